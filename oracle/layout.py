"""Paged compressed-KV store: byte layout of one layer's pool.

The pages describe a compressed store of packed records with norms
("turbo-attn 0.24.0", "Quickstart": compress_k returns packed codes and norms;
"How 0xsero/turboquant works", "Key Storage and Attention Scoring" and "Value
Compression": quantise/append records, per-group scale/zero metadata) living in
a paged KV cache with block tables ("How 0xsero/turboquant works", "vLLM
Integration and Cache Lifecycle").  The byte layout itself is not on the pages;
this is the format both the oracle and the library write and read:

  pool = uint8[num_blocks][n_kv_heads][block_bytes],  P = 16 tokens per block,
  slot = block * P + offset.

Inside one (block, head) region, five fields, each token-major:
  Kc  [P][d*k_bits/8]    key codebook indices, LSB-first bitstream
  Ks  [P][m/8]           QJL sign bits (bit j = 1 <=> y_j >= 0)
  Kn  [P][2] fp16        ||k|| then gamma = ||rho||   (little-endian)
  Vc  [P][d*v_bits/8]    value codes, LSB-first bitstream
  Vsz [P][d/G][2] fp16   per group: scale then zero
Bypass (uncompressed) layers: region = Kb [P][d] bf16 followed by Vb [P][d] bf16.
"""

import numpy as np

P = 16


class StoreLayout:
    def __init__(self, d=128, k_bits=4, v_bits=4, group=32, bypass=False, m=None):
        self.d, self.k_bits, self.v_bits, self.group, self.bypass = d, k_bits, v_bits, group, bypass
        self.m = d if m is None else m
        if bypass:
            self.kb_bytes = d * 2
            self.off_kb = 0
            self.off_vb = P * self.kb_bytes
            self.block_bytes = 2 * P * self.kb_bytes
            return
        self.kc_bytes = d * k_bits // 8
        self.ks_bytes = self.m // 8
        self.kn_bytes = 4
        self.vc_bytes = d * v_bits // 8
        self.vsz_bytes = 4 * (d // group)
        sizes = [self.kc_bytes, self.ks_bytes, self.kn_bytes, self.vc_bytes, self.vsz_bytes]
        offs, o = [], 0
        for s in sizes:
            offs.append(o)
            o += P * s
        self.off_kc, self.off_ks, self.off_kn, self.off_vc, self.off_vsz = offs
        self.block_bytes = o

    def field_offsets(self):
        if self.bypass:
            return [self.off_kb, self.off_vb]
        return [self.off_kc, self.off_ks, self.off_kn, self.off_vc, self.off_vsz]

    def record_bytes(self):
        """Bytes per (token, head), K and V together."""
        return self.block_bytes // P

    def region(self, n_kv_heads, slot, head):
        """Byte offset of the (block, head) region holding `slot`, and the in-block offset."""
        block, off = divmod(int(slot), P)
        return (block * n_kv_heads + head) * self.block_bytes, off


def new_pool(num_blocks, n_kv_heads, layout):
    return np.zeros(num_blocks * n_kv_heads * layout.block_bytes, dtype=np.uint8)


def _put(pool, at, data):
    data = np.asarray(data, dtype=np.uint8).ravel()
    pool[at: at + data.size] = data


def _get(pool, at, n):
    return pool[at: at + n]


def f16_bytes(values):
    return np.asarray(values, dtype=np.float16).view(np.uint8)


def write_compressed(pool, layout, n_kv_heads, slot, head, kc, ks, n16, g16, vc, scale16, zero16):
    """Store one compressed (token, head) record.  kc/ks/vc are packed bytes."""
    base, o = layout.region(n_kv_heads, slot, head)
    _put(pool, base + layout.off_kc + o * layout.kc_bytes, kc)
    _put(pool, base + layout.off_ks + o * layout.ks_bytes, ks)
    _put(pool, base + layout.off_kn + o * layout.kn_bytes, f16_bytes([n16, g16]))
    _put(pool, base + layout.off_vc + o * layout.vc_bytes, vc)
    sz = np.stack([np.asarray(scale16, np.float16), np.asarray(zero16, np.float16)], axis=-1)
    _put(pool, base + layout.off_vsz + o * layout.vsz_bytes, sz.view(np.uint8))


def read_compressed(pool, layout, n_kv_heads, slot, head):
    """Return the raw fields of one record: (kc, ks, n16, g16, vc, scale16, zero16)."""
    base, o = layout.region(n_kv_heads, slot, head)
    kc = _get(pool, base + layout.off_kc + o * layout.kc_bytes, layout.kc_bytes)
    ks = _get(pool, base + layout.off_ks + o * layout.ks_bytes, layout.ks_bytes)
    kn = _get(pool, base + layout.off_kn + o * layout.kn_bytes, 4).view(np.float16).astype(np.float64)
    vc = _get(pool, base + layout.off_vc + o * layout.vc_bytes, layout.vc_bytes)
    sz = _get(pool, base + layout.off_vsz + o * layout.vsz_bytes, layout.vsz_bytes)
    sz = sz.view(np.float16).astype(np.float64).reshape(-1, 2)
    return kc, ks, kn[0], kn[1], vc, sz[:, 0], sz[:, 1]


def write_bypass(pool, layout, n_kv_heads, slot, head, k_bf16_bits, v_bf16_bits):
    """Store raw bf16 K and V (given as uint16 bit patterns) of one (token, head)."""
    base, o = layout.region(n_kv_heads, slot, head)
    _put(pool, base + layout.off_kb + o * layout.kb_bytes, np.asarray(k_bf16_bits, np.uint16).view(np.uint8))
    _put(pool, base + layout.off_vb + o * layout.kb_bytes, np.asarray(v_bf16_bits, np.uint16).view(np.uint8))


def bf16_bits_to_f64(bits16):
    b = np.asarray(bits16, dtype=np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def read_bypass(pool, layout, n_kv_heads, slot, head):
    base, o = layout.region(n_kv_heads, slot, head)
    k = _get(pool, base + layout.off_kb + o * layout.kb_bytes, layout.kb_bytes).view(np.uint16)
    v = _get(pool, base + layout.off_vb + o * layout.kb_bytes, layout.kb_bytes).view(np.uint16)
    return bf16_bits_to_f64(k), bf16_bits_to_f64(v)
