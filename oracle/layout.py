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

Inside one (block, head) region (a "page"), five fields.  All bit packing is
LSB-first: element i of a b-bit stream occupies bits [b*i, b*i + b) of the
stream, bit k of the stream being bit k%8 of byte k//8.
  Kc  [d/32][P][4*k_bits]  key codebook indices: for each 32-dim block j and
                           token t, the b-bit stream of dims 32j .. 32j+31
  Ks  [m/32][P][4]         QJL sign bits (bit = 1 <=> y >= 0), same blocking
  Kn  [P][2] fp16          ||k|| then gamma = ||rho||   (little-endian)
  Vc  [2P][d/2] x v_bits   value codes in 32 lane blocks: for dim = 16i + c
                           and token t = 8h + k, block 16h + c, group
                           2i + k//4 of four codes, element k % 4; one b-bit
                           stream in the order (block, group, element)
  Vsz [P][d/G][2] fp16     per group: scale then zero
With MSE values (value_mode "mse": values coded like the keys' codebook part,
"5x Faster LLM Inference? ...", "What is TurboQuant-GPU?") Vc holds b_v-bit
codebook indices in the same stream order and the last field is
  Vn  [P] fp16             ||v||
so that K2 + QJL / V3 is 102 bytes per (token, head) and 1632 per page.
Key modes without the QJL residual signs ("turbo-attn 0.24.0", "How it works":
one magnitude and the shared-codebook codes per key) store neither the sign
field nor gamma: Ks has 0 bytes (its offset is Kn's) and
  Kn  [P] fp16             the stored magnitude only
so that K4 / V4 is 146 bytes per (token, head) instead of 164.
Bypass (uncompressed) layers: region = Kb [P][d] bf16 (token-major: one token's
d keys together) followed by Vb [d][P] bf16 (dim-major: the P tokens' values of
one dim together), so that a page's values load as the matrix-core operand of
P.V with one contiguous run per lane.
"""

import numpy as np

P = 16
VALUE_MODES = ("group", "mse")


class StoreLayout:
    def __init__(self, d=128, k_bits=4, v_bits=4, group=32, bypass=False, m=None, value_mode="group", qjl=True):
        if value_mode not in VALUE_MODES:
            raise ValueError("unknown value mode %r" % (value_mode,))
        self.d, self.k_bits, self.v_bits, self.group, self.bypass = d, k_bits, v_bits, group, bypass
        self.value_mode = value_mode
        self.qjl = bool(qjl)  # False: key modes without residual signs (no Ks field, no gamma)
        self.m = d if m is None else m
        if bypass:
            self.kb_bytes = d * 2
            self.off_kb = 0
            self.off_vb = P * self.kb_bytes
            self.block_bytes = 2 * P * self.kb_bytes
            return
        self.kc_bytes = d * k_bits // 8
        self.ks_bytes = self.m // 8 if self.qjl else 0
        self.kn_bytes = 4 if self.qjl else 2
        self.vc_bytes = d * v_bits // 8
        # the last field: group scale/zero, or one fp16 norm with MSE values
        self.vsz_bytes = 4 * (d // group) if value_mode == "group" else 2
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


def f16_bytes(values):
    return np.asarray(values, dtype=np.float16).view(np.uint8)


def _bit_read(pool, bitpos, nbits):
    """Unsigned ints from LSB-first bit fields starting at absolute bit positions."""
    bitpos = np.asarray(bitpos, dtype=np.int64)
    k = bitpos[..., None] + np.arange(nbits)
    b = (pool[k // 8] >> (k % 8).astype(np.uint8)) & 1
    return np.sum(b.astype(np.int64) << np.arange(nbits), axis=-1)


def _bit_write(pool, bitpos, nbits, values):
    """Write LSB-first bit fields (duplicate bytes across fields handled exactly)."""
    bitpos = np.asarray(bitpos, dtype=np.int64)
    values = np.broadcast_to(np.asarray(values, dtype=np.int64), bitpos.shape)
    k = (bitpos[..., None] + np.arange(nbits)).ravel()
    v = ((values[..., None] >> np.arange(nbits)) & 1).ravel().astype(np.uint8)
    byte, bit = k // 8, (k % 8).astype(np.uint8)
    np.bitwise_and.at(pool, byte, np.uint8(0xFF) ^ (np.uint8(1) << bit))
    np.bitwise_or.at(pool, byte, v << bit)


def _field_bits(layout, base, offs, name):
    """Absolute bit positions [N, n] of every element of one field of tokens (base, offs)."""
    base = np.asarray(base, dtype=np.int64)[:, None]
    offs = np.asarray(offs, dtype=np.int64)[:, None]
    if name == "idx":      # [N, d]: block j = dim // 32, element dim % 32 within the block's stream
        dim = np.arange(layout.d)[None, :]
        rec = (dim // 32) * P + offs
        return (base + layout.off_kc) * 8 + rec * (32 * layout.k_bits) + (dim % 32) * layout.k_bits
    if name == "z":        # [N, m]
        if not layout.qjl:
            raise KeyError("no sign field in a layout without QJL")
        j = np.arange(layout.m)[None, :]
        rec = (j // 32) * P + offs
        return (base + layout.off_ks) * 8 + rec * 32 + (j % 32)
    if name == "vcode":    # [N, d]: lane blocks of 8 tokens x 16-dim tiles
        dim = np.arange(layout.d)[None, :]
        i, c = dim // 16, dim % 16
        h, k = offs // 8, offs % 8
        block = 16 * h + c
        group = 2 * i + k // 4
        elem = (block * (layout.d // 16) * 2 + group) * 4 + k % 4
        return (base + layout.off_vc) * 8 + elem * layout.v_bits
    raise KeyError(name)


def put_records(pool, layout, n_kv_heads, slots, head, rec):
    """Store compressed records of one KV head at `slots`.

    rec: idx [N, d] and z [N, m] (ints), n16, g16 [N] (float16),
    vcode [N, d] (ints), scale16, zero16 [N, d/G] (float16); with MSE values
    vn16 [N] (float16) in place of scale16 and zero16.  A layout without QJL
    stores n16 only (z and g16 must then be zero).
    """
    slots = np.asarray(slots, dtype=np.int64)
    if slots.size == 0:  # no tokens: nothing to store
        return
    blocks, offs = np.divmod(slots, P)
    base = (blocks * n_kv_heads + head) * layout.block_bytes
    _bit_write(pool, _field_bits(layout, base, offs, "idx"), layout.k_bits, rec["idx"])
    if layout.qjl:
        _bit_write(pool, _field_bits(layout, base, offs, "z"), 1, rec["z"])
        kn = np.stack([np.asarray(rec["n16"], np.float16), np.asarray(rec["g16"], np.float16)], axis=-1)
    else:
        if np.any(np.asarray(rec["z"])) or np.any(np.asarray(rec["g16"], np.float64)):
            raise ValueError("a layout without QJL holds no residual signs or gamma")
        kn = np.asarray(rec["n16"], np.float16).reshape(len(slots), 1)
    _bit_write(pool, _field_bits(layout, base, offs, "vcode"), layout.v_bits, rec["vcode"])
    at = (base + layout.off_kn + offs * layout.kn_bytes)[:, None] + np.arange(layout.kn_bytes)
    pool[at] = np.ascontiguousarray(kn).view(np.uint8).reshape(len(slots), layout.kn_bytes)
    if layout.value_mode == "mse":
        sz = np.asarray(rec["vn16"], np.float16).reshape(len(slots), 1)
    else:
        sz = np.stack([np.asarray(rec["scale16"], np.float16), np.asarray(rec["zero16"], np.float16)], axis=-1)
    at = (base + layout.off_vsz + offs * layout.vsz_bytes)[:, None] + np.arange(layout.vsz_bytes)
    pool[at] = np.ascontiguousarray(sz.reshape(len(slots), -1)).view(np.uint8)


def get_records(pool, layout, n_kv_heads, slots, head):
    """Read the compressed records of one KV head at `slots` (fields as in put_records;
    n16, g16, scale16, zero16 or vn16 returned as float16)."""
    slots = np.asarray(slots, dtype=np.int64)
    blocks, offs = np.divmod(slots, P)
    base = (blocks * n_kv_heads + head) * layout.block_bytes
    kn = pool[(base + layout.off_kn + offs * layout.kn_bytes)[:, None] + np.arange(layout.kn_bytes)]
    kn = np.ascontiguousarray(kn).view(np.float16).reshape(len(slots), layout.kn_bytes // 2)
    sz = pool[(base + layout.off_vsz + offs * layout.vsz_bytes)[:, None] + np.arange(layout.vsz_bytes)]
    out = {
        "idx": _bit_read(pool, _field_bits(layout, base, offs, "idx"), layout.k_bits),
        "n16": kn[:, 0],
        "vcode": _bit_read(pool, _field_bits(layout, base, offs, "vcode"), layout.v_bits),
    }
    if layout.qjl:
        out["z"] = _bit_read(pool, _field_bits(layout, base, offs, "z"), 1)
        out["g16"] = kn[:, 1]
    else:  # no residual signs: the decoder's QJL term is zero
        out["z"] = np.zeros((len(slots), layout.m), dtype=np.int64)
        out["g16"] = np.zeros(len(slots), dtype=np.float16)
    if layout.value_mode == "mse":
        out["vn16"] = np.ascontiguousarray(sz).view(np.float16).reshape(len(slots))
    else:
        sz = np.ascontiguousarray(sz).view(np.float16).reshape(len(slots), layout.vsz_bytes // 4, 2)
        out["scale16"], out["zero16"] = sz[:, :, 0], sz[:, :, 1]
    return out


def bypass_byte_index(layout, base, offs):
    """Byte positions of the keys and of the values of tokens at in-page offsets
    `offs` [N] in the pages starting at `base` [N]: two [N, 2d] index arrays, bf16
    element e of a token at columns 2e (low byte) and 2e + 1."""
    base = np.asarray(base, dtype=np.int64)[:, None]
    offs = np.asarray(offs, dtype=np.int64)[:, None]
    byte = np.arange(2 * layout.d)
    k_at = base + layout.off_kb + offs * layout.kb_bytes + byte
    # value element e of token t: row e of the dim-major table, column t
    v_at = base + layout.off_vb + (byte // 2) * (2 * P) + 2 * offs + byte % 2
    return k_at, v_at


def write_bypass(pool, layout, n_kv_heads, slot, head, k_bf16_bits, v_bf16_bits):
    """Store raw bf16 K and V (given as uint16 bit patterns) of one (token, head)."""
    base, o = layout.region(n_kv_heads, slot, head)
    k_at, v_at = bypass_byte_index(layout, [base], [o])
    pool[k_at[0]] = np.asarray(k_bf16_bits, np.uint16).view(np.uint8)
    pool[v_at[0]] = np.asarray(v_bf16_bits, np.uint16).view(np.uint8)


def bf16_bits_to_f64(bits16):
    b = np.asarray(bits16, dtype=np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def read_bypass(pool, layout, n_kv_heads, slot, head):
    base, o = layout.region(n_kv_heads, slot, head)
    k_at, v_at = bypass_byte_index(layout, [base], [o])
    k = np.ascontiguousarray(pool[k_at[0]]).view(np.uint16)
    v = np.ascontiguousarray(pool[v_at[0]]).view(np.uint16)
    return bf16_bits_to_f64(k), bf16_bits_to_f64(v)
