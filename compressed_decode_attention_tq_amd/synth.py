"""Seeded synthetic workloads (inputs only -- no compression arithmetic here).

Both the library's tests/benchmarks and the reference oracle are fed from these
generators; nothing in this module quantises, rotates or attends.  The
workloads stand in for the pages' model KV caches (which need weights and
datasets): N(0,1) keys/values, optionally with a few outlier channels per head
scaled x10 (the outlier structure real K/V streams show), rounded to bf16
where the workload says bf16.
"""

import numpy as np

D = 128
PAGE = 16

# The five workloads.  Seeds: data 100+c, layer state 200+c, block table 300+c,
# mixed-bit allocation 405, ragged lengths 505.
WORKLOADS = {
    1: dict(name="tiny-parity", B=1, Hq=1, Hkv=1, ctx=1024, k_bits=2, v_bits=3, group=32,
            dtype="f32", outliers=0, table="identity"),
    2: dict(name="llama3-8b-decode-layer", B=16, Hq=32, Hkv=8, ctx=4096, k_bits=4, v_bits=4,
            group=32, dtype="bf16", outliers=4, table="identity"),
    3: dict(name="fused-compress", N=1 << 20, Hkv=8, k_bits=2, v_bits=3, group=32, dtype="bf16",
            outliers=0),
    4: dict(name="long-context-decode", B=1, Hq=32, Hkv=8, ctx=131072, k_bits=3, v_bits=2,
            group=32, dtype="bf16", outliers=4, table="random"),
    5: dict(name="ragged-mixed-bit-serving", B=64, Hq=32, Hkv=8, layers=32, min_len=512,
            max_len=32768, group=32, dtype="bf16", outliers=4, table="random"),
}


def seeds(c):
    return dict(data=100 + c, state=200 + c, table=300 + c, alloc=405, lens=505)


# ------------------------------------------------------------------ rounding
def bf16_bits(x):
    """float32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_to_f32(bits16):
    return (np.asarray(bits16, dtype=np.uint32) << 16).view(np.float32)


def bf16_round(x):
    return bf16_to_f32(bf16_bits(x))


# ------------------------------------------------------------------- host side
def outlier_channels(rng, n_heads, d, count):
    return np.stack([rng.choice(d, count, replace=False) for _ in range(n_heads)]) if count else None


def kv_host(seed, n_tokens, n_heads, d=D, outliers=0, dtype="bf16", factor=10.0):
    """K, V float32 arrays [n_tokens, n_heads, d]; values exactly representable in `dtype`."""
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((n_tokens, n_heads, d), dtype=np.float32)
    v = rng.standard_normal((n_tokens, n_heads, d), dtype=np.float32)
    ch = outlier_channels(rng, n_heads, d, outliers)
    if ch is not None:
        for h in range(n_heads):
            k[:, h, ch[h]] *= factor
            v[:, h, ch[h]] *= factor
    if dtype == "bf16":
        k, v = bf16_round(k), bf16_round(v)
    return k, v


def queries_host(seed, batch, n_q_heads, d=D, dtype="bf16"):
    rng = np.random.default_rng(seed + 7919)
    q = rng.standard_normal((batch, n_q_heads, d), dtype=np.float32)
    return bf16_round(q) if dtype == "bf16" else q


def block_table(seed, batch, blocks_per_seq, kind="identity"):
    """int32 [batch, blocks_per_seq] physical block ids, all distinct."""
    total = batch * blocks_per_seq
    if kind == "identity":
        ids = np.arange(total, dtype=np.int64)
    else:
        ids = np.random.default_rng(seed).permutation(total)
    return ids.reshape(batch, blocks_per_seq).astype(np.int32)


def slots_for(table, seq_len_of, positions_of):
    """Slots (block*16+offset) of token positions, per sequence."""
    out = []
    for b, pos in enumerate(positions_of):
        pos = np.asarray(pos, dtype=np.int64)
        out.append(table[b][pos // PAGE].astype(np.int64) * PAGE + pos % PAGE)
    return out


def ragged_lengths(seed, batch, lo, hi):
    return np.random.default_rng(seed).integers(lo, hi + 1, size=batch).astype(np.int32)


def mixed_bit_allocation(seed, layers=32, protect=2):
    """Per-layer (k_bits, v_bits), None for the protected (uncompressed bf16) layers.

    The middle layers get a seeded permutation of the fixed multiset
    {(4,4) x12, (4,3) x8, (3,3) x4, (3,2) x4}; with one QJL bit per key
    coordinate on top of k_bits, the mean of (k_bits + 1 + v_bits) / 2 over
    those 28 layers is exactly 4.0.
    """
    mid = layers - 2 * protect
    base = [(4, 4)] * 12 + [(4, 3)] * 8 + [(3, 3)] * 4 + [(3, 2)] * 4
    if mid != len(base):
        raise ValueError("the fixed allocation is defined for 28 compressed layers")
    perm = np.random.default_rng(seed).permutation(mid)
    alloc = [None] * layers
    for i, j in enumerate(perm):
        alloc[protect + i] = base[j]
    return alloc


# ----------------------------------------------------------------- device side
def kv_device(seed, n_tokens, n_heads, d=D, outliers=0, dtype="bf16", factor=10.0, device="cuda"):
    """Same recipe on the GPU with a seeded torch generator (for workloads too big for the host)."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)
    k = torch.randn((n_tokens, n_heads, d), generator=g, device=device, dtype=torch.float32)
    v = torch.randn((n_tokens, n_heads, d), generator=g, device=device, dtype=torch.float32)
    if outliers:
        ch = outlier_channels(np.random.default_rng(seed), n_heads, d, outliers)
        scale = torch.ones((n_heads, d), device=device)
        for h in range(n_heads):
            scale[h, torch.as_tensor(ch[h], device=device)] = factor
        k.mul_(scale)
        v.mul_(scale)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    return k.to(tdt), v.to(tdt)
