"""Reconstruction of keys and values from the compressed store, float64.

"turbo-attn 0.24.0", "How it works": a decompress path hands the cache to an
ordinary attention kernel; "tiny-turboquant 0.18.0", "Fused decode-attention
path": the codec is also used by decompressing to a dense buffer.  The
reconstruction is the one whose plain attention equals the decode's estimator:
for token i of KV head g,
    khat_i = (n16_i / sqrt d) R_g^T ( c[idx_i] + kappa * gamma16_i * S_g^T sigma_i ),
             sigma_ij = 2 z_ij - 1,  kappa = sqrt(pi/2) / m
    vhat_i = R_g^T ( zero16 + scale16 * code_i )          (per 32-wide group)
             or (nv16_i / sqrt d) R_g^T c_v[code_i]       (MSE values)
so q . khat_i = (n16_i / sqrt d) ( q'.c[idx_i] + kappa gamma16_i (S_g q').sigma_i )
with q' = R_g q, the score of "How 0xsero/turboquant works", "Key Storage and
Attention Scoring" before the softmax scale.  Without QJL (gamma16 = 0) khat is
the codebook reconstruction.  Bypass pages hold the bf16 values themselves.
"""

import math

import numpy as np

from . import layout as lay


def decompress(pool, layout, n_kv_heads, slots, state=None):
    """K, V [n, H, d] float64 for the tokens at `slots` [n] (negative: zero rows)."""
    slots = np.asarray(slots, dtype=np.int64)
    n, d = len(slots), layout.d
    K = np.zeros((n, n_kv_heads, d))
    V = np.zeros((n, n_kv_heads, d))
    keep = slots >= 0
    sl = slots[keep]
    if not len(sl):
        return K, V
    blocks, offs = np.divmod(sl, lay.P)
    for g in range(n_kv_heads):
        if layout.bypass:
            base = (blocks * n_kv_heads + g) * layout.block_bytes
            k_at, v_at = lay.bypass_byte_index(layout, base, offs)
            kb = np.ascontiguousarray(pool[k_at]).view(np.uint16)
            vb = np.ascontiguousarray(pool[v_at]).view(np.uint16)
            K[keep, g] = lay.bf16_bits_to_f64(kb)
            V[keep, g] = lay.bf16_bits_to_f64(vb)
            continue
        r = lay.get_records(pool, layout, n_kv_heads, sl, g)
        n16 = r["n16"].astype(np.float64)
        g16 = r["g16"].astype(np.float64)
        chat = np.asarray(state.centroids)[r["idx"]]
        sigma = 2.0 * r["z"] - 1.0
        kappa = math.sqrt(math.pi / 2.0) / state.S[g].shape[0]
        inner = chat + kappa * g16[:, None] * (sigma @ state.S[g])
        K[keep, g] = (n16 / math.sqrt(d))[:, None] * (inner @ state.R[g])
        if layout.value_mode == "mse":
            vn16 = r["vn16"].astype(np.float64)
            V[keep, g] = (vn16 / math.sqrt(d))[:, None] * (np.asarray(state.v_centroids)[r["vcode"]] @ state.R[g])
        else:
            scale = np.repeat(r["scale16"].astype(np.float64), layout.group, axis=1)
            zero = np.repeat(r["zero16"].astype(np.float64), layout.group, axis=1)
            V[keep, g] = (zero + scale * r["vcode"]) @ state.R[g]
    return K, V
