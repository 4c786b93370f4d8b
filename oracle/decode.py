"""Paged decode attention over the compressed store, float64.

"turbo-attn 0.24.0", "How it works": an orthogonal rotation applied to the
keys, the values and the query leaves attention unchanged, so the query is
rotated once per step and the scores, softmax and value sum are formed on the
rotated, compressed store in a single kernel.  "How 0xsero/turboquant works",
"Key Storage and Attention Scoring": the scores use only the compressed keys.  "turbo-attn 0.24.0",
"Configuration" (TKV_DECODE_SPLITS) and "tiny-turboquant 0.18.0", "Fused
decode-attention path": the context is split, partial results combined.

For query head h of sequence b, KV head g = h // (H_q / H_kv):
    q' = R_g q,   u = S_g q'
    token i < seq_len_b lives at slot block_table[b][i // 16] * 16 + i % 16
    s_i = tau * (n16_i / sqrt(d)) * ( q' . c[idx_i]  +  kappa * gamma16_i * (u . sigma_i) )
          sigma_ij = 2 z_ij - 1,   kappa = sqrt(pi/2) / m,   tau = 1/sqrt(d) by default
    p   = softmax(s)
    o'  = sum_i p_i * vhat'_i,     vhat'_ij = zero16_{i,g(j)} + scale16_{i,g(j)} * code_ij
                                   (with MSE values: vhat'_i = (nv16_i / sqrt d) c_v[code_i])
    out = R_g^T o'
The QJL term is the estimator <rho, q'> ~ ||rho|| sqrt(pi/2)/m <S q', sign(S rho)>
of the residual's inner product (QJL / TurboQuant, cited by the pages).
seq_len = 0 gives a zero output.
"""

import math

import numpy as np

from . import layout as lay


def gather(pool, layout, n_kv_heads, block_table_row, seq_len, head):
    """Raw fields of tokens 0..seq_len-1 of one sequence for one KV head."""
    i = np.arange(seq_len)
    blocks = np.asarray(block_table_row, dtype=np.int64)[i // lay.P]
    offs = i % lay.P
    base = (blocks * n_kv_heads + head) * layout.block_bytes

    def field(off, nbytes):
        idx = (base + off + offs * nbytes)[:, None] + np.arange(nbytes)
        return pool[idx]

    if layout.bypass:
        k_at, v_at = lay.bypass_byte_index(layout, base, offs)
        kb = np.ascontiguousarray(pool[k_at]).view(np.uint16)
        vb = np.ascontiguousarray(pool[v_at]).view(np.uint16)
        return {"k": lay.bf16_bits_to_f64(kb), "v": lay.bf16_bits_to_f64(vb)}
    slots = blocks * lay.P + offs
    r = lay.get_records(pool, layout, n_kv_heads, slots, head)
    for k in ("n16", "g16", "scale16", "zero16", "vn16"):
        if k in r:
            r[k] = r[k].astype(np.float64)
    return r


def value_rows(f, layout, state):
    """The gathered tokens' values in the rotated basis (group grid or MSE codebook)."""
    if layout.value_mode == "mse":
        return (f["vn16"] / math.sqrt(layout.d))[:, None] * np.asarray(state.v_centroids)[f["vcode"]]
    return dequant_values(f, layout.group)


def dequant_values(f, group):
    """vhat'[T, d] = zero + scale * code, per group."""
    T, d = f["vcode"].shape
    scale = np.repeat(f["scale16"], group, axis=1)
    zero = np.repeat(f["zero16"], group, axis=1)
    return zero + scale * f["vcode"]


def token_scores(qp, u, f, centroids, d, m, tau):
    chat = np.asarray(centroids)[f["idx"]]
    sigma = 2.0 * f["z"] - 1.0
    kappa = math.sqrt(math.pi / 2.0) / m
    return tau * (f["n16"] / math.sqrt(d)) * (chat @ qp + kappa * f["g16"] * (sigma @ u))


def _softmax_weighted_sum(s, vals):
    p = np.exp(s - np.max(s))
    return (p @ vals) / np.sum(p)


def _split_partials(s, vals, split_tokens):
    parts = []
    for start in range(0, len(s), split_tokens):
        ss = s[start: start + split_tokens]
        mx = np.max(ss)
        p = np.exp(ss - mx)
        parts.append((mx, np.sum(p), p @ vals[start: start + split_tokens]))
    return parts


def _combine(parts):
    m = max(pt[0] for pt in parts)
    num = sum(math.exp(pt[0] - m) * pt[2] for pt in parts)
    den = sum(math.exp(pt[0] - m) * pt[1] for pt in parts)
    return num / den


def decode(q, pool, layout, n_kv_heads, block_table, seq_lens, state=None,
           softmax_scale=None, split_tokens=None):
    """q: [B, H_q, d] float64 values.  Returns out [B, H_q, d] float64.

    split_tokens=None: one pass over all tokens; otherwise split-K partials of
    that many tokens each, merged with the running-max rescaling.
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hq, d = q.shape
    rep = Hq // n_kv_heads
    tau = 1.0 / math.sqrt(d) if not softmax_scale else softmax_scale
    out = np.zeros((B, Hq, d))
    for b in range(B):
        T = int(seq_lens[b])
        if T == 0:
            continue
        for g in range(n_kv_heads):
            f = gather(pool, layout, n_kv_heads, block_table[b], T, g)
            if layout.bypass:
                vals = f["v"]
            else:
                vals = value_rows(f, layout, state)
            for h in range(g * rep, (g + 1) * rep):
                if layout.bypass:
                    s = tau * (f["k"] @ q[b, h])
                else:
                    qp = state.R[g] @ q[b, h]
                    u = state.S[g] @ qp
                    s = token_scores(qp, u, f, state.centroids, d, layout.m, tau)
                if split_tokens is None:
                    o = _softmax_weighted_sum(s, vals)
                else:
                    o = _combine(_split_partials(s, vals, split_tokens))
                out[b, h] = o if layout.bypass else state.R[g].T @ o
    return out
