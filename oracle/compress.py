"""Key and value compression, float64, step by step.

Keys ("How 0xsero/turboquant works", "Compression Pipeline"; "turbo-attn
0.24.0", "How it works"; "5x Faster LLM Inference? ...", "Example 4:
Kernel-Level Operations": normalise -> rotate -> Lloyd-Max quantise -> pack,
plus a 1-bit QJL residual sign):
    n     = ||k||                                    stored as fp16
    t     = sqrt(d) * R k / n        (t = 0 if n = 0)
    idx_j = #{i : beta_i < t_j}                      b_k-bit codebook index
    rho   = t - c[idx]
    gamma = ||rho||                                  stored as fp16
    y     = S rho,   z_j = [y_j >= 0]                1 sign bit per coordinate
The code decisions use the unrounded n and gamma.

Key modes without the residual projection ("turbo-attn 0.24.0", "How it
works": normalise, store a single magnitude, quantise each rotated coordinate
to a shared codebook; "Configuration", TKV_K_NC: norm-correction of K reads):
    "mse"     the same n, t, idx; no residual signs (z = 0) and gamma = 0, so
              the decoder's QJL term vanishes and the score is the inner
              product with the codebook reconstruction (n/sqrt d) R^T c[idx]
    "mse_nc"  as "mse" with the stored magnitude n * sqrt(d) / ||c[idx]||: the
              reconstruction then has the key's own norm n (up to the fp16
              rounding of the stored value); the correction is folded into the
              stored magnitude, so the read path is the same for every mode

Values ("How 0xsero/turboquant works", "Value Compression": group
quantisation with per-group scale/zero; "tiny-turboquant 0.18.0",
"Measured quality": groups of 32 channels, each with its own scale/zero):
    v'     = R v                       (the same rotation as the head's keys)
    per group of G consecutive coordinates:
    scale  = fp16((max - min) / (2^b_v - 1)),   zero = fp16(min)
    code_j = clamp(round_half_even((v'_j - zero) / scale), 0, 2^b_v - 1)
             (code_j = 0 when scale == 0)
The codes are computed from the stored (fp16) scale and zero so that the
decoder's zero + scale * code is the nearest grid point.

Values coded like the keys' codebook part (value mode "mse"; "5x Faster LLM
Inference? ...", "What is TurboQuant-GPU?": 3-bit MSE values, and "Example 4:
Kernel-Level Operations": normalise -> rotate -> Lloyd-Max quantise -> pack for
both K and V), with the b_v-bit codebook of the same family:
    nv    = ||v||                                    stored as fp16
    t     = sqrt(d) * R v / nv       (t = 0 if nv = 0)
    idx_j = #{i : beta_i < t_j}
and the decoder's value is (nv16 / sqrt d) c[idx] in the rotated basis.
"""

import math

import numpy as np

from . import codebook, layout as lay


KEY_MODES = ("qjl", "mse", "mse_nc")
VALUE_MODES = ("group", "mse")


def compress_keys(K, R, S, centroids, boundaries, key_mode="qjl"):
    """K: [n, d] float64 (exact input values).  Returns a dict of per-vector arrays
    ("n16"/"gamma16" are what the store holds for the given key mode)."""
    if key_mode not in KEY_MODES:
        raise ValueError("unknown key mode %r" % (key_mode,))
    K = np.asarray(K, dtype=np.float64)
    d = K.shape[-1]
    n = np.sqrt(np.sum(K * K, axis=-1))
    rk = K @ R.T
    safe = np.where(n > 0.0, n, 1.0)
    t = np.where((n > 0.0)[:, None], (math.sqrt(d) / safe)[:, None] * rk, 0.0)
    idx = codebook.quantize_index(t, boundaries)
    chat = np.asarray(centroids)[idx]
    rho = t - chat
    if key_mode == "qjl":
        q = qjl_signs(t, idx, S, centroids)
        gamma, y, z = q["gamma"], q["y"], q["z"]
        n_store = n
    else:
        gamma = np.zeros_like(n)
        y = np.zeros_like(rho)
        z = np.zeros(rho.shape, dtype=np.int64)
        if key_mode == "mse":
            n_store = n
        else:
            # ||c[idx]|| > 0: the centroids of an even number of levels are all nonzero
            n_store = n * math.sqrt(d) / np.sqrt(np.sum(chat * chat, axis=-1))
    return {
        "n": n, "t": t, "idx": idx, "rho": rho, "gamma": gamma, "y": y, "z": z,
        "n16": n_store.astype(np.float16), "gamma16": gamma.astype(np.float16),
    }


def qjl_signs(t, idx, S, centroids):
    """The QJL step for given codebook decisions: rho = t - c[idx], gamma = ||rho||,
    y = S rho, z_j = [y_j >= 0] ("How 0xsero/turboquant works", "Compression
    Pipeline": the 1-bit sign sketch of the quantisation residual).  t: [n, d]
    standardised rotated coordinates, idx: [n, d] codes (any codes, not only the
    nearest ones: a checker uses it to recompute the signs that follow from codes
    taken elsewhere)."""
    rho = np.asarray(t, dtype=np.float64) - np.asarray(centroids, dtype=np.float64)[np.asarray(idx)]
    y = rho @ np.asarray(S, dtype=np.float64).T
    return {"rho": rho, "gamma": np.sqrt(np.sum(rho * rho, axis=-1)), "y": y, "z": (y >= 0.0).astype(np.int64)}


def quantize_groups(vrot, v_bits, group):
    """Group scale/zero quantisation of rotated values vrot: [n, d]."""
    n, d = vrot.shape
    g = vrot.reshape(n, d // group, group)
    mn = g.min(axis=-1)
    mx = g.max(axis=-1)
    top = (1 << v_bits) - 1
    scale16 = ((mx - mn) / top).astype(np.float16)
    zero16 = mn.astype(np.float16)
    s = scale16.astype(np.float64)[..., None]
    z = zero16.astype(np.float64)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.rint((g - z) / np.where(s > 0.0, s, 1.0))
    codes = np.where(s > 0.0, np.clip(q, 0, top), 0).astype(np.int64)
    return codes.reshape(n, d), scale16, zero16, mn, mx


def compress_values(V, R, v_bits, group):
    V = np.asarray(V, dtype=np.float64)
    vrot = V @ R.T
    codes, scale16, zero16, mn, mx = quantize_groups(vrot, v_bits, group)
    return {"vrot": vrot, "codes": codes, "scale16": scale16, "zero16": zero16, "mn": mn, "mx": mx}


def compress_values_mse(V, R, centroids, boundaries):
    """Values coded like the keys' codebook part: V [n, d] float64."""
    V = np.asarray(V, dtype=np.float64)
    d = V.shape[-1]
    n = np.sqrt(np.sum(V * V, axis=-1))
    vrot = V @ R.T
    safe = np.where(n > 0.0, n, 1.0)
    t = np.where((n > 0.0)[:, None], (math.sqrt(d) / safe)[:, None] * vrot, 0.0)
    idx = codebook.quantize_index(t, boundaries)
    return {"vrot": vrot, "n": n, "t": t, "codes": idx, "n16": n.astype(np.float16)}


def compress_into_pool(K, V, slots, pool, layout, state, keep=True):
    """Compress K, V [N, H_kv, d] (float64 values of the inputs) into `pool` at `slots` [N].

    Tokens with a negative slot are skipped.  `state` is an oracle.state.LayerState.
    Returns the per-head intermediate results ({head: (keys, values)}) if `keep`.
    """
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    slots = np.asarray(slots, dtype=np.int64)
    valid = slots >= 0
    K, V, slots = K[valid], V[valid], slots[valid]
    n_tok, H, d = K.shape
    value_mode = getattr(state, "value_mode", "group")
    if value_mode != layout.value_mode:
        raise ValueError("layer state (%s values) and layout (%s values) disagree" % (value_mode, layout.value_mode))
    if (getattr(state, "key_mode", "qjl") == "qjl") != layout.qjl:
        raise ValueError("layer state (%s keys) and layout (qjl=%s) disagree" % (state.key_mode, layout.qjl))
    out = {}
    for h in range(H):
        ck = compress_keys(K[:, h], state.R[h], state.S[h], state.centroids, state.boundaries,
                           getattr(state, "key_mode", "qjl"))
        rec = {"idx": ck["idx"], "z": ck["z"], "n16": ck["n16"], "g16": ck["gamma16"]}
        if value_mode == "mse":
            cv = compress_values_mse(V[:, h], state.R[h], state.v_centroids, state.v_boundaries)
            rec.update(vcode=cv["codes"], vn16=cv["n16"])
        else:
            cv = compress_values(V[:, h], state.R[h], layout.v_bits, layout.group)
            rec.update(vcode=cv["codes"], scale16=cv["scale16"], zero16=cv["zero16"])
        lay.put_records(pool, layout, H, slots, h, rec)
        if keep:
            out[h] = (ck, cv)
    return out


def store_bypass(K_bits16, V_bits16, slots, pool, layout, n_kv_heads):
    """Uncompressed layers: copy bf16 K, V bit patterns [N, H, d] into the pool."""
    slots = np.asarray(slots, dtype=np.int64)
    keep = slots >= 0
    Kb = np.asarray(K_bits16, np.uint16)[keep]
    Vb = np.asarray(V_bits16, np.uint16)[keep]
    blocks, offs = np.divmod(slots[keep], lay.P)
    for h in range(n_kv_heads):
        base = (blocks * n_kv_heads + h) * layout.block_bytes
        k_at, v_at = lay.bypass_byte_index(layout, base, offs)
        pool[k_at] = np.ascontiguousarray(Kb[:, h]).view(np.uint8).reshape(len(offs), -1)
        pool[v_at] = np.ascontiguousarray(Vb[:, h]).view(np.uint8).reshape(len(offs), -1)
