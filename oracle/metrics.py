"""Quality and byte-accounting metrics (reported, and used by the pins).

"5x Faster LLM Inference? ...", "Example 2: Manual Compression Pipeline":
compression ratio and cosine similarity statistics; "What is TurboQuant-GPU?":
2-bit keys + 1-bit QJL and 3-bit values, 5.02x against an FP16 cache at 0.98
cosine similarity.
"""

import math

import numpy as np


def reconstruct_keys_mse(ck, R, centroids, d):
    """k_hat = (n16 / sqrt(d)) R^T c[idx]  (codebook part only)."""
    chat = np.asarray(centroids)[ck["idx"]]
    return (ck["n16"].astype(np.float64) / math.sqrt(d))[:, None] * (chat @ R)


def reconstruct_keys_qjl(ck, R, S, centroids, d):
    """k_hat + the QJL residual estimate (n16/sqrt d) R^T (sqrt(pi/2)/m gamma16 S^T sigma)."""
    m = S.shape[0]
    chat = np.asarray(centroids)[ck["idx"]]
    sigma = 2.0 * ck["z"] - 1.0
    resid = (math.sqrt(math.pi / 2.0) / m) * ck["gamma16"].astype(np.float64)[:, None] * (sigma @ S)
    return (ck["n16"].astype(np.float64) / math.sqrt(d))[:, None] * ((chat + resid) @ R)


def reconstruct_values(cv, R, group):
    scale = np.repeat(cv["scale16"].astype(np.float64), group, axis=1)
    zero = np.repeat(cv["zero16"].astype(np.float64), group, axis=1)
    return (zero + scale * cv["codes"]) @ R


def reconstruct_values_mse(cv, R, centroids, d):
    """v_hat = (nv16 / sqrt(d)) R^T c[idx] for values coded like the keys' codebook part."""
    chat = np.asarray(centroids)[cv["codes"]]
    return (cv["n16"].astype(np.float64) / math.sqrt(d))[:, None] * (chat @ R)


def cosine_rows(a, b):
    num = np.sum(a * b, axis=-1)
    den = np.linalg.norm(a, axis=-1) * np.linalg.norm(b, axis=-1)
    return num / den


def record_bytes(d, k_bits, v_bits, group, m=None, value_mode="group"):
    """Bytes per (token, head): K codes + signs + 2 fp16 norms, V codes + fp16 scale/zero per
    group (or one fp16 norm with MSE values)."""
    m = d if m is None else m
    v_meta = 4 * (d // group) if value_mode == "group" else 2
    return d * k_bits // 8 + m // 8 + 4 + d * v_bits // 8 + v_meta


def compression_ratio(record, d=128, baseline_bits=16):
    """Against an uncompressed K+V cache of `baseline_bits` per element."""
    return 2 * d * baseline_bits / 8 / record
