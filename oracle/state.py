"""Per-(layer, KV head) rotation R and QJL projection S.

R: a Haar-random orthogonal d x d matrix ("How 0xsero/turboquant works",
"Compression Pipeline": random orthogonal rotation; "5x Faster LLM
Inference? ...", "What is TurboQuant-GPU?": random orthogonal rotation makes the
coordinates approximately Gaussian).  Drawn as in Mezzadri, "How to generate
random matrices from the classical compact groups" (2007): QR-factorise a
matrix of i.i.d. N(0,1) entries (filled row-major from the rotation stream)
and multiply column j of Q by the sign of R_jj (sign(0) taken as +1), which
makes the factor unique and Haar distributed.

S: an m x d matrix of i.i.d. N(0,1) entries from the projection stream, m = d
(the QJL residual-sign projection of the same sections).

Structured alternative ("turbo-attn 0.24.0", "How it works": there the KV
rotation is a fast Walsh-Hadamard transform): R = H D / sqrt(d), H the
Sylvester-ordered Hadamard matrix, H[i][j] = (-1)^popcount(i & j), and D a
diagonal of random signs from the tag-3 stream (a randomised Hadamard
transform).  Every entry of R is +-1/sqrt(d).

Both are stored, and used by every consumer, as float32-rounded values; the
oracle then computes in float64 on exactly those numbers.

Codebook state: the Lloyd-Max centroids (solved in float64) are stored rounded
to float16, and the decision boundaries are the exact midpoints of the stored
centroids (exactly representable in float32).  Compression and decode both use
these stored values, so the quantiser and the estimator see the same codebook.
"""

import numpy as np

from . import rng


def gaussian_matrix(seed, layer, head, tag, rows, cols):
    vals = rng.gaussians(seed, layer, head, tag, rows * cols)
    return np.array(vals, dtype=np.float64).reshape(rows, cols)


def haar_rotation_f64(seed, layer, head, d):
    g = gaussian_matrix(seed, layer, head, rng.TAG_ROTATION, d, d)
    q, r = np.linalg.qr(g)
    signs = np.where(np.diag(r) < 0.0, -1.0, 1.0)
    return q * signs[None, :]


def haar_rotation(seed, layer, head, d):
    """float32-rounded Haar rotation, returned as float64 values."""
    return haar_rotation_f64(seed, layer, head, d).astype(np.float32).astype(np.float64)


def sylvester_hadamard(d):
    """H[i][j] = (-1)^popcount(i & j) for d a power of two."""
    i = np.arange(d)
    bits = np.bitwise_and(i[:, None], i[None, :])
    par = np.zeros_like(bits)
    while bits.any():
        par ^= bits & 1
        bits >>= 1
    return np.where(par == 1, -1.0, 1.0)


def hadamard_rotation(seed, layer, head, d):
    """float32-rounded randomised Hadamard rotation H D / sqrt(d), as float64 values."""
    signs = np.array(rng.random_signs(seed, layer, head, d))
    r = sylvester_hadamard(d) * signs[None, :] / np.sqrt(d)
    return r.astype(np.float32).astype(np.float64)


ROTATIONS = ("haar", "hadamard")


def rotation(kind, seed, layer, head, d):
    if kind == "haar":
        return haar_rotation(seed, layer, head, d)
    if kind == "hadamard":
        return hadamard_rotation(seed, layer, head, d)
    raise ValueError("unknown rotation %r" % (kind,))


def qjl_projection(seed, layer, head, d, m=None):
    m = d if m is None else m
    s = gaussian_matrix(seed, layer, head, rng.TAG_PROJECTION, m, d)
    return s.astype(np.float32).astype(np.float64)


class LayerState:
    """All state of one compressed layer: R and S per KV head plus the key codebook
    (and, with MSE values, the b_v-bit value codebook of the same family)."""

    def __init__(self, seed, layer, n_kv_heads, d, k_bits, v_bits, group, dist="gaussian", key_mode="qjl",
                 rotation_kind="haar", value_mode="group"):
        self.seed, self.layer, self.n_kv_heads, self.d = seed, layer, n_kv_heads, d
        self.k_bits, self.v_bits, self.group, self.dist = k_bits, v_bits, group, dist
        self.key_mode = key_mode  # "qjl", "mse" or "mse_nc" (see compress.compress_keys)
        self.rotation_kind = rotation_kind  # "haar" or "hadamard"
        self.R = np.stack([rotation(rotation_kind, seed, layer, h, d) for h in range(n_kv_heads)])
        self.S = np.stack([qjl_projection(seed, layer, h, d) for h in range(n_kv_heads)])
        self.centroids, self.boundaries = stored_codebook(k_bits, dist, d)
        if value_mode not in ("group", "mse"):
            raise ValueError("unknown value mode %r" % (value_mode,))
        self.value_mode = value_mode
        if value_mode == "mse":
            self.v_centroids, self.v_boundaries = stored_codebook(v_bits, dist, d)


def stored_codebook(bits, dist="gaussian", d=128):
    """float16-rounded Lloyd-Max centroids and the midpoints between them (float64 values)."""
    from . import codebook

    c64, _, _ = codebook.lloyd_max(bits, dist, d)
    c16 = c64.astype(np.float16).astype(np.float64)
    return c16, 0.5 * (c16[:-1] + c16[1:])
