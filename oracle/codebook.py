"""Lloyd-Max scalar codebooks for the standardised rotated coordinates.

"How 0xsero/turboquant works", "Compression Pipeline": keys are quantised with
a Lloyd-Max scalar codebook, precomputed per (dimension, bit width).  "5x
Faster LLM Inference? ...", "What is TurboQuant-GPU?": Lloyd-Max quantisation
is MSE-optimal for Gaussian sources, and rotation makes coordinates
approximately Gaussian.  "tiny-turboquant 0.18.0", "The algorithm in three
lines", and its "References": the exact marginal of a rotated unit vector is a
(scaled) Beta law.

Units: the key coordinate t_j = sqrt(d) (R k)_j / ||k|| (unit variance).
  dist="gaussian": t_j ~ N(0, 1).
  dist="sphere":   t_j = sqrt(d) u_j with u uniform on the unit sphere S^{d-1};
                   (1 + u_j)/2 ~ Beta((d-1)/2, (d-1)/2).

Lloyd's algorithm (Lloyd 1957 / Max 1960) with L = 2**bits levels:
  boundaries  beta_i = (c_i + c_{i+1}) / 2                         (nearest neighbour)
  centroids   c_i = E[x | beta_{i-1} < x <= beta_i]                (centroid condition)
iterated from the quantile midpoints F^-1((i + 1/2) / L) until
max |c_new - c_old| < tol.  Both densities are even, so each iterate is
symmetrised (c_i = -c_{L-1-i}); the middle boundary is then exactly 0.
Cell probabilities and moments are evaluated in closed form (Gaussian: erfc and the density; sphere: the regularised
incomplete beta function and the closed-form first moment).
"""

import math

import numpy as np
from scipy import special

SQRT2 = math.sqrt(2.0)
INV_SQRT_2PI = 1.0 / math.sqrt(2.0 * math.pi)


# ----------------------------------------------------------------- Gaussian
def _phi(x):
    if math.isinf(x):
        return 0.0
    return INV_SQRT_2PI * math.exp(-0.5 * x * x)


def _cell_prob_gauss(a, b):
    # P(a < X <= b); use the upper tail on the right half to avoid cancellation.
    if a >= 0.0:
        return 0.5 * math.erfc(a / SQRT2) - 0.5 * math.erfc(b / SQRT2)
    return 0.5 * math.erfc(-b / SQRT2) - 0.5 * math.erfc(-a / SQRT2)


def _cell_moments_gauss(a, b):
    """(P, int x f, int x^2 f) over (a, b]."""
    p = _cell_prob_gauss(a, b)
    m1 = _phi(a) - _phi(b)
    xa = 0.0 if math.isinf(a) else a * _phi(a)
    xb = 0.0 if math.isinf(b) else b * _phi(b)
    m2 = p - (xb - xa)
    return p, m1, m2


# ------------------------------------------------------------------- sphere
def _sphere_cdf(x, d):
    lim = math.sqrt(d)
    if x <= -lim:
        return 0.0
    if x >= lim:
        return 1.0
    a = 0.5 * (d - 1)
    return float(special.betainc(a, a, 0.5 * (1.0 + x / lim)))


def _cell_moments_sphere(a, b, d):
    lim = math.sqrt(d)
    a = max(a, -lim)
    b = min(b, lim)
    alpha = 0.5 * (d - 3)
    p = _sphere_cdf(b, d) - _sphere_cdf(a, d)
    # f(x) = C (1 - x^2/d)^alpha on [-sqrt d, sqrt d], C = 1 / (sqrt(d) B(1/2, alpha+1))
    c_norm = 1.0 / (lim * math.exp(special.betaln(0.5, alpha + 1.0)))
    g = lambda x: max(0.0, 1.0 - x * x / d) ** (alpha + 1.0)  # noqa: E731
    m1 = c_norm * d / (2.0 * (alpha + 1.0)) * (g(a) - g(b))
    # int x^2 f_d = d P_d - (d - 1) P_{d+2} over the same u-interval
    p_d2 = _sphere_cdf(b * math.sqrt((d + 2) / d), d + 2) - _sphere_cdf(a * math.sqrt((d + 2) / d), d + 2)
    m2 = d * p - (d - 1) * p_d2
    return p, m1, m2


# ---------------------------------------------------------------- Lloyd-Max
def _moments(a, b, dist, d):
    if dist == "gaussian":
        return _cell_moments_gauss(a, b)
    if dist == "sphere":
        return _cell_moments_sphere(a, b, d)
    raise ValueError("dist must be 'gaussian' or 'sphere'")


def _initial(levels, dist, d):
    q = special.ndtri((np.arange(levels) + 0.5) / levels)
    if dist == "sphere":
        q = np.clip(q, -0.9 * math.sqrt(d), 0.9 * math.sqrt(d))
    return q.astype(np.float64)


def lloyd_max(bits, dist="gaussian", dim=128, tol=1e-14, max_iter=200000):
    """Return (centroids[L], boundaries[L-1], mse) in float64, ascending."""
    if bits < 1 or bits > 8:
        raise ValueError("bits must be in 1..8")
    if dist == "sphere" and dim < 3:
        raise ValueError("sphere codebook needs dim >= 3")
    levels = 1 << bits
    c = _initial(levels, dist, dim)
    for _ in range(max_iter):
        bnd = 0.5 * (c[:-1] + c[1:])
        edges = [-math.inf] + list(bnd) + [math.inf]
        new = np.empty_like(c)
        for i in range(levels):
            p, m1, _ = _moments(edges[i], edges[i + 1], dist, dim)
            new[i] = m1 / p
        new = 0.5 * (new - new[::-1])          # both densities are symmetric about 0
        delta = float(np.max(np.abs(new - c)))
        c = new
        if delta < tol:
            break
    bnd = 0.5 * (c[:-1] + c[1:])
    return c, bnd, distortion(c, bnd, dist, dim)


def distortion(centroids, boundaries, dist="gaussian", dim=128):
    """E[(x - Q(x))^2] for the quantiser (centroids, boundaries)."""
    edges = [-math.inf] + list(boundaries) + [math.inf]
    total = 0.0
    for i, c in enumerate(centroids):
        p, m1, m2 = _moments(edges[i], edges[i + 1], dist, dim)
        total += m2 - 2.0 * c * m1 + c * c * p
    return total


def centroid_residual(centroids, boundaries, dist="gaussian", dim=128):
    """max_i |c_i - E[x | cell i]| -- zero at a Lloyd-Max fixed point."""
    edges = [-math.inf] + list(boundaries) + [math.inf]
    worst = 0.0
    for i, c in enumerate(centroids):
        p, m1, _ = _moments(edges[i], edges[i + 1], dist, dim)
        worst = max(worst, abs(c - m1 / p))
    return worst


def quantize_index(t, boundaries):
    """idx = #{i : beta_i < t} -- a value on a boundary goes to the lower cell."""
    return np.searchsorted(np.asarray(boundaries), np.asarray(t), side="left")
