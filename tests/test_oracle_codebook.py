"""Pins of the Lloyd-Max codebooks: textbook tables, closed forms, Monte Carlo."""

import json
import math
import os

import numpy as np
import pytest

from oracle import codebook

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_gaussian_matches_tables(bits):
    ref = json.load(open(os.path.join(GOLDEN, "lloyd_max_gaussian.json")))["levels"][str(bits)]
    c, b, mse = codebook.lloyd_max(bits, "gaussian", 128)
    L = 1 << bits
    assert c.shape == (L,) and b.shape == (L - 1,)
    pos = c[L // 2:]
    assert np.max(np.abs(pos - ref["positive_centroids"])) < ref["tol"]
    if "positive_boundaries" in ref:
        assert np.max(np.abs(b[L // 2:] - ref["positive_boundaries"])) < ref["btol"]
    assert abs(mse - ref["mse"]) < ref["mse_tol"]


@pytest.mark.parametrize("dist", ["gaussian", "sphere"])
@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_fixed_point_conditions(bits, dist):
    c, b, _ = codebook.lloyd_max(bits, dist, 128)
    assert np.all(np.diff(c) > 0)
    assert np.allclose(b, 0.5 * (c[:-1] + c[1:]), atol=0, rtol=0)
    assert codebook.centroid_residual(c, b, dist, 128) < 1e-12
    assert np.max(np.abs(c + c[::-1])) < 1e-12       # symmetric density -> symmetric codebook


@pytest.mark.parametrize("bits", [1, 2, 3])
def test_sphere_d3_is_uniform_quantiser(bits):
    """For d = 3 a coordinate of a uniform point on S^2 is uniform on [-1, 1]
    (Archimedes), so sqrt(3) u is uniform on [-sqrt3, sqrt3] and Lloyd-Max is the
    uniform quantiser with MSE step^2/12."""
    L = 1 << bits
    c, b, mse = codebook.lloyd_max(bits, "sphere", 3)
    step = 2 * math.sqrt(3) / L
    expect = -math.sqrt(3) + (np.arange(L) + 0.5) * step
    assert np.max(np.abs(c - expect)) < 1e-9
    assert abs(mse - step * step / 12.0) < 1e-12


def test_sphere_tends_to_gaussian():
    for bits in (2, 3):
        cg, _, _ = codebook.lloyd_max(bits, "gaussian", 128)
        cs, _, _ = codebook.lloyd_max(bits, "sphere", 128)
        cb, _, _ = codebook.lloyd_max(bits, "sphere", 4096)
        assert 1e-4 < np.max(np.abs(cg - cs)) < 0.03
        assert np.max(np.abs(cg - cb)) < np.max(np.abs(cg - cs)) / 10


def _monte_carlo_cells(x, c, b):
    idx = np.searchsorted(b, x)
    means = np.array([x[idx == i].mean() for i in range(len(c))])
    ses = np.array([x[idx == i].std() / math.sqrt(np.sum(idx == i)) for i in range(len(c))])
    mse = np.mean((x - c[idx]) ** 2)
    return means, ses, mse


@pytest.mark.parametrize("bits", [2, 4])
def test_monte_carlo_gaussian(bits):
    x = np.random.default_rng(1).standard_normal(2_000_000)
    c, b, mse = codebook.lloyd_max(bits, "gaussian", 128)
    means, ses, emp = _monte_carlo_cells(x, c, b)
    assert np.all(np.abs(means - c) < 6 * ses)
    assert abs(emp - mse) < 0.02 * mse


def test_monte_carlo_sphere():
    d = 8
    g = np.random.default_rng(2).standard_normal((400_000, d))
    x = math.sqrt(d) * g[:, 0] / np.linalg.norm(g, axis=1)
    c, b, mse = codebook.lloyd_max(3, "sphere", d)
    means, ses, emp = _monte_carlo_cells(x, c, b)
    assert np.all(np.abs(means - c) < 6 * ses)
    assert abs(emp - mse) < 0.02 * mse


def test_quantize_index_nearest_centroid():
    c, b, _ = codebook.lloyd_max(3, "gaussian", 128)
    t = np.random.default_rng(3).standard_normal(10000) * 1.5
    idx = codebook.quantize_index(t, b)
    brute = np.argmin(np.abs(t[:, None] - c[None, :]), axis=1)
    assert np.array_equal(idx, brute)
    # ties go to the lower cell
    assert np.array_equal(codebook.quantize_index(b, b), np.arange(len(b)))


@pytest.mark.parametrize("dist", ["gaussian", "sphere"])
@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_stored_codebook(bits, dist):
    """The stored codebook: float16-rounded centroids, boundaries at their exact
    midpoints; its distortion is within a second-order hair of the optimum."""
    from oracle import state

    c, b = state.stored_codebook(bits, dist, 128)
    c64, b64, mse = codebook.lloyd_max(bits, dist, 128)
    assert np.array_equal(c, c.astype(np.float16).astype(np.float64))
    assert np.max(np.abs(c - c64) / np.abs(c64)) <= 2.0 ** -11
    assert np.array_equal(b, b.astype(np.float32).astype(np.float64))
    assert np.array_equal(b, (c[:-1] + c[1:]) / 2)
    d16 = codebook.distortion(c, b, dist, 128)
    assert mse <= d16 <= mse * (1 + 1e-5)
