"""Pins of the oracle's random state: SplitMix64, Box-Muller, Haar R and Gaussian S."""

import json
import os

import numpy as np
import pytest
from scipy import stats

from oracle import rng, state

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_splitmix64_published_outputs():
    cases = json.load(open(os.path.join(GOLDEN, "splitmix64.json")))["cases"]
    for case in cases:
        g = rng.SplitMix64(case["seed"])
        got = [g.next_u64() for _ in range(len(case.get("outputs", case.get("outputs_hex"))))]
        if "outputs_hex" in case:
            assert got == [int(h, 16) for h in case["outputs_hex"]]
        else:
            assert got == case["outputs"]


def test_box_muller_is_standard_normal():
    z = np.array(rng.gaussians(12345, 0, 0, 1, 200_000))
    se = 1.0 / np.sqrt(z.size)
    assert abs(z.mean()) < 5 * se
    assert abs(z.var() - 1.0) < 5 * np.sqrt(2.0) * se
    assert stats.kstest(z, "norm").pvalue > 1e-4
    # the two Box-Muller outputs of a pair are uncorrelated
    assert abs(np.corrcoef(z[0::2], z[1::2])[0, 1]) < 5 * np.sqrt(2.0) * se


def test_streams_are_distinct():
    a = rng.gaussians(7, 0, 0, 1, 64)
    for other in [(7, 0, 0, 2), (7, 0, 1, 1), (7, 1, 0, 1), (8, 0, 0, 1)]:
        assert not np.allclose(a, rng.gaussians(*other, 64))
    assert rng.gaussians(7, 3, 5, 2, 64) == rng.gaussians(7, 3, 5, 2, 64)


@pytest.mark.parametrize("d", [16, 128])
def test_rotation_orthogonal(d):
    r64 = state.haar_rotation_f64(200, 3, 1, d)
    assert np.abs(r64 @ r64.T - np.eye(d)).max() < 1e-12
    r32 = state.haar_rotation(200, 3, 1, d)
    assert np.all(r32 == r32.astype(np.float32))
    assert np.abs(r32 @ r32.T - np.eye(d)).max() < 1e-6
    assert abs(abs(np.linalg.det(r32)) - 1.0) < 1e-5
    assert abs((r32 ** 2).mean() - 1.0 / d) < 1e-9


def test_rotation_is_haar():
    """First entry of a Haar-random O(d) matrix: sqrt(d) R_00 has the sphere
    marginal, (1 + R_00)/2 ~ Beta((d-1)/2, (d-1)/2), and E[tr R] = 0, E[(tr R)^2] = 1.
    A QR without the sign fix fails all three (R_00 is then always negative)."""
    d, n = 16, 1500
    r00, tr = [], []
    for s in range(n):
        r = state.haar_rotation_f64(s, 0, 0, d)
        r00.append(r[0, 0])
        tr.append(np.trace(r))
    r00, tr = np.array(r00), np.array(tr)
    a = (d - 1) / 2.0
    assert stats.kstest((1.0 + r00) / 2.0, stats.beta(a, a).cdf).pvalue > 1e-3
    assert abs(tr.mean()) < 5 / np.sqrt(n)
    assert abs((tr ** 2).mean() - 1.0) < 5 * np.sqrt(2.0 / n)


def test_projection_gaussian():
    s = state.qjl_projection(200, 0, 0, 128)
    assert s.shape == (128, 128)
    assert np.all(s == s.astype(np.float32))
    z = s.ravel()
    assert abs(z.mean()) < 5 / np.sqrt(z.size)
    assert abs(z.var() - 1.0) < 5 * np.sqrt(2.0 / z.size)
    # independent of the same head's rotation stream
    g = state.gaussian_matrix(200, 0, 0, rng.TAG_ROTATION, 128, 128)
    assert abs(np.corrcoef(g.ravel(), z)[0, 1]) < 5 / np.sqrt(z.size)


def _fwht(x):
    """In-place fast Walsh-Hadamard butterflies (natural / Sylvester order), unnormalised."""
    x = np.array(x, dtype=np.float64)
    h = 1
    while h < len(x):
        for i in range(0, len(x), 2 * h):
            a = x[i:i + h].copy()
            b = x[i + h:i + 2 * h].copy()
            x[i:i + h] = a + b
            x[i + h:i + 2 * h] = a - b
        h *= 2
    return x


@pytest.mark.parametrize("d", [2, 8, 128])
def test_hadamard_rotation_is_the_fast_transform(d):
    """R x = FWHT(D x) / sqrt(d) for the butterfly algorithm (a different
    computation from the matrix definition), R is orthogonal, and every entry
    is +-1/sqrt(d) in float32."""
    r = state.hadamard_rotation(200, 3, 1, d)
    signs = np.array(rng.random_signs(200, 3, 1, d))
    x = np.random.default_rng(d).standard_normal(d)
    assert np.abs(r @ x - _fwht(signs * x) / np.sqrt(d)).max() < 1e-6 * np.abs(x).sum()
    assert np.abs(r @ r.T - np.eye(d)).max() < 1e-6
    assert np.all(np.abs(r) == np.float32(1.0 / np.sqrt(d)))
    if d == 2:
        assert np.array_equal(np.sign(r) * signs[None, :], np.array([[1.0, 1.0], [1.0, -1.0]]))


def test_random_signs_balanced_and_keyed():
    s = np.array(rng.random_signs(9, 2, 4, 4096))
    assert set(np.unique(s)) == {-1.0, 1.0}
    assert abs(s.mean()) < 5 / np.sqrt(s.size)
    assert rng.random_signs(9, 2, 4, 64) != rng.random_signs(9, 2, 5, 64)
    # first output of the tag-3 stream: its top bit is the first sign
    g = rng.SplitMix64(rng.stream_key(9, 2, 4, rng.TAG_SIGNS))
    assert s[0] == (1.0 if (g.next_u64() >> 63) == 0 else -1.0)
