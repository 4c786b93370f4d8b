"""Pins of the oracle's key/value compression."""

import math

import numpy as np
import pytest

from oracle import codebook, compress, metrics, state

D = 128


def _cb(bits):
    c, b = state.stored_codebook(bits, "gaussian", D)
    return c, b, codebook.distortion(c, b, "gaussian", D)


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("outliers", [False, True])
def test_mse_reconstruction_cosine(bits, outliers):
    """Mean cos(k, k_hat) -> sqrt(1 - D_b) for the codebook reconstruction (rotated
    coordinates are ~N(0,1) at d = 128 whatever the channel scales)."""
    rng = np.random.default_rng(bits)
    K = rng.standard_normal((4096, D))
    if outliers:
        K[:, rng.choice(D, 4, replace=False)] *= 10.0
    R = state.haar_rotation(11, 0, 0, D)
    S = state.qjl_projection(11, 0, 0, D)
    c, b, mse = _cb(bits)
    ck = compress.compress_keys(K, R, S, c, b)
    cos = metrics.cosine_rows(K, metrics.reconstruct_keys_mse(ck, R, c, D)).mean()
    assert abs(cos - math.sqrt(1.0 - mse)) < 3e-3
    if bits == 3:
        assert cos >= 0.98          # the target quality at 3 bits


def test_codes_are_nearest_centroid_of_rotated_standardised_key():
    rng = np.random.default_rng(5)
    K = rng.standard_normal((64, D)) * rng.uniform(0.1, 30.0, (64, 1))
    R = state.haar_rotation(3, 1, 2, D)
    S = state.qjl_projection(3, 1, 2, D)
    c, b, _ = _cb(4)
    ck = compress.compress_keys(K, R, S, c, b)
    # brute force, written from the definitions: unit vector, rotation, nearest centroid
    for i in range(64):
        unit = K[i] / math.sqrt(sum(x * x for x in K[i]))
        t = math.sqrt(D) * np.array([sum(R[r, j] * unit[j] for j in range(D)) for r in range(D)])
        idx = [int(np.argmin(np.abs(tj - c))) for tj in t]
        assert idx == list(ck["idx"][i])
        rho = t - c[idx]
        y = np.array([sum(S[r, j] * rho[j] for j in range(D)) for r in range(D)])
        assert list((y >= 0).astype(int)) == list(ck["z"][i])
    assert np.array_equal(ck["n16"], np.linalg.norm(K, axis=1).astype(np.float16))


def test_qjl_estimator_unbiased():
    """E_S[q'.c + sqrt(pi/2)/m gamma <S q', sign(S rho)>] = q'.t over random S,
    with standard deviation at most sqrt(pi/(2m)) ||q'|| gamma."""
    rng = np.random.default_rng(9)
    k = rng.standard_normal(D)
    qp = rng.standard_normal(D)
    R = np.eye(D)
    c, b, _ = _cb(2)
    n_seeds = 4000
    est = np.empty(n_seeds)
    from oracle import decode
    for s in range(n_seeds):
        S = np.random.default_rng(1000 + s).standard_normal((D, D))
        ck = compress.compress_keys(k[None, :], R, S, c, b)
        f = {"idx": ck["idx"], "z": ck["z"], "n16": np.array([math.sqrt(D)]),
             "g16": ck["gamma"]}
        est[s] = decode.token_scores(qp, S @ qp, f, c, D, D, 1.0)[0]
    truth = qp @ ck["t"][0]
    se = est.std() / math.sqrt(n_seeds)
    assert abs(est.mean() - truth) < 4 * se
    gamma = ck["gamma"][0]
    assert est.std() <= math.sqrt(math.pi / (2 * D)) * np.linalg.norm(qp) * gamma * 1.05


@pytest.mark.parametrize("v_bits", [2, 3, 4])
def test_value_group_quantiser_bounds(v_bits):
    rng = np.random.default_rng(v_bits)
    V = rng.standard_normal((512, D)) * 3.0
    R = state.haar_rotation(4, 0, 0, D)
    cv = compress.compress_values(V, R, v_bits, 32)
    top = (1 << v_bits) - 1
    assert cv["codes"].min() >= 0 and cv["codes"].max() <= top
    g = cv["vrot"].reshape(512, 4, 32)
    assert np.array_equal(cv["zero16"], g.min(axis=-1).astype(np.float16))
    assert np.array_equal(cv["scale16"], ((g.max(-1) - g.min(-1)) / top).astype(np.float16))
    s = np.repeat(cv["scale16"].astype(np.float64), 32, axis=1)
    z = np.repeat(cv["zero16"].astype(np.float64), 32, axis=1)
    err = np.abs(cv["vrot"] - (z + s * cv["codes"]))
    assert np.all(err <= 0.5 * s * (1 + 1e-9) + 1e-12)
    # every group uses its extreme codes
    codes = cv["codes"].reshape(512, 4, 32)
    assert np.all(codes.min(-1) == 0) and np.all(codes.max(-1) == top)


def test_value_grid_points_are_exact():
    """Rotated values already on an fp16 scale/zero grid come back exactly."""
    R = state.haar_rotation(4, 0, 1, D)
    rng = np.random.default_rng(0)
    codes = rng.integers(0, 8, (16, D))
    codes[:, ::32] = 0
    codes[:, 1::32] = 7
    scale = np.float16(0.375)
    zero = np.float16(-1.25)
    vrot = float(zero) + float(scale) * codes
    V = vrot @ R            # v = R^T v'
    cv = compress.compress_values(V, R, 3, 32)
    assert np.array_equal(cv["codes"], codes)
    assert np.all(cv["scale16"] == scale) and np.all(cv["zero16"] == zero)


def test_zero_norm_key():
    c, b, _ = _cb(3)
    ck = compress.compress_keys(np.zeros((1, D)), np.eye(D), np.eye(D), c, b)
    assert ck["n16"][0] == 0 and np.all(ck["t"] == 0)
    assert np.all(ck["idx"] == np.sum(b < 0))
    assert np.isfinite(ck["gamma"][0])


def test_norm_corrected_keys_keep_their_norm_and_direction():
    """Norm-corrected magnitude: the reconstruction (n16/sqrt d) R^T c[idx] has the
    key's own norm (to the fp16 rounding of the stored value, 2^-11 relative) and
    the direction of the plain codebook reconstruction (same codes)."""
    rng = np.random.default_rng(31)
    K = rng.standard_normal((300, D))
    K[:, 7] *= 10.0
    K[0] = 0.0  # zero-norm key: stored magnitude 0
    st = state.LayerState(41, 0, 1, D, 3, 3, 32)
    plain = compress.compress_keys(K, st.R[0], st.S[0], st.centroids, st.boundaries, "mse")
    nc = compress.compress_keys(K, st.R[0], st.S[0], st.centroids, st.boundaries, "mse_nc")
    assert np.array_equal(plain["idx"], nc["idx"])
    kp = metrics.reconstruct_keys_mse(plain, st.R[0], st.centroids, D)
    kn = metrics.reconstruct_keys_mse(nc, st.R[0], st.centroids, D)
    n = np.linalg.norm(K, axis=1)
    assert float(nc["n16"][0]) == 0.0 and not kn[0].any()
    rel = np.abs(np.linalg.norm(kn[1:], axis=1) - n[1:]) / n[1:]
    assert rel.max() <= 2.0 ** -11
    assert np.max(np.abs(metrics.cosine_rows(kp[1:], kn[1:]) - 1.0)) < 1e-12
    # the plain reconstruction is shorter on average (Lloyd-Max centroids shrink)
    assert np.mean(np.linalg.norm(kp[1:], axis=1) / n[1:]) < 1.0


def test_key_mode_rejects_unknown():
    st = state.LayerState(41, 0, 1, D, 3, 3, 32)
    with pytest.raises(ValueError):
        compress.compress_keys(np.ones((2, D)), st.R[0], st.S[0], st.centroids, st.boundaries, "qjl_off")


def test_hadamard_rotation_reconstruction_cosine():
    """The randomised Hadamard rotation spreads coordinates like the Haar one:
    the mean cosine of the 3-bit codebook reconstruction stays near sqrt(1 - D_3)."""
    rng = np.random.default_rng(5)
    K = rng.standard_normal((2000, D))
    K[:, 3] *= 10.0
    st = state.LayerState(77, 0, 1, D, 3, 3, 32, rotation_kind="hadamard")
    ck = compress.compress_keys(K, st.R[0], st.S[0], st.centroids, st.boundaries)
    cos = metrics.cosine_rows(K, metrics.reconstruct_keys_mse(ck, st.R[0], st.centroids, D)).mean()
    assert abs(cos - math.sqrt(1.0 - 0.03455)) < 0.004


# ------------------------------------------------ values coded like the keys
@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("outliers", [False, True])
def test_mse_values_reconstruction_cosine(bits, outliers):
    """Values normalised, rotated and Lloyd-Max quantised: mean cos(v, v_hat) ->
    sqrt(1 - D_b) (D_b the codebook's distortion, a closed-form integral); at 3 bits
    the 0.98 cosine the pages give for their 3-bit values."""
    rng = np.random.default_rng(100 + bits)
    V = rng.standard_normal((4096, D))
    if outliers:
        V[:, rng.choice(D, 4, replace=False)] *= 10.0
    R = state.haar_rotation(12, 0, 1, D)
    c, b, mse = _cb(bits)
    cv = compress.compress_values_mse(V, R, c, b)
    cos = metrics.cosine_rows(V, metrics.reconstruct_values_mse(cv, R, c, D)).mean()
    assert abs(cos - math.sqrt(1.0 - mse)) < 3e-3
    if bits == 3:
        assert cos >= 0.98


def test_mse_value_codes_are_nearest_centroid_of_rotated_standardised_value():
    """Brute force with pure-Python loops from the definitions: unit vector,
    rotation, nearest 3-bit centroid; the stored norm is fp16(||v||)."""
    rng = np.random.default_rng(15)
    V = rng.standard_normal((48, D)) * rng.uniform(0.05, 40.0, (48, 1))
    R = state.haar_rotation(4, 2, 0, D)
    c, b, _ = _cb(3)
    cv = compress.compress_values_mse(V, R, c, b)
    for i in range(48):
        unit = V[i] / math.sqrt(sum(x * x for x in V[i]))
        t = [math.sqrt(D) * sum(R[r, j] * unit[j] for j in range(D)) for r in range(D)]
        idx = [min(range(len(c)), key=lambda e: abs(tj - c[e])) for tj in t]
        assert idx == list(cv["codes"][i])
    assert np.array_equal(cv["n16"], np.linalg.norm(V, axis=1).astype(np.float16))


def test_mse_values_zero_vector():
    """A zero value vector stores norm 0, so its reconstruction is exactly zero."""
    c, b, _ = _cb(3)
    R = state.haar_rotation(1, 0, 0, D)
    cv = compress.compress_values_mse(np.zeros((2, D)), R, c, b)
    assert not cv["n16"].any()
    assert not metrics.reconstruct_values_mse(cv, R, c, D).any()


def test_value_mode_rejects_unknown():
    from oracle import layout
    with pytest.raises(ValueError):
        layout.StoreLayout(128, 2, 3, 32, value_mode="fp8")
    with pytest.raises(ValueError):
        state.LayerState(1, 0, 1, D, 2, 3, 32, value_mode="fp8")


def test_mse_values_under_hadamard_rotation_cosine():
    """The randomised Hadamard rotation Gaussianises values as well: mean cos(v, v_hat)
    at 3 bits stays at sqrt(1 - D_3) within the same tolerance, outlier channels
    included."""
    rng = np.random.default_rng(77)
    V = rng.standard_normal((4096, D))
    V[:, rng.choice(D, 4, replace=False)] *= 10.0
    R = state.hadamard_rotation(13, 0, 2, D)
    c, b, mse = _cb(3)
    cv = compress.compress_values_mse(V, R, c, b)
    cos = metrics.cosine_rows(V, metrics.reconstruct_values_mse(cv, R, c, D)).mean()
    assert abs(cos - math.sqrt(1.0 - mse)) < 3e-3
