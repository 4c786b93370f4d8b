"""The compress parity protocol (tests/parity.py) on the CPU: records written by the
oracle pass it, and mistakes planted in copies of those records (on the CPU, in
oracle output) are caught by the rule each one breaks."""

import numpy as np
import pytest

from compressed_decode_attention_tq_amd import synth
from oracle import compress
from tests import parity


def _case(key_mode="qjl", n=48, H=1):
    K, V = synth.kv_host(4321, n, H, outliers=4)
    slots = np.arange(n)
    st, layout, pool, res = parity.oracle_store(K, V, slots, (n + 15) // 16, H, 2, 3, 4322, key_mode=key_mode)
    ck, cv = res[0]
    rec = parity.fields_at(pool, layout, H, slots, 0)
    rec = {k: np.array(v) for k, v in rec.items()}
    return st, ck, cv, rec, V[:, 0]


def _stats(st, ck, cv, rec, V, key_mode="qjl"):
    return parity.compare_compress(rec, ck, cv, st.S[0], st.boundaries, V, 3, centroids=st.centroids,
                                   key_mode=key_mode)


def test_oracle_records_pass():
    st, ck, cv, rec, V = _case()
    s = _stats(st, ck, cv, rec, V)
    assert s["key_mismatch"] == s["sign_mismatch"] == s["value_mismatch"] == 0
    parity.assert_compress_ok(s)


def test_key_code_flip_outside_band_is_caught():
    st, ck, cv, rec, V = _case()
    i, j = 5, 17
    rec["idx"][i, j] = (rec["idx"][i, j] + 1) % 4
    s = _stats(st, ck, cv, rec, V)
    assert s["key_out_of_band"] == 1
    with pytest.raises(AssertionError):
        parity.assert_compress_ok(s)


def test_in_band_code_flip_needs_the_signs_of_the_new_codes():
    """A code flipped at an element placed (in the reference) 5e-7 from a boundary
    is accepted only together with the signs and gamma recomputed from the flipped
    codes; the original signs are then caught as out of band."""
    st, ck, cv, rec, V = _case()
    i, j = 7, 40
    b = int(np.argmin(np.abs(st.boundaries - ck["t"][i, j])))
    ck["t"][i, j] = st.boundaries[b] + 5e-7  # the reference's value sits just above boundary b
    ck["idx"][i, j] = b + 1
    flipped = rec["idx"].copy()
    flipped[i, j] = b  # the other side of the boundary, as a float32 decision may land
    good = dict(rec, idx=flipped)
    q = compress.qjl_signs(ck["t"][i:i + 1], flipped[i:i + 1], st.S[0], st.centroids)
    good["z"] = rec["z"].copy()
    good["z"][i] = q["z"][0]
    good["g16"] = rec["g16"].copy()
    good["g16"][i] = q["gamma"].astype(np.float16)[0]
    s = _stats(st, ck, cv, good, V)
    assert s["key_mismatch"] == 1 and s["key_out_of_band"] == 0 and s["sign_out_of_band"] == 0
    assert s["sign_rows_recomputed"] == 1
    parity.assert_compress_ok(s)
    # a compressor that flipped the code but kept the old code's signs
    stale = dict(good, z=rec["z"].copy())
    assert (q["z"][0] != rec["z"][i]).any()  # the flip moves the residual, so signs change
    s2 = _stats(st, ck, cv, stale, V)
    assert s2["sign_out_of_band"] > 0
    with pytest.raises(AssertionError):
        parity.assert_compress_ok(s2)


def test_sign_flip_is_caught():
    st, ck, cv, rec, V = _case()
    i = 3
    j = int(np.argmax(np.abs(ck["y"][i])))  # far from zero
    rec["z"][i, j] ^= 1
    s = _stats(st, ck, cv, rec, V)
    assert s["sign_out_of_band"] == 1
    with pytest.raises(AssertionError):
        parity.assert_compress_ok(s)


def test_value_code_and_metadata_mistakes_are_caught():
    st, ck, cv, rec, V = _case()
    bad = dict(rec, vcode=rec["vcode"].copy())
    bad["vcode"][2, 9] = (bad["vcode"][2, 9] + 1) % 8
    s = _stats(st, ck, cv, bad, V)
    assert s["value_out_of_band"] == 1
    with pytest.raises(AssertionError):
        parity.assert_compress_ok(s)
    # a norm two float16 ulps off
    bad = dict(rec, n16=rec["n16"].copy())
    bad["n16"][4] = (bad["n16"][4].view(np.uint16) + 2).view(np.float16)
    s = _stats(st, ck, cv, bad, V)
    assert s["n16_ulps"] == 2
    with pytest.raises(AssertionError):
        parity.assert_compress_ok(s)
    # a value scale one ulp off: the codes must then be the nearest points of that grid
    bad = dict(rec, scale16=rec["scale16"].copy())
    bad["scale16"][6, 1] = (bad["scale16"][6, 1].view(np.uint16) + 1).view(np.float16)
    s = _stats(st, ck, cv, bad, V)
    assert s["meta_ulps"] == 1 and s["value_meta_differs"] == 1
    # ... accepted only where the exact value is within the band of that ulp's
    # rounding boundary; two ulps off is always out of band
    bad["scale16"][6, 1] = (bad["scale16"][6, 1].view(np.uint16) + 1).view(np.float16)
    s = _stats(st, ck, cv, bad, V)
    assert s["meta_out_of_band"] == 1
    with pytest.raises(AssertionError):
        parity.assert_compress_ok(s)


def test_metadata_band_near_zero():
    """float16 spacing near zero is 2^-24 absolute: a zero computed as a rounding
    residue of a few 1e-8 may round to a few subnormal ulps, inside the 1e-6 ||v||
    band; the same distance on a normal value is outside."""
    g = np.array([3 * 2.0 ** -24, 2.0 ** -24 * 40, 1.0], np.float16)
    assert parity.f16_within(g, np.array([0.0, 0.0, 1.0 + 2 ** -9]), np.array([1e-6 * 0.2, 1e-6 * 0.2, 1e-6])).tolist() \
        == [True, False, False]


def test_key_modes_without_signs_must_store_zero_bits():
    st, ck, cv, rec, V = _case(key_mode="mse")
    s = _stats(st, ck, cv, rec, V, key_mode="mse")
    parity.assert_compress_ok(s)
    rec["z"][1, 2] = 1
    s = _stats(st, ck, cv, rec, V, key_mode="mse")
    assert s["sign_out_of_band"] == 1


def test_rate_is_asserted_on_large_samples_only():
    st = {"vectors": 10, "n16_ulps": 0, "g16_ulps": 0, "meta_ulps": 0, "meta_out_of_band": 0, "key_out_of_band": 0,
          "sign_out_of_band": 0, "value_out_of_band": 0, "value_invalid_other_meta": 0, "value_code_range": True,
          "key_mismatch": 1, "sign_mismatch": 0, "value_mismatch": 0}
    st["mismatch_rate"] = 1 / (3 * 10 * 128)
    before = parity.pooled()
    parity.assert_compress_ok(dict(st))  # 3840 decisions: the rate is not resolved, only pooled
    after = parity.pooled()
    assert after[0] - before[0] == 3840 and after[1] - before[1] == 1
    big = dict(st, vectors=3000, key_mismatch=30)
    big["mismatch_rate"] = 30 / (3 * 3000 * 128)  # 2.6e-5 over 1.15e6 decisions
    with pytest.raises(AssertionError):
        parity.assert_compress_ok(big)
