"""Parity helpers: oracle-side construction of workloads and the comparison protocol.

Test infrastructure (imports the oracle).  The GPU's results are only ever
compared here; nothing computed by the library is fed back into the oracle.

Compression protocol (packed codes are decisions taken in floating point, so
the GPU's float32 arithmetic and the oracle's float64 may legitimately disagree
next to a decision boundary):
  * fp16 norms (||k||, gamma): within 1 fp16 ulp.  Value scale and zero: the
    float16 rounding is a decision too, so each must be the float16 rounding of
    some value within the band of the exact one: zero16 of a value within
    1e-6 ||v|| of the group minimum, scale16 of one within 2e-6 ||v|| / (2^b - 1)
    of (max - min) / (2^b - 1).  For normal float16 values this is at most 1 ulp;
    near zero (subnormal float16, absolute spacing 2^-24) it admits the few ulps
    that float32 rotation rounding of an exactly-zero coordinate amounts to.
  * key codes: equal, except where the oracle's t_j lies within 1e-6 of a
    codebook boundary (t is the unit-variance coordinate).
  * sign bits: on vectors whose key codes all match, equal to the oracle's,
    except where |y_j| <= 1e-6 ||S_j|| ||rho|| (the cosine between projection
    row and residual is within 1e-6 of zero); on a vector whose codes differ
    (inside the band), the residual, its norm and the signs are recomputed from
    the GPU's own codes (oracle.compress.qjl_signs) and compared the same way,
    gamma16 within an ulp of the recomputed norm.
  * value codes, in groups whose scale/zero match: equal, except where the rotated
    value lies within 1e-6 ||v|| of the midpoint between the two codes; in groups
    whose fp16 scale/zero differ by an ulp, the GPU's code must be the nearest grid
    point of the GPU's own scale/zero (checked against the oracle's rotated value).
  * no mismatch outside those bands, in every case (the per-element rule).
  * mismatch rate <= 1e-5: asserted on any single comparison of at least 1e6
    decisions, and on the counts pooled over every comparison of a test session
    (record() / pooled()), since a small case cannot resolve a rate of 1e-5.
Decode protocol: both sides read the same pool; relative L2 of the whole output
and of the worst (b, h) row <= 1e-3 (float32 output) or <= 1e-2 (bf16 output).
"""

import math

import numpy as np

from oracle import compress, decode, layout as lay, state as ostate

BAND = 1e-6


def f16_ulps(a, b):
    def ordered(x):
        i = np.asarray(x, dtype=np.float16).view(np.uint16).astype(np.int32)
        mag = i & 0x7FFF
        return np.where(i & 0x8000, -mag, mag)
    return np.abs(ordered(a) - ordered(b))


def f16_within(g16, exact, delta):
    """True where the float16 value g16 is the round-to-nearest image of some real
    within delta of `exact`: its rounding interval (half its spacing either side)
    meets [exact - delta, exact + delta]."""
    g = np.asarray(g16, dtype=np.float16)
    half = np.spacing(np.abs(g)).astype(np.float64) / 2.0
    return np.abs(g.astype(np.float64) - np.asarray(exact, dtype=np.float64)) <= half + delta


def fields_at(pool_bytes, layout, n_heads, slots, head):
    """Parse the records at `slots` (one head) out of raw pool bytes."""
    return lay.get_records(pool_bytes, layout, n_heads, slots, head)


def compare_compress(gpu, ck, cv, S, boundaries, V, v_bits, group=32, centroids=None, key_mode="qjl",
                     v_boundaries=None):
    """Apply the protocol to one head's records.  Returns a dict of counts.

    With the norm-corrected magnitude (key_mode "mse_nc") the stored n16 depends on
    the codes, so for a vector whose codes differ (inside the decision band) the
    expected value is recomputed from the GPU's codes, as the signs are."""
    n, d = ck["idx"].shape
    st = {"vectors": n}
    n16_ref = ck["n16"]
    if key_mode == "mse_nc":
        chat = np.asarray(centroids)[gpu["idx"]]
        n16_ref = (ck["n"] * math.sqrt(d) / np.sqrt(np.sum(chat * chat, axis=-1))).astype(np.float16)
    st["n16_ulps"] = int(f16_ulps(gpu["n16"], n16_ref).max(initial=0))
    st["g16_ulps"] = int(f16_ulps(gpu["g16"], ck["gamma16"]).max(initial=0))
    # key codes
    kmis = gpu["idx"] != ck["idx"]
    t = ck["t"][kmis]
    near = np.min(np.abs(t[:, None] - np.asarray(boundaries)[None, :]), axis=1) if t.size else t
    st["key_mismatch"] = int(kmis.sum())
    st["key_out_of_band"] = int(np.sum(near > BAND))
    rows = ~kmis.any(axis=1)
    st["sign_rows_recomputed"] = 0
    if key_mode != "qjl":
        # no residual signs in this key mode: every stored sign bit must be zero
        st["sign_mismatch"] = st["sign_out_of_band"] = int(np.sum(gpu["z"] != 0))
    else:
        # signs on vectors whose codes all match
        smis = (gpu["z"] != ck["z"]) & rows[:, None]
        Snorm = np.linalg.norm(S, axis=1)[None, :]
        band = BAND * Snorm * ck["gamma"][:, None]
        st["sign_mismatch"] = int(smis.sum())
        st["sign_out_of_band"] = int(np.sum(smis & (np.abs(ck["y"]) > band)))
        # vectors whose codes differ: signs and gamma as they follow from the GPU's codes
        st["sign_rows_recomputed"] = int(np.sum(~rows))
        if (~rows).any():
            rq = compress.qjl_signs(ck["t"][~rows], gpu["idx"][~rows], S, centroids)
            rmis = gpu["z"][~rows] != rq["z"]
            rband = BAND * Snorm * rq["gamma"][:, None]
            st["sign_mismatch"] += int(rmis.sum())
            st["sign_out_of_band"] += int(np.sum(rmis & (np.abs(rq["y"]) > rband)))
            g_ref = ck["gamma16"].copy()
            g_ref[~rows] = rq["gamma"].astype(np.float16)
            st["g16_ulps"] = int(f16_ulps(gpu["g16"], g_ref).max(initial=0))
    # values
    top = (1 << v_bits) - 1
    if "vn16" in gpu:
        # codebook-coded values: codes as the keys' (band around the value
        # boundaries), the stored norm within an ulp
        st["meta_ulps"] = int(f16_ulps(gpu["vn16"], cv["n16"]).max(initial=0))
        st["meta_out_of_band"] = int(np.sum(st["meta_ulps"] > 1))
        vmis = gpu["vcode"] != cv["codes"]
        tv = cv["t"][vmis]
        near = np.min(np.abs(tv[:, None] - np.asarray(v_boundaries)[None, :]), axis=1) if tv.size else tv
        st["value_mismatch"] = int(vmis.sum())
        st["value_out_of_band"] = int(np.sum(near > BAND))
        st["value_meta_differs"] = 0
        st["value_invalid_other_meta"] = 0
        st["value_code_range"] = bool(gpu["vcode"].min(initial=0) >= 0 and gpu["vcode"].max(initial=0) <= top)
        st["mismatch_rate"] = (st["key_mismatch"] + st["sign_mismatch"] + st["value_mismatch"]) / max(3 * n * d, 1)
        return st
    st["meta_ulps"] = int(max(f16_ulps(gpu["scale16"], cv["scale16"]).max(initial=0),
                              f16_ulps(gpu["zero16"], cv["zero16"]).max(initial=0)))
    top_f = float((1 << v_bits) - 1)
    vn = np.linalg.norm(np.asarray(V, dtype=np.float64), axis=1)[:, None]
    st["meta_out_of_band"] = int(np.sum(~f16_within(gpu["zero16"], cv["mn"], BAND * vn)) +
                                 np.sum(~f16_within(gpu["scale16"], (cv["mx"] - cv["mn"]) / top_f,
                                                    2.0 * BAND * vn / top_f)))
    same = (gpu["scale16"] == cv["scale16"]) & (gpu["zero16"] == cv["zero16"])
    same_el = np.repeat(same, group, axis=1)
    vnorm = np.linalg.norm(np.asarray(V, dtype=np.float64), axis=1)[:, None]
    vmis = (gpu["vcode"] != cv["codes"]) & same_el
    s = np.repeat(cv["scale16"].astype(np.float64), group, axis=1)
    z = np.repeat(cv["zero16"].astype(np.float64), group, axis=1)
    k = np.minimum(gpu["vcode"], cv["codes"])
    dist = np.abs(cv["vrot"] - (z + (k + 0.5) * s))
    st["value_mismatch"] = int(vmis.sum())
    st["value_out_of_band"] = int(np.sum(vmis & ((dist > BAND * vnorm) | (np.abs(gpu["vcode"] - cv["codes"]) > 1))))
    st["value_meta_differs"] = int(np.sum(~same))
    gs = np.repeat(gpu["scale16"].astype(np.float64), group, axis=1)
    gz = np.repeat(gpu["zero16"].astype(np.float64), group, axis=1)
    err = np.abs(cv["vrot"] - (gz + gs * gpu["vcode"]))
    bad = (~same_el) & (err > 0.5 * gs + BAND * vnorm)
    st["value_invalid_other_meta"] = int(bad.sum())
    st["value_code_range"] = bool(gpu["vcode"].min(initial=0) >= 0 and gpu["vcode"].max(initial=0) <= top)
    total = 3 * n * d
    st["mismatch_rate"] = (st["key_mismatch"] + st["sign_mismatch"] + st["value_mismatch"]) / max(total, 1)
    return st


# Counts pooled over every comparison of a test session (one process).
_POOL = {"decisions": 0, "mismatches": 0, "comparisons": 0}
RATE = 1e-5
RATE_MIN_SAMPLE = 1_000_000  # decisions needed before a rate of 1e-5 means anything


def record(st):
    _POOL["decisions"] += 3 * st["vectors"] * 128
    _POOL["mismatches"] += st["key_mismatch"] + st["sign_mismatch"] + st["value_mismatch"]
    _POOL["comparisons"] += 1


def pooled():
    """(decisions, mismatches, comparisons) recorded so far in this session."""
    return _POOL["decisions"], _POOL["mismatches"], _POOL["comparisons"]


def assert_compress_ok(st, pool=True):
    """The per-element rule always; the rate on samples of at least 1e6 decisions.
    pool=False keeps a comparison out of the pooled rate: inputs built to sit on
    decision boundaries test the per-element rule, and the rate is a statement
    about ordinary inputs."""
    assert st["n16_ulps"] <= 1 and st["g16_ulps"] <= 1, st
    assert st["meta_out_of_band"] == 0, st
    assert st["key_out_of_band"] == 0, st
    assert st["sign_out_of_band"] == 0, st
    assert st["value_out_of_band"] == 0, st
    assert st["value_invalid_other_meta"] == 0, st
    assert st["value_code_range"], st
    if pool:
        record(st)
    if 3 * st["vectors"] * 128 >= RATE_MIN_SAMPLE:
        assert st["mismatch_rate"] <= RATE, st


def rel_l2(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm(got - ref) / np.linalg.norm(ref))


def decode_errors(got, ref):
    """Relative L2 of the whole output [B, H_q, d] and of its worst (b, h) row, over
    the rows whose reference is nonzero (an empty sequence's row must be exactly
    zero and is checked on its own).  Returns (whole, worst, (b, h) of the worst)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = np.linalg.norm(got - ref, axis=-1)
    den = np.linalg.norm(ref, axis=-1)
    live = den > 0
    assert not got[~live].any(), "rows with a zero reference must be zero"
    if not live.any():
        return 0.0, 0.0, None
    whole = float(np.linalg.norm(num[live]) / np.linalg.norm(den[live]))
    ratio = np.where(live, num / np.where(live, den, 1.0), 0.0)
    at = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
    return whole, float(ratio[at]), tuple(int(i) for i in at)


def assert_decode_ok(got, ref, out_dtype, label=""):
    """Decode parity on identical stores: whole output and worst (b, h) row within
    1e-3 (float32 output) or 1e-2 (bf16 output)."""
    whole, worst, at = decode_errors(got, ref)
    tol = 1e-3 if out_dtype == "f32" else 1e-2
    print("decode %s %s rel L2 %.3e, worst (b, h) %s %.3e" % (label, out_dtype, whole, at, worst), flush=True)
    assert whole <= tol and worst <= tol, (label, out_dtype, whole, worst, at)
    return whole, worst


def oracle_store(K, V, slots, num_blocks, n_heads, k_bits, v_bits, seed, layer=0, bypass=False,
                 K_bits16=None, V_bits16=None, keep=True, fill=0, key_mode="qjl", rotation_kind="haar",
                 value_mode="group"):
    """Oracle state + pool for the given inputs (float arrays [N, H, d]); every
    pool byte starts as `fill` (0xFF: all-ones fields, NaN norms and values)."""
    layout = lay.StoreLayout(128, k_bits, v_bits, 32, bypass=bypass, value_mode=value_mode, qjl=key_mode == "qjl")
    pool = lay.new_pool(num_blocks, n_heads, layout)
    pool[:] = fill
    if bypass:
        compress.store_bypass(K_bits16, V_bits16, slots, pool, layout, n_heads)
        return None, layout, pool, None
    st = ostate.LayerState(seed, layer, n_heads, 128, k_bits, v_bits, 32, key_mode=key_mode,
                           rotation_kind=rotation_kind, value_mode=value_mode)
    res = compress.compress_into_pool(K, V, slots, pool, layout, st, keep=keep)
    return st, layout, pool, res


def oracle_decode(q, pool, layout, n_heads, table, lens, st, scale=None):
    return decode.decode(q, pool, layout, n_heads, table, lens, st, softmax_scale=scale)


__all__ = ["f16_ulps", "f16_within", "fields_at", "compare_compress", "assert_compress_ok", "record", "pooled", "rel_l2", "decode_errors", "assert_decode_ok",
           "oracle_store", "oracle_decode", "math"]
