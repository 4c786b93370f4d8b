"""Parity helpers: oracle-side construction of workloads and the comparison protocol.

Test infrastructure (imports the oracle).  The GPU's results are only ever
compared here; nothing computed by the library is fed back into the oracle.

Compression protocol (packed codes are decisions taken in floating point, so
the GPU's float32 arithmetic and the oracle's float64 may legitimately disagree
next to a decision boundary):
  * fp16 norms (||k||, gamma) and value scale/zero: within 1 fp16 ulp.
  * key codes: equal, except where the oracle's t_j lies within 1e-6 of a
    codebook boundary (t is the unit-variance coordinate).
  * sign bits, compared on vectors whose key codes all match: equal, except where
    |y_j| <= 1e-6 ||S_j|| ||rho|| (the cosine between projection row and residual
    is within 1e-6 of zero).
  * value codes, in groups whose scale/zero match: equal, except where the rotated
    value lies within 1e-6 ||v|| of the midpoint between the two codes; in groups
    whose fp16 scale/zero differ by an ulp, the GPU's code must be the nearest grid
    point of the GPU's own scale/zero (checked against the oracle's rotated value).
  * all mismatches together: rate <= 1e-5.  Every mismatch must already lie in
    one of the bands above; the rate bounds how often that happens on a large
    sample.  On a sample too small for one allowed (in-band) mismatch to stay
    under the rate, up to two in-band mismatches are accepted.
Decode protocol: both sides read the same (oracle-written) pool; relative L2 of
the whole output <= 1e-3 (float32 output) or <= 1e-2 (bf16 output).
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
    # signs on vectors whose codes all match
    rows = ~kmis.any(axis=1)
    smis = (gpu["z"] != ck["z"]) & rows[:, None]
    band = BAND * np.linalg.norm(S, axis=1)[None, :] * ck["gamma"][:, None]
    st["sign_mismatch"] = int(smis.sum())
    st["sign_out_of_band"] = int(np.sum(smis & (np.abs(ck["y"]) > band)))
    st["sign_rows_skipped"] = int(np.sum(~rows))
    # values
    top = (1 << v_bits) - 1
    if "vn16" in gpu:
        # codebook-coded values: codes as the keys' (band around the value
        # boundaries), the stored norm within an ulp
        st["meta_ulps"] = int(f16_ulps(gpu["vn16"], cv["n16"]).max(initial=0))
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


def assert_compress_ok(st):
    assert st["n16_ulps"] <= 1 and st["g16_ulps"] <= 1, st
    assert st["meta_ulps"] <= 1, st
    assert st["key_out_of_band"] == 0, st
    assert st["sign_out_of_band"] == 0, st
    assert st["value_out_of_band"] == 0, st
    assert st["value_invalid_other_meta"] == 0, st
    assert st["value_code_range"], st
    n_mis = st["key_mismatch"] + st["sign_mismatch"] + st["value_mismatch"]
    total = 3 * st["vectors"] * 128
    assert st["mismatch_rate"] <= 1e-5 or n_mis <= max(2, 1e-5 * total), st


def rel_l2(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm(got - ref) / np.linalg.norm(ref))


def oracle_store(K, V, slots, num_blocks, n_heads, k_bits, v_bits, seed, layer=0, bypass=False,
                 K_bits16=None, V_bits16=None, keep=True, fill=0, key_mode="qjl", rotation_kind="haar",
                 value_mode="group"):
    """Oracle state + pool for the given inputs (float arrays [N, H, d]); every
    pool byte starts as `fill` (0xFF: all-ones fields, NaN norms and values)."""
    layout = lay.StoreLayout(128, k_bits, v_bits, 32, bypass=bypass, value_mode=value_mode)
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


__all__ = ["f16_ulps", "fields_at", "compare_compress", "assert_compress_ok", "rel_l2",
           "oracle_store", "oracle_decode", "math"]
