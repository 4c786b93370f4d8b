"""GPU parity: libtq's HIP kernels (through the C ABI) against the oracle."""

import os

import numpy as np
import pytest

import compressed_decode_attention_tq_amd as tq
from compressed_decode_attention_tq_amd import synth
from tests import parity

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a visible GPU")
    tq.lib()  # fails loudly if the library is missing
    return torch


def say(*a):
    print("[case]", *a, flush=True)


# ------------------------------------------------------------------ compress
def _gpu_compress(torch, K, V, slots, num_blocks, n_heads, kb, vb, seed, layer=0, dtype="bf16", key_mode=0,
                  rotation=0, value_mode=0, fill=None):
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    layer_obj = tq.Layer(tq.config(n_heads, kb, vb, seed=seed, layer=layer, key_mode=key_mode, rotation=rotation,
                                   value_mode=value_mode))
    k = torch.from_numpy(np.ascontiguousarray(K)).to("cuda", tdt)
    v = torch.from_numpy(np.ascontiguousarray(V)).to("cuda", tdt)
    pool = layer_obj.new_pool(num_blocks)
    if fill is not None:
        pool.fill_(fill)
    tq.compress_kv(layer_obj, k, v, torch.from_numpy(np.asarray(slots, np.int64)).cuda(), pool)
    torch.cuda.synchronize()
    out = pool.cpu().numpy()
    layer_obj.close()
    return out


def _check_compress(gpu_pool, res, st, layout, n_heads, slots, V, kb, vb, pool=True):
    keep = np.asarray(slots) >= 0
    sl = np.asarray(slots)[keep]
    for h in range(n_heads):
        f = parity.fields_at(gpu_pool, layout, n_heads, sl, h)
        ck, cv = res[h]
        stats = parity.compare_compress(f, ck, cv, st.S[h], st.boundaries, V[keep][:, h], vb,
                                        centroids=st.centroids, key_mode=st.key_mode,
                                        v_boundaries=getattr(st, "v_boundaries", None))
        print("head", h, stats)
        parity.assert_compress_ok(stats, pool=pool)


def _edge_rows(st, n_heads, kind):
    """K, V [16, H, 128] rows the compressors special-case, all exactly representable
    in bf16:
      "zero"   zero keys and values: t = 0 puts every coordinate on the codebook's
               middle boundary (the tie goes to the lower cell), n16 = 0, and every
               value group is constant (scale16 = 0, codes 0);
      "tiny"   N(0,1) rows scaled by 2^-70: ||k||^2 (about 2^-133) is a float32
               subnormal, n16 = 0, the codes are those of the unscaled direction,
               and the value scale rounds to float16 zero;
      "ones"   (randomised Hadamard layers) k = c sign(R_i,:), v likewise: R k is
               c sqrt(d) e_i exactly, so 127 coordinates of t are exactly 0 (on the
               boundary), 3 of the 4 value groups are exactly constant and the
               fourth holds one extreme value (codes 0 and 2^b - 1 exactly)."""
    K = np.zeros((16, n_heads, 128), np.float32)
    V = np.zeros((16, n_heads, 128), np.float32)
    if kind == "tiny":
        rng = np.random.default_rng(77)
        K = synth.bf16_round(rng.standard_normal(K.shape).astype(np.float32) * np.float32(2.0 ** -70))
        V = synth.bf16_round(rng.standard_normal(V.shape).astype(np.float32) * np.float32(2.0 ** -70))
    elif kind == "ones":
        for r in range(16):
            for h in range(n_heads):
                c = np.float32((-1.0) ** r * 2.0 ** -(r % 5))
                K[r, h] = c * np.sign(st.R[h][(5 * r + h) % 128])
                V[r, h] = -c * np.sign(st.R[h][(3 * r + 7 * h + 1) % 128])
    return K, V


@pytest.mark.parametrize("path,rotation,value_mode", [
    ("mfma-pages", 0, 0), ("mfma-pages", 1, 0), ("mfma-scattered", 1, 0), ("per-token-bf16", 0, 0),
    ("per-token-bf16", 1, 0), ("per-token-f32", 1, 0), ("mfma-pages", 1, 1), ("per-token-f32", 0, 1)])
def test_compress_edge_cases(path, rotation, value_mode):
    """Zero keys and values, keys with a subnormal squared norm, values whose float16
    scale is 0, coordinates exactly on the middle decision boundary and constant
    value groups, mixed with ordinary rows, through each compressor (the
    matrix-core kernel on whole pages and on scattered tokens; the per-token kernel
    for short bf16 appends and for fp32).  The exact-zero coordinates and constant
    groups of the "ones" rows need the Hadamard rotation's exact +-1 structure."""
    torch = _torch()
    say("compress edge cases", path, "hadamard" if rotation else "haar")
    H, kb, vb, seed = 2, 2, 3, 290 + rotation
    rot = "haar" if rotation == 0 else "hadamard"
    st0 = parity.ostate.LayerState(seed, 1, H, 128, kb, vb, 32, rotation_kind=rot)
    kinds = ["zero", "tiny"] + (["ones"] if rotation else [])
    parts = [_edge_rows(st0, H, k) for k in kinds]
    dtype = "f32" if path == "per-token-f32" else "bf16"
    n_plain = 8 if path == "per-token-bf16" else 208  # under / over the matrix-core kernel's 64 tokens
    Kp, Vp = synth.kv_host(291, n_plain, H, outliers=4, dtype=dtype)
    K = np.concatenate([p[0] for p in parts] + [Kp])
    V = np.concatenate([p[1] for p in parts] + [Vp])
    n = K.shape[0]
    nb = (n + 15) // 16 + 2
    if path == "mfma-pages":
        slots = np.arange(n, dtype=np.int64)
    else:
        slots = np.random.default_rng(292).permutation(nb * 16)[:n].astype(np.int64)
    gpu = _gpu_compress(torch, K, V, slots, nb, H, kb, vb, seed, layer=1, dtype=dtype, rotation=rotation,
                        value_mode=value_mode)
    st, layout, pool, res = parity.oracle_store(K, V, slots, nb, H, kb, vb, seed, layer=1, rotation_kind=rot,
                                                value_mode="mse" if value_mode else "group")
    _check_compress(gpu, res, st, layout, H, slots, V, kb, vb, pool=False)
    if value_mode:
        for h in range(H):
            f = parity.fields_at(gpu, layout, H, slots[:32], h)
            assert not f["n16"].astype(np.float64).any() and not f["vn16"].astype(np.float64).any()
            assert np.all(f["idx"][:16] == (1 << kb) // 2 - 1) and np.all(f["vcode"][:16] == (1 << vb) // 2 - 1)
        return
    # the special rows as the method defines them (read from the GPU's store)
    for h in range(H):
        f = parity.fields_at(gpu, layout, H, slots[:16 * len(kinds)], h)
        assert not f["n16"][:32].astype(np.float64).any()            # zero and tiny keys: n16 = 0
        assert np.all(f["idx"][:16] == (1 << kb) // 2 - 1)           # t = 0: the lower middle cell
        assert not f["scale16"][:32].astype(np.float64).any()        # zero and tiny values: scale 0
        assert not f["vcode"][:32].any()                             # ... and codes 0
        if rotation and path.startswith("mfma"):
            # the matrix-core kernel forms R k from the exact +-1 pattern, so the
            # zero coordinates are exactly 0 (the per-token kernel's dense float32
            # products leave rounding residues there, in band)
            ones = f["idx"][32:48]
            assert np.sum(ones == (1 << kb) // 2 - 1, axis=1).min() >= 127
            assert np.sum(f["scale16"][32:48].astype(np.float64) == 0.0, axis=1).min() == 3


def _operand_lanes(M, tiles, row_major=True):
    """[tiles][4 K-steps][64 lanes][8] views of a 2-D matrix in the matrix-core lane
    order: lane l of (tile t, step s) element j holds M[16t + l%16][32s + 8(l/16) + j]
    (row_major) or M[32s + 8(l/16) + j][16t + l%16]."""
    t = np.arange(tiles)[:, None, None, None]
    s = np.arange(4)[None, :, None, None]
    l = np.arange(64)[None, None, :, None]
    j = np.arange(8)[None, None, None, :]
    a, b = 16 * t + l % 16, 32 * s + 8 * (l // 16) + j
    return M[a, b] if row_major else M[b, a]


def _bf16_pieces(R):
    r = np.asarray(R, np.float32)
    p0 = synth.bf16_bits(r)
    p1 = synth.bf16_bits(r - synth.bf16_to_f32(p0))
    p2 = synth.bf16_bits(r - synth.bf16_to_f32(p0) - synth.bf16_to_f32(p1))
    return p0, p1, p2


def _f16_pieces(W):
    W = np.asarray(W, np.float64)
    hi = W.astype(np.float16)
    lo = (W - hi.astype(np.float64)).astype(np.float16)
    return hi.view(np.uint16), lo.view(np.uint16)


@pytest.mark.parametrize("kb,vb,rotation,value_mode,bypass", [
    (4, 4, 0, 0, False), (2, 3, 1, 0, False), (3, 2, 0, 1, False), (4, 4, 0, 0, True)])
def test_layer_export(kb, vb, rotation, value_mode, bypass):
    """The state a created layer holds on the device, read back: R, S and the
    codebooks bit for bit equal to the host recomputation and to the oracle's (R
    up to float32 rounding ties of the two QR factorisations), and every packed
    matrix-core operand buffer equal to one rebuilt here from the exported R and S
    (the compressor's bf16 pieces of R summing to R exactly)."""
    torch = _torch()
    say("layer export", kb, vb, rotation, value_mode, bypass)
    H, seed = 3, 330 + kb
    cfg = tq.config(H, kb, vb, seed=seed, layer=2, rotation=rotation, value_mode=value_mode, bypass=bypass)
    layer = tq.Layer(cfg)
    R, S, c, b, vc, vbd = layer.export()
    if bypass:
        assert not R.any() and not S.any() and c.size == 0
        with pytest.raises(tq.TQError):
            layer.export_operands(tq.OPERANDS_COMPRESS)
        layer.close()
        return
    Rh, Sh, ch, bh = tq.layer_state_host(cfg)
    assert np.array_equal(R.view(np.uint32), Rh.view(np.uint32)) and np.array_equal(S.view(np.uint32), Sh.view(np.uint32))
    assert np.array_equal(c, ch) and np.array_equal(b, bh)
    st = parity.ostate.LayerState(seed, 2, H, 128, kb, vb, 32, rotation_kind="haar" if rotation == 0 else "hadamard",
                                  value_mode="mse" if value_mode else "group")
    assert np.array_equal(S.astype(np.float64), st.S)
    ties = np.abs(R.astype(np.float64) - st.R) > 0
    assert ties.sum() <= 2 * H and np.abs(R.astype(np.float64) - st.R).max() <= 2.0 ** -30
    assert np.array_equal(c.astype(np.float64), st.centroids) and np.array_equal(b.astype(np.float64), st.boundaries)
    if value_mode:
        assert np.array_equal(vc.astype(np.float64), st.v_centroids)
        assert np.array_equal(vbd.astype(np.float64), st.v_boundaries)
    opa = layer.export_operands(tq.OPERANDS_COMPRESS).reshape(H, 8, 5, 4, 64, 8)
    opq = layer.export_operands(tq.OPERANDS_PROLOGUE).reshape(H, 16, 4, 2, 64, 8)
    opd = layer.export_operands(tq.OPERANDS_DECOMPRESS).reshape(H, 8, 4, 4, 64, 8)
    for h in range(H):
        Rf, Sf = R[h], S[h]
        if rotation == 0:
            pieces = _bf16_pieces(Rf)
            total = sum(synth.bf16_to_f32(p).astype(np.float64) for p in pieces)
            assert np.array_equal(total, Rf.astype(np.float64))  # hi + mid + lo = R exactly
        else:
            one = synth.bf16_bits(np.where(Rf < 0, -1.0, 1.0).astype(np.float32))
            pieces = (one, np.zeros_like(one), np.zeros_like(one))
        s0, s1 = _f16_pieces(Sf.astype(np.float64))
        s1 = (Sf.astype(np.float64) - s0.view(np.float16).astype(np.float64)).astype(np.float16).view(np.uint16)
        for k, P in enumerate(list(pieces) + [s0, s1]):
            assert np.array_equal(opa[h, :, k], _operand_lanes(P, 8)), (h, k)
        P64 = Sf.astype(np.float64) @ Rf.astype(np.float64)
        W = np.concatenate([Rf.astype(np.float64), P64])
        whi, wlo = _f16_pieces(W)
        assert np.array_equal(opq[h, :, :, 0], _operand_lanes(whi, 16)), h
        assert np.array_equal(opq[h, :, :, 1], _operand_lanes(wlo, 16)), h
        for k, M in enumerate(_f16_pieces(Rf.astype(np.float64)) + _f16_pieces(P64)):
            assert np.array_equal(opd[h, :, :, k], _operand_lanes(M, 8, row_major=False)), (h, k)
    layer.close()


def test_compress_tiny_fp32():
    """1 KV head, 1024 tokens, fp32 N(0,1), keys 2-bit + QJL, values 3-bit g32."""
    torch = _torch()
    say("compress tiny fp32 K2/V3")
    K, V = synth.kv_host(101, 1024, 1, dtype="f32")
    slots = np.arange(1024)
    gpu = _gpu_compress(torch, K, V, slots, 64, 1, 2, 3, 201, dtype="f32")
    st, layout, pool, res = parity.oracle_store(K, V, slots, 64, 1, 2, 3, 201)
    _check_compress(gpu, res, st, layout, 1, slots, V, 2, 3)


@pytest.mark.parametrize("kb,vb", [(2, 2), (3, 2), (3, 3), (4, 3), (4, 4), (2, 4), (1, 3), (1, 2)])
def test_compress_bits_ragged_slots(kb, vb):
    """8 heads, bf16 with outlier channels, shuffled slots with skipped (-1) tokens."""
    torch = _torch()
    say("compress ragged", kb, vb)
    n = 301
    K, V = synth.kv_host(110 + kb * 10 + vb, n, 8, outliers=4)
    rng = np.random.default_rng(kb * 7 + vb)
    slots = rng.permutation(40 * 16)[:n].astype(np.int64)
    slots[rng.choice(n, 20, replace=False)] = -1
    gpu = _gpu_compress(torch, K, V, slots, 40, 8, kb, vb, 210, layer=kb + vb)
    st, layout, pool, res = parity.oracle_store(K, V, slots, 40, 8, kb, vb, 210, layer=kb + vb)
    _check_compress(gpu, res, st, layout, 8, slots, V, kb, vb)
    # slots nobody wrote stay untouched
    written = set((slots[slots >= 0] // 16).tolist())
    untouched = [b for b in range(40) if b not in written]
    for b in untouched:
        assert not gpu[b * 8 * layout.block_bytes:(b + 1) * 8 * layout.block_bytes].any()


@pytest.mark.parametrize("kb,vb,key_mode,value_mode", [
    (2, 3, tq.KEY_QJL, "group"), (4, 4, tq.KEY_QJL, "group"), (3, 2, tq.KEY_MSE, "group"),
    (1, 3, tq.KEY_QJL, "mse"), (2, 4, tq.KEY_MSE_NC, "mse"), (3, 3, tq.KEY_QJL, "group")])
def test_compress_prefill_batch(kb, vb, key_mode, value_mode):
    """A prefill batch through the matrix-core compressor: 14 sequences of ragged
    lengths laid end to end in the input, each from offset 0 of its own shuffled
    pages, so the 16-token tiles straddle two pages at many rotations (and a tile
    holding a sequence's end and the next one's start goes token by token).
    Written records against the oracle; every offset nobody wrote (the tail of
    each sequence's last page, pages left free) keeps the pool's prior bytes, read
    field by field against the oracle's pool filled the same way."""
    torch = _torch()
    say("compress prefill batch", kb, vb, key_mode, value_mode)
    rng = np.random.default_rng(400 + 10 * kb + vb)
    lens = rng.integers(17, 200, 14)
    lens[3] = 16  # one sequence of exactly a page
    npg = (lens + 15) // 16
    nb = int(npg.sum()) + 3
    perm = rng.permutation(nb)
    slots, o = [], 0
    for L, m in zip(lens, npg):
        pages = perm[o:o + m]
        o += m
        pos = np.arange(L)
        slots.append(pages[pos // 16].astype(np.int64) * 16 + pos % 16)
    slots = np.concatenate(slots)
    n = len(slots)
    H = 8
    K, V = synth.kv_host(410 + kb, n, H, outliers=4)
    vm = tq.VAL_MSE if value_mode == "mse" else tq.VAL_GROUP
    gpu = _gpu_compress(torch, K, V, slots, nb, H, kb, vb, 420, layer=kb, key_mode=key_mode, value_mode=vm,
                        fill=0xA5)
    st, layout, pool, res = parity.oracle_store(K, V, slots, nb, H, kb, vb, 420, layer=kb, fill=0xA5,
                                                key_mode=KEY_MODE_NAMES[key_mode], value_mode=value_mode)
    _check_compress(gpu, res, st, layout, H, slots, V, kb, vb)
    unwritten = np.setdiff1d(np.arange(nb * 16), slots)
    assert len(unwritten) > 16 * 3
    for h in range(H):
        g = parity.fields_at(gpu, layout, H, unwritten, h)
        o_ = parity.fields_at(pool, layout, H, unwritten, h)
        for key in o_:
            a_, b_ = np.ascontiguousarray(g[key]), np.ascontiguousarray(o_[key])
            assert a_.shape == b_.shape and a_.tobytes() == b_.tobytes(), (h, key)


@pytest.mark.parametrize("kb,vb,n,dtype,key_mode,rotation,pages", [
    (2, 3, 301, "bf16", 0, 0, False), (4, 4, 500, "bf16", 0, 0, False), (3, 2, 200, "f32", 0, 0, False),
    (2, 3, 2003, "bf16", 0, 0, False), (3, 3, 300, "bf16", 2, 1, False), (2, 3, 1024, "bf16", 0, 0, True),
    (1, 4, 777, "bf16", 1, 1, True), (2, 2, 40, "bf16", 0, 0, False)])
def test_compress_mse_values(kb, vb, n, dtype, key_mode, rotation, pages):
    """Values coded like the keys' codebook part (the 102-byte record at K2/V3): 8
    heads with outlier channels; bf16 runs of 64+ tokens through the matrix-core
    compressor, on whole pages (identity slots) and on shuffled slots with skipped
    tokens; fp32 inputs and a 40-token append through the per-token compressor;
    together with norm-corrected or plain keys and the Hadamard rotation.  Codes as
    the keys' protocol, the value norm within an fp16 ulp, slots nobody wrote
    untouched."""
    torch = _torch()
    say("compress mse values", kb, vb, n, dtype)
    K, V = synth.kv_host(340 + kb * 10 + vb, n, 8, outliers=4, dtype=dtype)
    rng = np.random.default_rng(340 + kb)
    nb = max(40, (n + 15) // 16 + 4)  # 2003 tokens: 16 per workgroup, a ragged last run
    if pages:
        slots = np.arange(n, dtype=np.int64)
    else:
        slots = rng.permutation(nb * 16)[:n].astype(np.int64)
        slots[rng.choice(n, min(15, n // 3), replace=False)] = -1
    gpu = _gpu_compress(torch, K, V, slots, nb, 8, kb, vb, 341, layer=kb, dtype=dtype, key_mode=key_mode,
                        rotation=rotation, value_mode=tq.VAL_MSE)
    st, layout, pool, res = parity.oracle_store(K, V, slots, nb, 8, kb, vb, 341, layer=kb, value_mode="mse",
                                                key_mode=KEY_MODE_NAMES[key_mode],
                                                rotation_kind="haar" if rotation == tq.ROT_HAAR else "hadamard")
    # key metadata: 16 B of signs + (n, gamma) with QJL, the magnitude alone without
    assert layout.record_bytes() == 16 * kb + (20 if key_mode == tq.KEY_QJL else 2) + 16 * vb + 2
    _check_compress(gpu, res, st, layout, 8, slots, V, kb, vb)
    written = set((slots[slots >= 0] // 16).tolist())
    for b in range(nb):
        if b not in written:
            assert not gpu[b * 8 * layout.block_bytes:(b + 1) * 8 * layout.block_bytes].any()


@pytest.mark.parametrize("kb,vb,rep,splits", [(2, 3, 4, 0), (4, 4, 8, 0), (3, 2, 1, 3), (1, 3, 2, 64),
                                               (4, 3, 4, 1)])
def test_decode_mse_values(kb, vb, rep, splits):
    """Decode over stores with MSE-coded values (norm + value codebook; the 102-byte
    record at K2/V3): ragged lengths, random block tables, GQA 1/2/4/8, forced splits,
    float32 and bf16 output, against the oracle on the same store."""
    torch = _torch()
    say("decode mse values", kb, vb, rep, splits)
    Hkv = 4
    _decode_case(torch, 4, Hkv * rep, Hkv, [700, 1, 129, 2050], kb, vb, 360 + kb, num_splits=splits,
                 value_mode=tq.VAL_MSE)


@pytest.mark.parametrize("key_mode,kb,vb,rep,value_mode", [
    (1, 4, 4, 4, 0), (2, 3, 2, 8, 0), (1, 2, 3, 1, 1), (2, 1, 3, 2, 0), (1, 4, 3, 4, 1)])
def test_decode_compact_layout_without_qjl(key_mode, kb, vb, rep, value_mode):
    """Key modes without QJL store no sign field and no gamma (the compact page); the
    decode variant without sign products, over oracle-written compact stores at every
    GQA ratio, with group- and MSE-coded values, and 0xFF-filled pools."""
    torch = _torch()
    say("decode compact layout", key_mode, kb, vb, rep, value_mode)
    Hkv = 2
    _decode_case(torch, 4, Hkv * rep, Hkv, [1, 700, 129, 2050], kb, vb, 380 + kb, key_mode=key_mode,
                 value_mode=value_mode, fill=0xFF)


def test_decode_mse_values_unwritten_slots():
    """MSE-value pools filled with 0xFF before the records are written: the slots
    past each context end hold NaN norms, which must not reach the output."""
    torch = _torch()
    say("decode mse values, unwritten slots")
    _decode_case(torch, 5, 8, 2, [1, 17, 40, 129, 1000], 2, 3, 371, fill=0xFF, value_mode=tq.VAL_MSE)


def test_end_to_end_mse_values():
    """The pages' 102-byte format (2-bit keys + QJL, 3-bit MSE values): GPU compress ->
    GPU decode against oracle compress -> oracle decode."""
    torch = _torch()
    say("end to end mse values K2/V3")
    B, Hq, Hkv, T = 3, 32, 8, 700
    lens = np.array([T, 300, 64], np.int32)
    maxb = (T + 15) // 16
    table = synth.block_table(372, B, maxb, "random")
    K, V = synth.kv_host(373, B * T, Hkv, outliers=4)
    pos = np.tile(np.arange(T), B)
    seq = np.repeat(np.arange(B), T)
    slots = table[seq, pos // 16].astype(np.int64) * 16 + pos % 16
    _end_to_end(torch, K, V, slots, table, lens, Hq, Hkv, 2, 3, 372, value_mode=tq.VAL_MSE, label="mse K2/V3")


@pytest.mark.parametrize("kb,vb,out_dtype", [(2, 3, "f32"), (4, 4, "bf16"), (3, 2, "f32")])
def test_decompress_mse_values(kb, vb, out_dtype):
    """MSE-value stores written by the GPU (shuffled slots; some read slots
    negative: zero rows; tiles mixing whole pages and scattered tokens),
    reconstructed on the GPU against the oracle's reconstruction of the same bytes."""
    from oracle import decompress as odec
    torch = _torch()
    say("decompress mse values", kb, vb, out_dtype)
    H, n = 8, 517
    K, V = synth.kv_host(350 + kb, n, H, outliers=4)
    rng = np.random.default_rng(350 + vb)
    slots = np.concatenate([np.arange(64), 64 + rng.permutation(40 * 16)[: n - 64]]).astype(np.int64)
    layer = tq.Layer(tq.config(H, kb, vb, seed=351, layer=kb, value_mode=tq.VAL_MSE))
    pool = layer.new_pool(45)
    tq.compress_kv(layer, torch.from_numpy(K).to("cuda", torch.bfloat16),
                   torch.from_numpy(V).to("cuda", torch.bfloat16), torch.from_numpy(slots).cuda(), pool)
    q_slots = slots.copy()
    q_slots[rng.choice(np.arange(64, n), 9, replace=False)] = -1
    tdt = torch.float32 if out_dtype == "f32" else torch.bfloat16
    kd, vd = tq.decompress_kv(layer, pool, torch.from_numpy(q_slots).cuda(), out_dtype=tdt)
    torch.cuda.synchronize()
    kd, vd = kd.float().cpu().numpy(), vd.float().cpu().numpy()
    st = parity.ostate.LayerState(351, kb, H, 128, kb, vb, 32, value_mode="mse")
    layout = parity.lay.StoreLayout(128, kb, vb, 32, value_mode="mse")
    kr, vr = odec.decompress(pool.cpu().numpy(), layout, H, q_slots, st)
    neg = q_slots < 0
    assert not kd[neg].any() and not vd[neg].any()
    for got, ref, name in ((kd, kr, "K"), (vd, vr, "V")):
        err = np.abs(got - ref)
        scale = np.abs(ref).max(axis=-1, keepdims=True) + 1e-30
        if out_dtype == "f32":
            print(name, "max err / row max %.2e, rel L2 %.2e" % ((err / scale).max(), parity.rel_l2(got, ref)))
            assert (err / scale).max() <= 2e-6 and parity.rel_l2(got, ref) <= 1e-6
        else:
            assert np.all(err <= np.abs(ref) * 2.0 ** -8 + 1e-6 * scale), name
    layer.close()


@pytest.mark.parametrize("kb,vb,n,offset", [(4, 4, 2000, 37), (3, 2, 1000, 0), (2, 3, 777, 16), (1, 4, 500, 5)])
def test_compress_page_runs(kb, vb, n, offset):
    """bf16 runs of consecutive slots: whole aligned pages (stored whole), a ragged
    last tile, and runs that start mid-page (every tile scattered token by token)."""
    torch = _torch()
    say("compress page runs", kb, vb, n, offset)
    K, V = synth.kv_host(150 + kb * 10 + vb, n, 8, outliers=4)
    slots = np.arange(n, dtype=np.int64) + offset
    nb = (n + offset + 15) // 16 + 1
    gpu = _gpu_compress(torch, K, V, slots, nb, 8, kb, vb, 220, layer=kb * vb)
    st, layout, pool, res = parity.oracle_store(K, V, slots, nb, 8, kb, vb, 220, layer=kb * vb)
    _check_compress(gpu, res, st, layout, 8, slots, V, kb, vb)
    # pages before the run and after it are untouched
    first, last = offset // 16, (n + offset - 1) // 16
    assert not gpu[:first * 8 * layout.block_bytes].any()
    assert not gpu[(last + 1) * 8 * layout.block_bytes:].any()


def test_compress_full_size_sampled():
    """1,048,576 tokens x 8 KV heads bf16 (K2+QJL / V3), checked on 2048 sampled tokens."""
    torch = _torch()
    say("compress 1M tokens x 8 heads")
    N, H = 1 << 20, 8
    k, v = synth.kv_device(103, N, H)
    layer = tq.Layer(tq.config(H, 2, 3, seed=203))
    pool = layer.new_pool(N // 16)
    slots = torch.arange(N, dtype=torch.int64, device="cuda")
    tq.compress_kv(layer, k, v, slots, pool)
    torch.cuda.synchronize()
    idx = np.sort(np.random.default_rng(0).choice(N, 2048, replace=False))
    ti = torch.from_numpy(idx).cuda()
    K = k[ti].float().cpu().numpy()
    V = v[ti].float().cpu().numpy()
    lay_bytes = layer.block_bytes * H
    # gather the sampled tokens' blocks from the GPU pool
    blocks = np.unique(idx // 16)
    sub = pool.view(-1, lay_bytes)[torch.from_numpy(blocks).cuda()].cpu().numpy().ravel()
    remap = {b: i for i, b in enumerate(blocks)}
    local = np.array([remap[s // 16] * 16 + s % 16 for s in idx])
    st, layout, opool, res = parity.oracle_store(K, V, local, len(blocks), H, 2, 3, 203)
    _check_compress(sub, res, st, layout, H, local, V, 2, 3)
    layer.close()


def test_compress_bypass_bit_exact():
    """Bypass layers store the bf16 key rows and the dim-major value table: the
    GPU pool equals the oracle's byte for byte (shuffled slots, skipped tokens,
    untouched slots left as they were)."""
    torch = _torch()
    say("compress bypass")
    n, H, nb = 300, 4, 30
    K, V = synth.kv_host(280, n, H, outliers=4)
    rng = np.random.default_rng(280)
    slots = rng.permutation(nb * 16)[:n].astype(np.int64)
    slots[rng.choice(n, 10, replace=False)] = -1
    layer = tq.Layer(tq.config(H, seed=280, bypass=True))
    pool = layer.new_pool(nb)
    tq.compress_kv(layer, torch.from_numpy(K).to("cuda", torch.bfloat16),
                   torch.from_numpy(V).to("cuda", torch.bfloat16), torch.from_numpy(slots).cuda(), pool)
    torch.cuda.synchronize()
    got = pool.cpu().numpy()
    layer.close()
    _, _, ref, _ = parity.oracle_store(None, None, slots, nb, H, 4, 4, 280, bypass=True,
                                       K_bits16=synth.bf16_bits(K), V_bits16=synth.bf16_bits(V))
    assert got.shape == ref.shape
    assert np.array_equal(got, ref), int(np.count_nonzero(got != ref))


# -------------------------------------------------------------------- decode
def _gpu_decode(torch, layer_cfg, pool_np, q, table, lens, max_len, out_dtype="f32", num_splits=0,
                scale=0.0, q_dtype="bf16"):
    layer = tq.Layer(layer_cfg)
    pool = torch.from_numpy(pool_np).cuda()
    qdt = torch.bfloat16 if q_dtype == "bf16" else torch.float32
    qt = torch.from_numpy(np.ascontiguousarray(q)).to("cuda", qdt)
    bt = torch.from_numpy(np.ascontiguousarray(table, dtype=np.int32)).cuda()
    sl = torch.from_numpy(np.ascontiguousarray(lens, dtype=np.int32)).cuda()
    odt = torch.bfloat16 if out_dtype == "bf16" else torch.float32
    out = tq.decode_attn(layer, qt, pool, bt, sl, max_len, out_dtype=odt, num_splits=num_splits,
                         softmax_scale=scale)
    torch.cuda.synchronize()
    res = out.float().cpu().numpy()
    layer.close()
    return res


def _decode_case(torch, B, Hq, Hkv, lens, kb, vb, seed, table_kind="random", q_dtype="bf16",
                 outliers=4, out_dtypes=("f32", "bf16"), num_splits=0, scale=0.0, layer=0, bypass=False,
                 fill=0, value_mode=0, key_mode=0, orders=(None,)):
    """orders: split-K item orders to run (TQ_DECODE_WORK_LIST values, None = automatic);
    every order must give the same output bit for bit."""
    lens = np.asarray(lens, dtype=np.int32)
    maxb = max(1, (int(lens.max()) + 15) // 16)
    table = synth.block_table(seed, B, maxb, table_kind)
    nblk = B * maxb
    K, V, slots = [], [], []
    for b in range(B):
        kk, vv = synth.kv_host(seed * 1000 + b, int(lens[b]), Hkv, outliers=outliers,
                               dtype="bf16" if q_dtype == "bf16" else "f32")
        pos = np.arange(int(lens[b]))
        K.append(kk)
        V.append(vv)
        slots.append(table[b][pos // 16].astype(np.int64) * 16 + pos % 16)
    K = np.concatenate(K) if K else np.zeros((0, Hkv, 128), np.float32)
    V = np.concatenate(V) if V else np.zeros((0, Hkv, 128), np.float32)
    slots = np.concatenate(slots)
    if bypass:
        st, layout, pool, _ = parity.oracle_store(None, None, slots, nblk, Hkv, 4, 4, seed, bypass=True,
                                                  K_bits16=synth.bf16_bits(K), V_bits16=synth.bf16_bits(V),
                                                  fill=fill)
    else:
        st, layout, pool, _ = parity.oracle_store(K, V, slots, nblk, Hkv, kb, vb, seed, layer=layer, keep=False,
                                                  fill=fill, value_mode="mse" if value_mode else "group",
                                                  key_mode=("qjl", "mse", "mse_nc")[key_mode])
    q = synth.queries_host(seed, B, Hq, dtype=q_dtype)
    ref = parity.oracle_decode(q.astype(np.float64), pool, layout, Hkv, table, lens, st,
                               scale=scale if scale else None)
    cfg = tq.config(Hkv, kb, vb, seed=seed, layer=layer, bypass=bypass, value_mode=value_mode, key_mode=key_mode)
    results = {}
    for od in out_dtypes:
        first = None
        for order in orders:
            saved = os.environ.pop("TQ_DECODE_WORK_LIST", None)
            try:
                if order is not None:
                    os.environ["TQ_DECODE_WORK_LIST"] = order
                got = _gpu_decode(torch, cfg, pool, q, table, lens, int(lens.max()), od, num_splits, scale,
                                  q_dtype=q_dtype)
            finally:
                os.environ.pop("TQ_DECODE_WORK_LIST", None)
                if saved is not None:
                    os.environ["TQ_DECODE_WORK_LIST"] = saved
            results[od], _ = parity.assert_decode_ok(got, ref, od, label="order %s" % order)
            if first is None:
                first = got
            else:
                assert np.array_equal(got.view(np.uint32), first.view(np.uint32)), ("orders differ", order)
    return results


@pytest.mark.parametrize("bypass,kb,vb,value_mode,key_mode", [
    (False, 3, 3, 0, 0), (True, 4, 4, 0, 0), (False, 2, 3, 1, 0), (False, 4, 2, 0, 2)])
def test_decode_work_list_matches_plain_order(bypass, kb, vb, value_mode, key_mode):
    """Ragged batches through the split-K work list and through the plain item order:
    the same output bit for bit (each item's arithmetic does not depend on where
    it sits in the grid) and parity with the oracle.  300 sequences (two passes of
    the per-wave count), empty and one-token sequences, lengths on and around the
    split boundary, 64-token splits (a grid of 9,600 workgroups), 2 KV heads; group
    or codebook-coded values, keys with QJL or the compact page without it, and
    uncompressed layers."""
    torch = _torch()
    say("decode work list vs plain order", bypass, kb, vb, value_mode, key_mode)
    rng = np.random.default_rng(63)
    lens = rng.integers(1, 300, 300).astype(np.int32)
    lens[::11] = 0
    lens[[3, 4, 5, 6]] = [1, 64, 65, 128]
    lens[200] = 1000
    _decode_case(torch, 300, 8, 2, lens, kb, vb, 291, num_splits=16, out_dtypes=("f32",), bypass=bypass,
                 value_mode=value_mode, key_mode=key_mode, orders=("1", "0"))


def test_decode_tiny_fp32():
    """1 head, 1024 tokens, fp32 q/K/V, K2/V3, identity table."""
    torch = _torch()
    say("decode tiny fp32")
    _decode_case(torch, 1, 1, 1, [1024], 2, 3, 201, table_kind="identity", q_dtype="f32", outliers=0)


def test_decode_llama_layer_full():
    """B=16, 32/8 heads, ctx 4096, bf16 with outliers, K4/V4, identity table."""
    torch = _torch()
    say("decode B16 ctx4096 K4V4")
    _decode_case(torch, 16, 32, 8, [4096] * 16, 4, 4, 202, table_kind="identity")


def test_decode_long_context_full():
    """B=1, 32/8 heads, ctx 131072, bf16 with outliers, K3/V2, random block table."""
    torch = _torch()
    say("decode B1 ctx131072 K3V2")
    _decode_case(torch, 1, 32, 8, [131072], 3, 2, 204, out_dtypes=("f32",))


@pytest.mark.parametrize("kb,vb", [(4, 4), (4, 3), (3, 3), (3, 2), (2, 3), (2, 2), (1, 3), (1, 4)])
def test_decode_ragged_bits(kb, vb):
    """Ragged lengths with tails, a zero-length row, every supported bit pair."""
    torch = _torch()
    say("decode ragged", kb, vb)
    _decode_case(torch, 6, 8, 2, [1, 0, 17, 64, 300, 1000], kb, vb, 220 + kb * 10 + vb)


@pytest.mark.parametrize("rep", [1, 2, 8])
def test_decode_gqa_ratios(rep):
    torch = _torch()
    say("decode rep", rep)
    _decode_case(torch, 3, 2 * rep, 2, [33, 513, 257], 4, 3, 230 + rep)


@pytest.mark.parametrize("splits", [1, 3, 64])
def test_decode_forced_splits_and_scale(splits):
    torch = _torch()
    say("decode splits", splits)
    _decode_case(torch, 2, 8, 2, [700, 1500], 3, 3, 240 + splits, num_splits=splits, scale=0.05)


@pytest.mark.parametrize("rep,bypass", [(1, False), (8, False), (8, True)])
def test_decode_many_splits_per_head_combine(rep, bypass):
    """A small batch over many splits (40 requested, 21 made): the combine runs one
    workgroup per query head, the splits shared by four lane quarters. GQA ratios 1
    and 8, a one-split row (three empty quarters) and an empty row."""
    torch = _torch()
    say("decode per-head combine", rep, bypass)
    kb, vb = (0, 0) if bypass else (4, 4)
    _decode_case(torch, 3, 2 * rep, 2, [0, 15, 2600], kb, vb, 290 + rep, num_splits=40, bypass=bypass)


def test_decode_split_cap():
    """One requested split over 20000 tokens: the library raises the split count so
    that no split spans more than 4096 tokens (five splits here)."""
    torch = _torch()
    say("decode split cap")
    _decode_case(torch, 1, 8, 2, [20000], 4, 4, 245, num_splits=1, out_dtypes=("f32",))


def test_decode_bypass_layer():
    torch = _torch()
    say("decode bypass")
    _decode_case(torch, 3, 8, 2, [16, 200, 1031], 0, 0, 250, bypass=True)


@pytest.mark.parametrize("rep,q_dtype,splits", [(1, "bf16", 0), (2, "f32", 3), (8, "bf16", 0), (4, "f32", 64)])
def test_decode_bypass_variants(rep, q_dtype, splits):
    """Bypass layers: every GQA ratio, float32 and bf16 queries, forced splits,
    ragged lengths with a zero-length row and page tails."""
    torch = _torch()
    say("decode bypass", rep, q_dtype, splits)
    _decode_case(torch, 4, 2 * rep, 2, [0, 15, 333, 2100], 0, 0, 260 + rep, q_dtype=q_dtype, num_splits=splits,
                 bypass=True)


@pytest.mark.parametrize("bypass", [False, True])
def test_decode_empty_table(bypass):
    """Every sequence empty and a block table of zero blocks per row: no split
    kernel runs and the output is exact zeros."""
    torch = _torch()
    say("decode empty table, bypass", bypass)
    layer = tq.Layer(tq.config(2, 4, 4, seed=1, bypass=bypass))
    pool = layer.new_pool(1)
    q = torch.randn(3, 8, 128, device="cuda").to(torch.bfloat16)
    bt = torch.zeros((3, 1), dtype=torch.int32, device="cuda")  # passed with 0 blocks per row
    sl = torch.zeros(3, dtype=torch.int32, device="cuda")
    out = torch.full((3, 8, 128), float("nan"), device="cuda")
    ws = tq.new_workspace(layer, 3, 8, 0)
    st = tq.lib().tq_decode_attn(layer.handle, tq._ptr(q), tq._dtype_code(q), 3, 8, tq._ptr(pool), 1,
                                 tq._ptr(bt), 0, tq._ptr(sl), 0, 0.0, 0, tq._ptr(out), tq._dtype_code(out),
                                 tq._ptr(ws), ws.numel(), tq._stream(None))
    assert st == 0, tq.lib().tq_last_error().decode()
    torch.cuda.synchronize()
    assert torch.count_nonzero(out).item() == 0
    layer.close()


@pytest.mark.parametrize("bypass", [False, True])
def test_decode_ignores_unwritten_slots(bypass):
    """Pool bytes all 0xFF before the records are written: the slots past each
    context end hold NaN norms, scales, zeros and values, which must not reach
    the output (page and chunk tails of every length class)."""
    torch = _torch()
    say("decode unwritten slots, bypass", bypass)
    _decode_case(torch, 5, 8, 2, [1, 17, 40, 129, 1000], 3, 2, 270, bypass=bypass, fill=0xFF)


def test_decode_ragged_serving_sampled():
    """64 sequences with lengths U{512..32768}, 32/8 heads; the oracle fills only
    sequences 0, 31, 63 and the outputs of those are compared."""
    torch = _torch()
    say("decode ragged serving sample")
    B, Hq, Hkv = 64, 32, 8
    lens = synth.ragged_lengths(505, B, 512, 32768)
    maxb = (int(lens.max()) + 15) // 16
    table = synth.block_table(305, B, maxb, "random")
    sample = [0, 31, 63]
    for kb, vb in [(4, 4), (3, 2)]:
        K, V, slots = [], [], []
        for b in sample:
            kk, vv = synth.kv_host(105000 + b, int(lens[b]), Hkv, outliers=4)
            pos = np.arange(int(lens[b]))
            K.append(kk)
            V.append(vv)
            slots.append(table[b][pos // 16].astype(np.int64) * 16 + pos % 16)
        K, V, slots = np.concatenate(K), np.concatenate(V), np.concatenate(slots)
        st, layout, pool, _ = parity.oracle_store(K, V, slots, B * maxb, Hkv, kb, vb, 205, layer=kb + vb,
                                                  keep=False)
        q = synth.queries_host(205, B, Hq)
        sub_lens = np.zeros(B, np.int32)
        sub_lens[sample] = lens[sample]
        ref = parity.oracle_decode(q.astype(np.float64), pool, layout, Hkv, table, sub_lens, st)
        got = _gpu_decode(torch, tq.config(Hkv, kb, vb, seed=205, layer=kb + vb), pool, q, table, lens,
                          int(lens.max()))
        parity.assert_decode_ok(got[sample], ref[sample], "f32", "ragged serving %d/%d" % (kb, vb))


def _end_to_end(torch, K, V, slots, table, lens, Hq, Hkv, kb, vb, seed, key_mode=0, rotation=0, label="",
                value_mode=0):
    """GPU compress, then: the GPU store against the oracle's (compress protocol);
    GPU decode of the GPU store against the oracle decode of the same store, and
    of the oracle store likewise (decode protocol, whole output and worst row);
    and GPU compress -> GPU decode against oracle compress -> oracle decode
    (whole output within the benchmark spec's 1e-3, worst row reported)."""
    B = len(lens)
    T = int(lens.max())
    nblk = table.size
    rot = "haar" if rotation == tq.ROT_HAAR else "hadamard"
    st, layout, opool, res = parity.oracle_store(K, V, slots, nblk, Hkv, kb, vb, seed,
                                                 key_mode=KEY_MODE_NAMES[key_mode], rotation_kind=rot,
                                                 value_mode="mse" if value_mode else "group")
    q = synth.queries_host(seed, B, Hq)
    ref = parity.oracle_decode(q.astype(np.float64), opool, layout, Hkv, table, lens, st)
    layer = tq.Layer(tq.config(Hkv, kb, vb, seed=seed, key_mode=key_mode, rotation=rotation, value_mode=value_mode))
    pool = layer.new_pool(nblk)
    tq.compress_kv(layer, torch.from_numpy(K).to("cuda", torch.bfloat16),
                   torch.from_numpy(V).to("cuda", torch.bfloat16), torch.from_numpy(slots).cuda(), pool)
    qt = torch.from_numpy(q).to("cuda", torch.bfloat16)
    bt = torch.from_numpy(table).cuda()
    sl = torch.from_numpy(lens).cuda()
    out = tq.decode_attn(layer, qt, pool, bt, sl, T)
    out_o = tq.decode_attn(layer, qt, torch.from_numpy(opool).cuda(), bt, sl, T)
    torch.cuda.synchronize()
    gpu_pool = pool.cpu().numpy()
    _check_compress(gpu_pool, res, st, layout, Hkv, slots, V, kb, vb)
    ref_g = parity.oracle_decode(q.astype(np.float64), gpu_pool, layout, Hkv, table, lens, st)
    parity.assert_decode_ok(out.cpu().numpy(), ref_g, "f32", label + " GPU store")
    parity.assert_decode_ok(out_o.cpu().numpy(), ref, "f32", label + " oracle store")
    whole, worst, at = parity.decode_errors(out.cpu().numpy(), ref)
    print("%s end to end rel L2 %.3e, worst (b, h) %s %.3e" % (label, whole, at, worst), flush=True)
    assert whole <= 1e-3, whole
    layer.close()


def test_end_to_end_gpu_compress_then_decode():
    """GPU compress -> GPU decode against oracle compress -> oracle decode."""
    torch = _torch()
    say("end to end")
    B, Hq, Hkv, T = 4, 16, 4, 777
    lens = np.full(B, T, np.int32)
    maxb = (T + 15) // 16
    table = synth.block_table(260, B, maxb, "random")
    K, V = synth.kv_host(160, B * T, Hkv, outliers=4)
    pos = np.tile(np.arange(T), B)
    seq = np.repeat(np.arange(B), T)
    slots = table[seq, pos // 16].astype(np.int64) * 16 + pos % 16
    _end_to_end(torch, K, V, slots, table, lens, Hq, Hkv, 3, 3, 260, label="K3/V3")


def test_end_to_end_one_bit_keys():
    """1-bit key codebook (+-0.7979) with QJL signs, 2-bit values: GPU compress -> GPU
    decode against the oracle (the matrix-core compressor and the 1-bit decode table)."""
    torch = _torch()
    say("end to end K1/V2")
    B, Hq, Hkv, T = 3, 32, 8, 600
    lens = np.array([T, 333, 1], np.int32)
    maxb = (T + 15) // 16
    table = synth.block_table(262, B, maxb, "random")
    K, V = synth.kv_host(162, B * T, Hkv, outliers=4)
    pos = np.tile(np.arange(T), B)
    seq = np.repeat(np.arange(B), T)
    slots = table[seq, pos // 16].astype(np.int64) * 16 + pos % 16
    _end_to_end(torch, K, V, slots, table, lens, Hq, Hkv, 1, 2, 262, label="K1/V2")


KEY_MODE_NAMES = {tq.KEY_QJL: "qjl", tq.KEY_MSE: "mse", tq.KEY_MSE_NC: "mse_nc"}


@pytest.mark.parametrize("key_mode,kb,vb,n,dtype,value_mode,scattered", [
    (tq.KEY_MSE, 4, 4, 700, "bf16", "group", False), (tq.KEY_MSE_NC, 3, 2, 700, "bf16", "group", False),
    (tq.KEY_MSE_NC, 2, 3, 1024, "f32", "group", False), (tq.KEY_MSE, 3, 3, 40, "bf16", "group", False),
    (tq.KEY_MSE_NC, 1, 3, 500, "bf16", "group", False), (tq.KEY_MSE, 1, 2, 100, "f32", "group", False),
    (tq.KEY_MSE, 4, 3, 613, "bf16", "group", True), (tq.KEY_MSE_NC, 2, 4, 509, "bf16", "mse", True),
    (tq.KEY_MSE, 3, 2, 300, "f32", "group", True)])
def test_compress_key_modes(key_mode, kb, vb, n, dtype, value_mode, scattered):
    """Keys without the residual projection (plain and norm-corrected magnitude):
    the matrix-core compressor (bf16: whole pages and a ragged last tile) and the
    per-token one (fp32 inputs; a 40-token append).  Scattered: every page starts
    at offset 5 of a shuffled block, so no 16-token tile fills one page and each
    record goes through the token-by-token store."""
    torch = _torch()
    say("compress key mode", key_mode, kb, vb, n, dtype, value_mode, scattered)
    H = 8 if dtype == "bf16" else 1
    K, V = synth.kv_host(170 + key_mode, n, H, dtype=dtype, outliers=4 if dtype == "bf16" else 0)
    if scattered:
        pos = np.arange(n) + 5
        perm = np.random.default_rng(171 + kb).permutation((n + 5 + 15) // 16)
        slots = (perm[pos // 16] * 16 + pos % 16).astype(np.int64)
        nb = len(perm)
    else:
        slots = np.arange(n, dtype=np.int64)
        nb = (n + 15) // 16
    vm = tq.VAL_MSE if value_mode == "mse" else tq.VAL_GROUP
    gpu = _gpu_compress(torch, K, V, slots, nb, H, kb, vb, 230, layer=key_mode, dtype=dtype, key_mode=key_mode,
                        value_mode=vm)
    st, layout, pool, res = parity.oracle_store(K, V, slots, nb, H, kb, vb, 230, layer=key_mode,
                                                key_mode=KEY_MODE_NAMES[key_mode], value_mode=value_mode)
    _check_compress(gpu, res, st, layout, H, slots, V, kb, vb)
    # no residual signs and gamma 0 in the store
    for h in range(H):
        f = parity.fields_at(gpu, layout, H, slots, h)
        assert not np.asarray(f["z"]).any() and not np.asarray(f["g16"], np.float64).any()


@pytest.mark.parametrize("key_mode", [tq.KEY_MSE, tq.KEY_MSE_NC])
def test_end_to_end_key_modes(key_mode):
    """GPU compress -> GPU decode against the oracle for the key modes without QJL
    (the decode kernels read the same page layout; gamma 0 removes the QJL term)."""
    torch = _torch()
    say("end to end key mode", key_mode)
    B, Hq, Hkv, T = 3, 16, 4, 613
    lens = np.array([T, 400, 97], np.int32)
    maxb = (T + 15) // 16
    table = synth.block_table(270 + key_mode, B, maxb, "random")
    K, V = synth.kv_host(180 + key_mode, B * T, Hkv, outliers=4)
    pos = np.tile(np.arange(T), B)
    seq = np.repeat(np.arange(B), T)
    slots = table[seq, pos // 16].astype(np.int64) * 16 + pos % 16
    _end_to_end(torch, K, V, slots, table, lens, Hq, Hkv, 4, 3, 270, key_mode=key_mode,
                label="key mode %d" % key_mode)


@pytest.mark.parametrize("kb,vb,n,dtype,key_mode", [
    (4, 4, 700, "bf16", tq.KEY_QJL), (2, 3, 500, "bf16", tq.KEY_MSE_NC), (3, 2, 300, "f32", tq.KEY_QJL)])
def test_compress_hadamard_rotation(kb, vb, n, dtype, key_mode):
    """Randomised Hadamard layers: the matrix-core compressor's one-pass +-1 rotation
    (bf16, whole pages and a ragged tile) and the per-token compressor (fp32)."""
    torch = _torch()
    say("compress hadamard", kb, vb, n, dtype, key_mode)
    H = 8 if dtype == "bf16" else 2
    K, V = synth.kv_host(190 + kb, n, H, dtype=dtype, outliers=4)
    slots = np.arange(n, dtype=np.int64)
    nb = (n + 15) // 16
    gpu = _gpu_compress(torch, K, V, slots, nb, H, kb, vb, 240, layer=kb, dtype=dtype, key_mode=key_mode,
                        rotation=tq.ROT_HADAMARD)
    st, layout, pool, res = parity.oracle_store(K, V, slots, nb, H, kb, vb, 240, layer=kb,
                                                key_mode=KEY_MODE_NAMES[key_mode], rotation_kind="hadamard")
    _check_compress(gpu, res, st, layout, H, slots, V, kb, vb)


def test_end_to_end_hadamard_rotation():
    """GPU compress -> GPU decode on a randomised Hadamard layer against the oracle
    (the decode prologue and epilogue use the layer's R as stored)."""
    torch = _torch()
    say("end to end hadamard")
    B, Hq, Hkv, T = 2, 32, 8, 1000
    lens = np.array([T, 333], np.int32)
    maxb = (T + 15) // 16
    table = synth.block_table(280, B, maxb, "random")
    K, V = synth.kv_host(200, B * T, Hkv, outliers=4)
    pos = np.tile(np.arange(T), B)
    seq = np.repeat(np.arange(B), T)
    slots = table[seq, pos // 16].astype(np.int64) * 16 + pos % 16
    _end_to_end(torch, K, V, slots, table, lens, Hq, Hkv, 4, 4, 280, rotation=tq.ROT_HADAMARD, label="hadamard")


@pytest.mark.parametrize("kb,vb,key_mode,rotation,out_dtype,slot_kind", [
    (4, 4, tq.KEY_QJL, tq.ROT_HAAR, "f32", "shuffled"), (3, 2, tq.KEY_MSE_NC, tq.ROT_HADAMARD, "f32", "shuffled"),
    (2, 3, tq.KEY_QJL, tq.ROT_HAAR, "bf16", "shuffled"), (1, 3, tq.KEY_QJL, tq.ROT_HADAMARD, "f32", "shuffled"),
    (4, 4, tq.KEY_QJL, tq.ROT_HAAR, "f32", "pages"), (3, 2, tq.KEY_MSE_NC, tq.ROT_HADAMARD, "bf16", "pages"),
    (2, 3, tq.KEY_QJL, tq.ROT_HAAR, "bf16", "pages"), (3, 4, tq.KEY_MSE, tq.ROT_HAAR, "f32", "pages")])
def test_decompress_matches_oracle(kb, vb, key_mode, rotation, out_dtype, slot_kind):
    """Keys and values reconstructed from a GPU-written store against the oracle's
    reconstruction of the same bytes.  Shuffled slots (every tile read record by
    record), or consecutive slots (whole pages through the kernel's page ring, a
    ragged last tile); some read slots negative (zero rows, and a tile that is no
    longer one whole page)."""
    from oracle import decompress as odec
    torch = _torch()
    say("decompress", kb, vb, key_mode, rotation, out_dtype, slot_kind)
    H, n = 8, 613
    K, V = synth.kv_host(300 + kb, n, H, outliers=4)
    rng = np.random.default_rng(kb)
    if slot_kind == "pages":
        slots = np.arange(n, dtype=np.int64)
    else:
        slots = rng.permutation(48 * 16)[:n].astype(np.int64)
    layer = tq.Layer(tq.config(H, kb, vb, seed=290, layer=kb, key_mode=key_mode, rotation=rotation))
    pool = layer.new_pool(48)
    tq.compress_kv(layer, torch.from_numpy(K).to("cuda", torch.bfloat16),
                   torch.from_numpy(V).to("cuda", torch.bfloat16), torch.from_numpy(slots).cuda(), pool)
    q_slots = slots.copy()
    q_slots[rng.choice(n, 9, replace=False)] = -1
    tdt = torch.float32 if out_dtype == "f32" else torch.bfloat16
    kd, vd = tq.decompress_kv(layer, pool, torch.from_numpy(q_slots).cuda(), out_dtype=tdt)
    torch.cuda.synchronize()
    kd, vd = kd.float().cpu().numpy(), vd.float().cpu().numpy()
    st = parity.ostate.LayerState(290, kb, H, 128, kb, vb, 32, key_mode=KEY_MODE_NAMES[key_mode],
                                  rotation_kind="haar" if rotation == tq.ROT_HAAR else "hadamard")
    layout = parity.lay.StoreLayout(128, kb, vb, 32, qjl=key_mode == tq.KEY_QJL)
    kr, vr = odec.decompress(pool.cpu().numpy(), layout, H, q_slots, st)
    neg = q_slots < 0
    assert not kd[neg].any() and not vd[neg].any()
    for got, ref, name in ((kd, kr, "K"), (vd, vr, "V")):
        err = np.abs(got - ref)
        scale = np.abs(ref).max(axis=-1, keepdims=True) + 1e-30
        if out_dtype == "f32":
            print(name, "max err / row max %.2e, rel L2 %.2e" % ((err / scale).max(), parity.rel_l2(got, ref)))
            assert (err / scale).max() <= 2e-6 and parity.rel_l2(got, ref) <= 1e-6
        else:
            # bf16 of the fp32 result: within one bf16 rounding of the exact value
            assert np.all(err <= np.abs(ref) * 2.0 ** -8 + 1e-6 * scale), name
            print(name, "bf16 rel L2 %.2e" % parity.rel_l2(got, ref))
    layer.close()


@pytest.mark.parametrize("n", [1, 5, 16, 63, 64, 65, 80])
@pytest.mark.parametrize("kb,vb,key_mode,out_dtype,slot_kind", [
    (4, 4, tq.KEY_QJL, "bf16", "shuffled"), (3, 2, tq.KEY_MSE_NC, "f32", "shuffled"),
    (4, 4, tq.KEY_QJL, "f32", "pages")])
def test_decompress_short_and_boundary_lengths(n, kb, vb, key_mode, out_dtype, slot_kind):
    """Decompress at the lengths around the switch between the per-tile kernel
    (fewer than 64 tokens) and the persistent ring kernel (64 and more: exactly
    four tiles, then a ragged last tile of one or sixteen tokens), against the
    oracle's reconstruction.  Shuffled slots with one negative read slot, or
    consecutive slots (whole pages through the page ring) whose last read slot
    is negative."""
    from oracle import decompress as odec
    torch = _torch()
    say("decompress length", n, kb, vb, key_mode, out_dtype, slot_kind)
    H = 4
    K, V = synth.kv_host(500 + n, 96, H, outliers=4)
    rng = np.random.default_rng(n)
    if slot_kind == "pages":
        slots = np.arange(96, dtype=np.int64)
    else:
        slots = rng.permutation(12 * 16)[:96].astype(np.int64)
    layer = tq.Layer(tq.config(H, kb, vb, seed=501, layer=kb, key_mode=key_mode))
    pool = layer.new_pool(12)
    tq.compress_kv(layer, torch.from_numpy(K).to("cuda", torch.bfloat16),
                   torch.from_numpy(V).to("cuda", torch.bfloat16), torch.from_numpy(slots).cuda(), pool)
    if slot_kind == "pages":
        q_slots = slots[:n].copy()
        q_slots[n - 1] = -1
    else:
        q_slots = slots[rng.permutation(96)[:n]].copy()
        q_slots[rng.integers(n)] = -1
    tdt = torch.float32 if out_dtype == "f32" else torch.bfloat16
    kd, vd = tq.decompress_kv(layer, pool, torch.from_numpy(q_slots).cuda(), out_dtype=tdt)
    torch.cuda.synchronize()
    kd, vd = kd.float().cpu().numpy(), vd.float().cpu().numpy()
    assert kd.shape == (n, H, 128) and vd.shape == (n, H, 128)
    st = parity.ostate.LayerState(501, kb, H, 128, kb, vb, 32, key_mode=KEY_MODE_NAMES[key_mode])
    layout = parity.lay.StoreLayout(128, kb, vb, 32, qjl=key_mode == tq.KEY_QJL)
    kr, vr = odec.decompress(pool.cpu().numpy(), layout, H, q_slots, st)
    neg = q_slots < 0
    assert not kd[neg].any() and not vd[neg].any()
    for got, ref, name in ((kd, kr, "K"), (vd, vr, "V")):
        err = np.abs(got - ref)
        scale = np.abs(ref).max(axis=-1, keepdims=True) + 1e-30
        if out_dtype == "f32":
            assert (err / scale).max() <= 2e-6, name
        else:
            assert np.all(err <= np.abs(ref) * 2.0 ** -8 + 1e-6 * scale), name
    layer.close()


@pytest.mark.parametrize("case", range(12))
def test_decompress_random_configurations(case):
    """Seeded random decompress cases: KV heads, bit widths, key mode, value mode,
    rotation, output type, input length (both kernels), and read slots that mix
    runs of whole pages, a run starting inside a page, shuffled slots, repeats
    and negative slots; GPU-written store, GPU reconstruction against the
    oracle's reconstruction of the same bytes."""
    from oracle import decompress as odec
    torch = _torch()
    rng = np.random.default_rng(4000 + case)
    H = int(rng.choice([1, 2, 4, 8]))
    kb, vb = int(rng.choice([1, 2, 3, 4])), int(rng.choice([2, 3, 4]))
    value_mode = int(rng.choice([tq.VAL_GROUP, tq.VAL_MSE]))
    key_mode = int(rng.choice([tq.KEY_QJL, tq.KEY_MSE, tq.KEY_MSE_NC]))
    rotation = int(rng.choice([tq.ROT_HAAR, tq.ROT_HADAMARD]))
    out_dtype = str(rng.choice(["f32", "bf16"]))
    n_blocks = 40
    n = int(rng.choice([int(rng.integers(1, 64)), int(rng.integers(64, 600))]))
    say("random decompress", case, dict(H=H, kb=kb, vb=vb, key_mode=key_mode, value_mode=value_mode,
                                         rotation=rotation, out=out_dtype, n=n))
    # every slot of the pool written once, in a shuffled order
    wslots = rng.permutation(n_blocks * 16).astype(np.int64)
    K, V = synth.kv_host(4100 + case, n_blocks * 16, H, outliers=4)
    layer = tq.Layer(tq.config(H, kb, vb, seed=4200 + case, layer=case, key_mode=key_mode, rotation=rotation,
                               value_mode=value_mode))
    pool = layer.new_pool(n_blocks)
    tq.compress_kv(layer, torch.from_numpy(K).to("cuda", torch.bfloat16),
                   torch.from_numpy(V).to("cuda", torch.bfloat16), torch.from_numpy(wslots).cuda(), pool)
    # read slots: consecutive whole pages, a run from inside a page, shuffled, repeated, negative
    parts, left = [], n
    while left > 0:
        kind = int(rng.integers(4))
        m = min(left, int(rng.integers(1, 80)))
        if kind == 0:
            b0 = int(rng.integers(0, n_blocks - (m + 15) // 16 + 1)) if m <= n_blocks * 16 else 0
            parts.append(np.arange(b0 * 16, b0 * 16 + m) % (n_blocks * 16))
        elif kind == 1:
            s0 = int(rng.integers(0, n_blocks * 16 - m + 1))
            parts.append(np.arange(s0, s0 + m))
        elif kind == 2:
            parts.append(rng.integers(0, n_blocks * 16, m))
        else:
            parts.append(np.full(m, int(rng.integers(0, n_blocks * 16))))
        left -= m
    q_slots = np.concatenate(parts).astype(np.int64)[:n]
    q_slots[rng.random(n) < 0.03] = -1
    tdt = torch.float32 if out_dtype == "f32" else torch.bfloat16
    kd, vd = tq.decompress_kv(layer, pool, torch.from_numpy(q_slots).cuda(), out_dtype=tdt)
    torch.cuda.synchronize()
    kd, vd = kd.float().cpu().numpy(), vd.float().cpu().numpy()
    st = parity.ostate.LayerState(4200 + case, case, H, 128, kb, vb, 32, key_mode=KEY_MODE_NAMES[key_mode],
                                  rotation_kind="haar" if rotation == tq.ROT_HAAR else "hadamard",
                                  value_mode="mse" if value_mode == tq.VAL_MSE else "group")
    layout = parity.lay.StoreLayout(128, kb, vb, 32, qjl=key_mode == tq.KEY_QJL,
                                    value_mode="mse" if value_mode == tq.VAL_MSE else "group")
    kr, vr = odec.decompress(pool.cpu().numpy(), layout, H, q_slots, st)
    neg = q_slots < 0
    assert not kd[neg].any() and not vd[neg].any()
    for got, ref, name in ((kd, kr, "K"), (vd, vr, "V")):
        err = np.abs(got - ref)
        scale = np.abs(ref).max(axis=-1, keepdims=True) + 1e-30
        if out_dtype == "f32":
            assert (err / scale).max() <= 2e-6, name
        else:
            assert np.all(err <= np.abs(ref) * 2.0 ** -8 + 1e-6 * scale), name
    layer.close()


def test_decompress_full_size_sampled():
    """The headline store (16 x 4096 tokens x 8 KV heads, K4/V4, outlier channels,
    random block table) written by the GPU compressor, all 65,536 tokens
    reconstructed to bf16 in one launch in page order (every tile one whole page,
    as timed), checked on 1024 sampled tokens against the oracle's reconstruction
    of their pages gathered into a small store."""
    from oracle import decompress as odec
    torch = _torch()
    say("decompress full size")
    B, T, H, kb, vb, seed = 16, 4096, 8, 4, 4, 330
    N = B * T
    k, v = synth.kv_device(seed, N, H, outliers=4)
    layer = tq.Layer(tq.config(H, kb, vb, seed=seed))
    pool = layer.new_pool(N // 16)
    table = synth.block_table(seed, B, T // 16, "random")
    b_of = np.repeat(np.arange(B), T)
    pos = np.tile(np.arange(T), B)
    slots = table[b_of, pos // 16].astype(np.int64) * 16 + pos % 16
    slots_t = torch.from_numpy(slots).cuda()
    tq.compress_kv(layer, k, v, slots_t, pool)
    kd, vd = tq.decompress_kv(layer, pool, slots_t, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    idx = np.sort(np.random.default_rng(seed).choice(N, 1024, replace=False))
    lay_bytes = layer.block_bytes * H
    blocks = np.unique(slots[idx] // 16)
    sub = pool.view(-1, lay_bytes)[torch.from_numpy(blocks).cuda()].cpu().numpy().ravel()
    remap = {int(b): i for i, b in enumerate(blocks)}
    local = np.array([remap[int(x) // 16] * 16 + int(x) % 16 for x in slots[idx]], np.int64)
    st = parity.ostate.LayerState(seed, 0, H, 128, kb, vb, 32)
    layout = parity.lay.StoreLayout(128, kb, vb, 32)
    kr, vr = odec.decompress(sub, layout, H, local, st)
    ti = torch.from_numpy(idx).cuda()
    for got, ref, name in ((kd[ti].float().cpu().numpy(), kr, "K"), (vd[ti].float().cpu().numpy(), vr, "V")):
        scale = np.abs(ref).max(axis=-1, keepdims=True) + 1e-30
        # bf16 of the fp32 result: within one bf16 rounding of the exact value
        assert np.all(np.abs(got - ref) <= np.abs(ref) * 2.0 ** -8 + 1e-6 * scale), name
        print(name, "bf16 rel L2 %.2e" % parity.rel_l2(got, ref))
    layer.close()


def test_decompress_bypass_exact():
    """Bypass layers return their stored bf16 values bit for bit."""
    torch = _torch()
    say("decompress bypass")
    H, n = 4, 100
    K, V = synth.kv_host(310, n, H, outliers=4)
    slots = np.random.default_rng(3).permutation(8 * 16)[:n].astype(np.int64)
    layer = tq.Layer(tq.config(H, seed=311, bypass=True))
    pool = layer.new_pool(8)
    kt = torch.from_numpy(K).to("cuda", torch.bfloat16)
    vt = torch.from_numpy(V).to("cuda", torch.bfloat16)
    tq.compress_kv(layer, kt, vt, torch.from_numpy(slots).cuda(), pool)
    kd, vd = tq.decompress_kv(layer, pool, torch.from_numpy(slots).cuda(), out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(kd, kt) and torch.equal(vd, vt)
    layer.close()


def test_store_past_4gib():
    """A 4.6 GiB store with every record in its top 66 blocks, so that each page
    address is past 2^32 bytes: the GPU compress of those pages against the
    oracle, the decode over them and the decompress from them against the
    oracle on the same pages gathered into a small store."""
    from oracle import decompress as odec
    torch = _torch()
    say("store past 4 GiB")
    H, kb, vb, B, seed = 2, 4, 4, 2, 320
    layer = tq.Layer(tq.config(H, kb, vb, seed=seed))
    lay_bytes = layer.block_bytes * H
    nblk = int(4.6 * 2 ** 30) // lay_bytes + 1
    lens = np.array([300, 517], np.int32)
    maxb = (int(lens.max()) + 15) // 16
    rng = np.random.default_rng(seed)
    ids = (nblk - 1 - rng.permutation(B * maxb)).reshape(B, maxb).astype(np.int32)
    assert int(ids.min()) * lay_bytes > 2 ** 32
    N = int(lens.sum())
    K, V = synth.kv_host(seed + 1, N, H, outliers=4)
    seq = np.repeat(np.arange(B), lens)
    pos = np.concatenate([np.arange(n) for n in lens])
    slots = ids[seq, pos // 16].astype(np.int64) * 16 + pos % 16
    pool = layer.new_pool(nblk)
    assert pool.numel() > 2 ** 32
    tq.compress_kv(layer, torch.from_numpy(K).to("cuda", torch.bfloat16),
                   torch.from_numpy(V).to("cuda", torch.bfloat16), torch.from_numpy(slots).cuda(), pool)
    torch.cuda.synchronize()
    # the used pages, gathered into a small store with renumbered blocks
    used = np.unique(ids)
    remap = {int(b): i for i, b in enumerate(used)}
    sub = pool.view(-1, lay_bytes)[torch.from_numpy(used.astype(np.int64)).cuda()].cpu().numpy().ravel()
    local_slots = np.array([remap[int(x) // 16] * 16 + int(x) % 16 for x in slots], np.int64)
    local_ids = np.vectorize(lambda b: remap[int(b)])(ids).astype(np.int32)
    st, layout, _, res = parity.oracle_store(K, V, local_slots, len(used), H, kb, vb, seed)
    _check_compress(sub, res, st, layout, H, local_slots, V, kb, vb)
    # decode over the top of the store
    q = synth.queries_host(seed + 2, B, 4 * H)
    ref = parity.oracle_decode(q.astype(np.float64), sub, layout, H, local_ids, lens, st)
    out = tq.decode_attn(layer, torch.from_numpy(q).to("cuda", torch.bfloat16), pool, torch.from_numpy(ids).cuda(),
                         torch.from_numpy(lens).cuda(), int(lens.max()))
    torch.cuda.synchronize()
    parity.assert_decode_ok(out.float().cpu().numpy(), ref, "f32", "store past 4 GiB")
    # decompress from the top of the store
    kd, vd = tq.decompress_kv(layer, pool, torch.from_numpy(slots).cuda())
    torch.cuda.synchronize()
    kr, vr = odec.decompress(sub, layout, H, local_slots, st)
    for got, want, name in ((kd.cpu().numpy(), kr, "K"), (vd.cpu().numpy(), vr, "V")):
        assert parity.rel_l2(got, want) <= 1e-6, name
    del pool
    layer.close()


def test_decode_step_graph_capture():
    """Appending a token and decoding allocate and synchronise nothing, so the step
    can be captured in a HIP graph: every replay, with eager work between replays,
    gives the eager step's output bit for bit."""
    torch = _torch()
    say("graph capture of append + decode")
    B, Hq, Hkv, T = 4, 32, 8, 1000
    maxb = (T + 15) // 16
    table = synth.block_table(320, B, maxb, "random")
    K, V = synth.kv_host(320, B * T, Hkv, outliers=4)
    pos = np.tile(np.arange(T), B)
    seq = np.repeat(np.arange(B), T)
    slots = torch.from_numpy(table[seq, pos // 16].astype(np.int64) * 16 + pos % 16).cuda()
    kt = torch.from_numpy(K).to("cuda", torch.bfloat16)
    vt = torch.from_numpy(V).to("cuda", torch.bfloat16)
    layer = tq.Layer(tq.config(Hkv, 4, 4, seed=320))
    pool = layer.new_pool(B * maxb)
    tq.compress_kv(layer, kt, vt, slots, pool)  # the whole context; the step re-appends the last token
    last = torch.arange(B, device="cuda") * T + (T - 1)
    k_new, v_new, s_new = kt[last].contiguous(), vt[last].contiguous(), slots[last].contiguous()
    q = torch.from_numpy(synth.queries_host(320, B, Hq)).to("cuda", torch.bfloat16)
    bt = torch.from_numpy(table).cuda()
    sl = torch.full((B,), T, dtype=torch.int32, device="cuda")
    ws = tq.new_workspace(layer, B, Hq, T)
    out = torch.empty((B, Hq, 128), dtype=torch.float32, device="cuda")

    def step():
        tq.compress_kv(layer, k_new, v_new, s_new, pool)
        tq.decode_attn(layer, q, pool, bt, sl, T, out=out, workspace=ws)

    step()
    torch.cuda.synchronize()
    ref = out.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    x = torch.randn(512, 512, device="cuda")
    for i in range(4):
        out.fill_(float("nan"))
        y = x @ x  # eager work between replays
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), i
        assert torch.isfinite(y).all()
    layer.close()


# seeds 17 and 21 draw a batch whose every sequence is empty (a store of no tokens)
@pytest.mark.parametrize("case", list(range(6)) + [17, 21])
def test_random_layer_configurations(case):
    """Seeded random layers: KV heads, GQA ratio, bit widths, key mode, rotation,
    value coding (group scale/zero or codebook with a norm), ragged lengths (some
    zero), a random block table, K/V rows with a token stride wider than the row,
    split count, query and output types: GPU compress against the oracle's store,
    then GPU decode of the GPU store against the oracle decode."""
    torch = _torch()
    rng = np.random.default_rng(1000 + case)
    Hkv = int(rng.choice([1, 2, 4, 8]))
    rep = int(rng.choice([1, 2, 4, 8]))
    Hq = Hkv * rep
    kb, vb = int(rng.choice([1, 2, 3, 4])), int(rng.choice([2, 3, 4]))
    key_mode = int(rng.choice([tq.KEY_QJL, tq.KEY_MSE, tq.KEY_MSE_NC]))
    rotation = int(rng.choice([tq.ROT_HAAR, tq.ROT_HADAMARD]))
    B = int(rng.integers(1, 5))
    lens = rng.integers(1, 700, B).astype(np.int32)
    lens[rng.random(B) < 0.2] = 0
    splits = int(rng.choice([0, 0, 1, 3, 8]))
    q_dtype = str(rng.choice(["bf16", "f32"]))
    out_dtype = str(rng.choice(["f32", "bf16"]))
    value_mode = str(rng.choice(["group", "group", "mse"]))
    say("random layer", case, dict(Hkv=Hkv, rep=rep, kb=kb, vb=vb, key_mode=key_mode, rotation=rotation,
                                   value_mode=value_mode, lens=lens.tolist(), splits=splits, q=q_dtype,
                                   out=out_dtype))
    maxb = max(1, int((lens.max() + 15) // 16) + 1)
    table = rng.permutation(B * maxb).reshape(B, maxb).astype(np.int32)
    N = int(lens.sum())
    K, V = synth.kv_host(2000 + case, max(N, 1), Hkv, outliers=4)
    K, V = K[:N], V[:N]
    seq = np.repeat(np.arange(B), lens)
    pos = np.concatenate([np.arange(n) for n in lens]) if N else np.zeros(0, np.int64)
    slots = (table[seq, pos // 16].astype(np.int64) * 16 + pos % 16) if N else np.zeros(0, np.int64)
    layer = tq.Layer(tq.config(Hkv, kb, vb, seed=3000 + case, layer=case, key_mode=key_mode, rotation=rotation,
                               value_mode=tq.VAL_MSE if value_mode == "mse" else tq.VAL_GROUP))
    pool = layer.new_pool(B * maxb)
    # K and V as views into wider rows: token stride (Hkv + 1) * 128
    kw = torch.zeros((N, Hkv + 1, 128), dtype=torch.bfloat16, device="cuda")
    vw = torch.zeros_like(kw)
    kw[:, :Hkv] = torch.from_numpy(K).to("cuda", torch.bfloat16)
    vw[:, 1:] = torch.from_numpy(V).to("cuda", torch.bfloat16)
    tq.compress_kv(layer, kw[:, :Hkv], vw[:, 1:], torch.from_numpy(slots).cuda(), pool)
    torch.cuda.synchronize()
    gpu_pool = pool.cpu().numpy()
    if not N:
        assert not gpu_pool.any()  # no tokens: the store is left as allocated
    st, layout, opool, res = parity.oracle_store(K, V, slots, B * maxb, Hkv, kb, vb, 3000 + case, layer=case,
                                                 key_mode=KEY_MODE_NAMES[key_mode],
                                                 rotation_kind="haar" if rotation == tq.ROT_HAAR else "hadamard",
                                                 value_mode=value_mode)
    if N:
        _check_compress(gpu_pool, res, st, layout, Hkv, slots, V, kb, vb)
    q = synth.queries_host(4000 + case, B, Hq, dtype=q_dtype)
    ref = parity.oracle_decode(q.astype(np.float64), gpu_pool, layout, Hkv, table, lens, st)
    tq_dt = torch.bfloat16 if q_dtype == "bf16" else torch.float32
    od = torch.bfloat16 if out_dtype == "bf16" else torch.float32
    out = tq.decode_attn(layer, torch.from_numpy(q).to("cuda", tq_dt), pool, torch.from_numpy(table).cuda(),
                         torch.from_numpy(lens).cuda(), max(int(lens.max()), 1), num_splits=splits, out_dtype=od)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    assert not got[lens == 0].any()
    live = lens > 0
    if live.any():
        parity.assert_decode_ok(got[live], ref[live], out_dtype, "random layer %d" % case)
    layer.close()


@pytest.mark.parametrize("bypass", [False, True])
def test_decode_table_rows_padded_with_minus_one(bypass):
    """Block-table entries past each sequence's last page hold -1 (a caller's
    padding): no kernel dereferences them, whatever the split count (the waves
    and splits that start past a sequence's end read no page of it)."""
    torch = _torch()
    say("decode with -1 padded table rows, bypass", bypass)
    B, Hq, Hkv, kb, vb, seed = 5, 8, 2, 4, 4, 296
    lens = np.array([1, 33, 130, 700, 0], np.int32)
    maxb = 64  # rows much longer than any sequence
    K, V, slots = [], [], []
    table = np.full((B, maxb), -1, np.int32)
    nxt = 0
    for b in range(B):
        npg = (int(lens[b]) + 15) // 16
        table[b, :npg] = np.arange(nxt, nxt + npg)
        nxt += npg
        kk, vv = synth.kv_host(seed * 100 + b, int(lens[b]), Hkv, outliers=4)
        pos = np.arange(int(lens[b]))
        K.append(kk)
        V.append(vv)
        slots.append(table[b][pos // 16].astype(np.int64) * 16 + pos % 16)
    K, V, slots = np.concatenate(K), np.concatenate(V), np.concatenate(slots)
    nblk = max(nxt, 1)
    if bypass:
        st, layout, pool, _ = parity.oracle_store(None, None, slots, nblk, Hkv, kb, vb, seed, bypass=True,
                                                  K_bits16=synth.bf16_bits(K), V_bits16=synth.bf16_bits(V))
    else:
        st, layout, pool, _ = parity.oracle_store(K, V, slots, nblk, Hkv, kb, vb, seed, keep=False)
    q = synth.queries_host(seed, B, Hq)
    ref = parity.oracle_decode(q.astype(np.float64), pool, layout, Hkv, np.maximum(table, 0), lens, st)
    for splits in (0, 1, 5, 64):
        got = _gpu_decode(torch, tq.config(Hkv, kb, vb, seed=seed, bypass=bypass), pool, q, table, lens,
                          maxb * 16, num_splits=splits)
        parity.assert_decode_ok(got, ref, "f32", "padded table, %d splits" % splits)


def test_pooled_mismatch_rate():
    """The compress mismatch rate (codes, signs, value codes that differ from the
    oracle's, all inside their 1e-6 bands) over every compress comparison of this
    session, pooled: <= 1e-5 once at least 1e6 decisions are pooled."""
    n_dec, n_mis, n_cmp = parity.pooled()
    print("pooled compress decisions %d, mismatches %d, comparisons %d" % (n_dec, n_mis, n_cmp))
    if n_dec < parity.RATE_MIN_SAMPLE:
        pytest.skip("fewer than 1e6 compress decisions compared in this session")
    assert n_mis <= parity.RATE * n_dec, (n_mis, n_dec)


def test_debug_checks_refuse_bad_indices(monkeypatch):
    """With TQ_DEBUG_CHECKS=1 the entry points copy the index arrays to the host
    and refuse, before any launch, a slot past the pool, a block id past the pool
    in a used page and a length past the table; unused padding entries pass."""
    torch = _torch()
    say("debug checks")
    monkeypatch.setenv("TQ_DEBUG_CHECKS", "1")
    layer = tq.Layer(tq.config(2, 4, 4, seed=9))
    pool = layer.new_pool(4)
    k = torch.zeros(3, 2, 128, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(tq.TQError) as e:
        tq.compress_kv(layer, k, k, torch.tensor([0, 5, 64], device="cuda"), pool)
    assert e.value.status == tq.ERR_INVALID_ARGUMENT and "slot_mapping[2]" in str(e.value)
    with pytest.raises(tq.TQError):
        tq.decompress_kv(layer, pool, torch.tensor([70], device="cuda"))
    tq.compress_kv(layer, k, k, torch.tensor([0, 5, -1], device="cuda"), pool)
    q = torch.zeros(2, 8, 128, dtype=torch.bfloat16, device="cuda")
    sl = torch.tensor([17, 0], dtype=torch.int32, device="cuda")
    bt = torch.tensor([[1, 4, -1], [-1, -1, -1]], dtype=torch.int32, device="cuda")
    with pytest.raises(tq.TQError) as e:
        tq.decode_attn(layer, q, pool, bt, sl, 48)
    assert "block_table[0][1]" in str(e.value)
    bt[0, 1] = 3
    out = tq.decode_attn(layer, q, pool, bt, sl, 48)  # padding entries (-1) past each sequence pass
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    sl[1] = 49  # past max_seq_len 48 = 16 * 3 blocks per row
    with pytest.raises(tq.TQError) as e:
        tq.decode_attn(layer, q, pool, bt, sl, 48)
    assert "seq_lens[1]" in str(e.value)
    layer.close()


def test_decode_plan_grid_limit():
    """The split-K grid (batch x KV heads x splits workgroups, one-dimensional) must
    stay below 2^31: the plan refuses larger ones with TQ_ERR_UNSUPPORTED instead of
    launching a truncated grid (host arithmetic only, no kernel)."""
    _torch()
    layer = tq.Layer(tq.config(8, 4, 4))
    try:
        ok = tq.decode_workspace_size(layer, 1 << 16, 32, 1 << 20)  # 65,536 x 8 x 256 splits = 2^27
        assert ok > 0
        with pytest.raises(tq.TQError) as e:
            tq.decode_workspace_size(layer, 1 << 20, 32, 1 << 20)  # 2^20 x 8 x 256 = 2^31
        assert e.value.status == tq.ERR_UNSUPPORTED and "exceeds" in str(e.value)
    finally:
        layer.close()
