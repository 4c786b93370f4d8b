"""GPU parity: libtq's HIP kernels (through the C ABI) against the oracle."""

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
                  rotation=0, value_mode=0):
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    layer_obj = tq.Layer(tq.config(n_heads, kb, vb, seed=seed, layer=layer, key_mode=key_mode, rotation=rotation,
                                   value_mode=value_mode))
    k = torch.from_numpy(np.ascontiguousarray(K)).to("cuda", tdt)
    v = torch.from_numpy(np.ascontiguousarray(V)).to("cuda", tdt)
    pool = layer_obj.new_pool(num_blocks)
    tq.compress_kv(layer_obj, k, v, torch.from_numpy(np.asarray(slots, np.int64)).cuda(), pool)
    torch.cuda.synchronize()
    out = pool.cpu().numpy()
    layer_obj.close()
    return out


def _check_compress(gpu_pool, res, st, layout, n_heads, slots, V, kb, vb):
    keep = np.asarray(slots) >= 0
    sl = np.asarray(slots)[keep]
    for h in range(n_heads):
        f = parity.fields_at(gpu_pool, layout, n_heads, sl, h)
        ck, cv = res[h]
        stats = parity.compare_compress(f, ck, cv, st.S[h], st.boundaries, V[keep][:, h], vb,
                                        centroids=st.centroids, key_mode=st.key_mode,
                                        v_boundaries=getattr(st, "v_boundaries", None))
        print("head", h, stats)
        parity.assert_compress_ok(stats)


def test_compress_tiny_fp32():
    """1 KV head, 1024 tokens, fp32 N(0,1), keys 2-bit + QJL, values 3-bit g32."""
    torch = _torch()
    say("compress tiny fp32 K2/V3")
    K, V = synth.kv_host(101, 1024, 1, dtype="f32")
    slots = np.arange(1024)
    gpu = _gpu_compress(torch, K, V, slots, 64, 1, 2, 3, 201, dtype="f32")
    st, layout, pool, res = parity.oracle_store(K, V, slots, 64, 1, 2, 3, 201)
    _check_compress(gpu, res, st, layout, 1, slots, V, 2, 3)


@pytest.mark.parametrize("kb,vb", [(2, 2), (3, 2), (3, 3), (4, 3), (4, 4), (2, 4)])
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


@pytest.mark.parametrize("kb,vb,n,dtype,key_mode,rotation", [
    (2, 3, 301, "bf16", 0, 0), (4, 4, 500, "bf16", 0, 0), (3, 2, 200, "f32", 0, 0), (2, 3, 2003, "bf16", 0, 0),
    (3, 3, 300, "bf16", 2, 1)])
def test_compress_mse_values(kb, vb, n, dtype, key_mode, rotation):
    """Values coded like the keys' codebook part (the 102-byte record at K2/V3): 8
    heads with outlier channels, shuffled slots with skipped tokens, bf16 (more
    than 64 tokens, which the matrix-core compressor would otherwise take) and
    fp32; and together with norm-corrected keys and the Hadamard rotation. Codes as
    the keys' protocol, the value norm within an fp16 ulp, slots nobody wrote
    untouched."""
    torch = _torch()
    say("compress mse values", kb, vb, n, dtype)
    K, V = synth.kv_host(340 + kb * 10 + vb, n, 8, outliers=4, dtype=dtype)
    rng = np.random.default_rng(340 + kb)
    nb = max(40, (n + 15) // 16 + 4)  # 2003 tokens: 16 per workgroup, a ragged last run
    slots = rng.permutation(nb * 16)[:n].astype(np.int64)
    slots[rng.choice(n, 15, replace=False)] = -1
    gpu = _gpu_compress(torch, K, V, slots, nb, 8, kb, vb, 341, layer=kb, dtype=dtype, key_mode=key_mode,
                        rotation=rotation, value_mode=tq.VAL_MSE)
    st, layout, pool, res = parity.oracle_store(K, V, slots, nb, 8, kb, vb, 341, layer=kb, value_mode="mse",
                                                key_mode=KEY_MODE_NAMES[key_mode],
                                                rotation_kind="haar" if rotation == tq.ROT_HAAR else "hadamard")
    assert layout.record_bytes() == 16 * kb + 16 + 4 + 16 * vb + 2
    _check_compress(gpu, res, st, layout, 8, slots, V, kb, vb)
    written = set((slots[slots >= 0] // 16).tolist())
    for b in range(nb):
        if b not in written:
            assert not gpu[b * 8 * layout.block_bytes:(b + 1) * 8 * layout.block_bytes].any()


def test_mse_value_layers_refuse_decode():
    """Decode of MSE-value layers is not built: it returns TQ_ERR_UNSUPPORTED
    before any launch (no silent fallback)."""
    torch = _torch()
    say("mse values: decode refused")
    layer = tq.Layer(tq.config(2, 2, 3, seed=5, value_mode=tq.VAL_MSE))
    pool = layer.new_pool(4)
    q = torch.zeros((1, 8, 128), dtype=torch.bfloat16, device="cuda")
    bt = torch.zeros((1, 4), dtype=torch.int32, device="cuda")
    sl = torch.full((1,), 16, dtype=torch.int32, device="cuda")
    out = torch.zeros((1, 8, 128), device="cuda")
    ws = tq.new_workspace(layer, 1, 8, 64)
    st = tq.lib().tq_decode_attn(layer.handle, tq._ptr(q), tq._dtype_code(q), 1, 8, tq._ptr(pool), 4,
                                 tq._ptr(bt), 4, tq._ptr(sl), 64, 0.0, 0, tq._ptr(out), tq._dtype_code(out),
                                 tq._ptr(ws), ws.numel(), tq._stream(None))
    assert st == tq.ERR_UNSUPPORTED and b"MSE" in tq.lib().tq_last_error()
    torch.cuda.synchronize()
    assert not out.any()
    layer.close()


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


@pytest.mark.parametrize("kb,vb,n,offset", [(4, 4, 2000, 37), (3, 2, 1000, 0), (2, 3, 777, 16)])
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
                 fill=0):
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
                                                  fill=fill)
    q = synth.queries_host(seed, B, Hq, dtype=q_dtype)
    ref = parity.oracle_decode(q.astype(np.float64), pool, layout, Hkv, table, lens, st,
                               scale=scale if scale else None)
    cfg = tq.config(Hkv, kb, vb, seed=seed, layer=layer, bypass=bypass)
    results = {}
    for od in out_dtypes:
        got = _gpu_decode(torch, cfg, pool, q, table, lens, int(lens.max()), od, num_splits, scale,
                          q_dtype=q_dtype)
        err = parity.rel_l2(got, ref)
        results[od] = err
        print("decode", od, "rel L2 %.3e" % err)
        assert err <= (1e-3 if od == "f32" else 1e-2), (od, err)
    return results


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


@pytest.mark.parametrize("kb,vb", [(4, 4), (4, 3), (3, 3), (3, 2), (2, 3), (2, 2)])
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
        err = parity.rel_l2(got[sample], ref[sample])
        print("ragged serving", kb, vb, "rel L2 %.3e" % err)
        assert err <= 1e-3


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
    st, layout, opool, _ = parity.oracle_store(K, V, slots, B * maxb, Hkv, 3, 3, 260, keep=False)
    q = synth.queries_host(260, B, Hq)
    ref = parity.oracle_decode(q.astype(np.float64), opool, layout, Hkv, table, lens, st)
    layer = tq.Layer(tq.config(Hkv, 3, 3, seed=260))
    pool = layer.new_pool(B * maxb)
    tq.compress_kv(layer, torch.from_numpy(K).to("cuda", torch.bfloat16),
                   torch.from_numpy(V).to("cuda", torch.bfloat16), torch.from_numpy(slots).cuda(), pool)
    out = tq.decode_attn(layer, torch.from_numpy(q).to("cuda", torch.bfloat16), pool,
                         torch.from_numpy(table).cuda(), torch.from_numpy(lens).cuda(), T)
    torch.cuda.synchronize()
    err = parity.rel_l2(out.cpu().numpy(), ref)
    print("end-to-end rel L2 %.3e" % err)
    assert err <= 2e-3
    layer.close()


KEY_MODE_NAMES = {tq.KEY_QJL: "qjl", tq.KEY_MSE: "mse", tq.KEY_MSE_NC: "mse_nc"}


@pytest.mark.parametrize("key_mode,kb,vb,n,dtype", [
    (tq.KEY_MSE, 4, 4, 700, "bf16"), (tq.KEY_MSE_NC, 3, 2, 700, "bf16"),
    (tq.KEY_MSE_NC, 2, 3, 1024, "f32"), (tq.KEY_MSE, 3, 3, 40, "bf16")])
def test_compress_key_modes(key_mode, kb, vb, n, dtype):
    """Keys without the residual projection (plain and norm-corrected magnitude):
    the matrix-core compressor (bf16: whole pages and a ragged last tile) and the
    per-token one (fp32 inputs; a 40-token append)."""
    torch = _torch()
    say("compress key mode", key_mode, kb, vb, n, dtype)
    H = 8 if dtype == "bf16" else 1
    K, V = synth.kv_host(170 + key_mode, n, H, dtype=dtype, outliers=4 if dtype == "bf16" else 0)
    slots = np.arange(n, dtype=np.int64)
    nb = (n + 15) // 16
    gpu = _gpu_compress(torch, K, V, slots, nb, H, kb, vb, 230, layer=key_mode, dtype=dtype, key_mode=key_mode)
    st, layout, pool, res = parity.oracle_store(K, V, slots, nb, H, kb, vb, 230, layer=key_mode,
                                                key_mode=KEY_MODE_NAMES[key_mode])
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
    st, layout, opool, _ = parity.oracle_store(K, V, slots, B * maxb, Hkv, 4, 3, 270, keep=False,
                                               key_mode=KEY_MODE_NAMES[key_mode])
    q = synth.queries_host(270, B, Hq)
    ref = parity.oracle_decode(q.astype(np.float64), opool, layout, Hkv, table, lens, st)
    layer = tq.Layer(tq.config(Hkv, 4, 3, seed=270, key_mode=key_mode))
    pool = layer.new_pool(B * maxb)
    tq.compress_kv(layer, torch.from_numpy(K).to("cuda", torch.bfloat16),
                   torch.from_numpy(V).to("cuda", torch.bfloat16), torch.from_numpy(slots).cuda(), pool)
    qt = torch.from_numpy(q).to("cuda", torch.bfloat16)
    bt = torch.from_numpy(table).cuda()
    sl = torch.from_numpy(lens).cuda()
    out = tq.decode_attn(layer, qt, pool, bt, sl, T)
    out_o = tq.decode_attn(layer, qt, torch.from_numpy(opool).cuda(), bt, sl, T)
    torch.cuda.synchronize()
    same = parity.rel_l2(out_o.cpu().numpy(), ref)
    err = parity.rel_l2(out.cpu().numpy(), ref)
    print("key mode %d: decode on oracle store rel L2 %.3e, end-to-end %.3e" % (key_mode, same, err))
    assert same <= 1e-3 and err <= 2e-3
    layer.close()


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
    st, layout, opool, _ = parity.oracle_store(K, V, slots, B * maxb, Hkv, 4, 4, 280, keep=False,
                                               rotation_kind="hadamard")
    q = synth.queries_host(280, B, Hq)
    ref = parity.oracle_decode(q.astype(np.float64), opool, layout, Hkv, table, lens, st)
    layer = tq.Layer(tq.config(Hkv, 4, 4, seed=280, rotation=tq.ROT_HADAMARD))
    pool = layer.new_pool(B * maxb)
    tq.compress_kv(layer, torch.from_numpy(K).to("cuda", torch.bfloat16),
                   torch.from_numpy(V).to("cuda", torch.bfloat16), torch.from_numpy(slots).cuda(), pool)
    qt = torch.from_numpy(q).to("cuda", torch.bfloat16)
    bt = torch.from_numpy(table).cuda()
    sl = torch.from_numpy(lens).cuda()
    out = tq.decode_attn(layer, qt, pool, bt, sl, T)
    out_o = tq.decode_attn(layer, qt, torch.from_numpy(opool).cuda(), bt, sl, T)
    torch.cuda.synchronize()
    same = parity.rel_l2(out_o.cpu().numpy(), ref)
    err = parity.rel_l2(out.cpu().numpy(), ref)
    print("hadamard: decode on oracle store rel L2 %.3e, end-to-end %.3e" % (same, err))
    assert same <= 1e-3 and err <= 2e-3
    layer.close()


@pytest.mark.parametrize("kb,vb,key_mode,rotation,out_dtype", [
    (4, 4, tq.KEY_QJL, tq.ROT_HAAR, "f32"), (3, 2, tq.KEY_MSE_NC, tq.ROT_HADAMARD, "f32"),
    (2, 3, tq.KEY_QJL, tq.ROT_HAAR, "bf16")])
def test_decompress_matches_oracle(kb, vb, key_mode, rotation, out_dtype):
    """Keys and values reconstructed from a GPU-written store (shuffled slots, some
    negative: zero rows) against the oracle's reconstruction of the same bytes."""
    from oracle import decompress as odec
    torch = _torch()
    say("decompress", kb, vb, key_mode, rotation, out_dtype)
    H, n = 8, 613
    K, V = synth.kv_host(300 + kb, n, H, outliers=4)
    rng = np.random.default_rng(kb)
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
    layout = parity.lay.StoreLayout(128, kb, vb, 32)
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
    err = parity.rel_l2(out.float().cpu().numpy(), ref)
    print("decode rel L2 %.3e" % err)
    assert err <= 1e-3, err
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


@pytest.mark.parametrize("case", range(6))
def test_random_layer_configurations(case):
    """Seeded random layers: KV heads, GQA ratio, bit widths, key mode, rotation,
    ragged lengths (some zero), a random block table, K/V rows with a token stride
    wider than the row, split count, query and output types: GPU compress against
    the oracle's store, then GPU decode of the GPU store against the oracle decode."""
    torch = _torch()
    rng = np.random.default_rng(1000 + case)
    Hkv = int(rng.choice([1, 2, 4, 8]))
    rep = int(rng.choice([1, 2, 4, 8]))
    Hq = Hkv * rep
    kb, vb = int(rng.choice([2, 3, 4])), int(rng.choice([2, 3, 4]))
    key_mode = int(rng.choice([tq.KEY_QJL, tq.KEY_MSE, tq.KEY_MSE_NC]))
    rotation = int(rng.choice([tq.ROT_HAAR, tq.ROT_HADAMARD]))
    B = int(rng.integers(1, 5))
    lens = rng.integers(1, 700, B).astype(np.int32)
    lens[rng.random(B) < 0.2] = 0
    splits = int(rng.choice([0, 0, 1, 3, 8]))
    q_dtype = str(rng.choice(["bf16", "f32"]))
    out_dtype = str(rng.choice(["f32", "bf16"]))
    say("random layer", case, dict(Hkv=Hkv, rep=rep, kb=kb, vb=vb, key_mode=key_mode, rotation=rotation,
                                   lens=lens.tolist(), splits=splits, q=q_dtype, out=out_dtype))
    maxb = max(1, int((lens.max() + 15) // 16) + 1)
    table = rng.permutation(B * maxb).reshape(B, maxb).astype(np.int32)
    N = int(lens.sum())
    K, V = synth.kv_host(2000 + case, max(N, 1), Hkv, outliers=4)
    K, V = K[:N], V[:N]
    seq = np.repeat(np.arange(B), lens)
    pos = np.concatenate([np.arange(n) for n in lens]) if N else np.zeros(0, np.int64)
    slots = (table[seq, pos // 16].astype(np.int64) * 16 + pos % 16) if N else np.zeros(0, np.int64)
    layer = tq.Layer(tq.config(Hkv, kb, vb, seed=3000 + case, layer=case, key_mode=key_mode, rotation=rotation))
    pool = layer.new_pool(B * maxb)
    if N:
        # K and V as views into wider rows: token stride (Hkv + 1) * 128
        kw = torch.zeros((N, Hkv + 1, 128), dtype=torch.bfloat16, device="cuda")
        vw = torch.zeros_like(kw)
        kw[:, :Hkv] = torch.from_numpy(K).to("cuda", torch.bfloat16)
        vw[:, 1:] = torch.from_numpy(V).to("cuda", torch.bfloat16)
        tq.compress_kv(layer, kw[:, :Hkv], vw[:, 1:], torch.from_numpy(slots).cuda(), pool)
    torch.cuda.synchronize()
    gpu_pool = pool.cpu().numpy()
    st, layout, opool, res = parity.oracle_store(K, V, slots, B * maxb, Hkv, kb, vb, 3000 + case, layer=case,
                                                 key_mode=KEY_MODE_NAMES[key_mode],
                                                 rotation_kind="haar" if rotation == tq.ROT_HAAR else "hadamard")
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
        err = parity.rel_l2(got[live], ref[live])
        print("decode rel L2 %.3e" % err)
        assert err <= (1e-3 if out_dtype == "f32" else 1e-2), err
    layer.close()
