"""tq_decode_attn_noalloc (through the C ABI) against tq_decode_attn on the same
inputs: two calls in a row, the second with a smaller batch and context, each
equal bit for bit to the workspace entry point's output and within the decode
protocol of the oracle; a shape needing more than the static workspace is
refused before any launch."""

import ctypes

import numpy as np
import pytest

import compressed_decode_attention_tq_amd as tq
from compressed_decode_attention_tq_amd import synth
from tests import parity

pytestmark = pytest.mark.gpu


def _noalloc(layer, q, pool, bt, sl, max_len, out, num_splits=0):
    lib = tq.lib()
    num_blocks = pool.numel() // (layer.cfg.n_kv_heads * layer.block_bytes)
    return lib.tq_decode_attn_noalloc(layer.handle, tq._ptr(q), tq._dtype_code(q), q.shape[0], q.shape[1],
                                      tq._ptr(pool), num_blocks, tq._ptr(bt), bt.shape[1], tq._ptr(sl), max_len,
                                      ctypes.c_float(0.0), num_splits, tq._ptr(out), tq._dtype_code(out),
                                      tq._stream(None))


def test_noalloc_matches_workspace_entry_point():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a visible GPU")
    print("[case] decode without allocation", flush=True)
    Hq, Hkv, kb, vb, seed = 32, 8, 4, 4, 410
    lens_all = np.array([1000, 517, 2048, 37], np.int32)
    B = len(lens_all)
    maxb = (int(lens_all.max()) + 15) // 16
    table = synth.block_table(seed, B, maxb, "random")
    K, V, slots = [], [], []
    for b in range(B):
        kk, vv = synth.kv_host(seed * 10 + b, int(lens_all[b]), Hkv, outliers=4)
        pos = np.arange(int(lens_all[b]))
        K.append(kk)
        V.append(vv)
        slots.append(table[b][pos // 16].astype(np.int64) * 16 + pos % 16)
    K, V, slots = np.concatenate(K), np.concatenate(V), np.concatenate(slots)
    st, layout, opool, _ = parity.oracle_store(K, V, slots, B * maxb, Hkv, kb, vb, seed, keep=False)
    q_all = synth.queries_host(seed, B, Hq)
    layer = tq.Layer(tq.config(Hkv, kb, vb, seed=seed))
    pool = torch.from_numpy(opool).cuda()
    # second call: a smaller batch over shorter contexts (a prefix of each sequence)
    for B_, cut in ((B, None), (2, 300)):
        lens = lens_all[:B_].copy() if cut is None else np.minimum(lens_all[:B_], cut).astype(np.int32)
        max_len = int(lens.max())
        nbt = (max_len + 15) // 16
        bt = torch.from_numpy(np.ascontiguousarray(table[:B_, :nbt])).cuda()
        sl = torch.from_numpy(lens).cuda()
        q = torch.from_numpy(np.ascontiguousarray(q_all[:B_])).to("cuda", torch.bfloat16)
        ref = tq.decode_attn(layer, q, pool, bt, sl, max_len)
        out = torch.full((B_, Hq, 128), float("nan"), device="cuda")
        assert _noalloc(layer, q, pool, bt, sl, max_len, out) == tq.OK, tq.lib().tq_last_error()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), (B_, (out - ref).abs().max().item())
        oref = parity.oracle_decode(q_all[:B_].astype(np.float64), opool, layout, Hkv, table[:B_], lens, st)
        parity.assert_decode_ok(out.cpu().numpy(), oref, "f32", "no-alloc B=%d" % B_)
    # a workspace larger than the static array: refused before any launch
    big_b = 512
    need = tq.decode_workspace_size(layer, big_b, Hq, 4096, 8)
    assert need > 16 << 20
    qb = torch.zeros((big_b, Hq, 128), dtype=torch.bfloat16, device="cuda")
    btb = torch.zeros((big_b, 256), dtype=torch.int32, device="cuda")
    slb = torch.zeros(big_b, dtype=torch.int32, device="cuda")
    outb = torch.zeros((big_b, Hq, 128), device="cuda")
    assert _noalloc(layer, qb, pool, btb, slb, 4096, outb, num_splits=8) == tq.ERR_UNSUPPORTED
    assert b"static scratch" in tq.lib().tq_last_error()
    torch.cuda.synchronize()
    assert not outb.any()
    layer.close()
