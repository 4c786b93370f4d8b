"""The Python binding refuses tensors whose layout the library would misread
(CPU only: every refusal happens before any library call)."""

import pytest
import torch

import compressed_decode_attention_tq_amd as tq


class _Layer:
    """Stand-in with the attributes the binding reads before calling the library."""

    def __init__(self, H=2, kb=4, vb=4):
        self.cfg = tq.config(H, kb, vb)
        self.block_bytes = 256 * (kb + vb) + 576
        self.handle = None


def _refused(fn, *a, **kw):
    with pytest.raises(tq.TQError) as e:
        fn(*a, **kw)
    assert e.value.status == tq.ERR_INVALID_ARGUMENT
    return str(e.value)


def _kv(n=32, H=2, dtype=torch.bfloat16):
    return torch.zeros(n, H, 128, dtype=dtype), torch.zeros(n, H, 128, dtype=dtype)


def test_compress_refusals():
    L = _Layer()
    k, v = _kv()
    slots = torch.arange(32, dtype=torch.int64)
    pool = torch.zeros(4 * 2 * L.block_bytes, dtype=torch.uint8)
    assert "dtype" in _refused(tq.compress_kv, L, k, v.float(), slots, pool)
    assert "shape" in _refused(tq.compress_kv, L, k[:, :1], v[:, :1], slots, pool)
    assert "rows" in _refused(tq.compress_kv, L, k, v, slots[:31], pool)
    wide = torch.zeros(32, 2, 256, dtype=torch.bfloat16)
    assert "shape" in _refused(tq.compress_kv, L, wide, v, slots, pool)
    strided = torch.zeros(32, 2, 256, dtype=torch.bfloat16)[:, :, ::2]
    assert "stride" in _refused(tq.compress_kv, L, strided, v, slots, pool)
    heads_apart = torch.zeros(32, 2, 2, 128, dtype=torch.bfloat16)[:, :, 0]
    assert "stride" in _refused(tq.compress_kv, L, heads_apart, v, slots, pool)
    assert "slot_mapping" in _refused(tq.compress_kv, L, k, v, slots.int(), pool)
    assert "slot_mapping" in _refused(tq.compress_kv, L, k, v, torch.arange(64)[::2], pool)
    assert "pool" in _refused(tq.compress_kv, L, k, v, slots, pool[:-1])
    assert "pool" in _refused(tq.compress_kv, L, k, v, slots, pool.view(2, -1)[:, ::2])


def test_decode_refusals():
    L = _Layer()
    B, Hq = 3, 8
    q = torch.zeros(B, Hq, 128, dtype=torch.bfloat16)
    pool = torch.zeros(4 * 2 * L.block_bytes, dtype=torch.uint8)
    bt = torch.zeros(B, 4, dtype=torch.int32)
    sl = torch.zeros(B, dtype=torch.int32)
    qkv = torch.zeros(B, 3 * Hq, 128, dtype=torch.bfloat16)
    assert "q must" in _refused(tq.decode_attn, L, qkv[:, :Hq], pool, bt, sl, 64)
    assert "block_table" in _refused(tq.decode_attn, L, q, pool, bt.t().contiguous().t(), sl, 64)
    assert "block_table" in _refused(tq.decode_attn, L, q, pool, bt[:2], sl, 64)
    assert "block_table" in _refused(tq.decode_attn, L, q, pool, bt.long(), sl, 64)
    assert "seq_lens" in _refused(tq.decode_attn, L, q, pool, bt, sl[:2], 64)
    assert "seq_lens" in _refused(tq.decode_attn, L, q, pool, bt, sl.long(), 64)
    out = torch.zeros(B, 2 * Hq, 128)[:, ::2]
    assert "out must" in _refused(tq.decode_attn, L, q, pool, bt, sl, 64, out=out)
    assert "out must" in _refused(tq.decode_attn, L, q, pool, bt, sl, 64, out=torch.zeros(B, Hq, 64))
    assert "pool" in _refused(tq.decode_attn, L, q, pool[:100], bt, sl, 64)


def test_decompress_refusals():
    L = _Layer()
    pool = torch.zeros(4 * 2 * L.block_bytes, dtype=torch.uint8)
    slots = torch.arange(10, dtype=torch.int64)
    k_out = torch.zeros(10, 2, 128)
    assert "k_out" in _refused(tq.decompress_kv, L, pool, slots, k_out=k_out[:, :1], v_out=k_out)
    assert "dtype" in _refused(tq.decompress_kv, L, pool, slots, k_out=k_out, v_out=k_out.bfloat16())
    assert "slot_mapping" in _refused(tq.decompress_kv, L, pool, slots.int(), k_out=k_out, v_out=k_out)
