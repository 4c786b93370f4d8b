"""Pins of the oracle's packing, store layout and byte accounting."""

import json
import os

import numpy as np
import pytest

from oracle import bits, layout, metrics

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_worked_bytes():
    for case in json.load(open(os.path.join(GOLDEN, "packing.json")))["cases"]:
        packed = bits.pack(np.array(case["values"]), case["bits"])
        assert packed.tobytes().hex() == case["bytes_hex"]
        back = bits.unpack(packed, case["bits"], len(case["values"]))
        assert list(back) == case["values"]


@pytest.mark.parametrize("b", [1, 2, 3, 4])
def test_round_trip(b):
    v = np.random.default_rng(b).integers(0, 1 << b, size=(37, 128))
    p = bits.pack(v, b)
    assert p.shape == (37, 128 * b // 8)
    assert np.array_equal(bits.unpack(p, b, 128), v)


def test_pack_rejects_out_of_range():
    with pytest.raises(ValueError):
        bits.pack(np.array([4, 0, 0, 0]), 2)


def test_block_and_record_bytes():
    ref = json.load(open(os.path.join(GOLDEN, "byte_accounting.json")))
    for row in ref["this_store"]:
        lay = layout.StoreLayout(128, row["k_bits"], row["v_bits"], 32)
        assert lay.block_bytes == row["block_bytes"]
        assert lay.record_bytes() == row["record_bytes"]
        assert metrics.record_bytes(128, row["k_bits"], row["v_bits"], 32) == row["record_bytes"]
        assert all(o % 64 == 0 for o in lay.field_offsets())
    assert layout.StoreLayout(bypass=True).block_bytes == ref["bypass_block_bytes"]
    blog = 2 * 128 // 8 + 128 // 8 + 4 + 3 * 128 // 8 + 2
    assert blog == ref["blog_layout_bytes"]
    assert abs(metrics.compression_ratio(blog) - ref["blog_ratio"]) < 1e-4


def _records(lay, n, seed):
    rng = np.random.default_rng(seed)
    G = lay.d // lay.group
    return {
        "idx": rng.integers(0, 1 << lay.k_bits, (n, lay.d)),
        "z": rng.integers(0, 2, (n, lay.m)),
        "n16": rng.standard_normal(n).astype(np.float16),
        "g16": rng.standard_normal(n).astype(np.float16),
        "vcode": rng.integers(0, 1 << lay.v_bits, (n, lay.d)),
        "scale16": rng.standard_normal((n, G)).astype(np.float16),
        "zero16": rng.standard_normal((n, G)).astype(np.float16),
    }


@pytest.mark.parametrize("kb,vb", [(4, 4), (3, 2), (2, 3)])
def test_record_round_trip(kb, vb):
    """Records written at scattered slots (several sharing pages) read back exactly,
    and neighbouring tokens of a page are not disturbed."""
    lay = layout.StoreLayout(128, kb, vb, 32)
    pool = layout.new_pool(6, 2, lay)
    slots = np.array([37, 5, 36, 80, 38, 0, 95, 17])
    rec = _records(lay, len(slots), kb * 10 + vb)
    layout.put_records(pool, lay, 2, slots, 1, rec)
    got = layout.get_records(pool, lay, 2, slots, 1)
    for k in rec:
        assert np.array_equal(got[k], rec[k]), k
    # rewriting one token leaves the others of its page intact
    rec2 = _records(lay, 1, 99)
    layout.put_records(pool, lay, 2, [36], 1, rec2)
    again = layout.get_records(pool, lay, 2, slots, 1)
    for k in rec:
        assert np.array_equal(np.delete(again[k], 2, axis=0), np.delete(rec[k], 2, axis=0)), k
        assert np.array_equal(again[k][2], rec2[k][0]), k
    # head 0 untouched
    for b in range(6):
        base = (b * 2) * lay.block_bytes
        assert np.count_nonzero(pool[base: base + lay.block_bytes]) == 0


def test_record_placement_by_hand():
    """Hand-computed positions of single set bits (K3/V3 store, slot 37 = block 2
    offset 5, head 1 of 2 -> region 5)."""
    lay = layout.StoreLayout(128, 3, 3, 32)
    base = 5 * lay.block_bytes
    zero = {k: np.zeros_like(v) for k, v in _records(lay, 1, 0).items()}
    # key dim 33 = block 1, element 1, code 0b100 -> stream bit 3*1 + 2 = 5 of
    # record (block 1, token 5) = record index 1*16 + 5 = 21, 12 bytes each
    r = dict(zero, idx=zero["idx"].copy())
    r["idx"][0, 33] = 4
    pool = layout.new_pool(3, 2, lay)
    layout.put_records(pool, lay, 2, [37], 1, r)
    nz = np.flatnonzero(pool)
    assert list(nz) == [base + lay.off_kc + 21 * 12] and pool[nz[0]] == 1 << 5
    # sign 70 = block 2, element 6 -> record 2*16 + 5 = 37 (4 bytes), bit 6
    r = dict(zero, z=zero["z"].copy())
    r["z"][0, 70] = 1
    pool = layout.new_pool(3, 2, lay)
    layout.put_records(pool, lay, 2, [37], 1, r)
    nz = np.flatnonzero(pool)
    assert list(nz) == [base + lay.off_ks + 37 * 4] and pool[nz[0]] == 1 << 6
    # value dim 9 = tile 0, column 9; token 5 = half 0, element 5: block 9, group
    # 0*2 + 5//4 = 1, element 1 -> stream element (9*16 + 1)*4 + 1 = 581, bits
    # 1743..1745; code 0b010 -> bit 1744 = byte 218, bit 0
    r = dict(zero, vcode=zero["vcode"].copy())
    r["vcode"][0, 9] = 2
    pool = layout.new_pool(3, 2, lay)
    layout.put_records(pool, lay, 2, [37], 1, r)
    nz = np.flatnonzero(pool)
    assert list(nz) == [base + lay.off_vc + 218] and pool[nz[0]] == 1 << 0
    # norms and group metadata are token-major fp16 pairs
    r = dict(zero, n16=np.float16([1.0]), zero16=zero["zero16"].copy())
    r["zero16"][0, 2] = np.float16(-2.0)
    pool = layout.new_pool(3, 2, lay)
    layout.put_records(pool, lay, 2, [37], 1, r)
    assert pool[base + lay.off_kn + 20: base + lay.off_kn + 22].view(np.float16)[0] == 1.0
    at = base + lay.off_vsz + 5 * 16 + 2 * 4 + 2
    assert pool[at: at + 2].view(np.float16)[0] == -2.0
    assert np.count_nonzero(pool) == 2      # 0x3C00 and 0xC000: one nonzero byte each


@pytest.mark.parametrize("vb", [2, 3, 4])
def test_value_code_map_is_a_bijection(vb):
    """Every bit of a page's Vc field is taken by exactly one (token, dim, bit) and
    the 8 codes of (tile i, column c, half h) are one contiguous v_bits*8-bit run."""
    lay = layout.StoreLayout(128, 2, vb, 32)
    offs = np.arange(16)
    bits = layout._field_bits(lay, np.zeros(16, np.int64), offs, "vcode") - lay.off_vc * 8   # [16, 128]
    allbits = (bits[..., None] + np.arange(vb)).ravel()
    assert np.array_equal(np.sort(allbits), np.arange(16 * 128 * vb))
    for h in range(2):
        for c in (0, 7, 15):
            for i in (0, 5, 7):
                run = bits[8 * h: 8 * h + 8, 16 * i + c]
                start = ((16 * h + c) * 8 + i) * 8 * vb
                assert list(run) == [start + k * vb for k in range(8)]


def test_bypass_placement_by_hand():
    """Bypass pages: keys token-major, values dim-major.  Token 5 of block 2, head 1
    of 3: page base (2*3 + 1) * 8192; key e at base + 5*256 + 2e, value e at
    base + 4096 + 32e + 2*5 (little-endian bf16 patterns)."""
    lay = layout.StoreLayout(bypass=True)
    assert lay.block_bytes == 8192
    pool = layout.new_pool(4, 3, lay)
    kbits = np.arange(128, dtype=np.uint16) + 0x3f00
    vbits = np.arange(128, dtype=np.uint16) + 0x4100
    layout.write_bypass(pool, lay, 3, 2 * 16 + 5, 1, kbits, vbits)
    base = 7 * 8192
    for e in (0, 1, 77, 127):
        ka, va = base + 5 * 256 + 2 * e, base + 4096 + 32 * e + 10
        assert pool[ka] == (0x3f00 + e) & 0xff and pool[ka + 1] == 0x3f
        assert pool[va] == (0x4100 + e) & 0xff and pool[va + 1] == 0x41
    assert np.count_nonzero(pool) == np.count_nonzero(kbits.view(np.uint8)) + np.count_nonzero(vbits.view(np.uint8))
    k, v = layout.read_bypass(pool, lay, 3, 2 * 16 + 5, 1)
    assert np.array_equal(k, layout.bf16_bits_to_f64(kbits))
    assert np.array_equal(v, layout.bf16_bits_to_f64(vbits))
    # a neighbouring token's values interleave with these, one bf16 apart
    layout.write_bypass(pool, lay, 3, 2 * 16 + 6, 1, kbits, vbits + 1)
    assert pool[base + 4096 + 32 * 3 + 12] == (0x4100 + 3 + 1) & 0xff
    k2, v2 = layout.read_bypass(pool, lay, 3, 2 * 16 + 5, 1)
    assert np.array_equal(v2, v)


def test_mse_value_layout_is_the_pages_102_byte_record():
    """K2 + QJL / V3 with MSE values: the worked 102-byte record and 5.02x of the
    byte-accounting fixture; the key fields keep their offsets."""
    ref = json.load(open(os.path.join(GOLDEN, "byte_accounting.json")))
    lay = layout.StoreLayout(128, 2, 3, 32, value_mode="mse")
    assert lay.record_bytes() == ref["blog_layout_bytes"]
    assert lay.block_bytes == 16 * ref["blog_layout_bytes"]
    assert metrics.record_bytes(128, 2, 3, 32, value_mode="mse") == ref["blog_layout_bytes"]
    assert abs(metrics.compression_ratio(lay.record_bytes()) - ref["blog_ratio"]) < 1e-4
    assert all(o % 64 == 0 for o in lay.field_offsets())
    assert lay.field_offsets()[:4] == layout.StoreLayout(128, 2, 3, 32).field_offsets()[:4]


@pytest.mark.parametrize("kb,vb", [(2, 3), (4, 4)])
def test_mse_value_record_round_trip(kb, vb):
    """MSE-value records (codes + one fp16 norm) at scattered slots read back exactly;
    rewriting one token leaves its page neighbours intact."""
    lay = layout.StoreLayout(128, kb, vb, 32, value_mode="mse")
    pool = layout.new_pool(6, 2, lay)
    slots = np.array([37, 5, 36, 80, 38, 0, 95, 17])
    rng = np.random.default_rng(kb * 7 + vb)

    def recs(n):
        return {"idx": rng.integers(0, 1 << kb, (n, 128)), "z": rng.integers(0, 2, (n, 128)),
                "n16": rng.standard_normal(n).astype(np.float16), "g16": rng.standard_normal(n).astype(np.float16),
                "vcode": rng.integers(0, 1 << vb, (n, 128)), "vn16": rng.standard_normal(n).astype(np.float16)}

    rec = recs(len(slots))
    layout.put_records(pool, lay, 2, slots, 0, rec)
    got = layout.get_records(pool, lay, 2, slots, 0)
    assert set(got) == set(rec)
    for k in rec:
        assert np.array_equal(got[k], rec[k]), k
    rec2 = recs(1)
    layout.put_records(pool, lay, 2, [36], 0, rec2)
    again = layout.get_records(pool, lay, 2, slots, 0)
    for k in rec:
        assert np.array_equal(np.delete(again[k], 2, axis=0), np.delete(rec[k], 2, axis=0)), k
        assert np.array_equal(again[k][2], rec2[k][0]), k


def test_mse_value_norm_placement_by_hand():
    """The fp16 norm of slot 21 (block 1, offset 5) of head 1 of 2, K2/V3: region
    3 (1632 bytes each), field offset 1600, token offset 2 * 5."""
    lay = layout.StoreLayout(128, 2, 3, 32, value_mode="mse")
    pool = layout.new_pool(2, 2, lay)
    rec = {"idx": np.zeros((1, 128), int), "z": np.zeros((1, 128), int), "n16": np.zeros(1, np.float16),
           "g16": np.zeros(1, np.float16), "vcode": np.zeros((1, 128), int), "vn16": np.array([1.5], np.float16)}
    layout.put_records(pool, lay, 2, [21], 1, rec)
    at = 3 * 1632 + 1600 + 10
    assert list(np.nonzero(pool)[0]) == [at + 1]  # 1.5 = 0x3E00: low byte 0, high byte 0x3E
    assert pool[at + 1] == 0x3E


def test_layout_without_qjl_by_hand():
    """Key modes without residual signs: no sign field, no gamma.  K4/V4 page =
    16 x (64 Kc + 2 Kn + 64 Vc + 16 Vsz) = 2336 bytes (146 per token-head, against
    164 with QJL); offsets Kc 0, Ks = Kn 1024 (0 bytes), Kn 1024, Vc 1056, Vsz 2080."""
    lay = layout.StoreLayout(128, 4, 4, 32, qjl=False)
    assert lay.block_bytes == 2336 and lay.record_bytes() == 146
    assert lay.field_offsets() == [0, 1024, 1024, 1056, 2080]
    mse = layout.StoreLayout(128, 2, 3, 32, value_mode="mse", qjl=False)
    assert mse.record_bytes() == 32 + 2 + 48 + 2  # 84
    # one token's magnitude at slot 37 (block 2, offset 5), head 1 of 2: bytes
    # off_kn + 2*5 of region 5, nothing else written
    zero = {k: np.zeros_like(v) for k, v in _records(lay, 1, 0).items()}
    r = dict(zero, n16=np.float16([2.0]))
    pool = layout.new_pool(3, 2, lay)
    layout.put_records(pool, lay, 2, [37], 1, r)
    base = 5 * lay.block_bytes
    assert list(np.flatnonzero(pool)) == [base + 1024 + 11] and pool[base + 1024 + 11] == 0x40  # fp16 2.0 = 0x4000
    got = layout.get_records(pool, lay, 2, [37], 1)
    assert got["n16"][0] == 2.0 and not got["z"].any() and got["g16"][0] == 0
    # signs or gamma handed to a layout without QJL are refused
    bad = dict(zero, z=zero["z"].copy())
    bad["z"][0, 3] = 1
    with pytest.raises(ValueError):
        layout.put_records(pool, lay, 2, [37], 1, bad)
    with pytest.raises(ValueError):
        layout.put_records(pool, lay, 2, [37], 1, dict(zero, g16=np.float16([0.5])))


@pytest.mark.parametrize("key_mode,value_mode", [("qjl", "group"), ("mse_nc", "group"), ("qjl", "mse")])
def test_store_of_no_tokens_writes_nothing(key_mode, value_mode):
    """A batch with no tokens (every sequence empty) stores nothing: the pool keeps
    its bytes, and reading no slots gives empty fields of the right widths."""
    from oracle import compress, state
    lay = layout.StoreLayout(128, 3, 2, 32, qjl=key_mode == "qjl", value_mode=value_mode)
    st = state.LayerState(7, 0, 2, 128, 3, 2, 32, key_mode=key_mode, value_mode=value_mode)
    pool = np.full(2 * 2 * lay.block_bytes, 0xA5, dtype=np.uint8)
    empty = np.zeros((0, 2, 128))
    compress.compress_into_pool(empty, empty, np.zeros(0, np.int64), pool, lay, st)
    assert np.all(pool == 0xA5)
    got = layout.get_records(pool, lay, 2, np.zeros(0, np.int64), 1)
    assert got["idx"].shape == (0, 128) and got["vcode"].shape == (0, 128)
    assert got["n16"].shape == (0,) and got["g16"].shape == (0,) and got["z"].shape[0] == 0
    if value_mode == "mse":
        assert got["vn16"].shape == (0,)
    else:
        assert got["scale16"].shape == (0, 4) and got["zero16"].shape == (0, 4)
