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


def test_record_round_trip():
    lay = layout.StoreLayout(128, 3, 2, 32)
    pool = layout.new_pool(4, 2, lay)
    rng = np.random.default_rng(0)
    kc = rng.integers(0, 256, lay.kc_bytes)
    ks = rng.integers(0, 256, lay.ks_bytes)
    vc = rng.integers(0, 256, lay.vc_bytes)
    sc = np.float16([0.5, 0.25, 2.0, 1.5])
    ze = np.float16([-1.0, -2.0, 0.125, 3.0])
    layout.write_compressed(pool, lay, 2, 37, 1, kc, ks, 3.5, 0.75, vc, sc, ze)
    got = layout.read_compressed(pool, lay, 2, 37, 1)
    assert np.array_equal(got[0], kc) and np.array_equal(got[1], ks) and np.array_equal(got[4], vc)
    assert got[2] == 3.5 and got[3] == 0.75
    assert np.array_equal(got[5], sc) and np.array_equal(got[6], ze)
    # slot 37 = block 2, offset 5, head 1 -> region 5
    base = (2 * 2 + 1) * lay.block_bytes
    assert pool[base + lay.off_kc + 5 * lay.kc_bytes] == kc[0]
    assert np.count_nonzero(pool[:base]) == 0
