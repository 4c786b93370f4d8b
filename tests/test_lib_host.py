"""libtq on the CPU: exported symbols, host state against the oracle, error paths.

No compute call here touches a device.
"""

import ctypes
import os
import re

import numpy as np
import pytest

import compressed_decode_attention_tq_amd as tq
from oracle import codebook, layout, state

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_symbols():
    text = open(os.path.join(ROOT, "include", "tq.h")).read()
    return sorted(set(re.findall(r"^\s*(?:tq_status|const char\*|int)\s+(tq_\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_symbol():
    lib = tq.lib()
    names = _declared_symbols()
    assert len(names) == 17
    assert sorted(names) == sorted(tq.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n
    assert lib.tq_abi_version() == tq.ABI_VERSION == 6


def test_export_error_paths_without_a_device():
    lib = tq.lib()
    assert lib.tq_layer_export(None, None, None, None, None, None, None, None) == tq.ERR_INVALID_ARGUMENT
    n = ctypes.c_size_t(0)
    assert lib.tq_layer_export_operands(None, 0, None, 0, ctypes.byref(n), None) == tq.ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("dist,name", [(tq.DIST_GAUSSIAN, "gaussian"), (tq.DIST_SPHERE, "sphere")])
@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_codebook_matches_oracle(bits, dist, name):
    c, b, mse = tq.codebook_build(bits, dist, 128)
    oc, ob, om = codebook.lloyd_max(bits, name, 128)
    assert np.max(np.abs(c - oc)) < 1e-12
    assert np.max(np.abs(b - ob)) < 1e-12
    assert abs(mse - om) < 1e-12
    # the stored (float16-rounded) codebook the kernels use is identical
    assert np.array_equal(c.astype(np.float16), oc.astype(np.float16))


@pytest.mark.parametrize("layer,heads,kb", [(0, 1, 2), (3, 8, 4), (17, 2, 3), (5, 2, 1)])
def test_layer_state_matches_oracle(layer, heads, kb):
    cfg = tq.config(heads, kb, 3, seed=205, layer=layer)
    R, S, c, b = tq.layer_state_host(cfg)
    st = state.LayerState(205, layer, heads, 128, kb, 3, 32)
    # same generators, same float32 rounding: bit-identical except at rare rounding ties
    assert np.count_nonzero(R.astype(np.float64) != st.R) <= 2
    assert np.max(np.abs(R - st.R)) <= 1.2e-7
    assert np.array_equal(S.astype(np.float64), st.S)
    assert np.array_equal(c.astype(np.float64), st.centroids)
    assert np.array_equal(b.astype(np.float64), st.boundaries)


@pytest.mark.parametrize("kb,vb", [(1, 2), (1, 3), (2, 2), (2, 3), (3, 2), (3, 3), (4, 3), (4, 4)])
def test_store_layout_matches_oracle(kb, vb):
    bb, offs = tq.store_layout(tq.config(8, kb, vb))
    lay = layout.StoreLayout(128, kb, vb, 32)
    assert bb == lay.block_bytes
    assert offs == lay.field_offsets()
    bb, offs = tq.store_layout(tq.config(8, bypass=True))
    lay = layout.StoreLayout(bypass=True)
    assert bb == lay.block_bytes and offs[:2] == lay.field_offsets()


def _status_of(fn):
    with pytest.raises(tq.TQError) as e:
        fn()
    assert str(e.value)
    return e.value.status


def test_config_errors():
    bad = [
        (dict(head_dim=64), tq.ERR_UNSUPPORTED), (dict(k_bits=5), tq.ERR_UNSUPPORTED),
        (dict(k_bits=0), tq.ERR_UNSUPPORTED), (dict(v_bits=1), tq.ERR_UNSUPPORTED),
        (dict(v_group=16), tq.ERR_UNSUPPORTED), (dict(block_size=32), tq.ERR_UNSUPPORTED),
        (dict(n_kv_heads=0), tq.ERR_INVALID_ARGUMENT), (dict(layer=-1), tq.ERR_INVALID_ARGUMENT),
        (dict(dist=7), tq.ERR_INVALID_ARGUMENT), (dict(key_mode=3), tq.ERR_INVALID_ARGUMENT),
        (dict(key_mode=-1), tq.ERR_INVALID_ARGUMENT), (dict(rotation=2), tq.ERR_INVALID_ARGUMENT),
        (dict(value_mode=2), tq.ERR_INVALID_ARGUMENT),
    ]
    for kw, want in bad:
        args = dict(n_kv_heads=8)
        args.update(kw)
        cfg = tq.config(**args)
        assert _status_of(lambda: tq.store_layout(cfg)) == want, kw
        assert _status_of(lambda: tq.layer_state_host(cfg)) == want, kw


def test_codebook_errors():
    assert _status_of(lambda: tq.codebook_build(0)) == tq.ERR_INVALID_ARGUMENT
    assert _status_of(lambda: tq.codebook_build(9)) == tq.ERR_INVALID_ARGUMENT
    assert _status_of(lambda: tq.codebook_build(2, tq.DIST_SPHERE, 2)) == tq.ERR_INVALID_ARGUMENT


def test_null_and_bad_arguments_on_device_entry_points():
    lib = tq.lib()
    vp = ctypes.c_void_p
    assert lib.tq_compress_kv(None, vp(1), vp(1), tq.BF16, 1, 1024, 1024, vp(1), vp(1), 1, None) == tq.ERR_INVALID_ARGUMENT
    assert b"null layer" in lib.tq_last_error()
    out = ctypes.c_size_t(0)
    assert lib.tq_decode_workspace_size(None, 1, 1, 1, 0, ctypes.byref(out)) == tq.ERR_INVALID_ARGUMENT
    assert lib.tq_decode_attn(None, vp(1), tq.BF16, 1, 1, vp(1), 1, vp(1), 1, vp(1), 16, 0.0, 0,
                              vp(1), tq.F32, vp(256), 1 << 20, None) == tq.ERR_INVALID_ARGUMENT
    assert lib.tq_decompress_kv(None, vp(1), 1, vp(1), 1, vp(1), vp(1), tq.F32, None) == tq.ERR_INVALID_ARGUMENT
    assert lib.tq_layer_destroy(None) == tq.OK
    assert lib.tq_layer_create(None, None, ctypes.byref(vp())) == tq.ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("kb,vb,value_mode", [(2, 3, 0), (4, 4, 0), (1, 2, 0), (2, 3, 1)])
def test_key_modes_without_qjl_use_the_compact_layout(kb, vb, value_mode):
    """The two key modes without QJL store no sign field and no gamma: the library's
    layout equals the oracle's compact layout (Ks 0 bytes at Kn's offset, Kn [16]
    fp16), 18 bytes per token-head less than with QJL."""
    vm = "mse" if value_mode else "group"
    ref = tq.store_layout(tq.config(8, kb, vb, value_mode=value_mode))
    for km in (tq.KEY_MSE, tq.KEY_MSE_NC):
        bb, offs = tq.store_layout(tq.config(8, kb, vb, key_mode=km, value_mode=value_mode))
        lay = layout.StoreLayout(128, kb, vb, 32, value_mode=vm, qjl=False)
        assert bb == lay.block_bytes and offs == lay.field_offsets()
        assert ref[0] - bb == 16 * 18
        assert all(o % 16 == 0 for o in offs)


@pytest.mark.parametrize("layer,heads", [(0, 1), (5, 3)])
def test_hadamard_layer_state_matches_oracle(layer, heads):
    cfg = tq.config(heads, 3, 3, seed=207, layer=layer, rotation=tq.ROT_HADAMARD)
    R, S, c, b = tq.layer_state_host(cfg)
    st = state.LayerState(207, layer, heads, 128, 3, 3, 32, rotation_kind="hadamard")
    assert np.array_equal(R.astype(np.float64), st.R)
    assert np.array_equal(S.astype(np.float64), st.S)


@pytest.mark.parametrize("kb,vb", [(2, 3), (4, 4), (3, 2)])
def test_mse_value_layout_matches_oracle(kb, vb):
    """Values coded like the keys: the library's page layout equals the oracle's
    (one fp16 norm per token in the last field; 102 bytes per token-head at K2/V3)."""
    bb, offs = tq.store_layout(tq.config(8, kb, vb, value_mode=tq.VAL_MSE))
    lay = layout.StoreLayout(128, kb, vb, 32, value_mode="mse")
    assert bb == lay.block_bytes
    assert offs == lay.field_offsets()
    if (kb, vb) == (2, 3):
        assert bb == 16 * 102


def test_bench_refuses_several_gpus():
    """bench.py measures one GPU: --gpus 2 exits with status 2 and says why,
    before any device is touched."""
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and "--gpus 2" in r.stderr
    assert r.stdout == ""
