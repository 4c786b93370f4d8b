"""Python binding of libtq (TurboQuant-style compressed KV cache for MI355X).

Argument marshalling only: every step of compression and decode attention runs
in the library's HIP kernels.  PyTorch supplies device memory and the current
HIP stream.  If libtq.so is missing the calls raise; there is no fallback.
"""

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libtq.so")

OK, ERR_INVALID_ARGUMENT, ERR_UNSUPPORTED, ERR_OUT_OF_MEMORY, ERR_HIP, ERR_NOT_CONVERGED = range(6)
F32, BF16, F16 = 0, 1, 2
DIST_GAUSSIAN, DIST_SPHERE = 0, 1
KEY_QJL, KEY_MSE, KEY_MSE_NC = 0, 1, 2  # key estimator (tq_key_mode)
ROT_HAAR, ROT_HADAMARD = 0, 1  # rotation family (tq_rotation)
VAL_GROUP, VAL_MSE = 0, 1  # value coding (tq_value_mode)
ABI_VERSION = 6  # TQ_ABI_VERSION of include/tq.h that this binding mirrors
EXPORTED = [
    "tq_last_error", "tq_abi_version", "tq_codebook_build", "tq_layer_state_host",
    "tq_layer_create", "tq_layer_destroy", "tq_store_layout", "tq_compress_kv",
    "tq_decode_workspace_size", "tq_decode_attn", "tq_profile_enable", "tq_profile_read",
    "tq_profile_reset", "tq_decompress_kv", "tq_layer_export", "tq_layer_export_operands",
    "tq_decode_attn_noalloc",
]
OPERANDS_COMPRESS, OPERANDS_PROLOGUE, OPERANDS_DECOMPRESS = range(3)  # tq_operands
K_COMPRESS, K_PROLOGUE, K_SPLITK, K_COMBINE = range(4)


class TQError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__("libtq status %d: %s" % (status, msg))
        self.status = status


class LayerConfig(ctypes.Structure):
    _fields_ = [
        ("head_dim", ctypes.c_int), ("n_kv_heads", ctypes.c_int), ("k_bits", ctypes.c_int),
        ("v_bits", ctypes.c_int), ("v_group", ctypes.c_int), ("block_size", ctypes.c_int),
        ("layer", ctypes.c_int), ("dist", ctypes.c_int), ("seed", ctypes.c_ulonglong),
        ("bypass", ctypes.c_int), ("key_mode", ctypes.c_int), ("rotation", ctypes.c_int),
        ("value_mode", ctypes.c_int),
    ]


def config(n_kv_heads, k_bits=4, v_bits=4, seed=0, layer=0, dist=DIST_GAUSSIAN, bypass=False,
           head_dim=128, v_group=32, block_size=16, key_mode=KEY_QJL, rotation=ROT_HAAR, value_mode=VAL_GROUP):
    return LayerConfig(head_dim, n_kv_heads, k_bits, v_bits, v_group, block_size, layer, dist, seed,
                       int(bool(bypass)), key_mode, rotation, value_mode)


_LIB = None


def lib():
    """Load libtq.so (raises if it has not been built)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libtq.so not built: run `python -m compressed_decode_attention_tq_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    c_int, c_ll, c_size, vp = ctypes.c_int, ctypes.c_longlong, ctypes.c_size_t, ctypes.c_void_p
    dp, fp = ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_float)
    L.tq_last_error.restype = ctypes.c_char_p
    L.tq_abi_version.restype = c_int
    if L.tq_abi_version() != ABI_VERSION:
        # the config struct and entry points of another version would be misread
        raise RuntimeError("libtq.so has ABI %d, this binding expects %d: rebuild it"
                           % (L.tq_abi_version(), ABI_VERSION))
    L.tq_codebook_build.argtypes = [c_int, c_int, c_int, dp, dp, dp]
    L.tq_layer_state_host.argtypes = [ctypes.POINTER(LayerConfig), fp, fp, fp, fp]
    L.tq_layer_create.argtypes = [ctypes.POINTER(LayerConfig), vp, ctypes.POINTER(vp)]
    L.tq_layer_destroy.argtypes = [vp]
    L.tq_store_layout.argtypes = [ctypes.POINTER(LayerConfig), ctypes.POINTER(c_size), ctypes.POINTER(c_size)]
    L.tq_compress_kv.argtypes = [vp, vp, vp, c_int, c_ll, c_ll, c_ll, vp, vp, c_ll, vp]
    L.tq_decompress_kv.argtypes = [vp, vp, c_ll, vp, c_ll, vp, vp, c_int, vp]
    L.tq_decode_workspace_size.argtypes = [vp, c_int, c_int, c_int, c_int, ctypes.POINTER(c_size)]
    L.tq_decode_attn.argtypes = [vp, vp, c_int, c_int, c_int, vp, c_ll, vp, c_int, vp, c_int,
                                 ctypes.c_float, c_int, vp, c_int, vp, c_size, vp]
    L.tq_decode_attn_noalloc.argtypes = [vp, vp, c_int, c_int, c_int, vp, c_ll, vp, c_int, vp, c_int,
                                         ctypes.c_float, c_int, vp, c_int, vp]
    L.tq_layer_export.argtypes = [vp, fp, fp, fp, fp, fp, fp, vp]
    L.tq_layer_export_operands.argtypes = [vp, c_int, vp, c_size, ctypes.POINTER(c_size), vp]
    L.tq_profile_enable.argtypes = [ctypes.c_uint]
    L.tq_profile_read.argtypes = [c_int, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(c_ll)]
    L.tq_profile_reset.argtypes = []
    for name in ["tq_codebook_build", "tq_layer_state_host", "tq_layer_create", "tq_layer_destroy",
                 "tq_store_layout", "tq_compress_kv", "tq_decode_workspace_size", "tq_decode_attn",
                 "tq_profile_enable", "tq_profile_read", "tq_profile_reset", "tq_layer_export",
                 "tq_layer_export_operands", "tq_decompress_kv", "tq_decode_attn_noalloc"]:
        getattr(L, name).restype = c_int
    _LIB = L
    return L


def _check(status):
    if status != OK:
        raise TQError(status, lib().tq_last_error().decode())


def _dptr(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _fptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.POINTER(ctypes.c_float))


# ------------------------------------------------------------------- host only
def codebook_build(bits, dist=DIST_GAUSSIAN, dim=128):
    L = 1 << bits
    c = np.zeros(L)
    b = np.zeros(max(L - 1, 1))
    mse = ctypes.c_double(0.0)
    _check(lib().tq_codebook_build(bits, dist, dim, _dptr(c), _dptr(b), ctypes.byref(mse)))
    return c, b[: L - 1], mse.value


def layer_state_host(cfg):
    H, d = cfg.n_kv_heads, cfg.head_dim
    R = np.zeros((H, d, d), np.float32)
    S = np.zeros((H, d, d), np.float32)
    nl = 0 if cfg.bypass else (1 << cfg.k_bits)
    c = np.zeros(max(nl, 1), np.float32)
    b = np.zeros(max(nl - 1, 1), np.float32)
    _check(lib().tq_layer_state_host(ctypes.byref(cfg), _fptr(R), _fptr(S), _fptr(c), _fptr(b)))
    return R, S, c[:nl], b[: max(nl - 1, 0)]


def store_layout(cfg):
    bb = ctypes.c_size_t(0)
    offs = (ctypes.c_size_t * 5)()
    _check(lib().tq_store_layout(ctypes.byref(cfg), ctypes.byref(bb), offs))
    return bb.value, list(offs)


# ------------------------------------------------------------------ device side
def _torch():
    import torch
    return torch


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float16:
        return F16
    raise TQError(ERR_UNSUPPORTED, "unsupported tensor dtype %s" % t.dtype)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


class Layer:
    """Device state of one layer (R, S, codebook).  Owns it until close()."""

    def __init__(self, cfg, stream=None):
        self.cfg = cfg
        self.handle = ctypes.c_void_p()
        _check(lib().tq_layer_create(ctypes.byref(cfg), _stream(stream), ctypes.byref(self.handle)))
        self.block_bytes, self.field_offsets = store_layout(cfg)

    def close(self):
        if self.handle:
            _check(lib().tq_layer_destroy(self.handle))
            self.handle = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def export(self, stream=None):
        """(R, S, centroids, boundaries, v_centroids, v_boundaries) as the device holds them."""
        cfg = self.cfg
        H = cfg.n_kv_heads
        R = np.zeros((H, 128, 128), np.float32)
        S = np.zeros((H, 128, 128), np.float32)
        nk = 0 if cfg.bypass else 1 << cfg.k_bits
        nv = (1 << cfg.v_bits) if (not cfg.bypass and cfg.value_mode == VAL_MSE) else 0
        c, b = np.zeros(max(nk, 1), np.float32), np.zeros(max(nk - 1, 1), np.float32)
        vc, vb = np.zeros(max(nv, 1), np.float32), np.zeros(max(nv - 1, 1), np.float32)
        _check(lib().tq_layer_export(self.handle, _fptr(R), _fptr(S), _fptr(c), _fptr(b), _fptr(vc), _fptr(vb),
                                     _stream(stream)))
        return R, S, c[:nk], b[:max(nk - 1, 0)], vc[:nv], vb[:max(nv - 1, 0)]

    def export_operands(self, which, stream=None):
        """One matrix-core operand buffer of the layer as uint16 words (tq_layer_export_operands)."""
        n = ctypes.c_size_t(0)
        _check(lib().tq_layer_export_operands(self.handle, which, None, 0, ctypes.byref(n), _stream(stream)))
        out = np.zeros(n.value // 2, np.uint16)
        _check(lib().tq_layer_export_operands(self.handle, which, out.ctypes.data_as(ctypes.c_void_p), n.value,
                                              ctypes.byref(n), _stream(stream)))
        return out

    def new_pool(self, num_blocks):
        torch = _torch()
        return torch.zeros(num_blocks * self.cfg.n_kv_heads * self.block_bytes, dtype=torch.uint8, device="cuda")


def _require(cond, msg):
    if not cond:
        raise TQError(ERR_INVALID_ARGUMENT, msg)


def _check_pool(layer, pool):
    torch = _torch()
    _require(pool.dtype == torch.uint8 and pool.is_contiguous(), "pool must be a contiguous uint8 tensor")
    per_block = layer.cfg.n_kv_heads * layer.block_bytes
    _require(pool.numel() % per_block == 0 and pool.numel() > 0,
             "pool size %d is not a positive multiple of n_kv_heads*block_bytes = %d" % (pool.numel(), per_block))
    return pool.numel() // per_block


def _check_rows(name, t, n, H):
    """[n, H, 128] with unit element stride and head stride 128 (any token stride)."""
    _require(t.dim() == 3 and tuple(t.shape[1:]) == (H, 128),
             "%s must have shape [N, %d, 128], got %s" % (name, H, tuple(t.shape)))
    _require(t.shape[0] == n, "%s has %d rows, slot_mapping has %d" % (name, t.shape[0], n))
    _require(t.stride(2) == 1 and t.stride(1) == 128,
             "%s must have element stride 1 and head stride 128, got strides %s" % (name, tuple(t.stride())))


def compress_kv(layer, k, v, slot_mapping, pool, stream=None):
    """k, v: [N, H_kv, 128] (f32 or bf16, token stride = k.stride(0)); slot_mapping int64 [N]."""
    torch = _torch()
    _require(slot_mapping.dtype == torch.int64 and slot_mapping.dim() == 1 and slot_mapping.is_contiguous(),
             "slot_mapping must be a contiguous 1-D int64 tensor")
    n = slot_mapping.shape[0]
    H = layer.cfg.n_kv_heads
    _check_rows("k", k, n, H)
    _check_rows("v", v, n, H)
    _require(k.dtype == v.dtype, "k and v must have the same dtype (%s vs %s)" % (k.dtype, v.dtype))
    num_blocks = _check_pool(layer, pool)
    _check(lib().tq_compress_kv(layer.handle, _ptr(k), _ptr(v), _dtype_code(k), n, k.stride(0), v.stride(0),
                                _ptr(slot_mapping), _ptr(pool), num_blocks, _stream(stream)))


def decompress_kv(layer, pool, slot_mapping, out_dtype=None, k_out=None, v_out=None, stream=None):
    """K, V [N, H_kv, 128] (f32 or bf16) reconstructed from the store at slot_mapping int64 [N]."""
    torch = _torch()
    _require(slot_mapping.dtype == torch.int64 and slot_mapping.dim() == 1 and slot_mapping.is_contiguous(),
             "slot_mapping must be a contiguous 1-D int64 tensor")
    n, H = slot_mapping.shape[0], layer.cfg.n_kv_heads
    dt = out_dtype or (k_out.dtype if k_out is not None else torch.float32)
    if k_out is None:
        k_out = torch.empty((n, H, 128), dtype=dt, device=pool.device)
    if v_out is None:
        v_out = torch.empty((n, H, 128), dtype=dt, device=pool.device)
    for name, t in (("k_out", k_out), ("v_out", v_out)):
        _require(t.is_contiguous() and tuple(t.shape) == (n, H, 128),
                 "%s must be a contiguous [%d, %d, 128] tensor" % (name, n, H))
    _require(k_out.dtype == v_out.dtype, "k_out and v_out must have the same dtype")
    num_blocks = _check_pool(layer, pool)
    _check(lib().tq_decompress_kv(layer.handle, _ptr(pool), num_blocks, _ptr(slot_mapping), n, _ptr(k_out),
                                  _ptr(v_out), _dtype_code(k_out), _stream(stream)))
    return k_out, v_out


def decode_workspace_size(layer, batch, n_q_heads, max_seq_len, num_splits=0):
    out = ctypes.c_size_t(0)
    _check(lib().tq_decode_workspace_size(layer.handle, batch, n_q_heads, max_seq_len, num_splits,
                                          ctypes.byref(out)))
    return out.value


def new_workspace(layer, batch, n_q_heads, max_seq_len, num_splits=0):
    torch = _torch()
    nbytes = decode_workspace_size(layer, batch, n_q_heads, max_seq_len, num_splits)
    return torch.empty(nbytes, dtype=torch.uint8, device="cuda")


def _check_decode_args(layer, q, pool, block_table, seq_lens, out):
    torch = _torch()
    _require(q.dim() == 3 and q.shape[2] == 128 and q.is_contiguous(),
             "q must be a contiguous [B, H_q, 128] tensor, got shape %s strides %s" % (tuple(q.shape), tuple(q.stride())))
    B, Hq = q.shape[0], q.shape[1]
    _require(block_table.dtype == torch.int32 and block_table.dim() == 2 and block_table.is_contiguous()
             and block_table.shape[0] == B, "block_table must be a contiguous int32 [%d, max_blocks] tensor" % B)
    _require(seq_lens.dtype == torch.int32 and seq_lens.dim() == 1 and seq_lens.is_contiguous()
             and seq_lens.shape[0] == B, "seq_lens must be a contiguous int32 [%d] tensor" % B)
    if out is not None:
        _require(out.is_contiguous() and tuple(out.shape) == (B, Hq, 128),
                 "out must be a contiguous [%d, %d, 128] tensor" % (B, Hq))
    return _check_pool(layer, pool)


def decode_attn(layer, q, pool, block_table, seq_lens, max_seq_len, out=None, workspace=None,
                softmax_scale=0.0, num_splits=0, out_dtype=None, stream=None):
    """q: [B, H_q, 128]; block_table int32 [B, max_blocks]; seq_lens int32 [B]."""
    torch = _torch()
    num_blocks = _check_decode_args(layer, q, pool, block_table, seq_lens, out)
    B, Hq = q.shape[0], q.shape[1]
    if out is None:
        out = torch.empty((B, Hq, 128), dtype=out_dtype or torch.float32, device=q.device)
    if workspace is None:
        workspace = new_workspace(layer, B, Hq, max_seq_len, num_splits)
    _require(workspace.dtype == torch.uint8 and workspace.is_contiguous(), "workspace must be a contiguous uint8 tensor")
    _check(lib().tq_decode_attn(layer.handle, _ptr(q), _dtype_code(q), B, Hq, _ptr(pool), num_blocks,
                                _ptr(block_table), block_table.shape[1], _ptr(seq_lens), max_seq_len,
                                float(softmax_scale), num_splits, _ptr(out), _dtype_code(out),
                                _ptr(workspace), workspace.numel(), _stream(stream)))
    return out


def decode_attn_noalloc(layer, q, pool, block_table, seq_lens, max_seq_len, out, softmax_scale=0.0, num_splits=0,
                        stream=None):
    """decode_attn with the library's static per-GPU workspace (tq_decode_attn_noalloc):
    nothing is allocated, `out` is required."""
    num_blocks = _check_decode_args(layer, q, pool, block_table, seq_lens, out)
    _check(lib().tq_decode_attn_noalloc(layer.handle, _ptr(q), _dtype_code(q), q.shape[0], q.shape[1], _ptr(pool),
                                        num_blocks, _ptr(block_table), block_table.shape[1], _ptr(seq_lens),
                                        max_seq_len, float(softmax_scale), num_splits, _ptr(out), _dtype_code(out),
                                        _stream(stream)))
    return out


# ------------------------------------------------------------------- profiling
def profile_enable(mask):
    _check(lib().tq_profile_enable(mask))


def profile_read(kernel):
    """(total milliseconds, launches) of the timed launches of `kernel` since the last reset."""
    ms = ctypes.c_double(0.0)
    n = ctypes.c_longlong(0)
    _check(lib().tq_profile_read(kernel, ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


def profile_reset():
    _check(lib().tq_profile_reset())
