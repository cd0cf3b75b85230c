"""ctypes binding of libqmoe.so (include/qmoe.h), argument marshalling only.

Every function takes torch tensors that already live on the GPU, passes their
data pointers and torch's current HIP stream to the C entry point of the same
name, and raises QmError on a negative status.  No computation happens here;
if the library is missing the import fails loudly (there is no fallback).
"""
import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
# QMOE_LIB_PATH names another build of the same sources (e.g. a sanitized host build)
LIB_PATH = os.environ.get("QMOE_LIB_PATH", os.path.join(HERE, "libqmoe.so"))

QM_OK, QM_ERR_INVALID, QM_ERR_UNSUPPORTED, QM_ERR_WORKSPACE, QM_ERR_LAUNCH, QM_ERR_TOO_LARGE = 0, -1, -2, -3, -4, -5
QM_FMT_INT8_ROW, QM_FMT_INT4 = 1, 4
QM_F32, QM_BF16 = 0, 1
QM_SMALL_MAX, QM_TOPK_MAX, QM_DECODE_MAX_TOKENS = 8, 32, 8
QM_NOALLOC_SCRATCH_BYTES = 32 << 20
QM_PATH_AUTO, QM_PATH_DECODE, QM_PATH_PREFILL = 0, 1, 2

EXPORTS = ("qgemv", "qgemv_pair", "qgemv_norm_chain", "qgemm_small", "moe_expert_ffn_workspace", "moe_expert_ffn", "moe_expert_ffn_path",
           "moe_gate_up", "moe_down", "moe_expert_ffn_noalloc", "qm_strerror",
           "qm_pack_int4", "qm_pack_int8", "qm_validate", "qm_quantize_int4", "qm_quantize_int8")
QM_FMT_INT3 = 5


class QmError(RuntimeError):
    def __init__(self, status, lib):
        self.status = status
        super().__init__("qmoe status %d: %s" % (status, lib.qm_strerror(status).decode()))


class QMat(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int32), ("n", ctypes.c_int32), ("k", ctypes.c_int32),
                ("group_size", ctypes.c_int32), ("q", ctypes.c_void_p), ("scales", ctypes.c_void_p)]


class Experts(ctypes.Structure):
    _fields_ = [("n_experts", ctypes.c_int32), ("hidden", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("fmt", ctypes.c_int32), ("group_size", ctypes.c_int32),
                ("gate_q", ctypes.c_void_p), ("up_q", ctypes.c_void_p), ("down_q", ctypes.c_void_p),
                ("gate_s", ctypes.c_void_p), ("up_s", ctypes.c_void_p), ("down_s", ctypes.c_void_p)]


def load(path=LIB_PATH):
    if not os.path.exists(path):
        raise ImportError("libqmoe.so not built at %s (run python -m int4_expert_gemv_amd.build)" % path)
    L = ctypes.CDLL(path)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    L.qgemv.argtypes = [ctypes.POINTER(QMat), vp, i32, vp, vp]
    L.qgemv.restype = ctypes.c_int
    L.qgemv_pair.argtypes = [ctypes.POINTER(QMat), ctypes.POINTER(QMat), vp, i32, vp, vp, vp]
    L.qgemv_pair.restype = ctypes.c_int
    L.qgemv_norm_chain.argtypes = [ctypes.POINTER(QMat), ctypes.POINTER(QMat), vp, ctypes.c_float,
                                   ctypes.POINTER(QMat), vp, i32, vp, vp, vp, vp]
    L.qgemv_norm_chain.restype = ctypes.c_int
    L.qgemm_small.argtypes = [ctypes.POINTER(QMat), vp, i32, i32, i64, vp, i64, vp]
    L.qgemm_small.restype = ctypes.c_int
    L.moe_expert_ffn_workspace.argtypes = [ctypes.POINTER(Experts), i32, i32]
    L.moe_expert_ffn_workspace.restype = sz
    L.moe_expert_ffn.argtypes = [ctypes.POINTER(Experts), vp, i32, i32, vp, vp, i32, vp, vp, sz, vp]
    L.moe_expert_ffn.restype = ctypes.c_int
    L.moe_expert_ffn_path.argtypes = [ctypes.POINTER(Experts), vp, i32, i32, vp, vp, i32, vp, vp, sz, vp, i32]
    L.moe_expert_ffn_path.restype = ctypes.c_int
    L.moe_gate_up.argtypes = [ctypes.POINTER(Experts), vp, i32, i32, vp, i32, vp, vp, sz, vp]
    L.moe_gate_up.restype = ctypes.c_int
    L.moe_down.argtypes = [ctypes.POINTER(Experts), vp, i32, vp, vp, i32, vp, vp, sz, vp]
    L.moe_down.restype = ctypes.c_int
    L.moe_expert_ffn_noalloc.argtypes = [ctypes.POINTER(Experts), vp, i32, i32, vp, vp, i32, vp, vp]
    L.moe_expert_ffn_noalloc.restype = ctypes.c_int
    L.qm_strerror.argtypes = [ctypes.c_int]
    L.qm_strerror.restype = ctypes.c_char_p
    L.qm_pack_int4.argtypes = [vp, i64, i64, vp]
    L.qm_pack_int8.argtypes = [vp, i64, i64, vp]
    L.qm_validate.argtypes = [i32, i64, i64, i32, vp]
    L.qm_quantize_int4.argtypes = [vp, i64, i64, i32, vp, vp]
    L.qm_quantize_int8.argtypes = [vp, i64, i64, vp, vp]
    for f in (L.qm_pack_int4, L.qm_pack_int8, L.qm_validate, L.qm_quantize_int4, L.qm_quantize_int8):
        f.restype = ctypes.c_int
    return L


lib = load()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _dtype_code(x):
    if x.dtype == torch.bfloat16:
        return QM_BF16
    if x.dtype == torch.float32:
        return QM_F32
    raise TypeError("activations must be float32 or bfloat16")


def _check(st):
    if st != QM_OK:
        raise QmError(st, lib)


def qmat(fmt, q, scales, n, k, group_size=0):
    """Describe a device-resident quantized matrix (keeps the tensors alive)."""
    m = QMat(fmt, n, k, group_size, q.data_ptr(), scales.data_ptr())
    m._keep = (q, scales)
    return m


def experts(fmt, group_size, gate_q, up_q, down_q, gate_s, up_s, down_s):
    E, I = gate_q.shape[0], gate_q.shape[1]
    H = down_q.shape[1]
    ex = Experts(E, H, I, fmt, group_size, gate_q.data_ptr(), up_q.data_ptr(), down_q.data_ptr(),
                 gate_s.data_ptr(), up_s.data_ptr(), down_s.data_ptr())
    ex._keep = (gate_q, up_q, down_q, gate_s, up_s, down_s)
    return ex


def qgemv(w, x, y, stream=None):
    _check(lib.qgemv(ctypes.byref(w), _ptr(x), _dtype_code(x), _ptr(y), _stream(stream)))
    return y


def qgemv_pair(w1, w2, x, y1, y2, stream=None):
    _check(lib.qgemv_pair(ctypes.byref(w1), ctypes.byref(w2), _ptr(x), _dtype_code(x), _ptr(y1), _ptr(y2),
                          _stream(stream)))
    return y1, y2


def qgemv_norm_chain(w_a, w_kv, norm_w, eps, w_b, x, u, kv, q, stream=None):
    """u = rmsnorm(W_a x) * norm_w (norm_w None: ones), kv = W_kv x, q = W_b u."""
    _check(lib.qgemv_norm_chain(ctypes.byref(w_a), ctypes.byref(w_kv), None if norm_w is None else _ptr(norm_w),
                                eps, ctypes.byref(w_b), _ptr(x), _dtype_code(x), _ptr(u), _ptr(kv), _ptr(q),
                                _stream(stream)))
    return u, kv, q


def qgemm_small(w, x, y, stream=None):
    """x: [batch][ldx] device tensor; y: [batch][ldy] fp32."""
    _check(lib.qgemm_small(ctypes.byref(w), _ptr(x), _dtype_code(x), x.shape[0], x.stride(0), _ptr(y),
                           y.stride(0), _stream(stream)))
    return y


def moe_expert_ffn_workspace(ex, n_tokens, top_k):
    return lib.moe_expert_ffn_workspace(ctypes.byref(ex), n_tokens, top_k)


def moe_expert_ffn(ex, x, topk_ids, topk_w, y, workspace, stream=None, path=QM_PATH_AUTO):
    T, k = topk_ids.shape
    _check(lib.moe_expert_ffn_path(ctypes.byref(ex), _ptr(x), _dtype_code(x), T, _ptr(topk_ids), _ptr(topk_w), k,
                                   _ptr(y), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                   _stream(stream), path))
    return y


def moe_expert_ffn_noalloc(ex, x, topk_ids, topk_w, y, stream=None):
    """moe_expert_ffn on the library's fixed per-GPU scratch (no workspace)."""
    T, k = topk_ids.shape
    _check(lib.moe_expert_ffn_noalloc(ctypes.byref(ex), _ptr(x), _dtype_code(x), T, _ptr(topk_ids), _ptr(topk_w), k,
                                      _ptr(y), _stream(stream)))
    return y


def moe_gate_up(ex, x, topk_ids, h, workspace, stream=None):
    """h: fp32 [T*k][inter] device tensor (stage 1 of the decode path)."""
    T, k = topk_ids.shape
    _check(lib.moe_gate_up(ctypes.byref(ex), _ptr(x), _dtype_code(x), T, _ptr(topk_ids), k, _ptr(h),
                           _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))
    return h


def moe_down(ex, h, topk_ids, topk_w, y, workspace, stream=None):
    """Stage 2 of the decode path: y from the hidden rows of moe_gate_up."""
    T, k = topk_ids.shape
    _check(lib.moe_down(ctypes.byref(ex), _ptr(h), T, _ptr(topk_ids), _ptr(topk_w), k, _ptr(y), _ptr(workspace),
                        workspace.numel() * workspace.element_size(), _stream(stream)))
    return y


def raw_status(fn, *args):
    """Call an entry point with raw ctypes arguments and return its status
    (used by the host-side validation tests)."""
    return getattr(lib, fn)(*args)


# ---- host packing (numpy arrays in host memory; no GPU) -----------------------------

def _host(a, dtype):
    import numpy as np
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError("expected %s, got %s" % (np.dtype(dtype), a.dtype))
    return a


def pack_int4(v):
    """int8 values in [-8, 7], shape [n][k] -> packed uint8 [n][k/2]."""
    import numpy as np
    v = _host(v, np.int8)
    n, k = v.shape
    q = np.empty((n, k // 2), np.uint8)
    _check(lib.qm_pack_int4(v.ctypes.data, n, k, q.ctypes.data))
    return q


def pack_int8(v):
    """int8 values [n][k] -> the int8 layout [n][k]."""
    import numpy as np
    v = _host(v, np.int8)
    q = np.empty_like(v)
    _check(lib.qm_pack_int8(v.ctypes.data, v.shape[0], v.shape[1], q.ctypes.data))
    return q


def validate(fmt, n, k, group_size, scales):
    """QM_OK when the format's shape rules hold and every scale is finite."""
    import numpy as np
    s = _host(scales, np.float32)
    return lib.qm_validate(fmt, n, k, group_size, s.ctypes.data)


def quantize_int4(w, group_size):
    """fp32 [n][k] -> (packed uint8 [n][k/2], fp32 scales [n][groups])."""
    import numpy as np
    w = _host(w, np.float32)
    n, k = w.shape
    groups = 1 if group_size in (0, k) else k // group_size
    q = np.empty((n, k // 2), np.uint8)
    s = np.empty((n, groups), np.float32)
    _check(lib.qm_quantize_int4(w.ctypes.data, n, k, group_size, q.ctypes.data, s.ctypes.data))
    return q, s


def quantize_int8(w):
    """fp32 [n][k] -> (int8 [n][k], fp32 scales [n][1])."""
    import numpy as np
    w = _host(w, np.float32)
    n, k = w.shape
    q = np.empty((n, k), np.int8)
    s = np.empty((n, 1), np.float32)
    _check(lib.qm_quantize_int8(w.ctypes.data, n, k, q.ctypes.data, s.ctypes.data))
    return q, s
