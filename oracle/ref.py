"""ctypes front end of the fp64 CPU oracle (oracle/qmref.c).

TEST INFRASTRUCTURE ONLY: imported by the tests, the package smoke check and
the bench's CPU-baseline leg.  The product library never imports it.

Arrays are numpy arrays on the host:
  q       uint8  [n][k/2] (int4) or int8/uint8 [n][k] (int8 per-row)
  scales  float32 [n][ceil(k/gs)] (int4 grouped) or [n] (per-row / int8)
  x       float32 (dtype F32) or uint16 bf16 bit patterns (dtype BF16)
Outputs are float64.
"""
import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "qmref.c")
LIB = os.path.join(HERE, "libqmref.so")

FMT_INT8_ROW = 1
FMT_INT4 = 4
FMT_INT3 = 5
F32 = 0
BF16 = 1
BF16_ACT = 1
F64 = 2


def gcc_cmd(out, mutant=0, openmp=True):
    cmd = ["gcc", "-std=c99", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
           "-Wall", "-Wextra", "-o", out, SRC, "-lm"]
    if openmp:
        cmd.insert(1, "-fopenmp")
    if mutant:
        cmd.insert(1, "-DQMREF_MUTANT=%d" % mutant)
    return cmd


def build(out=LIB, mutant=0):
    """Compile the oracle into a shared library (gcc, no GPU code)."""
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.run(gcc_cmd(tmp, mutant), check=True)
    os.replace(tmp, out)
    return out


class _Experts(ctypes.Structure):
    _fields_ = [("n_experts", ctypes.c_int), ("hidden", ctypes.c_int), ("inter", ctypes.c_int),
                ("fmt", ctypes.c_int), ("gs", ctypes.c_int),
                ("gate_q", ctypes.c_void_p), ("up_q", ctypes.c_void_p), ("down_q", ctypes.c_void_p),
                ("gate_s", ctypes.c_void_p), ("up_s", ctypes.c_void_p), ("down_s", ctypes.c_void_p)]


class Oracle:
    """One loaded copy of the oracle library (the normal build or a mutant)."""

    def __init__(self, path=LIB):
        if not os.path.exists(path):
            build(path)
        L = ctypes.CDLL(path)
        vp, i32, i64, dp = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_void_p
        L.qmref_gemv.argtypes = [i32, i32, i32, i32, vp, vp, vp, i32, dp, dp]
        L.qmref_gemv.restype = i32
        L.qmref_gemm_small.argtypes = [i32, i32, i32, i32, vp, vp, vp, i32, i32, i64, dp, i64, dp]
        L.qmref_gemm_small.restype = i32
        L.qmref_moe_ffn.argtypes = [ctypes.POINTER(_Experts), vp, i32, i32, vp, vp, i32, i32, dp, dp, dp]
        L.qmref_moe_ffn.restype = i32
        L.qmref_silu.argtypes = [ctypes.c_double]
        L.qmref_silu.restype = ctypes.c_double
        L.qmref_f32_to_bf16.argtypes = [ctypes.c_float]
        L.qmref_f32_to_bf16.restype = ctypes.c_uint16
        L.qmref_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.qmref_bf16_to_f32.restype = ctypes.c_float
        L.qmref_round_bf16.argtypes = [ctypes.c_double]
        L.qmref_round_bf16.restype = ctypes.c_double
        L.qmref_weight.argtypes = [i32, i32, i32, vp, vp, i64, i64, ctypes.POINTER(ctypes.c_double)]
        L.qmref_weight.restype = ctypes.c_double
        L.qmref_set_threads.argtypes = [i32]
        L.qmref_rmsnorm.argtypes = [i32, dp, vp, ctypes.c_double, dp]
        L.qmref_rmsnorm.restype = i32
        L.qmref_set_threads.restype = i32
        self.L = L

    # -- helpers -----------------------------------------------------------
    @staticmethod
    def _p(a):
        return None if a is None else a.ctypes.data_as(ctypes.c_void_p)

    @staticmethod
    def _x_dtype(x):
        if x.dtype == np.float32:
            return F32
        if x.dtype == np.uint16:
            return BF16
        if x.dtype == np.float64:
            return F64
        raise TypeError("x must be float32, float64 or uint16 (bf16 bits)")

    # -- API ----------------------------------------------------------------
    def set_threads(self, n):
        return self.L.qmref_set_threads(int(n))

    def silu(self, z):
        return self.L.qmref_silu(float(z))

    def f32_to_bf16(self, f):
        return self.L.qmref_f32_to_bf16(float(f))

    def bf16_to_f32(self, b):
        return self.L.qmref_bf16_to_f32(int(b))

    def round_bf16(self, v):
        return self.L.qmref_round_bf16(float(v))

    def weight(self, fmt, k, gs, q, scales, row, col):
        s = ctypes.c_double()
        v = self.L.qmref_weight(fmt, k, gs, self._p(q), self._p(scales), row, col, ctypes.byref(s))
        return v, s.value

    def gemv(self, fmt, n, k, gs, q, scales, x, want_norm=True):
        q = np.ascontiguousarray(q)
        scales = np.ascontiguousarray(scales, dtype=np.float32)
        x = np.ascontiguousarray(x)
        y = np.zeros(n, np.float64)
        nrm = np.zeros(n, np.float64) if want_norm else None
        rc = self.L.qmref_gemv(fmt, n, k, gs, self._p(q), self._p(scales), self._p(x),
                               self._x_dtype(x), self._p(y), self._p(nrm))
        if rc:
            raise ValueError("qmref_gemv rejected its arguments")
        return y, nrm

    def rmsnorm(self, u, g=None, eps=0.0):
        """out = u / sqrt(mean(u^2) + eps) * g, in fp64."""
        u = np.ascontiguousarray(u, dtype=np.float64)
        gp = None if g is None else np.ascontiguousarray(g, dtype=np.float32)
        out = np.zeros(u.shape[0], np.float64)
        if self.L.qmref_rmsnorm(u.shape[0], self._p(u), None if gp is None else self._p(gp), eps, self._p(out)):
            raise ValueError("qmref_rmsnorm rejected its arguments")
        return out

    def gemm_small(self, fmt, n, k, gs, q, scales, x, want_norm=True):
        """x: [batch][k]; returns y [batch][n] and norm [batch][n]."""
        q = np.ascontiguousarray(q)
        scales = np.ascontiguousarray(scales, dtype=np.float32)
        x = np.ascontiguousarray(x)
        batch = x.shape[0]
        y = np.zeros((batch, n), np.float64)
        nrm = np.zeros((batch, n), np.float64) if want_norm else None
        rc = self.L.qmref_gemm_small(fmt, n, k, gs, self._p(q), self._p(scales), self._p(x),
                                     self._x_dtype(x), batch, k, self._p(y), n, self._p(nrm))
        if rc:
            raise ValueError("qmref_gemm_small rejected its arguments")
        return y, nrm

    def moe_ffn(self, ex, x, ids, w, flags=0, want_h=False, want_norm=True):
        """ex: dict with n_experts, hidden, inter, fmt, gs and the six arrays
        gate_q, up_q, down_q, gate_s, up_s, down_s (experts stacked first).
        x: [T][hidden]; ids int32 [T][k]; w float32 [T][k]."""
        arrs = {key: np.ascontiguousarray(ex[key]) for key in
                ("gate_q", "up_q", "down_q", "gate_s", "up_s", "down_s")}
        s = _Experts(ex["n_experts"], ex["hidden"], ex["inter"], ex["fmt"], ex["gs"],
                     *[arrs[k].ctypes.data for k in ("gate_q", "up_q", "down_q",
                                                     "gate_s", "up_s", "down_s")])
        x = np.ascontiguousarray(x)
        ids = np.ascontiguousarray(ids, dtype=np.int32)
        w = np.ascontiguousarray(w, dtype=np.float32)
        T, k = ids.shape
        H, I = ex["hidden"], ex["inter"]
        y = np.zeros((T, H), np.float64)
        h = np.zeros((T * k, I), np.float64) if want_h else None
        nrm = np.zeros((T, H), np.float64) if want_norm else None
        rc = self.L.qmref_moe_ffn(ctypes.byref(s), self._p(x), self._x_dtype(x), T,
                                  self._p(ids), self._p(w), k, flags,
                                  self._p(y), self._p(h), self._p(nrm))
        if rc:
            raise ValueError("qmref_moe_ffn rejected its arguments")
        return y, h, nrm


_default = None


def oracle():
    """The shared oracle instance (builds the library on first use if absent;
    QMREF_LIB names another build of the same source, e.g. a sanitized one)."""
    global _default
    if _default is None:
        _default = Oracle(os.environ.get("QMREF_LIB", LIB))
    return _default


def max_norm_err(y_test, y_ref, norm):
    """Max over outputs of |y_test - y_ref| / norm; where norm == 0 the test
    value must be exactly 0 (reported as inf otherwise)."""
    y_test = np.asarray(y_test, np.float64)
    y_ref = np.asarray(y_ref, np.float64)
    norm = np.asarray(norm, np.float64)
    diff = np.abs(y_test - y_ref)
    zero = norm == 0
    err = np.where(zero, np.where(y_test == 0, 0.0, np.inf), diff / np.where(zero, 1.0, norm))
    return float(err.max()) if err.size else 0.0
