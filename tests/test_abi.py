"""Host-side checks of the C ABI (no GPU needed).

The library must load on a machine without a GPU, export every entry point
declared in include/qmoe.h, size workspaces on the host, and reject every
malformed call during host-side validation -- before any HIP call -- with the
documented status.  Pointers passed here are fake addresses: a call that got
past validation would fail (or fault), so each case must be rejected by the
host checks alone.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qmoe.h")
LIB = os.environ.get("QMOE_LIB_PATH", os.path.join(ROOT, "int4_expert_gemv_amd", "libqmoe.so"))

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libqmoe.so not built")


def declared_functions():
    text = open(HEADER).read()
    return re.findall(r"QM_API\s+[\w\s\*]+?\b(\w+)\s*\(", text)


@pytest.fixture(scope="module")
def q():
    from int4_expert_gemv_amd import qmoe
    return qmoe


def test_header_declares_expected_entry_points():
    names = declared_functions()
    assert set(names) == {"qgemv", "qgemv_pair", "qgemv_norm_chain", "qgemm_small", "moe_expert_ffn_workspace", "moe_expert_ffn",
                          "moe_expert_ffn_path", "moe_gate_up", "moe_down", "moe_expert_ffn_noalloc",
                          "qm_strerror", "qm_pack_int4", "qm_pack_int8", "qm_validate", "qm_quantize_int4",
                          "qm_quantize_int8"}


def test_library_exports_every_declared_symbol(q):
    lib = ctypes.CDLL(LIB)
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(q.EXPORTS) == set(declared_functions())


def test_strerror(q):
    for st in (0, -1, -2, -3, -4, -5):
        assert q.lib.qm_strerror(st)
    assert q.lib.qm_strerror(12345) == b"unknown status"


FAKE = 0x7F0000000000  # 16-byte aligned, never dereferenced


def _mat(q, fmt=4, n=64, k=512, gs=64, qp=FAKE, sp=FAKE):
    return q.QMat(fmt, n, k, gs, qp, sp)


@pytest.mark.parametrize("case,want", [
    (dict(fmt=3), -1),                 # unknown format
    (dict(n=-1), -1),                  # negative size
    (dict(k=511), -1),                 # odd K for int4
    (dict(fmt=1, gs=64), -1),          # int8 has per-row scales only
    (dict(qp=0), -1),                  # null weights
    (dict(sp=0), -1),                  # null scales
    (dict(k=496), -2),                 # K not a multiple of 32
    (dict(k=512, gs=48), -2),          # group size not a multiple of 32
    (dict(k=576, gs=96), -2),          # group size not a power-of-two multiple of 32
    (dict(k=544, gs=64), -2),          # K not a multiple of the group size (ragged group)
    (dict(fmt=1, k=520, gs=0), -2),    # int8 K not a multiple of 16
    (dict(qp=FAKE + 8), -2),           # weights not 16-byte aligned
])
def test_qgemv_rejects(q, case, want):
    m = _mat(q, **case)
    st = q.raw_status("qgemv", ctypes.byref(m), ctypes.c_void_p(FAKE), 1, ctypes.c_void_p(FAKE), None)
    assert st == want


def test_qgemv_bad_dtype_and_nulls(q):
    m = _mat(q)
    assert q.raw_status("qgemv", ctypes.byref(m), ctypes.c_void_p(FAKE), 7, ctypes.c_void_p(FAKE), None) == -1
    assert q.raw_status("qgemv", ctypes.byref(m), None, 1, ctypes.c_void_p(FAKE), None) == -1
    assert q.raw_status("qgemv", ctypes.byref(m), ctypes.c_void_p(FAKE), 1, None, None) == -1
    assert q.raw_status("qgemv", None, ctypes.c_void_p(FAKE), 1, ctypes.c_void_p(FAKE), None) == -1
    # x not 16-byte aligned
    assert q.raw_status("qgemv", ctypes.byref(m), ctypes.c_void_p(FAKE + 2), 1, ctypes.c_void_p(FAKE), None) == -2


def test_qgemv_zero_rows_is_a_noop(q):
    m = _mat(q, n=0, qp=0, sp=0)
    assert q.raw_status("qgemv", ctypes.byref(m), None, 1, None, None) == 0


def test_qgemv_pair_rejects(q):
    """Both matrices are validated before anything is enqueued: any invalid
    one, or two different K, rejects the pair (nothing touches FAKE)."""
    f = ctypes.c_void_p(FAKE)
    call = lambda m1, m2, dt=1, x=f: q.raw_status("qgemv_pair", ctypes.byref(m1), ctypes.byref(m2), x, dt, f, f,
                                                  None)
    assert call(_mat(q), _mat(q, k=1024)) == -1           # different K
    assert call(_mat(q), _mat(q, fmt=3)) == -1            # second matrix invalid
    assert call(_mat(q, sp=0), _mat(q)) == -1             # first matrix invalid
    assert call(_mat(q), _mat(q, qp=FAKE + 8)) == -2      # second matrix unsupported (alignment)
    assert call(_mat(q), _mat(q), dt=7) == -1             # bad activation type
    assert call(_mat(q), _mat(q), x=None) == -1           # null x
    assert q.raw_status("qgemv_pair", None, ctypes.byref(_mat(q)), f, 1, f, f, None) == -1
    z = _mat(q, n=0, qp=0, sp=0)
    assert q.raw_status("qgemv_pair", ctypes.byref(z), ctypes.byref(z), None, 1, None, None, None) == 0


def test_qgemv_norm_chain_rejects(q):
    """Shape links between the three matrices and every operand are checked
    before anything is enqueued."""
    f = ctypes.c_void_p(FAKE)

    def call(wa, wkv, wb, eps=1e-6, dt=1, u=FAKE):
        return q.raw_status("qgemv_norm_chain", ctypes.byref(wa), ctypes.byref(wkv), f, ctypes.c_float(eps),
                            ctypes.byref(wb), f, dt, ctypes.c_void_p(u), f, f, None)

    a, kv, b = _mat(q, n=64, k=512), _mat(q, n=32, k=512), _mat(q, n=128, k=64)
    assert call(a, kv, _mat(q, n=128, k=128)) == -1       # q_b's K is not q_a's N
    assert call(a, _mat(q, n=32, k=1024), b) == -1        # kv_a reads another x length
    assert call(a, kv, b, eps=-1.0) == -1                 # negative eps
    assert call(a, kv, b, dt=5) == -1                     # bad activation type
    assert call(a, kv, _mat(q, n=128, k=64, sp=0)) == -1  # q_b invalid
    assert call(a, kv, b, u=FAKE + 4) == -2               # latent not 16-byte aligned (it is q_b's input)
    assert q.raw_status("qgemv_norm_chain", None, ctypes.byref(kv), f, ctypes.c_float(0), ctypes.byref(b), f, 1, f,
                        f, f, None) == -1


def test_int3_limits(q):
    """int3-g64: group size 64 only, k <= 16384, batches as for int4;
    as an expert format, the decode kernels' limits (no prefill path)."""
    f = ctypes.c_void_p(FAKE)
    st = lambda m: q.raw_status("qgemv", ctypes.byref(m), f, 1, f, None)
    assert st(_mat(q, fmt=5, gs=0)) == -1                  # int3 needs group size 64
    assert st(_mat(q, fmt=5, gs=128)) == -1
    assert st(_mat(q, fmt=5, k=16416)) == -2               # k above the staged maximum
    assert st(_mat(q, fmt=5, k=80)) == -2                  # k not a multiple of 32
    m = _mat(q, fmt=5)
    assert q.raw_status("qgemm_small", ctypes.byref(m), f, 1, 9, ctypes.c_int64(512), f, ctypes.c_int64(64),
                        None) == -2                        # batch above QM_SMALL_MAX
    assert _moe(q, _experts(q, fmt=5, gs=0)) == -1         # group size 64 only
    assert _moe(q, _experts(q, fmt=5, gs=64), path=2) == -2  # no prefill kernels for int3
    assert _moe(q, _experts(q, fmt=5, gs=64, I=16384), k=32) == -2  # inter past the down kernel's limit
    assert _moe(q, _experts(q, fmt=5, gs=64, H=16416)) == -2
    assert _moe(q, _experts(q, fmt=5, gs=64), ws_bytes=16) == -3  # workspace too small
    ex = _experts(q, fmt=5, gs=64)
    assert q.moe_expert_ffn_workspace(ex, 3, 8) >= 3 * 8 * 128 * 4  # at least h's records for every pair


def test_qgemm_small_rejects(q):
    m = _mat(q)
    f = ctypes.c_void_p(FAKE)
    call = lambda batch, ldx, ldy, dt=1: q.raw_status("qgemm_small", ctypes.byref(m), f, dt, batch,
                                                      ctypes.c_int64(ldx), f, ctypes.c_int64(ldy), None)
    assert call(0, 512, 64) == -1          # empty batch
    assert call(9, 512, 64) == -2          # batch above QM_SMALL_MAX
    assert call(2, 511, 64) == -1          # ldx < k
    assert call(2, 512, 63) == -1          # ldy < n
    assert call(2, 516, 64) == -2          # bf16 row stride not a multiple of 16 bytes
    assert call(2, 514, 64, dt=0) == -2    # fp32 row stride not a multiple of 16 bytes


def _experts(q, E=8, H=256, I=128, fmt=4, gs=64, **ptrs):
    p = dict(gate_q=FAKE, up_q=FAKE, down_q=FAKE, gate_s=FAKE, up_s=FAKE, down_s=FAKE)
    p.update(ptrs)
    return q.Experts(E, H, I, fmt, gs, p["gate_q"], p["up_q"], p["down_q"], p["gate_s"], p["up_s"], p["down_s"])


def _moe(q, ex, T=1, k=8, ws_bytes=1 << 30, path=0, x=FAKE, ws=FAKE, dt=1):
    f = ctypes.c_void_p(FAKE)
    return q.raw_status("moe_expert_ffn_path", ctypes.byref(ex), ctypes.c_void_p(x), dt, T, f, f, k, f,
                        ctypes.c_void_p(ws), ctypes.c_size_t(ws_bytes), None, path)


def test_moe_rejects(q):
    assert _moe(q, _experts(q, fmt=3)) == -1
    assert _moe(q, _experts(q, E=0)) == -1
    assert _moe(q, _experts(q, down_s=0)) == -1
    assert _moe(q, _experts(q), k=0) == -1
    assert _moe(q, _experts(q), T=-1) == -1
    assert _moe(q, _experts(q), path=9) == -1
    assert _moe(q, _experts(q), dt=5) == -1
    assert _moe(q, _experts(q), x=0) == -1
    assert _moe(q, _experts(q), k=33) == -2                  # top_k above QM_TOPK_MAX
    assert _moe(q, _experts(q, H=250)) == -2                 # hidden not a multiple of 32
    assert _moe(q, _experts(q, gate_q=FAKE + 4)) == -2       # misaligned weights
    assert _moe(q, _experts(q, fmt=1, gs=0), T=16, path=2) == -2   # prefill kernels: int4 only
    assert _moe(q, _experts(q, gs=32), T=16, path=2) == -2         # prefill kernels: group size >= 64
    assert _moe(q, _experts(q, H=288, gs=0), T=16, path=2) == -2   # prefill kernels: hidden % 512
    assert _moe(q, _experts(q, H=512, I=160, gs=0), T=16, path=2) == -2   # prefill kernels: inter % 256
    assert _moe(q, _experts(q, H=256, I=96, gs=64)) == -2    # I=96 with g64: ragged group
    assert _moe(q, _experts(q), ws_bytes=16) == -3           # workspace too small
    assert _moe(q, _experts(q), ws=0) == -3                  # no workspace
    assert _moe(q, _experts(q), ws=FAKE + 64) == -3          # workspace not 256-byte aligned


def test_moe_zero_tokens_is_a_noop(q):
    assert _moe(q, _experts(q), T=0, x=0, ws=0, ws_bytes=0) == 0


def test_workspace_sizes(q):
    ex = _experts(q, E=320, H=6144, I=2048)
    w1 = q.lib.moe_expert_ffn_workspace(ctypes.byref(ex), 1, 8)
    w8 = q.lib.moe_expert_ffn_workspace(ctypes.byref(ex), 8, 8)
    assert w1 >= 8 * (2048 + 6144) * 4 and w8 >= 64 * (2048 + 6144) * 4 and w8 > w1
    # the 512-token batch-union: per-pair outputs alone are 4096 x 6144 fp32
    w512 = q.lib.moe_expert_ffn_workspace(ctypes.byref(_experts(q, E=256, H=6144, I=2048)), 512, 8)
    assert w512 >= 4096 * 6144 * 4 + 4096 * 2048 * 2 + 512 * 6144 * 2
    # int8 experts never take the prefill kernels: a large batch needs one decode pass of 8 tokens
    ex8 = _experts(q, E=320, H=6144, I=2048, fmt=1, gs=0)
    assert q.lib.moe_expert_ffn_workspace(ctypes.byref(ex8), 512, 8) == \
        q.lib.moe_expert_ffn_workspace(ctypes.byref(ex8), 8, 8)
    assert q.lib.moe_expert_ffn_workspace(ctypes.byref(ex), 1, 0) == 0
    assert q.lib.moe_expert_ffn_workspace(None, 1, 8) == 0


def _moe_noalloc(q, ex, T=1, k=8, x=FAKE, dt=1):
    f = ctypes.c_void_p(FAKE)
    return q.raw_status("moe_expert_ffn_noalloc", ctypes.byref(ex), ctypes.c_void_p(x), dt, T, f, f, k, f, None)


def test_moe_noalloc_rejects_before_any_hip_call(q):
    """Malformed calls and calls needing more than the fixed scratch are
    refused on the host, before the scratch address is looked up."""
    assert _moe_noalloc(q, _experts(q), dt=5) == -1
    assert _moe_noalloc(q, _experts(q), k=0) == -1
    assert _moe_noalloc(q, _experts(q), x=0) == -1
    assert _moe_noalloc(q, _experts(q, E=0)) == -1
    assert _moe_noalloc(q, _experts(q), k=33) == -2
    assert _moe_noalloc(q, _experts(q), T=0, x=0) == 0
    big = _experts(q, E=256, H=6144, I=2048)
    need = q.lib.moe_expert_ffn_workspace(ctypes.byref(big), 512, 8)
    assert need > q.QM_NOALLOC_SCRATCH_BYTES
    assert _moe_noalloc(q, big, T=512) == q.QM_ERR_TOO_LARGE
    assert b"scratch" in q.lib.qm_strerror(q.QM_ERR_TOO_LARGE)
