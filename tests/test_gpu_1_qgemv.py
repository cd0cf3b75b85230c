"""GPU parity of qgemv / qgemm_small against the fp64 oracle.

Bar: max over outputs of |y_gpu - y_oracle| / sum_k |w x| <= 2e-4 (fp32
accumulation), and bit-exact equality on integer-valued data with
power-of-two scales, where every partial sum is exact in fp32.
"""
import numpy as np
import pytest
import torch

from gpu_util import TOL, dev, host, norm_err
from int4_expert_gemv_amd import synth
from oracle import ref

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    from int4_expert_gemv_amd import qmoe
    assert torch.cuda.is_available()
    return qmoe


def _case(seed, fmt, n, k, gs, xdt, batch=None):
    g = np.random.default_rng([seed, fmt, n, k, gs])
    qw, s = synth.quant_matrix(g, fmt, n, k, gs)
    shape = (k,) if batch is None else (batch, k)
    x = synth.activations(g, shape, xdt)
    return qw, s, x


def _run_gemv(q, fmt, n, k, gs, qw, s, x):
    m = q.qmat(fmt, dev(qw), dev(s), n, k, gs)
    y = torch.full((n,), float("nan"), device="cuda")
    q.qgemv(m, dev(x), y)
    torch.cuda.synchronize()
    return host(y)


@pytest.mark.parametrize("fmt,n,k,gs,xdt", [
    (4, 256, 512, 64, "f32"),      # the 256x512 parity configuration, fp32 x
    (4, 256, 512, 64, "bf16"),
    (4, 6144, 6144, 64, "bf16"),   # dense decode shapes
    (4, 6144, 16384, 64, "bf16"),
    (4, 6144, 6144, 0, "bf16"),    # per-row int4
    (4, 6144, 16384, 0, "bf16"),
    (1, 6144, 6144, 0, "bf16"),    # int8 per-row
    (1, 6144, 16384, 0, "bf16"),
    (1, 512, 1024, 0, "f32"),
    (4, 1000, 2048, 64, "f32"),    # ragged row count
    (4, 77, 96, 0, "bf16"),        # 3 chunks per row (lanes idle), ragged rows
    (4, 33, 6176, 0, "f32"),       # K not a multiple of 64 lanes * 32
    (4, 130, 1024, 128, "bf16"),   # group size 128
    (4, 130, 1024, 32, "bf16"),    # group size 32
    (1, 19, 48, 0, "bf16"),        # tiny int8
])
def test_qgemv_parity(q, oracle, fmt, n, k, gs, xdt):
    print("qgemv parity fmt=%d n=%d k=%d gs=%d x=%s" % (fmt, n, k, gs, xdt), flush=True)
    qw, s, x = _case(0, fmt, n, k, gs, xdt)
    y = _run_gemv(q, fmt, n, k, gs, qw, s, x)
    yr, nr = oracle.gemv(fmt, n, k, gs, qw, s, x)
    err = norm_err(y, yr, nr)
    assert err <= TOL, err


@pytest.mark.parametrize("fmt,gs,xdt", [(4, 64, "bf16"), (4, 64, "f32"), (4, 0, "bf16"), (1, 0, "bf16"),
                                        (1, 0, "f32")])
def test_qgemv_exact_integer_data(q, oracle, fmt, gs, xdt):
    g = np.random.default_rng(42)
    n, k = 300, 4096
    qw, _ = synth.quant_matrix(g, fmt, n, k, gs)
    s = synth.pow2_scales(g, (n, k // gs if gs else 1))
    x = synth.small_int_activations(g, (k,), xdt)
    y = _run_gemv(q, fmt, n, k, gs, qw, s, x)
    yr, _ = oracle.gemv(fmt, n, k, gs, qw, s, x)
    assert np.array_equal(y.astype(np.float64), yr)


def test_qgemv_deterministic(q):
    qw, s, x = _case(1, 4, 6144, 6144, 64, "bf16")
    m = q.qmat(4, dev(qw), dev(s), 6144, 6144, 64)
    xd = dev(x)
    y1 = torch.empty(6144, device="cuda")
    y2 = torch.empty(6144, device="cuda")
    q.qgemv(m, xd, y1)
    q.qgemv(m, xd, y2)
    assert torch.equal(y1, y2)


@pytest.mark.parametrize("fmt,n,k,gs,xdt,batch", [
    (4, 6144, 6144, 64, "bf16", 1), (4, 6144, 6144, 64, "bf16", 2), (4, 6144, 6144, 64, "bf16", 3),
    (4, 2048, 6144, 64, "bf16", 8), (4, 512, 16384, 64, "bf16", 8), (4, 512, 16384, 64, "f32", 8),
    (4, 1536, 6144, 0, "f32", 4), (1, 1536, 6144, 0, "bf16", 5), (1, 1024, 16384, 0, "f32", 8),
])
def test_qgemm_small_parity(q, oracle, fmt, n, k, gs, xdt, batch):
    print("qgemm_small parity fmt=%d n=%d k=%d gs=%d x=%s b=%d" % (fmt, n, k, gs, xdt, batch), flush=True)
    qw, s, x = _case(2, fmt, n, k, gs, xdt, batch)
    m = q.qmat(fmt, dev(qw), dev(s), n, k, gs)
    y = torch.full((batch, n), float("nan"), device="cuda")
    q.qgemm_small(m, dev(x), y)
    torch.cuda.synchronize()
    yr, nr = oracle.gemm_small(fmt, n, k, gs, qw, s, x)
    err = norm_err(host(y), yr, nr)
    assert err <= TOL, err


def test_qgemm_small_strided(q, oracle):
    """ldx > k and ldy > n: padding columns are neither read into the result
    nor written."""
    fmt, n, k, gs, batch = 4, 640, 2048, 64, 3
    qw, s, x = _case(3, fmt, n, k, gs, "bf16", batch)
    xpad = np.zeros((batch, k + 64), np.uint16)
    xpad[:, :k] = x
    xpad[:, k:] = synth.to_bf16_bits(np.full((batch, 64), 1e30, np.float32))
    m = q.qmat(fmt, dev(qw), dev(s), n, k, gs)
    y = torch.full((batch, n + 16), -7.0, device="cuda")
    q.qgemm_small(m, dev(xpad), y)
    torch.cuda.synchronize()
    yh = host(y)
    assert np.all(yh[:, n:] == -7.0)
    yr, nr = oracle.gemm_small(fmt, n, k, gs, qw, s, x)
    assert norm_err(yh[:, :n], yr, nr) <= TOL


def test_rejected_call_leaves_output(q):
    qw, s, x = _case(4, 4, 64, 512, 64, "bf16")
    m = q.qmat(4, dev(qw), dev(s), 64, 544, 64)  # ragged group: unsupported
    y = torch.full((64,), 3.0, device="cuda")
    with pytest.raises(q.QmError):
        q.qgemv(m, dev(np.zeros(544, np.uint16)), y)
    torch.cuda.synchronize()
    assert torch.all(y == 3.0)


def _wide_range_x(seed, k, xdt):
    """Activations spanning six decades, with all-zero groups of 16 and groups
    holding one large value among tiny ones (the single-token fast paths give
    each group of 16 activations its own power-of-two scale)."""
    g = np.random.default_rng([seed, 21])
    x = synth.normal_f32(g, (k,)) * (10.0 ** g.uniform(-3, 3, size=k)).astype(np.float32)
    xg = x.reshape(k // 16, 16)
    xg[::5] = 0.0
    xg[2::9] *= 1e-4
    xg[2::9, 7] = -50.0
    x = xg.reshape(k).astype(np.float32)
    return synth.to_bf16_bits(x) if xdt == "bf16" else x


@pytest.mark.parametrize("fmt,n,k,gs,xdt", [
    (4, 512, 6144, 64, "bf16"), (4, 512, 16384, 0, "f32"), (4, 300, 2048, 32, "bf16"),
    (1, 512, 6144, 0, "bf16"), (1, 300, 16384, 0, "f32"), (1, 64, 2048, 0, "bf16"),
])
def test_qgemv_one_token_wide_activation_range(q, oracle, fmt, n, k, gs, xdt):
    """The GEMV on activation digit planes within the bar for activations of
    very different magnitudes (groups whose values span many binades need
    more planes)."""
    print("qgemv wide-range fmt=%d n=%d k=%d gs=%d x=%s" % (fmt, n, k, gs, xdt), flush=True)
    g = np.random.default_rng([9, fmt, n, k])
    qw, s = synth.quant_matrix(g, fmt, n, k, gs)
    x = _wide_range_x(9, k, xdt)
    y = _run_gemv(q, fmt, n, k, gs, qw, s, x)
    yr, nr = oracle.gemv(fmt, n, k, gs, qw, s, x)
    assert norm_err(y, yr, nr) <= TOL
