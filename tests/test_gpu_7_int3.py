"""GPU parity of the int3-g64 two-plane GEMV (fmt 5) against the fp64
oracle: dense decode shapes, fp32 and bf16 activations, ragged rows, a
ragged tail group (k not a multiple of 64), the largest k, several
activation rows per weight read, the pair entry point, and bit-exact
results on integer-valued data with power-of-two scales (every partial sum
exact in fp32, so any decode slip shows).  Activations with an outlier on a
zero weight are in test_gpu_8_outliers.py.
Bar: max normalised error <= 2e-4.
"""
import numpy as np
import pytest
import torch

from gpu_util import TOL, dev, host, norm_err
from int4_expert_gemv_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    from int4_expert_gemv_amd import qmoe
    assert torch.cuda.is_available()
    return qmoe


def _run(q, n, k, qw, s, x):
    m = q.qmat(5, dev(qw), dev(s), n, k, 64)
    y = torch.full((n,), float("nan"), device="cuda")
    q.qgemv(m, dev(x), y)
    torch.cuda.synchronize()
    return host(y)


@pytest.mark.parametrize("n,k,xdt", [
    (6144, 6144, "bf16"), (6144, 16384, "bf16"), (256, 512, "f32"), (1000, 2048, "f32"),
    (77, 96, "bf16"), (19, 64, "bf16"), (130, 16384, "f32"), (33, 160, "f32"),
])
def test_int3_qgemv_parity(q, oracle, n, k, xdt):
    print("int3 qgemv n=%d k=%d x=%s" % (n, k, xdt), flush=True)
    g = np.random.default_rng([31, n, k])
    qw, s = synth.quant_matrix(g, 5, n, k, 64)
    x = synth.activations(g, (k,), xdt)
    y = _run(q, n, k, qw, s, x)
    yr, nr = oracle.gemv(5, n, k, 64, qw, s, x)
    err = norm_err(y, yr, nr)
    print("  max normalised error %.3g" % err, flush=True)
    assert err <= TOL, err


@pytest.mark.parametrize("xdt", ["bf16", "f32"])
def test_int3_exact_integer_data(q, oracle, xdt):
    n, k = 300, 2048
    g = np.random.default_rng(32)
    qw = g.integers(0, 256, (n, (k // 64) * 24), dtype=np.uint8)
    s = np.ldexp(1.0, g.integers(-3, 3, (n, k // 64))).astype(np.float32)
    xv = g.integers(-8, 9, k).astype(np.float32)
    x = synth.to_bf16_bits(xv) if xdt == "bf16" else xv
    y = _run(q, n, k, qw, s, x)
    yr, _ = oracle.gemv(5, n, k, 64, qw, s, x)
    assert np.array_equal(y.astype(np.float64), yr)


@pytest.mark.parametrize("batch,xdt", [(2, "bf16"), (5, "f32"), (8, "bf16")])
def test_int3_qgemm_small(q, oracle, batch, xdt):
    """Several activation rows per weight read."""
    n, k = 1000, 6144
    g = np.random.default_rng([34, batch])
    qw, s = synth.quant_matrix(g, 5, n, k, 64)
    x = synth.activations(g, (batch, k), xdt)
    m = q.qmat(5, dev(qw), dev(s), n, k, 64)
    y = torch.full((batch, n), float("nan"), device="cuda")
    q.qgemm_small(m, dev(x), y)
    torch.cuda.synchronize()
    yr, nr = oracle.gemm_small(5, n, k, 64, qw, s, x)
    assert norm_err(host(y), yr, nr) <= TOL


def test_int3_pair(q, oracle):
    """Two int3 projections of one x (two launches behind qgemv_pair)."""
    k = 6144
    g = np.random.default_rng(33)
    q1, s1 = synth.quant_matrix(g, 5, 2048, k, 64)
    q2, s2 = synth.quant_matrix(g, 5, 576, k, 64)
    x = synth.activations(g, (k,), "bf16")
    m1, m2 = q.qmat(5, dev(q1), dev(s1), 2048, k, 64), q.qmat(5, dev(q2), dev(s2), 576, k, 64)
    y1, y2 = torch.empty(2048, device="cuda"), torch.empty(576, device="cuda")
    q.qgemv_pair(m1, m2, dev(x), y1, y2)
    torch.cuda.synchronize()
    r1, n1 = oracle.gemv(5, 2048, k, 64, q1, s1, x)
    r2, n2 = oracle.gemv(5, 576, k, 64, q2, s2, x)
    assert max(norm_err(host(y1), r1, n1), norm_err(host(y2), r2, n2)) <= TOL
