"""GPU parity of qgemv_pair (two projections of one x in one launch) against
the fp64 oracle, and its equality with two separate qgemv calls (the fused
launch runs the same per-row arithmetic, so the results are bit-identical).
Shapes: the attention-input pair 6144 -> (2048, 576), ragged tile tails,
both formats, and the cases that fall back to two launches (fp32 x, mixed
formats).  Bar: max normalised error <= 2e-4.
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


def _mat(q, seed, fmt, n, k, gs):
    qw, s = synth.quant_matrix(np.random.default_rng([seed, fmt, n, k, gs]), fmt, n, k, gs)
    return qw, s, q.qmat(fmt, dev(qw), dev(s), n, k, gs)


@pytest.mark.parametrize("f1,gs1,n1,f2,gs2,n2,k,xdt", [
    (4, 64, 2048, 4, 64, 576, 6144, "bf16"),   # q_a + kv_a shapes, one launch
    (4, 0, 2048, 4, 0, 576, 6144, "bf16"),     # per-row int4, one launch
    (1, 0, 1536, 1, 0, 576, 6144, "bf16"),     # int8 per-row, one launch
    (4, 64, 100, 4, 64, 37, 512, "bf16"),      # ragged tiles in both halves
    (4, 64, 2048, 4, 64, 576, 6144, "f32"),    # fp32 x: two launches
    (4, 64, 512, 1, 0, 192, 2048, "bf16"),     # mixed formats: two launches
])
def test_qgemv_pair_parity(q, oracle, f1, gs1, n1, f2, gs2, n2, k, xdt):
    print("qgemv_pair fmt %d/%d gs %d/%d n %d/%d k=%d x=%s" % (f1, f2, gs1, gs2, n1, n2, k, xdt), flush=True)
    q1, s1, m1 = _mat(q, 1, f1, n1, k, gs1)
    q2, s2, m2 = _mat(q, 2, f2, n2, k, gs2)
    x = synth.activations(np.random.default_rng([3, k]), (k,), xdt)
    xd = dev(x)
    y1 = torch.full((n1,), float("nan"), device="cuda")
    y2 = torch.full((n2,), float("nan"), device="cuda")
    q.qgemv_pair(m1, m2, xd, y1, y2)
    r1 = torch.full((n1,), float("nan"), device="cuda")
    r2 = torch.full((n2,), float("nan"), device="cuda")
    q.qgemv(m1, xd, r1)
    q.qgemv(m2, xd, r2)
    torch.cuda.synchronize()
    a1, a2 = host(y1), host(y2)
    assert np.array_equal(a1, host(r1)) and np.array_equal(a2, host(r2))
    yr1, nr1 = oracle.gemv(f1, n1, k, gs1, q1, s1, x)
    yr2, nr2 = oracle.gemv(f2, n2, k, gs2, q2, s2, x)
    err = max(norm_err(a1, yr1, nr1), norm_err(a2, yr2, nr2))
    print("  max normalised error %.3g" % err, flush=True)
    assert err <= TOL, err


def test_qgemv_pair_one_empty(q, oracle):
    """An empty second matrix: the pair is the first GEMV alone."""
    q1, s1, m1 = _mat(q, 4, 4, 256, 1024, 64)
    m2 = q.qmat(4, torch.empty(0, dtype=torch.uint8, device="cuda"), torch.empty(0, device="cuda"), 0, 1024, 64)
    x = synth.activations(np.random.default_rng(5), (1024,), "bf16")
    y1 = torch.full((256,), float("nan"), device="cuda")
    y2 = torch.empty(0, device="cuda")
    q.qgemv_pair(m1, m2, dev(x), y1, y2)
    torch.cuda.synchronize()
    yr, nr = oracle.gemv(4, 256, 1024, 64, q1, s1, x)
    assert norm_err(host(y1), yr, nr) <= TOL
