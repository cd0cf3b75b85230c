"""GPU parity of qgemv_norm_chain, the q-prep chain: u = W_a x and
kv = W_kv x (one launch), u RMS-normalised in place with weight g, then
q = W_b u; all on one stream.  Against the oracle: kv = gemv(W_a's pair),
un = rmsnorm(gemv(W_a, x)) and q = gemv(W_b, un) in fp64.

Bar (max normalised error <= 2e-4): kv with the GEMV normaliser sum|w x|;
the latent with that normaliser carried through the norm (times
|g| / sqrt(mean u^2 + eps)); q with sum|w_b un|.  The GPU's q is computed
from its own fp32 latent, so q's error also carries the latent's.
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
    return (fmt, n, k, gs, qw, s), q.qmat(fmt, dev(qw), dev(s), n, k, gs)


@pytest.mark.parametrize("fa,gsa,fb,gsb,na,nkv,k,nq,xdt,eps,weighted", [
    (4, 64, 4, 64, 2048, 576, 6144, 4096, "bf16", 1e-6, True),   # attention-input shapes, one pair launch
    (4, 0, 1, 0, 1536, 576, 6144, 2048, "bf16", 1e-6, False),    # per-row int4 pair, int8 q_b
    (4, 64, 4, 64, 64, 32, 256, 128, "f32", 1.0, True),          # fp32 x (pair as two launches), large eps
])
def test_qgemv_norm_chain_parity(q, oracle, fa, gsa, fb, gsb, na, nkv, k, nq, xdt, eps, weighted):
    print("q-prep chain: %d -> (%d, %d) fmt %d gs %d, norm eps %g, q_b %d -> %d fmt %d gs %d, x %s" %
          (k, na, nkv, fa, gsa, eps, na, nq, fb, gsb, xdt), flush=True)
    A, ma = _mat(q, 1, fa, na, k, gsa)
    KV, mkv = _mat(q, 2, fa, nkv, k, gsa)
    B, mb = _mat(q, 3, fb, nq, na, gsb)
    g = np.random.default_rng(4)
    gw = (1.0 + 0.1 * g.standard_normal(na)).astype(np.float32) if weighted else None
    x = synth.activations(np.random.default_rng(5), (k,), xdt)
    u = torch.full((na,), float("nan"), device="cuda")
    kv = torch.full((nkv,), float("nan"), device="cuda")
    qo = torch.full((nq,), float("nan"), device="cuda")
    q.qgemv_norm_chain(ma, mkv, None if gw is None else dev(gw), eps, mb, dev(x), u, kv, qo)
    torch.cuda.synchronize()
    ua, kva, qa = host(u), host(kv), host(qo)

    yk, nk = oracle.gemv(*KV, x)
    ur, nu = oracle.gemv(*A, x)
    un = oracle.rmsnorm(ur, gw, eps)
    r = 1.0 / np.sqrt(np.mean(ur ** 2) + eps)
    gabs = np.ones(na) if gw is None else np.abs(gw.astype(np.float64))
    yq, nq_ = oracle.gemv(*B, un)
    e_kv, e_u, e_q = norm_err(kva, yk, nk), norm_err(ua, un, nu * r * gabs), norm_err(qa, yq, nq_)
    print("  max normalised error: kv %.3g  latent %.3g  q %.3g" % (e_kv, e_u, e_q), flush=True)
    assert max(e_kv, e_u, e_q) <= TOL, (e_kv, e_u, e_q)
