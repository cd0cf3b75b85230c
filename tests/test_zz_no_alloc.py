"""GPU check of moe_expert_ffn_noalloc, the allocation-free variant of
moe_expert_ffn whose scratch is a fixed per-GPU device array.

Two calls in a row (the second with fewer tokens, so it runs on whatever the
first left in the array) must each give exactly what moe_expert_ffn gives
with a workspace of its own, and meet the oracle's bar."""
import numpy as np
import pytest
import torch

from gpu_util import TOL, dev, host, norm_err, upload_experts
from int4_expert_gemv_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    from int4_expert_gemv_amd import qmoe
    assert torch.cuda.is_available()
    return qmoe


@pytest.mark.parametrize("E,H,I,gs,calls", [
    (32, 2048, 512, 64, (4, 1)),     # small experts: 4 tokens, then 1
    (24, 6144, 2048, 64, (3, 1)),    # large experts
    (16, 1024, 512, 0, (8, 2)),      # per-row scales, other kernels
])
def test_noalloc_matches_workspace_call(q, oracle, E, H, I, gs, calls):
    print("noalloc E=%d H=%d I=%d gs=%d calls=%s" % (E, H, I, gs, calls), flush=True)
    K = 8
    ex = synth.expert_set(31, synth.FMT_INT4, E, H, I, gs)
    d = upload_experts(ex)
    e = q.experts(4, gs, d["gate_q"], d["up_q"], d["down_q"], d["gate_s"], d["up_s"], d["down_s"])
    for i, T in enumerate(calls):
        g = np.random.default_rng([32, i])
        ids, w = synth.uniform_routing(g, T, E, K)
        x = synth.activations(g, (T, H), "bf16")
        xd, idd, wd = dev(x), dev(ids), dev(w)
        ws = torch.empty(q.moe_expert_ffn_workspace(e, T, K), dtype=torch.uint8, device="cuda")
        y_ws = torch.full((T, H), float("nan"), device="cuda")
        y_na = torch.full((T, H), float("nan"), device="cuda")
        q.moe_expert_ffn(e, xd, idd, wd, y_ws, ws)
        q.moe_expert_ffn_noalloc(e, xd, idd, wd, y_na)
        torch.cuda.synchronize()
        assert torch.equal(y_ws, y_na), i
        yr, _, nr = oracle.moe_ffn(ex, x, ids, w)
        assert norm_err(host(y_na), yr, nr) <= TOL
