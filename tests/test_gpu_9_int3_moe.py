"""GPU parity of the expert FFN with int3-g64 experts (fmt 5) against the
fp64 oracle: the 35B-like and large decode layers, several tokens, fp32
activations, ragged groups, top-k 32, invalid and repeated expert ids, the
two stage entry points, many tokens in one call, and the refusal of the
prefill path (int3 has decode kernels only).

Bar: max over outputs of |y_gpu - y_oracle| / N(t, i) <= 2e-4, with N the
oracle's normaliser of the final contraction.
"""
import numpy as np
import pytest
import torch

from gpu_util import TOL, dev, host, norm_err, upload_experts
from int4_expert_gemv_amd import synth

pytestmark = pytest.mark.gpu

FMT3 = 5


@pytest.fixture(scope="module")
def q():
    from int4_expert_gemv_amd import qmoe
    assert torch.cuda.is_available()
    return qmoe


def _experts(q, ex, d):
    return q.experts(FMT3, 64, d["gate_q"], d["up_q"], d["down_q"], d["gate_s"], d["up_s"], d["down_s"])


def _ws(q, e, T, k):
    return torch.empty(max(q.moe_expert_ffn_workspace(e, T, k), 256), dtype=torch.uint8, device="cuda")


def _run(q, ex, d, x, ids, w, path=0):
    T, k = ids.shape
    e = _experts(q, ex, d)
    y = torch.full((T, ex["hidden"]), float("nan"), device="cuda")
    q.moe_expert_ffn(e, dev(x), dev(ids), dev(w), y, _ws(q, e, T, k), path=path)
    torch.cuda.synchronize()
    return host(y)


def _case(seed, E, H, I, T, k, xdt="bf16", scales="wide", kind="uniform"):
    g = np.random.default_rng([seed, 7])
    ids, w = synth.zipf_routing(g, T, E, k) if kind == "zipf" else synth.uniform_routing(g, T, E, k)
    ex = synth.expert_set(seed, FMT3, E, H, I, 64, experts=np.unique(ids), scales=scales)
    x = synth.activations(np.random.default_rng([seed, 8]), (T, H), xdt)
    return ex, x, ids, w


def _check(q, oracle, seed, E, H, I, T, k, **kw):
    print("int3 moe parity E=%d H=%d I=%d T=%d k=%d %s" % (E, H, I, T, k, kw), flush=True)
    ex, x, ids, w = _case(seed, E, H, I, T, k, **kw)
    d = upload_experts(ex, only=np.unique(ids))
    y = _run(q, ex, d, x, ids, w)
    yr, _, nr = oracle.moe_ffn(ex, x, ids, w)
    err = norm_err(y, yr, nr)
    print("  max normalised error %.3g" % err, flush=True)
    assert err <= TOL, err
    return y


@pytest.mark.parametrize("scales", ["wide", "unit"])
def test_int3_moe_35b_like(q, oracle, scales):
    """hidden 2048, 256 experts, intermediate 512, top-8, one token."""
    _check(q, oracle, 40, 256, 2048, 512, 1, 8, scales=scales)


@pytest.mark.parametrize("T", [1, 3, 8])
def test_int3_moe_large(q, oracle, T):
    """hidden 6144, 320 experts, intermediate 2048, top-8, 1..8 tokens."""
    _check(q, oracle, 41, 320, 6144, 2048, T, 8)


def test_int3_moe_fp32_activations(q, oracle):
    _check(q, oracle, 42, 32, 2048, 512, 2, 8, xdt="f32")


def test_int3_moe_ragged_groups(q, oracle):
    """hidden 96 and intermediate 160: the last group of every row is half
    padding (rows are whole 24-byte groups)."""
    _check(q, oracle, 43, 5, 96, 160, 3, 2)
    _check(q, oracle, 44, 7, 160, 96, 4, 3, xdt="f32")


def test_int3_moe_topk_32(q, oracle):
    _check(q, oracle, 45, 64, 512, 256, 3, 32)


def test_int3_moe_zipf_tokens(q, oracle):
    """Skewed routing over few experts: most experts serve several tokens."""
    _check(q, oracle, 46, 16, 2048, 1024, 8, 6, kind="zipf")


def test_int3_moe_invalid_and_duplicate_ids(q, oracle):
    E, H, I, T, k = 12, 512, 256, 3, 4
    ex, x, ids, w = _case(47, E, H, I, T, k)
    ids[0, 1] = E + 3       # out of range: skipped
    ids[1, 2] = -1          # negative: skipped
    ids[2, 3] = ids[2, 0]   # same expert twice in one token: summed
    ex = synth.expert_set(47, FMT3, E, H, I, 64)
    d = upload_experts(ex)
    y = _run(q, ex, d, x, ids, w)
    yr, _, nr = oracle.moe_ffn(ex, x, ids, w)
    assert norm_err(y, yr, nr) <= TOL
    # the stage entry point leaves the h rows of invalid pairs unwritten
    e = _experts(q, ex, d)
    h = torch.full((T * k, I), float("nan"), device="cuda")
    q.moe_gate_up(e, dev(x), dev(ids), h, _ws(q, e, T, k))
    torch.cuda.synchronize()
    written = np.isfinite(host(h)).all(axis=1)
    assert np.array_equal(written, ((ids >= 0) & (ids < E)).ravel())
    ids[:] = -1             # no valid pair at all: y = 0
    assert np.array_equal(_run(q, ex, d, x, ids, w), np.zeros((T, H), np.float32))


def test_int3_moe_stages(q, oracle):
    """moe_gate_up then moe_down give the fused call's y bit for bit; down
    fed the oracle's own h meets the bar on its own; gate_up's h matches the
    oracle's h."""
    E, H, I, T, k = 40, 2048, 768, 3, 8
    ex, x, ids, w = _case(48, E, H, I, T, k)
    d = upload_experts(ex, only=np.unique(ids))
    e = _experts(q, ex, d)
    ws = _ws(q, e, T, k)
    h = torch.full((T * k, I), float("nan"), device="cuda")
    y2 = torch.full((T, H), float("nan"), device="cuda")
    q.moe_gate_up(e, dev(x), dev(ids), h, ws)
    q.moe_down(e, h, dev(ids), dev(w), y2, ws)
    torch.cuda.synchronize()
    y1 = _run(q, ex, d, x, ids, w)
    assert np.array_equal(host(y2), y1)
    yr, hr, nr = oracle.moe_ffn(ex, x, ids, w, want_h=True)
    # h: relative to the largest |h| of its row (silu(a) * b has no
    # per-element normaliser in the oracle)
    hg = host(h).astype(np.float64)
    scale = np.maximum(np.abs(hr).max(axis=1, keepdims=True), 1e-30)
    assert np.max(np.abs(hg - hr) / scale) <= TOL
    y3 = torch.full((T, H), float("nan"), device="cuda")
    q.moe_down(e, dev(hr.astype(np.float32)), dev(ids), dev(w), y3, ws)
    torch.cuda.synchronize()
    assert norm_err(host(y3), yr, nr) <= TOL


def test_int3_moe_many_tokens_and_no_prefill(q, oracle):
    """100 tokens in one call run the decode kernels (int3 has no prefill
    path); asking for the prefill path is refused without writing y."""
    E, H, I, T, k = 24, 512, 256, 100, 4
    ex, x, ids, w = _case(49, E, H, I, T, k)
    d = upload_experts(ex, only=np.unique(ids))
    y = _run(q, ex, d, x, ids, w)
    yr, _, nr = oracle.moe_ffn(ex, x, ids, w)
    assert norm_err(y, yr, nr) <= TOL
    e = _experts(q, ex, d)
    yt = torch.full((T, H), 7.0, device="cuda")
    with pytest.raises(q.QmError):
        q.moe_expert_ffn(e, dev(x), dev(ids), dev(w), yt, _ws(q, e, T, k), path=q.QM_PATH_PREFILL)
    torch.cuda.synchronize()
    assert bool((yt == 7.0).all())


def test_int3_moe_deterministic(q):
    E, H, I, T, k = 64, 2048, 1024, 4, 8
    ex, x, ids, w = _case(50, E, H, I, T, k)
    d = upload_experts(ex, only=np.unique(ids))
    assert np.array_equal(_run(q, ex, d, x, ids, w), _run(q, ex, d, x, ids, w))
