"""GPU parity of moe_expert_ffn against the fp64 oracle.

Bar: max over outputs of |y_gpu - y_oracle| / N(t, i) <= 2e-4 where
N(t, i) = sum_j |w_tj| * sum_m |d_{e,i,m} h_{tj,m}| (the normaliser of the
final contraction, from the oracle).
"""
import numpy as np
import pytest
import torch

from gpu_util import TOL, dev, host, norm_err, upload_experts
from int4_expert_gemv_amd import synth
from oracle import ref

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    from int4_expert_gemv_amd import qmoe
    assert torch.cuda.is_available()
    return qmoe


def _routing(seed, T, E, k, kind="uniform"):
    g = np.random.default_rng([seed, 7])
    if kind == "zipf":
        return synth.zipf_routing(g, T, E, k)
    return synth.uniform_routing(g, T, E, k)


def run_moe(q, ex, d, x, ids, w, path=0):
    T, k = ids.shape
    e = q.experts(ex["fmt"], ex["gs"], d["gate_q"], d["up_q"], d["down_q"], d["gate_s"], d["up_s"], d["down_s"])
    ws = torch.empty(max(q.moe_expert_ffn_workspace(e, T, k), 256), dtype=torch.uint8, device="cuda")
    y = torch.full((T, ex["hidden"]), float("nan"), device="cuda")
    q.moe_expert_ffn(e, dev(x), dev(ids), dev(w), y, ws, path=path)
    torch.cuda.synchronize()
    return host(y)


def _check(q, oracle, seed, fmt, gs, E, H, I, T, k, xdt="bf16", kind="uniform", path=0, flags=0):
    print("moe parity fmt=%d gs=%d E=%d H=%d I=%d T=%d k=%d x=%s %s path=%d" %
          (fmt, gs, E, H, I, T, k, xdt, kind, path), flush=True)
    ids, w = _routing(seed, T, E, k, kind)
    ex = synth.expert_set(seed, fmt, E, H, I, gs, experts=np.unique(ids))
    d = upload_experts(ex, only=np.unique(ids))
    x = synth.activations(np.random.default_rng([seed, 8]), (T, H), xdt)
    y = run_moe(q, ex, d, x, ids, w, path)
    yr, _, nr = oracle.moe_ffn(ex, x, ids, w, flags=flags)
    err = norm_err(y, yr, nr)
    assert err <= TOL, err
    return y


def test_moe_35b_like_decode(q, oracle):
    """hidden 2048, 256 experts, intermediate 512, top-8, one token, int4-g64."""
    _check(q, oracle, 0, 4, 64, 256, 2048, 512, 1, 8)


@pytest.mark.parametrize("gs", [64, 0])
@pytest.mark.parametrize("T", [1, 2, 4, 8])
def test_moe_large_decode(q, oracle, gs, T):
    """hidden 6144, 320 experts, intermediate 2048, top-8, 1..8 tokens."""
    _check(q, oracle, 1, 4, gs, 320, 6144, 2048, T, 8)


def test_moe_int8_experts(q, oracle):
    _check(q, oracle, 2, 1, 0, 16, 1024, 512, 3, 4)


def test_moe_fp32_activations(q, oracle):
    _check(q, oracle, 3, 4, 64, 32, 2048, 512, 2, 8, xdt="f32")


def test_moe_shared_experts_across_tokens(q, oracle):
    """Zipf routing over few experts: most experts serve several tokens."""
    _check(q, oracle, 4, 4, 64, 16, 2048, 1024, 8, 6, kind="zipf")


def test_moe_small_and_ragged(q, oracle):
    _check(q, oracle, 5, 4, 0, 5, 96, 160, 3, 2)
    _check(q, oracle, 6, 4, 32, 7, 256, 96, 5, 3)


def test_moe_topk_32(q, oracle):
    _check(q, oracle, 7, 4, 64, 64, 512, 256, 8, 32)


def test_moe_invalid_and_duplicate_ids(q, oracle):
    E, H, I, T, k = 12, 512, 256, 3, 4
    ids, w = _routing(8, T, E, k)
    ids[0, 1] = E + 3       # out of range: skipped
    ids[1, 2] = -1          # negative: skipped
    ids[2, 3] = ids[2, 0]   # same expert twice in one token: summed
    ex = synth.expert_set(8, 4, E, H, I, 64)
    d = upload_experts(ex)
    x = synth.activations(np.random.default_rng(9), (T, H), "bf16")
    y = run_moe(q, ex, d, x, ids, w)
    yr, _, nr = oracle.moe_ffn(ex, x, ids, w)
    assert norm_err(y, yr, nr) <= TOL


def test_moe_deterministic(q):
    E, H, I, T, k = 64, 2048, 1024, 4, 8
    ids, w = _routing(10, T, E, k)
    ex = synth.expert_set(10, 4, E, H, I, 64, experts=np.unique(ids))
    d = upload_experts(ex, only=np.unique(ids))
    x = synth.activations(np.random.default_rng(11), (T, H), "bf16")
    y1 = run_moe(q, ex, d, x, ids, w)
    y2 = run_moe(q, ex, d, x, ids, w)
    assert np.array_equal(y1, y2)


def _wide_range_x(seed, T, H, xdt):
    """Activations spanning six decades, with all-zero 16-value groups and
    groups holding one large value among tiny ones: the single-token kernels
    scale every group of 16 activations by its own power of two, and this
    case exercises that per-group exponent (and its zero case)."""
    g = np.random.default_rng([seed, 12])
    x = synth.normal_f32(g, (T, H)) * (10.0 ** g.uniform(-3, 3, size=(T, H))).astype(np.float32)
    xg = x.reshape(T, H // 16, 16)
    xg[:, ::7, :] = 0.0                          # whole groups of zeros
    xg[:, 3::11, :] *= 1e-4                      # tiny groups ...
    xg[:, 3::11, 5] = 40.0                       # ... with one large value
    x = xg.reshape(T, H).astype(np.float32)
    return synth.to_bf16_bits(x) if xdt == "bf16" else x


@pytest.mark.parametrize("xdt", ["bf16", "f32"])
def test_moe_one_token_wide_activation_range(q, oracle, xdt):
    """hidden 6144, inter 2048, top-8, one token (the single-token kernels):
    within the bar for activations of very different magnitudes."""
    E, H, I, T, k = 24, 6144, 2048, 1, 8
    ids, w = _routing(13, T, E, k)
    ex = synth.expert_set(13, 4, E, H, I, 64, experts=np.unique(ids))
    d = upload_experts(ex, only=np.unique(ids))
    x = _wide_range_x(13, T, H, xdt)
    y = run_moe(q, ex, d, x, ids, w)
    yr, _, nr = oracle.moe_ffn(ex, x, ids, w)
    assert norm_err(y, yr, nr) <= TOL


def test_moe_one_token_stages_match_layer(q):
    """moe_gate_up then moe_down (hidden vectors through the caller's buffer,
    turned into digit planes by their own kernel) give the same y, bit for
    bit, as moe_expert_ffn (planes written by the gate+up kernel itself)."""
    E, H, I, T, k = 24, 6144, 2048, 1, 8
    ids, w = _routing(14, T, E, k)
    ex = synth.expert_set(14, 4, E, H, I, 64, experts=np.unique(ids))
    d = upload_experts(ex, only=np.unique(ids))
    x = synth.activations(np.random.default_rng(15), (T, H), "bf16")
    e = q.experts(4, 64, d["gate_q"], d["up_q"], d["down_q"], d["gate_s"], d["up_s"], d["down_s"])
    ws = torch.empty(q.moe_expert_ffn_workspace(e, T, k), dtype=torch.uint8, device="cuda")
    y1 = torch.full((T, H), float("nan"), device="cuda")
    y2 = torch.full((T, H), float("nan"), device="cuda")
    h = torch.empty((T * k, I), dtype=torch.float32, device="cuda")
    xd, idd, wd = dev(x), dev(ids), dev(w)
    q.moe_expert_ffn(e, xd, idd, wd, y1, ws)
    q.moe_gate_up(e, xd, idd, h, ws)
    q.moe_down(e, h, idd, wd, y2, ws)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


def test_moe_stages_over_several_passes(q, oracle):
    """8 tokens at hidden 6144 run as two decode passes (the gate+up kernel
    holds the activations of fewer tokens at a time): the stage calls loop
    the same passes as the layer call and give the same y bit for bit; every
    token's experts drawn independently from 24, so tokens share experts."""
    E, H, I, T, k = 24, 6144, 2048, 8, 8
    print("moe stages over passes T=%d H=%d" % (T, H), flush=True)
    g = np.random.default_rng([14, 8])
    ids = np.stack([g.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    w = synth.uniform_f32(g, (T, k), 0.05, 0.3)
    ex = synth.expert_set(18, 4, E, H, I, 64, experts=np.unique(ids), threads=16)
    d = upload_experts(ex, only=np.unique(ids))
    x = synth.activations(np.random.default_rng(19), (T, H), "bf16")
    e = q.experts(4, 64, d["gate_q"], d["up_q"], d["down_q"], d["gate_s"], d["up_s"], d["down_s"])
    ws = torch.empty(q.moe_expert_ffn_workspace(e, T, k), dtype=torch.uint8, device="cuda")
    y1 = torch.full((T, H), float("nan"), device="cuda")
    y2 = torch.full((T, H), float("nan"), device="cuda")
    h = torch.empty((T * k, I), dtype=torch.float32, device="cuda")
    xd, idd, wd = dev(x), dev(ids), dev(w)
    q.moe_expert_ffn(e, xd, idd, wd, y1, ws)
    q.moe_gate_up(e, xd, idd, h, ws)
    q.moe_down(e, h, idd, wd, y2, ws)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    oracle.set_threads(16)
    yr, _, nr = oracle.moe_ffn(ex, x, ids, w)
    assert norm_err(host(y1), yr, nr) <= TOL


@pytest.mark.parametrize("H,k,bad", [(2048, 8, False), (2048, 8, True), (2048, 4, False), (4096, 8, True)])
def test_moe_small_experts(q, oracle, H, k, bad):
    """inter 512, one token (the small-expert decode layer), with fewer slots,
    invalid and duplicate ids, hidden 4096; two calls on one workspace give
    identical y (nothing the first call leaves in the workspace is read as
    the second call's data)."""
    E, I, T = 24, 512, 1
    print("moe small experts H=%d k=%d bad=%s" % (H, k, bad), flush=True)
    ids, w = _routing(16 + H + k, T, E, k)
    if bad:
        ids[0, 1] = -1          # skipped
        ids[0, 3] = E + 5       # skipped
        ids[0, 6] = ids[0, 0]   # the same expert twice: summed
    ex = synth.expert_set(17, 4, E, H, I, 64)
    d = upload_experts(ex)
    x = synth.activations(np.random.default_rng(18), (T, H), "bf16")
    e = q.experts(4, 64, d["gate_q"], d["up_q"], d["down_q"], d["gate_s"], d["up_s"], d["down_s"])
    ws = torch.empty(q.moe_expert_ffn_workspace(e, T, k), dtype=torch.uint8, device="cuda")
    ys = []
    for _ in range(2):
        y = torch.full((T, H), float("nan"), device="cuda")
        q.moe_expert_ffn(e, dev(x), dev(ids), dev(w), y, ws)
        torch.cuda.synchronize()
        ys.append(host(y))
    assert np.array_equal(ys[0], ys[1])
    yr, _, nr = oracle.moe_ffn(ex, x, ids, w)
    assert norm_err(ys[0], yr, nr) <= TOL
