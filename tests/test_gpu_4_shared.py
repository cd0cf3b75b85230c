"""GPU parity of a shared expert folded into the routed group (one launch
sequence instead of a separate dense FFN): the shared expert is stored in
the stacked expert arrays and every token gets one more slot routed to it
with weight 1.  The reference is the routed layer and the shared expert's
FFN as two separate oracle calls, added -- what running the shared expert
as its own FFN gives.  Single-token, batch-decode and prefill paths; the
normalised error uses the sum of the two calls' normalisers.
"""
import numpy as np
import pytest

from gpu_util import TOL, dev, host, norm_err, upload_experts
from int4_expert_gemv_amd import synth
from oracle import ref

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    import torch
    from int4_expert_gemv_amd import qmoe
    assert torch.cuda.is_available()
    return qmoe


def _folded(q, ex, d, x, ids, w):
    import torch
    T, k = ids.shape
    e = q.experts(ex["fmt"], ex["gs"], d["gate_q"], d["up_q"], d["down_q"], d["gate_s"], d["up_s"], d["down_s"])
    ws = torch.empty(max(q.moe_expert_ffn_workspace(e, T, k), 256), dtype=torch.uint8, device="cuda")
    y = torch.full((T, ex["hidden"]), float("nan"), device="cuda")
    q.moe_expert_ffn(e, dev(x), dev(ids), dev(w), y, ws)
    torch.cuda.synchronize()
    return host(y)


def _case(q, oracle, seed, E, H, I, T, k, flags):
    print("shared-expert slot seed=%d E=%d+1 H=%d I=%d T=%d top-%d+1" % (seed, E, H, I, T, k), flush=True)
    g = np.random.default_rng([seed, 41])
    ids, w = synth.uniform_routing(g, T, E, k)
    sid = np.full((T, 1), E, np.int32)  # the shared expert: index E of the stack
    ones = np.ones((T, 1), np.float32)
    ids_f, w_f = np.concatenate([ids, sid], 1), np.concatenate([w, ones], 1)
    used = np.unique(ids_f)
    ex = synth.expert_set(seed, 4, E + 1, H, I, 64, experts=used, threads=16)
    d = upload_experts(ex, only=used)
    x = synth.activations(np.random.default_rng([seed, 42]), (T, H), "bf16")
    y = _folded(q, ex, d, x, ids_f, w_f)
    yr, _, nr = oracle.moe_ffn(ex, x, ids, w, flags=flags)
    ys, _, ns = oracle.moe_ffn(ex, x, sid, ones, flags=flags)
    err = norm_err(y, yr + ys, nr + ns)
    print("  max normalised error %.3g" % err, flush=True)
    assert err <= TOL, err


@pytest.mark.parametrize("T", [1, 3])
def test_shared_slot_decode(q, oracle, T):
    _case(q, oracle, 1, 16, 512, 256, T, 4, 0)


def test_shared_slot_prefill(q, oracle):
    """20 tokens of int4-g64 take the prefill kernels (bf16 activations and h)."""
    _case(q, oracle, 2, 16, 512, 256, 20, 4, ref.BF16_ACT)


def test_shared_slot_full_size_one_token(q, oracle):
    """hidden 6144, inter 2048: top-8 routed + the shared expert = 9 slots."""
    oracle.set_threads(16)
    _case(q, oracle, 3, 320, 6144, 2048, 1, 8, 0)


@pytest.mark.parametrize("k", [9, 13, 16])
def test_two_pairs_per_wave_down(q, oracle, k):
    """One token with 9..16 slots and inter 2048: the register-h down kernel
    with two pairs per wave; slot 1 invalid (id -1) and the last slot a
    duplicate of slot 0."""
    E, H, I, T = 40, 512, 2048, 1
    print("two pairs per wave: top-%d E=%d H=%d I=%d" % (k, E, H, I), flush=True)
    g = np.random.default_rng([7, k])
    ids, w = synth.uniform_routing(g, T, E, k)
    ids[0, 1] = -1
    ids[0, k - 1] = ids[0, 0]
    used = np.unique(ids[ids >= 0])
    ex = synth.expert_set(7, 4, E, H, I, 64, experts=used)
    d = upload_experts(ex, only=used)
    x = synth.activations(np.random.default_rng([7, 43]), (T, H), "bf16")
    y = _folded(q, ex, d, x, ids, w)
    yr, _, nr = oracle.moe_ffn(ex, x, ids, w)
    err = norm_err(y, yr, nr)
    print("  max normalised error %.3g" % err, flush=True)
    assert err <= TOL, err
