"""GPU parity of the expert-grouped prefill path (many tokens, MFMA bf16)
against the fp64 oracle in its prefill-precision mode (activations and the
hidden vector rounded to bf16, QMREF_BF16_ACT), and of the chunked decode
path that takes batches the prefill kernels do not.

Bar: max normalised error <= 2e-4 (normaliser of the final contraction).
The full-size case runs the whole 512-token batch on the GPU and checks
every token against the oracle (about half a minute of the oracle on 16
host threads).
"""
import time

import numpy as np
import pytest
import torch

from gpu_util import TOL, dev, host, norm_err, upload_experts
from int4_expert_gemv_amd import synth
from oracle import ref

pytestmark = pytest.mark.gpu

PREFILL = 2
DECODE = 1


@pytest.fixture(scope="module")
def q():
    from int4_expert_gemv_amd import qmoe
    assert torch.cuda.is_available()
    return qmoe


def _experts_handle(q, ex, d):
    return q.experts(ex["fmt"], ex["gs"], d["gate_q"], d["up_q"], d["down_q"], d["gate_s"], d["up_s"], d["down_s"])


def _run(q, ex, d, x, ids, w, path):
    T, k = ids.shape
    e = _experts_handle(q, ex, d)
    ws = torch.empty(max(q.moe_expert_ffn_workspace(e, T, k), 256), dtype=torch.uint8, device="cuda")
    y = torch.full((T, ex["hidden"]), float("nan"), device="cuda")
    q.moe_expert_ffn(e, dev(x), dev(ids), dev(w), y, ws, path=path)
    torch.cuda.synchronize()
    return host(y)


def _case(q, oracle, seed, fmt, gs, E, H, I, T, k, xdt="bf16", kind="zipf", path=0, ids=None, w=None):
    print("prefill parity seed=%d fmt=%d gs=%d E=%d H=%d I=%d T=%d k=%d x=%s %s path=%d" %
          (seed, fmt, gs, E, H, I, T, k, xdt, kind, path), flush=True)
    g = np.random.default_rng([seed, 17])
    if ids is None:
        ids, w = (synth.zipf_routing if kind == "zipf" else synth.uniform_routing)(g, T, E, k)
    used = np.unique(ids[(ids >= 0) & (ids < E)])
    ex = synth.expert_set(seed, fmt, E, H, I, gs, experts=used)
    d = upload_experts(ex, only=used)
    x = synth.activations(np.random.default_rng([seed, 18]), (T, H), xdt)
    y = _run(q, ex, d, x, ids, w, path)
    prefill = path == PREFILL or (path == 0 and T > 8 and fmt == 4 and gs != 32)
    yr, _, nr = oracle.moe_ffn(ex, x, ids, w, flags=ref.BF16_ACT if prefill else 0)
    err = norm_err(y, yr, nr)
    print("  max normalised error %.3g" % err, flush=True)
    assert err <= TOL, err
    return y, (ex, d, x, ids, w)


@pytest.mark.parametrize("gs", [64, 0])
def test_prefill_small_g64_and_row(q, oracle, gs):
    """40 tokens, 16 experts, hidden 512, inter 256, top-4 (several M-tiles
    per popular expert, ragged last tiles)."""
    _case(q, oracle, 1, 4, gs, 16, 512, 256, 40, 4)


def test_prefill_group_128(q, oracle):
    _case(q, oracle, 2, 4, 128, 8, 1024, 512, 24, 4)


def test_prefill_group_256(q, oracle):
    """Groups as long as a whole pipeline stage: each group's offset
    correction is applied once, by the wave holding the stage's second K
    half, while both halves fold their partial sums."""
    _case(q, oracle, 11, 4, 256, 8, 1024, 1024, 40, 4)


def test_prefill_fp32_activations(q, oracle):
    _case(q, oracle, 3, 4, 64, 16, 512, 256, 33, 4, xdt="f32")


def test_prefill_one_expert_takes_all(q, oracle):
    """Every token routed to expert 3 in slot 0: 150 rows = 5 M-tiles (4 x 32
    + 22) of one expert; the other slots uniform."""
    T, E, k = 150, 12, 3
    g = np.random.default_rng(4)
    ids = np.zeros((T, k), np.int32)
    for t in range(T):
        ids[t] = np.concatenate([[3], g.choice(np.setdiff1d(np.arange(E), [3]), k - 1, replace=False)])
    w = synth.uniform_f32(g, (T, k), 0.1, 1.0)
    _case(q, oracle, 4, 4, 64, E, 512, 256, T, k, ids=ids, w=w)


@pytest.mark.parametrize("T", [1, 9, 32, 33])
def test_prefill_tile_edges(q, oracle, T):
    """Forced prefill at tiny batches and 32/33 rows per expert (one full
    M-tile, or a full one and a one-row tail)."""
    ids = np.tile(np.array([[0, 1]], np.int32), (T, 1))
    w = np.tile(np.array([[0.75, 0.25]], np.float32), (T, 1))
    _case(q, oracle, 5, 4, 64, 4, 512, 256, T, 2, path=PREFILL, ids=ids, w=w)


def test_prefill_invalid_and_duplicate_ids(q, oracle):
    T, E, k = 20, 10, 4
    g = np.random.default_rng(6)
    ids, w = synth.uniform_routing(g, T, E, k)
    ids[0, 1] = E + 3
    ids[5, 2] = -1
    ids[7, 3] = ids[7, 0]
    ids[9, :] = -7  # a token with no valid slot: y row must be 0
    y, _ = _case(q, oracle, 6, 4, 64, E, 512, 256, T, k, ids=ids, w=w)
    assert np.all(y[9] == 0)


def test_prefill_deterministic(q):
    """Bit-identical outputs across calls although pairs are bucketed with
    atomics (a pair's M-tile and row within it may change between calls);
    Zipf routing puts more than one M-tile on the popular experts."""
    T, E, H, I, k = 64, 16, 512, 256, 8
    g = np.random.default_rng(7)
    ids, w = synth.zipf_routing(g, T, E, k)
    ex = synth.expert_set(7, 4, E, H, I, 64)
    d = upload_experts(ex)
    x = synth.activations(np.random.default_rng(8), (T, H), "bf16")
    y1 = _run(q, ex, d, x, ids, w, PREFILL)
    y2 = _run(q, ex, d, x, ids, w, PREFILL)
    assert np.array_equal(y1, y2)


@pytest.mark.parametrize("fmt,gs", [(1, 0), (4, 32)])
def test_chunked_decode_for_other_formats(q, oracle, fmt, gs):
    """int8 and int4-g32 experts with more than 8 tokens run the decode
    kernels 8 tokens per pass (fp32 hidden vector: no bf16 rounding)."""
    _case(q, oracle, 9, fmt, gs, 12, 512, 256, 20, 4)
    with pytest.raises(q.QmError):
        _case(q, oracle, 9, fmt, gs, 12, 512, 256, 20, 4, path=PREFILL)


def test_decode_path_forced_on_large_batch(q, oracle):
    _case(q, oracle, 10, 4, 64, 12, 512, 256, 19, 4, path=DECODE)


def test_prefill_full_size(q, oracle):
    """512 tokens, 256 experts, hidden 6144, inter 2048, top-8, int4-g64,
    Zipf-skewed routing: the whole batch runs as one call and all 512
    tokens are checked."""
    T, E, H, I, k = 512, 256, 6144, 2048, 8
    print("prefill full size T=%d E=%d H=%d I=%d k=%d" % (T, E, H, I, k), flush=True)
    g = np.random.default_rng([0, 17])
    ids, w = synth.zipf_routing(g, T, E, k)
    used = np.unique(ids)
    ex = synth.expert_set(0, 4, E, H, I, 64, experts=used, threads=16)
    d = upload_experts(ex, only=used)
    x = synth.activations(np.random.default_rng([0, 18]), (T, H), "bf16")
    y = _run(q, ex, d, x, ids, w, 0)
    counts = np.bincount(ids.ravel(), minlength=E)
    oracle.set_threads(16)
    t0 = time.time()
    yr, _, nr = oracle.moe_ffn(ex, x, ids, w, flags=ref.BF16_ACT)
    err = norm_err(y, yr, nr)
    print("  all %d tokens (oracle %.1f s), busiest expert %d tokens: max normalised error %.3g" %
          (T, time.time() - t0, counts.max(), err), flush=True)
    assert err <= TOL, err
    assert np.all(np.isfinite(y))
