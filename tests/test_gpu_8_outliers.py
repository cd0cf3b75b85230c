"""GPU parity on activations with an outlier that meets a zero weight.

The bar is per output, for any input: |y_gpu - y_ref| <= 2e-4 * sum|w x|.
Here x is zero except one group of 16 consecutive activations: an outlier R
times larger than its 15 neighbours (R = 2^8 .. 2^24, and 2^60 for fp32),
placed on a column whose weight is zero (nibble 8, or int8 0) in every row,
so the outlier adds nothing to the result or to the normaliser while any
error it causes would.  A kernel that rounds each activation relative to
the largest one near it fails this; one whose error is relative to each
activation itself passes.  The same construction is applied to the hidden
vector of the down projection (caller-supplied h) and to x of the whole
expert layer (zero gate and up columns), for int4, int8 and int3 weights.
"""
import numpy as np
import pytest
import torch

from gpu_util import TOL, dev, host, norm_err, upload_experts
from int4_expert_gemv_amd import synth

pytestmark = pytest.mark.gpu

RATIOS = (2.0 ** 8, 2.0 ** 12, 2.0 ** 16, 2.0 ** 24)


@pytest.fixture(scope="module")
def q():
    from int4_expert_gemv_amd import qmoe
    assert torch.cuda.is_available()
    return qmoe


def outlier_vec(g, k, ratio, pos, background=0.0):
    """fp32 vector: zero (or tiny noise) except group pos // 16, whose element
    pos is `ratio` times the scale of its N(0,1) neighbours."""
    x = (g.standard_normal(k) * background).astype(np.float32)
    g0 = pos // 16
    x[16 * g0:16 * g0 + 16] = g.standard_normal(16).astype(np.float32)
    x[pos] = np.float32(ratio * (1.0 + g.random()))
    return x


def as_dtype(x, xdt):
    return synth.to_bf16_bits(x) if xdt == "bf16" else x.astype(np.float32)


def zero_column(fmt, qw, col):
    """Set element `col` of every row to the zero weight (nibble 8 / int8 0 /
    int3 value 4: low part 0, high bit 1)."""
    qw = qw.copy()
    if fmt == 5:
        g, i = col // 64, col % 64
        b = np.ascontiguousarray(qw[:, 24 * g:24 * g + 24])
        lo = np.ascontiguousarray(b[:, :16]).view("<u4")
        hi = np.ascontiguousarray(b[:, 16:]).view("<u8")
        lo[:, i // 16] &= np.uint32(~(3 << (2 * (i % 16))) & 0xFFFFFFFF)
        hi[:, 0] |= np.uint64(1) << np.uint64(i)
        qw[:, 24 * g:24 * g + 16] = lo.view(np.uint8)
        qw[:, 24 * g + 16:24 * g + 24] = hi.view(np.uint8)
        return qw
    if fmt == 4:
        b = qw[:, col // 2]
        qw[:, col // 2] = (b & 0xF0) | 8 if col % 2 == 0 else (b & 0x0F) | 0x80
    else:
        qw[:, col] = 0
    return qw


GEMV_SHAPES = [
    (4, 512, 6144, 64, "bf16"), (4, 300, 16384, 0, "f32"), (4, 256, 2048, 32, "bf16"),
    (1, 512, 6144, 0, "bf16"), (1, 300, 2048, 0, "f32"),
    (4, 256, 512, 64, "f32"), (4, 77, 96, 0, "bf16"), (1, 19, 48, 0, "bf16"),
    (5, 512, 6144, 64, "bf16"), (5, 300, 16384, 64, "f32"), (5, 77, 96, 64, "bf16"), (5, 256, 2048, 64, "bf16"),
]


@pytest.mark.parametrize("fmt,n,k,gs,xdt", GEMV_SHAPES)
@pytest.mark.parametrize("ratio", RATIOS)
def test_qgemv_outlier_on_zero_weight(q, oracle, fmt, n, k, gs, xdt, ratio):
    print("qgemv outlier fmt=%d n=%d k=%d gs=%d x=%s R=2^%d" % (fmt, n, k, gs, xdt, np.log2(ratio)), flush=True)
    g = np.random.default_rng([61, fmt, n, k])
    pos = 16 * ((k // 16) // 3) + 7
    qw, s = synth.quant_matrix(g, fmt, n, k, gs)
    qw = zero_column(fmt, qw, pos)
    x = as_dtype(outlier_vec(g, k, ratio, pos), xdt)
    m = q.qmat(fmt, dev(qw), dev(s), n, k, gs)
    y = torch.full((n,), float("nan"), device="cuda")
    q.qgemv(m, dev(x), y)
    torch.cuda.synchronize()
    yr, nr = oracle.gemv(fmt, n, k, gs, qw, s, x)
    assert norm_err(host(y), yr, nr) <= TOL


@pytest.mark.parametrize("ratio", (2.0 ** 40, 2.0 ** 60, 2.0 ** 100))
def test_qgemv_extreme_fp32_outlier(q, oracle, ratio):
    fmt, n, k, gs = 4, 256, 4096, 64
    g = np.random.default_rng([62, int(np.log2(ratio))])
    pos = 16 * 100 + 3
    qw, s = synth.quant_matrix(g, fmt, n, k, gs)
    qw = zero_column(fmt, qw, pos)
    x = outlier_vec(g, k, ratio, pos, background=1e-3)
    m = q.qmat(fmt, dev(qw), dev(s), n, k, gs)
    y = torch.full((n,), float("nan"), device="cuda")
    q.qgemv(m, dev(x), y)
    torch.cuda.synchronize()
    yr, nr = oracle.gemv(fmt, n, k, gs, qw, s, x)
    assert norm_err(host(y), yr, nr) <= TOL


@pytest.mark.parametrize("fmt,gs", [(4, 64), (1, 0), (5, 64)])
@pytest.mark.parametrize("ratio", RATIOS)
def test_qgemv_pair_outlier(q, oracle, fmt, gs, ratio):
    k, n1, n2 = 6144, 2048, 576
    g = np.random.default_rng([63, fmt])
    pos = 16 * 200 + 11
    q1, s1 = synth.quant_matrix(g, fmt, n1, k, gs)
    q2, s2 = synth.quant_matrix(g, fmt, n2, k, gs)
    q1, q2 = zero_column(fmt, q1, pos), zero_column(fmt, q2, pos)
    x = as_dtype(outlier_vec(g, k, ratio, pos), "bf16")
    y1 = torch.full((n1,), float("nan"), device="cuda")
    y2 = torch.full((n2,), float("nan"), device="cuda")
    q.qgemv_pair(q.qmat(fmt, dev(q1), dev(s1), n1, k, gs), q.qmat(fmt, dev(q2), dev(s2), n2, k, gs), dev(x), y1, y2)
    torch.cuda.synchronize()
    for y, qq, ss, n in ((y1, q1, s1, n1), (y2, q2, s2, n2)):
        yr, nr = oracle.gemv(fmt, n, k, gs, qq, ss, x)
        assert norm_err(host(y), yr, nr) <= TOL


@pytest.mark.parametrize("fmt,gs,xdt,batch", [(4, 64, "bf16", 2), (4, 64, "f32", 8), (1, 0, "bf16", 4),
                                              (5, 64, "bf16", 3)])
@pytest.mark.parametrize("ratio", (2.0 ** 12, 2.0 ** 24))
def test_qgemm_small_outlier(q, oracle, fmt, gs, xdt, batch, ratio):
    n, k = 1024, 6144
    g = np.random.default_rng([64, fmt, batch])
    qw, s = synth.quant_matrix(g, fmt, n, k, gs)
    xs = []
    for t in range(batch):
        pos = 16 * (37 * t + 5) + (5 * t) % 16
        qw = zero_column(fmt, qw, pos)
        xs.append(outlier_vec(g, k, ratio, pos))
    x = as_dtype(np.stack(xs), xdt)
    m = q.qmat(fmt, dev(qw), dev(s), n, k, gs)
    y = torch.full((batch, n), float("nan"), device="cuda")
    q.qgemm_small(m, dev(x), y)
    torch.cuda.synchronize()
    yr, nr = oracle.gemm_small(fmt, n, k, gs, qw, s, x)
    assert norm_err(host(y), yr, nr) <= TOL


def _experts_zero_cols(seed, fmt, E, H, I, gs, xcol=None, hcol=None):
    ex = synth.expert_set(seed, fmt, E, H, I, gs)
    if xcol is not None:
        for key in ("gate_q", "up_q"):
            ex[key] = np.stack([zero_column(fmt, ex[key][e], xcol) for e in range(E)])
    if hcol is not None:
        ex["down_q"] = np.stack([zero_column(fmt, ex["down_q"][e], hcol) for e in range(E)])
    return ex


def _qexperts(q, ex):
    d = upload_experts(ex)
    return q.experts(ex["fmt"], ex["gs"], d["gate_q"], d["up_q"], d["down_q"], d["gate_s"], d["up_s"], d["down_s"])


@pytest.mark.parametrize("fmt,gs,E,H,I,T", [
    (4, 64, 16, 6144, 2048, 1), (4, 64, 16, 6144, 2048, 3), (4, 0, 16, 6144, 2048, 1),
    (4, 64, 32, 2048, 512, 1), (1, 0, 8, 1024, 512, 2), (4, 64, 12, 1024, 256, 5),
    (5, 64, 16, 6144, 2048, 1), (5, 64, 32, 2048, 512, 3),
])
@pytest.mark.parametrize("ratio", RATIOS)
def test_moe_down_outlier_h(q, oracle, fmt, gs, E, H, I, T, ratio):
    """The down stage on caller-supplied h with an outlier on a zero column
    of every expert's down matrix."""
    print("moe_down outlier fmt=%d gs=%d E=%d H=%d I=%d T=%d R=2^%d" % (fmt, gs, E, H, I, T, np.log2(ratio)),
          flush=True)
    K = 8
    pos = 16 * ((I // 16) // 2) + 9
    ex = _experts_zero_cols(71, fmt, E, H, I, gs, hcol=pos)
    g = np.random.default_rng([72, T])
    ids, w = synth.uniform_routing(g, T, E, K)
    h = np.stack([outlier_vec(g, I, ratio, pos) for _ in range(T * K)])
    e = _qexperts(q, ex)
    ws = torch.empty(q.moe_expert_ffn_workspace(e, T, K), dtype=torch.uint8, device="cuda")
    y = torch.full((T, H), float("nan"), device="cuda")
    q.moe_down(e, dev(h), dev(ids), dev(w), y, ws)
    torch.cuda.synchronize()
    yr = np.zeros((T, H))
    nr = np.zeros((T, H))
    D = ex["down_q"]
    for t in range(T):
        for j in range(K):
            ee = int(ids[t, j])
            o, no = oracle.gemv(fmt, H, I, gs, D[ee], ex["down_s"][ee], h[t * K + j].astype(np.float64))
            yr[t] += float(w[t, j]) * o
            nr[t] += abs(float(w[t, j])) * no
    assert norm_err(host(y), yr, nr) <= TOL


def _silu(z):
    return z / (1.0 + np.exp(-z))


@pytest.mark.parametrize("fmt,gs,E,H,I,T", [
    (4, 64, 16, 6144, 2048, 1), (4, 64, 32, 2048, 512, 1), (4, 0, 16, 6144, 2048, 2), (1, 0, 8, 1024, 512, 1),
    (5, 64, 16, 6144, 2048, 1), (5, 64, 32, 2048, 512, 2),
])
@pytest.mark.parametrize("ratio", RATIOS)
def test_moe_gate_up_outlier_x(q, oracle, fmt, gs, E, H, I, T, ratio):
    """The gate+up stage: h within the bar propagated from the gate and up
    contractions, |silu'(a) b| sum|g x| + |silu(a)| sum|u x|."""
    K = 8
    pos = 16 * ((H // 16) // 3) + 5
    ex = _experts_zero_cols(73, fmt, E, H, I, gs, xcol=pos)
    g = np.random.default_rng([74, T])
    ids, w = synth.uniform_routing(g, T, E, K)
    x32 = np.stack([outlier_vec(g, H, ratio, pos) for _ in range(T)])
    x = as_dtype(x32, "bf16")
    e = _qexperts(q, ex)
    h = torch.full((T * K, I), float("nan"), device="cuda")
    ws = torch.empty(q.moe_expert_ffn_workspace(e, T, K), dtype=torch.uint8, device="cuda")
    q.moe_gate_up(e, dev(x), dev(ids), h, ws)
    torch.cuda.synchronize()
    hg = host(h).astype(np.float64)
    for t in range(T):
        for j in range(K):
            ee = int(ids[t, j])
            a, na = oracle.gemv(fmt, I, H, gs, ex["gate_q"][ee], ex["gate_s"][ee], x[t])
            b, nb = oracle.gemv(fmt, I, H, gs, ex["up_q"][ee], ex["up_s"][ee], x[t])
            sg = 1.0 / (1.0 + np.exp(-a))
            dsilu = sg * (1.0 + a * (1.0 - sg))
            href = _silu(a) * b
            nh = np.abs(dsilu * b) * na + np.abs(_silu(a)) * nb
            assert norm_err(hg[t * K + j], href, nh) <= TOL, (t, j)


@pytest.mark.parametrize("fmt,gs,E,H,I,T", [
    (4, 64, 64, 2048, 512, 1),     # small experts
    (4, 64, 24, 6144, 2048, 1),    # large experts, one token
    (4, 0, 24, 6144, 2048, 1),
    (4, 64, 24, 6144, 2048, 4),
    (1, 0, 8, 1024, 512, 2),
    (5, 64, 24, 6144, 2048, 1),    # int3-g64 experts
    (5, 64, 64, 2048, 512, 2),
])
@pytest.mark.parametrize("ratio", RATIOS)
def test_moe_layer_outlier_x(q, oracle, fmt, gs, E, H, I, T, ratio):
    print("moe layer outlier fmt=%d gs=%d E=%d H=%d I=%d T=%d R=2^%d" % (fmt, gs, E, H, I, T, np.log2(ratio)),
          flush=True)
    K = 8
    pos = 16 * ((H // 16) // 4) + 12
    ex = _experts_zero_cols(75, fmt, E, H, I, gs, xcol=pos)
    g = np.random.default_rng([76, T])
    ids, w = synth.uniform_routing(g, T, E, K)
    x = as_dtype(np.stack([outlier_vec(g, H, ratio, pos) for _ in range(T)]), "bf16")
    e = _qexperts(q, ex)
    ws = torch.empty(q.moe_expert_ffn_workspace(e, T, K), dtype=torch.uint8, device="cuda")
    y = torch.full((T, H), float("nan"), device="cuda")
    q.moe_expert_ffn(e, dev(x), dev(ids), dev(w), y, ws)
    torch.cuda.synchronize()
    yr, _, nr = oracle.moe_ffn(ex, x, ids, w)
    assert norm_err(host(y), yr, nr) <= TOL
