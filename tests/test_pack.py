"""Host packing, validation and quantization (include/qmoe.h, no GPU).

The packed layouts are checked against the oracle's own reading of them: the
oracle GEMV of a one-hot x (x = e_c) returns column c of the dequantized
matrix, which must equal value x scale exactly for every row and column (the
oracle computes in fp64; int x fp32 products are exact there).
"""
import numpy as np
import pytest

from int4_expert_gemv_amd import synth

pytestmark = pytest.mark.filterwarnings("ignore")


@pytest.fixture(scope="module")
def q():
    from int4_expert_gemv_amd import qmoe
    return qmoe


def _columns(oracle, fmt, n, k, gs, qm, sc, cols):
    """Dequantized columns through the oracle: y = W e_c."""
    out = np.zeros((n, len(cols)))
    for j, c in enumerate(cols):
        x = np.zeros(k, np.float64)
        x[c] = 1.0
        y, _ = oracle.gemv(fmt, n, k, gs, qm, sc, x)
        out[:, j] = y
    return out


@pytest.mark.parametrize("n,k,gs", [(8, 256, 64), (5, 64, 0), (3, 96, 32), (4, 128, 128)])
def test_pack_int4_round_trip(q, oracle, n, k, gs):
    g = synth.rng(41, n, k, gs)
    v = g.integers(-8, 8, size=(n, k), dtype=np.int8)
    groups = 1 if gs in (0, k) else k // gs
    s = synth.uniform_f32(g, (n, groups), 0.01, 2.0)
    qm = q.pack_int4(v)
    assert qm.shape == (n, k // 2)
    assert q.validate(q.QM_FMT_INT4, n, k, gs, s) == q.QM_OK
    cols = list(range(k))
    got = _columns(oracle, 4, n, k, gs, qm, s, cols)
    want = v.astype(np.float64) * np.repeat(s.astype(np.float64), k // groups, axis=1)
    np.testing.assert_array_equal(got, want)


def test_pack_int4_nibble_order(q):
    """Element 2i in the low nibble, 2i+1 in the high nibble, value + 8."""
    v = np.array([[-8, 7, 0, -1]], np.int8)
    assert q.pack_int4(v).tolist() == [[0x00 | (15 << 4), 8 | (7 << 4)]]


def test_pack_int8_round_trip(q, oracle):
    n, k = 6, 80
    g = synth.rng(42)
    v = g.integers(-128, 128, size=(n, k), dtype=np.int8)
    s = synth.uniform_f32(g, (n, 1), 0.01, 2.0)
    qm = q.pack_int8(v)
    assert q.validate(q.QM_FMT_INT8_ROW, n, k, 0, s) == q.QM_OK
    got = _columns(oracle, 1, n, k, 0, qm, s, list(range(k)))
    np.testing.assert_array_equal(got, v.astype(np.float64) * s.astype(np.float64))


def test_pack_rejects(q):
    with pytest.raises(q.QmError):
        q.pack_int4(np.array([[8, 0]], np.int8))         # outside [-8, 7]
    with pytest.raises(q.QmError):
        q.pack_int4(np.array([[-9, 0]], np.int8))
    with pytest.raises(q.QmError):
        q.pack_int4(np.zeros((2, 3), np.int8))           # odd k
    assert q.lib.qm_pack_int4(None, 1, 2, None) == q.QM_ERR_INVALID
    assert q.lib.qm_pack_int8(None, 1, 2, None) == q.QM_ERR_INVALID
    s = np.ones((2, 4), np.float32)
    assert q.validate(q.QM_FMT_INT4, 2, 256, 64, s) == q.QM_OK
    assert q.validate(q.QM_FMT_INT4, 2, 256, 48, s) == q.QM_ERR_INVALID   # not a multiple of 32
    assert q.validate(q.QM_FMT_INT4, 2, 256, 96, s) == q.QM_ERR_INVALID   # does not divide k
    assert q.validate(q.QM_FMT_INT8_ROW, 2, 256, 64, s) == q.QM_ERR_INVALID
    assert q.validate(9, 2, 256, 64, s) == q.QM_ERR_INVALID
    for bad in (np.nan, np.inf, -np.inf):
        t = s.copy()
        t[1, 3] = bad
        assert q.validate(q.QM_FMT_INT4, 2, 256, 64, t) == q.QM_ERR_INVALID
    assert q.validate(q.QM_FMT_INT3, 2, 200, 64, s) == q.QM_OK            # ceil(200 / 64) = 4 groups
    with pytest.raises(q.QmError):
        q.quantize_int4(np.array([[np.nan, 0.0]], np.float32), 0)


@pytest.mark.parametrize("gs", [64, 0])
def test_quantize_int4(q, oracle, gs):
    n, k = 4, 256
    g = synth.rng(43, gs)
    w = synth.normal_f32(g, (n, k))
    w[1, 64:128] = 0.0                                   # an all-zero group: scale 0, codes 0
    qm, s = q.quantize_int4(w, gs)
    groups = s.shape[1]
    ws = k // groups
    amax = np.abs(w.reshape(n, groups, ws)).max(axis=2)
    np.testing.assert_array_equal(s, (amax / np.float32(7)).astype(np.float32))
    deq = _columns(oracle, 4, n, k, gs, qm, s, list(range(k)))
    sfull = np.repeat(s.astype(np.float64), ws, axis=1)
    # nearest code: within half a step of the weight; the group's largest
    # magnitude lands on +-7 exactly
    assert np.all(np.abs(deq - w) <= 0.5 * sfull * (1 + 1e-6) + 1e-30)
    codes = np.rint(np.divide(deq, sfull, out=np.zeros_like(deq), where=sfull > 0))
    assert codes.min() >= -7 and codes.max() <= 7
    for r in range(n):
        for gi in range(groups):
            if amax[r, gi] > 0:
                i = np.argmax(np.abs(w[r, gi * ws:(gi + 1) * ws])) + gi * ws
                assert abs(codes[r, i]) == 7
    if gs:
        assert np.all(deq[1, 64:128] == 0) and s[1, 1] == 0


def test_quantize_int8(q, oracle):
    n, k = 3, 96
    w = synth.normal_f32(synth.rng(44), (n, k))
    qm, s = q.quantize_int8(w)
    np.testing.assert_array_equal(s[:, 0], (np.abs(w).max(axis=1) / np.float32(127)).astype(np.float32))
    deq = _columns(oracle, 1, n, k, 0, qm, s, list(range(k)))
    assert np.all(np.abs(deq - w) <= 0.5 * s.astype(np.float64) * (1 + 1e-6))
    assert np.abs(qm).max() == 127
