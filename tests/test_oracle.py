"""Pins of the fp64 CPU oracle against facts fixed outside it.

Each pin checks the oracle against something other than itself: hand-worked
exact cases (tests/golden/hand_cases.json), one-hot closed forms built from
the encoding direction of the format, invariants of the definition, a dense
float64 numpy/BLAS restatement (tests/bruteforce.py), exact rational
arithmetic on integer data, textbook SiLU values and torch's bf16 cast.
`test_mutants_are_caught` plants known mistakes in the oracle (compile-time
switch, CPU only) and checks that the pin battery fails for every one.
"""
import bisect
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import bruteforce as bf
from int4_expert_gemv_amd import synth
from oracle import ref

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")))


def _rel_close(got, want, tol):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    if tol == 0:
        return np.array_equal(got, want)
    return bool(np.all(np.abs(got - want) <= tol * np.maximum(np.abs(want), 1e-300)))


# --------------------------------------------------------------------------
# pin battery: each function raises AssertionError on a mismatch.  The same
# functions run on the real oracle (tests below) and on planted mutants.
# --------------------------------------------------------------------------

def pin_hand_gemv(o):
    for case in GOLD["gemv"]:
        fmt, n, k, gs = case["fmt"], case["n"], case["k"], case["gs"]
        if fmt == 4:
            q = bf.pack_nibbles(case["nibbles"])
            assert q.tolist() == case["bytes"], case["name"]
        else:
            q = np.array(case["int8"], np.int8)
        s = np.array(case["scales"], np.float32)
        x = np.array(case["x"], np.float32)
        y, nrm = o.gemv(fmt, n, k, gs, q, s, x)
        assert _rel_close(y, case["y"], case["rel_tol"]), (case["name"], y)
        if "norm" in case:
            assert _rel_close(nrm, case["norm"], case["rel_tol"]), (case["name"], nrm)


def pin_one_hot(o, gs, n=3, k=16, seed=1):
    """x = e_c gives y_n = (nibble(n, c) - 8) * s[n][c // gs] exactly."""
    g = np.random.default_rng([seed, gs])
    nib = np.stack([g.permutation(16)[:k] if k <= 16 else g.integers(0, 16, k) for _ in range(n)])
    q = bf.pack_nibbles(nib)
    G = 1 if gs == 0 else -(-k // gs)
    s = g.uniform(-2, 2, size=(n, G)).astype(np.float32)
    for c in range(k):
        x = np.zeros(k, np.float32)
        x[c] = 1.0
        y, _ = o.gemv(4, n, k, gs, q, s, x)
        sc = s[:, 0 if gs == 0 else c // gs].astype(np.float64)
        want = (nib[:, c].astype(np.float64) - 8.0) * sc
        assert np.array_equal(y, want), (gs, c, y, want)


def pin_one_hot_int8(o, n=4, k=8, seed=2):
    g = np.random.default_rng(seed)
    v = g.integers(-128, 128, size=(n, k)).astype(np.int8)
    v[0, 0], v[1, 1] = -128, 127
    s = g.uniform(-2, 2, size=(n, 1)).astype(np.float32)
    for c in range(k):
        x = np.zeros(k, np.float32)
        x[c] = 1.0
        y, _ = o.gemv(1, n, k, 0, v, s, x)
        assert np.array_equal(y, v[:, c].astype(np.float64) * s[:, 0].astype(np.float64)), c


def pin_silu(o):
    for z, want in GOLD["silu"]["points"]:
        assert _rel_close(o.silu(z), want, GOLD["silu"]["rel_tol"]), z


def pin_hand_moe(o):
    c = GOLD["moe"]
    ex = {"n_experts": c["n_experts"], "hidden": c["hidden"], "inter": c["inter"],
          "fmt": c["fmt"], "gs": c["gs"]}
    for name in ("gate", "up", "down"):
        ex[name + "_q"] = np.stack([bf.pack_nibbles(m) for m in c[name + "_nibbles"]])
        ex[name + "_s"] = np.array(c[name + "_scales"], np.float32)
    x = np.array([c["x"]], np.float32)
    y, h, _ = o.moe_ffn(ex, x, np.array(c["ids"], np.int32), np.array(c["w"], np.float32), want_h=True)
    assert _rel_close(y[0], c["y"], c["rel_tol"]), y
    assert _rel_close(h[0], c["h0"], c["rel_tol"]), h


def _bf16_table():
    """All finite non-negative bf16 values, exactly, with their bit patterns."""
    bits = np.arange(0, 0x7F80, dtype=np.uint32)
    vals = (bits << 16).view(np.float32).astype(np.float64)
    return vals.tolist(), bits.tolist()


_BF16_VALS, _BF16_BITS = _bf16_table()


def _exact_bf16(v):
    """Nearest bf16 to the double v by table search; ties go to the even
    pattern; past the largest finite value's rounding midpoint -> inf."""
    if v == 0 or math.isnan(v) or math.isinf(v):
        return v
    a = abs(v)
    top = _BF16_VALS[-1]
    half_ulp_top = Fraction(top) - Fraction(_BF16_VALS[-2])
    if Fraction(a) >= Fraction(top) + half_ulp_top / 2:
        r = math.inf
    else:
        i = bisect.bisect_left(_BF16_VALS, a)
        if i < len(_BF16_VALS) and _BF16_VALS[i] == a:
            r = a
        elif i == len(_BF16_VALS):
            r = top  # above the largest finite value but below its rounding midpoint
        else:
            lo, hi = _BF16_VALS[i - 1], _BF16_VALS[i]
            dlo, dhi = Fraction(a) - Fraction(lo), Fraction(hi) - Fraction(a)
            if dlo < dhi:
                r = lo
            elif dhi < dlo:
                r = hi
            else:
                r = lo if (_BF16_BITS[i - 1] & 1) == 0 else hi
    return -r if v < 0 else r


def pin_bf16(o):
    edge = [0.0, -0.0, 1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -8 + 2 ** -20, -(1 + 2 ** -8),
            1e-40, -1e-40, 2 ** -133, 3 * 2 ** -134, 1.17e-38, 3.3895e38, 3.39e38, 3.4028234e38,
            65504.0, 0.1, -0.3, 7.0, 1e30, 2.5e-20, float("inf"), -float("inf")]
    g = np.random.default_rng(7)
    rnd = (g.standard_normal(200) * np.exp2(g.integers(-130, 127, 200))).astype(np.float32)
    vals = np.array(edge + rnd.tolist(), np.float32)
    want = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    for v, w in zip(vals.tolist(), want.tolist()):
        assert o.f32_to_bf16(v) == w, (v, o.f32_to_bf16(v), w)
        assert o.bf16_to_f32(w) == float(np.float32((np.uint32(w) << 16).view(np.float32)))
    nan = o.f32_to_bf16(float("nan"))
    assert (nan & 0x7F80) == 0x7F80 and (nan & 0x007F) != 0
    dvals = [1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -8 + 2 ** -40, 2 ** -130 * 1.5, 2 ** -140,
             3.3895313892515355e38, 3.3961e38, -2.7182818284590455, 1e-45]
    dvals += (g.standard_normal(200) * np.exp2(g.integers(-140, 120, 200))).tolist()
    for v in dvals:
        assert o.round_bf16(v) == _exact_bf16(v), (v, o.round_bf16(v), _exact_bf16(v))


def pin_bruteforce_gemv(o, fmt, n, k, gs, xdt, seed=3):
    g = np.random.default_rng([seed, fmt, n, k, gs])
    q, s = synth.quant_matrix(g, fmt, n, k, gs)
    x = synth.activations(g, (k,), xdt)
    xf = synth.bf16_bits_to_f32(x) if xdt == "bf16" else x
    y, nrm = o.gemv(fmt, n, k, gs, q, s, x)
    yb, nb = bf.gemv(fmt, q, s, k, gs, xf)
    assert np.all(np.abs(y - yb) <= 1e-12 * nb), np.max(np.abs(y - yb) / nb)
    assert np.all(np.abs(nrm - nb) <= 1e-12 * nb)


def pin_bruteforce_moe(o, fmt, gs, T=3, E=5, H=128, I=64, k=3, seed=4):
    """y and the parity normaliser against the dense numpy restatement, with
    routing weights of both signs (the normaliser takes |w|)."""
    ex = synth.expert_set(seed, fmt, E, H, I, gs)
    g = np.random.default_rng([seed, 99])
    x = synth.activations(g, (T, H), "f32")
    ids, w = synth.uniform_routing(g, T, E, k)
    w = (w * np.where(g.random(w.shape) < 0.5, -1.0, 1.0) * g.uniform(0.5, 3.0, w.shape)).astype(np.float32)
    y, _, nrm = o.moe_ffn(ex, x, ids, w)
    yb, nb = bf.moe(ex, x, ids, w)
    assert np.all(np.abs(y - yb) <= 1e-12 * nb), np.max(np.abs(y - yb) / nb)
    assert np.all(np.abs(nrm - nb) <= 1e-12 * nb), np.max(np.abs(nrm - nb) / nb)


def pin_bf16_act(o, T=2, E=4, H=64, I=32, k=2, seed=14):
    """Prefill precision mode with fp32 activations that bf16 cannot hold:
    the oracle must give exactly what it gives for the same x rounded to
    bf16 by torch, and match the dense restatement with x and every hidden
    vector rounded to the nearest bf16 (exact table search)."""
    ex = synth.expert_set(seed, 4, E, H, I, 64)
    g = np.random.default_rng(seed)
    x = (g.standard_normal((T, H)) * (1.0 + 2.0 ** -12)).astype(np.float32)
    xb = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    xr = (xb.astype(np.uint32) << 16).view(np.float32)
    assert not np.array_equal(xr, x)  # the rounding is visible
    ids, w = synth.uniform_routing(g, T, E, k)
    y1, h1, n1 = o.moe_ffn(ex, x, ids, w, flags=ref.BF16_ACT, want_h=True)
    y2, h2, n2 = o.moe_ffn(ex, xb, ids, w, flags=ref.BF16_ACT, want_h=True)
    assert np.array_equal(y1, y2) and np.array_equal(h1, h2) and np.array_equal(n1, n2)
    yb, nb = bf.moe(ex, xr, ids, w, round_h=lambda h: np.array([_exact_bf16(v) for v in h]))
    assert np.all(np.abs(y1 - yb) <= 1e-12 * nb), np.max(np.abs(y1 - yb) / nb)


def pin_rmsnorm(o):
    """Closed forms of out = u / sqrt(mean(u^2) + eps) * g."""
    r = np.sqrt(12.5)  # [3, 4]: mean of squares 12.5
    assert _rel_close(o.rmsnorm([3.0, 4.0]), [3 / r, 4 / r], 1e-15)
    g = np.arange(1, 8, dtype=np.float32)
    assert _rel_close(o.rmsnorm(np.full(7, -2.5), g), -g.astype(np.float64), 1e-15)  # constant vector -> sign * g
    assert _rel_close(o.rmsnorm([1.0, 1.0], np.array([2, -6], np.float32), eps=3.0), [1.0, -3.0], 1e-15)
    u = np.random.default_rng(11).standard_normal(1536)
    out = o.rmsnorm(u)
    assert abs(np.mean(out ** 2) - 1.0) < 1e-12  # unit mean square with eps = 0, g = 1
    assert _rel_close(o.rmsnorm(u * 1024.0), out, 1e-14)  # scale invariance


def pin_f64_input(o):
    """A float64 activation vector gives what the same values in float32 give."""
    g = np.random.default_rng(12)
    nib = g.integers(0, 16, (5, 64))
    q = bf.pack_nibbles(nib)
    s = g.uniform(0.5, 2.0, (5, 1)).astype(np.float32)
    x32 = g.standard_normal(64).astype(np.float32)
    y32, _ = o.gemv(4, 5, 64, 0, q, s, x32)
    y64, _ = o.gemv(4, 5, 64, 0, q, s, x32.astype(np.float64))
    assert np.array_equal(y32, y64)


def pack_int3(vals):
    """Test-side packer for the int3 two-plane layout (independent of the
    generators): per 64-group, four little-endian 32-bit words of 2-bit low
    parts (value i of the group at bits 2 (i % 16) of word i // 16), then a
    64-bit word of high bits (value i at bit i); a ragged last group is
    padded with zeros."""
    vals = np.asarray(vals)
    n, k = vals.shape
    G = (k + 63) // 64
    out = np.zeros((n, G * 24), np.uint8)
    for r in range(n):
        for g in range(G):
            lo, hi = [0, 0, 0, 0], 0
            for i in range(64):
                c = 64 * g + i
                v = int(vals[r, c]) if c < k else 0
                lo[i // 16] |= (v & 3) << (2 * (i % 16))
                hi |= ((v >> 2) & 1) << i
            raw = b"".join(w.to_bytes(4, "little") for w in lo) + hi.to_bytes(8, "little")
            out[r, 24 * g:24 * g + 24] = np.frombuffer(raw, np.uint8)
    return out


def pin_int3(o):
    """One-hot columns (every bit position class, a ragged tail group) give
    (v - 4) * scale exactly; an int3 matrix equals the int4-g64 matrix with
    nibbles v + 4 and the same scales."""
    g = np.random.default_rng(13)
    n, k = 3, 96
    vals = g.integers(0, 8, (n, k))
    s = g.uniform(0.5, 2.0, (n, 2)).astype(np.float32)
    q3 = pack_int3(vals)
    for c in (0, 1, 7, 15, 16, 30, 31, 47, 48, 63, 64, 70, 95):
        x = np.zeros(k, np.float32)
        x[c] = 1.0
        y, _ = o.gemv(5, n, k, 64, q3, s, x)
        assert np.array_equal(y, (vals[:, c] - 4) * s[:, c // 64].astype(np.float64)), c
    k2 = 256
    vals2 = g.integers(0, 8, (n, k2))
    s2 = g.uniform(0.5, 2.0, (n, 4)).astype(np.float32)
    x2 = g.standard_normal(k2).astype(np.float32)
    y3, n3 = o.gemv(5, n, k2, 64, pack_int3(vals2), s2, x2)
    y4, n4 = o.gemv(4, n, k2, 64, bf.pack_nibbles(vals2 + 4), s2, x2)
    assert np.array_equal(y3, y4) and np.array_equal(n3, n4)


def _int3_layer(g, E, H, I):
    """An int3-g64 layer from known values v in 0..7 and the int4-g64 layer
    with nibbles v + 4 (the same elements v - 4) and the same scales."""
    ex3 = {"n_experts": E, "hidden": H, "inter": I, "fmt": 5, "gs": 64}
    ex4 = {"n_experts": E, "hidden": H, "inter": I, "fmt": 4, "gs": 64}
    vals = {}
    for name, n, k in (("gate", I, H), ("up", I, H), ("down", H, I)):
        v = g.integers(0, 8, (E, n, k))
        s = g.uniform(0.5, 2.0, (E, n, k // 64)).astype(np.float32)
        ex3[name + "_q"] = np.stack([pack_int3(v[e]) for e in range(E)])
        ex4[name + "_q"] = np.stack([bf.pack_nibbles(v[e] + 4) for e in range(E)])
        ex3[name + "_s"] = ex4[name + "_s"] = s
        vals[name] = v
    return ex3, ex4, vals


def pin_int3_moe(o):
    """A whole int3 layer: bit for bit the int4-g64 layer with nibbles v + 4
    (y, h and the normaliser); the dense numpy restatement; and, with each
    token's x one-hot on a column c, h = silu(a) * b with a, b the known
    elements (v - 4) times their scales in column c, then y = sum_j w_j D h."""
    E, H, I, T, k = 4, 192, 128, 3, 2
    g = np.random.default_rng(15)
    ex3, ex4, vals = _int3_layer(g, E, H, I)
    x = g.standard_normal((T, H)).astype(np.float32)
    ids = np.array([[0, 3], [2, 1], [3, 3]], np.int32)
    w = np.array([[0.7, -1.3], [0.25, 2.0], [1.5, 0.5]], np.float32)
    y3, h3, n3 = o.moe_ffn(ex3, x, ids, w, want_h=True)
    y4, h4, n4 = o.moe_ffn(ex4, x, ids, w, want_h=True)
    assert np.array_equal(y3, y4) and np.array_equal(h3, h4) and np.array_equal(n3, n4)
    yb, nb = bf.moe(ex3, x, ids, w)
    assert np.all(np.abs(y3 - yb) <= 1e-12 * nb) and np.all(np.abs(n3 - nb) <= 1e-12 * nb)
    cols = [5, 64 + 17, 191]
    xo = np.zeros((T, H), np.float32)
    for t, c in enumerate(cols):
        xo[t, c] = 1.0
    yo, ho, _ = o.moe_ffn(ex3, xo, ids, w, want_h=True)
    for t, c in enumerate(cols):
        yt, nt = np.zeros(H), np.zeros(H)
        for j in range(k):
            e = ids[t, j]
            a = (vals["gate"][e][:, c] - 4) * ex3["gate_s"][e][:, c // 64].astype(np.float64)
            b = (vals["up"][e][:, c] - 4) * ex3["up_s"][e][:, c // 64].astype(np.float64)
            h = a / (1.0 + np.exp(-a)) * b
            assert _rel_close(ho[t * k + j], h, 1e-14)
            D = (vals["down"][e] - 4) * np.repeat(ex3["down_s"][e].astype(np.float64), 64, axis=1)
            yt += float(w[t, j]) * (D @ h)
            nt += abs(float(w[t, j])) * (np.abs(D) @ np.abs(h))
        assert np.all(np.abs(yo[t] - yt) <= 1e-12 * nt)


def run_battery(o):
    pin_int3(o)
    pin_int3_moe(o)
    pin_rmsnorm(o)
    pin_f64_input(o)
    pin_hand_gemv(o)
    for gs in (0, 2, 4, 8):
        pin_one_hot(o, gs)
    pin_one_hot_int8(o)
    pin_silu(o)
    pin_hand_moe(o)
    pin_bf16(o)
    pin_bruteforce_gemv(o, 4, 7, 128, 64, "f32")
    pin_bruteforce_gemv(o, 1, 5, 48, 0, "bf16")
    pin_bruteforce_moe(o, 4, 64)
    pin_bruteforce_moe(o, 1, 0)
    pin_bf16_act(o)


# --------------------------------------------------------------------------
# tests on the real oracle
# --------------------------------------------------------------------------

def test_hand_gemv(oracle):
    pin_hand_gemv(oracle)


def test_int3_decode(oracle):
    pin_int3(oracle)


def test_int3_moe_layer(oracle):
    pin_int3_moe(oracle)


def test_rmsnorm_closed_forms(oracle):
    pin_rmsnorm(oracle)
    pin_f64_input(oracle)


@pytest.mark.parametrize("gs", [0, 2, 4, 8, 64])
def test_one_hot_int4(oracle, gs):
    pin_one_hot(oracle, gs, k=16 if gs != 64 else 128)


def test_one_hot_int8(oracle):
    pin_one_hot_int8(oracle)


def test_silu_closed_form(oracle):
    pin_silu(oracle)
    assert oracle.silu(-800.0) == 0.0 and math.copysign(1, oracle.silu(-800.0)) == -1
    assert oracle.silu(800.0) == 800.0


def test_hand_moe(oracle):
    pin_hand_moe(oracle)


def test_bf16_helpers(oracle):
    pin_bf16(oracle)


@pytest.mark.parametrize("fmt,n,k,gs,xdt", [
    (4, 7, 128, 64, "f32"), (4, 5, 96, 64, "f32"), (4, 9, 512, 64, "bf16"), (4, 4, 128, 0, "f32"),
    (4, 3, 256, 32, "bf16"), (4, 6, 64, 16, "f32"), (1, 5, 48, 0, "bf16"), (1, 8, 512, 0, "f32"),
])
def test_bruteforce_gemv(oracle, fmt, n, k, gs, xdt):
    pin_bruteforce_gemv(oracle, fmt, n, k, gs, xdt)


def test_every_nibble_in_every_position(oracle):
    """All 16 nibble values at every position of a 32-element word span."""
    k, n = 32, 16
    nib = (np.arange(n)[:, None] + np.arange(k)[None, :]) % 16
    q = bf.pack_nibbles(nib)
    g = np.random.default_rng(5)
    s = g.uniform(0.5, 2, size=(n, 1)).astype(np.float32)
    x = g.standard_normal(k).astype(np.float32)
    y, nrm = oracle.gemv(4, n, k, 0, q, s, x)
    yb, nb = bf.gemv(4, q, s, k, 0, x)
    assert np.all(np.abs(y - yb) <= 1e-13 * nb)


@pytest.mark.parametrize("fmt,gs", [(4, 64), (4, 0), (1, 0), (5, 64)])
def test_bruteforce_moe(oracle, fmt, gs):
    pin_bruteforce_moe(oracle, fmt, gs)


def test_exact_integer_data(oracle):
    """Integer x in [-4, 4] and power-of-two scales: the exact rational result
    (python Fractions) is representable and the oracle must hit it exactly."""
    g = np.random.default_rng(6)
    n, k, gs = 4, 192, 64
    q, _ = synth.quant_matrix(g, 4, n, k, gs)
    s = synth.pow2_scales(g, (n, k // gs))
    x = synth.small_int_activations(g, (k,), "f32")
    y, _ = oracle.gemv(4, n, k, gs, q, s, x)
    for r in range(n):
        tot = Fraction(0)
        for c in range(k):
            nibv = (int(q[r, c // 2]) >> (4 * (c % 2))) & 15
            tot += Fraction(nibv - 8) * Fraction(float(s[r, c // gs])) * Fraction(float(x[c]))
        assert y[r] == float(tot)


# ---- invariants of the definition ------------------------------------------

def _mat(seed, fmt, n, k, gs):
    g = np.random.default_rng(seed)
    q, s = synth.quant_matrix(g, fmt, n, k, gs)
    return g, q, s


def test_all_nibbles_eight_is_zero(oracle):
    q = np.full((5, 64), 0x88, np.uint8)
    s = np.random.default_rng(8).uniform(0.1, 1, (5, 2)).astype(np.float32)
    x = np.random.default_rng(9).standard_normal(128).astype(np.float32)
    y, nrm = oracle.gemv(4, 5, 128, 64, q, s, x)
    assert np.all(y == 0) and np.all(nrm == 0)


def test_zero_scale_group_contributes_nothing(oracle):
    g, q, s = _mat(10, 4, 6, 256, 64)
    x = g.standard_normal(256).astype(np.float32)
    s2 = s.copy()
    s2[:, 2] = 0
    x2 = x.copy()
    x2[128:192] = 0
    y2, _ = oracle.gemv(4, 6, 256, 64, q, s2, x)
    y3, _ = oracle.gemv(4, 6, 256, 64, q, s, x2)
    assert np.allclose(y2, y3, rtol=1e-14, atol=1e-14)


def test_linear_in_x(oracle):
    g, q, s = _mat(11, 4, 8, 256, 64)
    # multiples of 2^-10 below 8 in magnitude: a*x1 + b*x2 stays exact in fp32
    x1 = (np.round(np.clip(g.standard_normal(256), -7, 7) * 1024) / 1024).astype(np.float32)
    x2 = (np.round(np.clip(g.standard_normal(256), -7, 7) * 1024) / 1024).astype(np.float32)
    a, b = 0.5, -2.0
    y1, n1 = oracle.gemv(4, 8, 256, 64, q, s, x1)
    y2, n2 = oracle.gemv(4, 8, 256, 64, q, s, x2)
    x3 = (a * x1.astype(np.float64) + b * x2.astype(np.float64))
    assert np.array_equal(x3.astype(np.float32).astype(np.float64), x3)
    y3, _ = oracle.gemv(4, 8, 256, 64, q, s, x3.astype(np.float32))
    assert np.all(np.abs(y3 - (a * y1 + b * y2)) <= 1e-14 * (abs(a) * n1 + abs(b) * n2))


def test_group_k_equals_per_row(oracle):
    g, q, s = _mat(12, 4, 6, 128, 0)
    x = g.standard_normal(128).astype(np.float32)
    y0, _ = oracle.gemv(4, 6, 128, 0, q, s, x)
    yk, _ = oracle.gemv(4, 6, 128, 128, q, s, x)
    assert np.array_equal(y0, yk)
    # g64 with the same scale in every group of a row == per-row with that scale
    s64 = np.repeat(s, 2, axis=1)
    y64, _ = oracle.gemv(4, 6, 128, 64, q, s64, x)
    assert np.allclose(y64, y0, rtol=1e-14, atol=1e-12)


def test_int4_embedded_as_int8(oracle):
    g, q, s = _mat(13, 4, 5, 64, 0)
    x = g.standard_normal(64).astype(np.float32)
    v = np.empty((5, 64), np.int8)
    v[:, 0::2] = (q & 15).astype(np.int8) - 8
    v[:, 1::2] = (q >> 4).astype(np.int8) - 8
    y4, _ = oracle.gemv(4, 5, 64, 0, q, s, x)
    y8, _ = oracle.gemv(1, 5, 64, 0, v, s, x)
    assert np.array_equal(y4, y8)


def test_gemm_small_columns_equal_gemv(oracle):
    g, q, s = _mat(14, 4, 9, 256, 64)
    X = synth.activations(g, (5, 256), "bf16")
    Y, N = oracle.gemm_small(4, 9, 256, 64, q, s, X)
    for t in range(5):
        y, n = oracle.gemv(4, 9, 256, 64, q, s, X[t])
        assert np.array_equal(Y[t], y) and np.array_equal(N[t], n)


def test_thread_count_does_not_change_results(oracle):
    g, q, s = _mat(15, 4, 257, 512, 64)
    x = g.standard_normal(512).astype(np.float32)
    prev = oracle.set_threads(1)
    y1, _ = oracle.gemv(4, 257, 512, 64, q, s, x)
    oracle.set_threads(4)
    y4, _ = oracle.gemv(4, 257, 512, 64, q, s, x)
    oracle.set_threads(prev)
    assert np.array_equal(y1, y4)


def test_rejects_invalid(oracle):
    q = np.zeros((2, 3), np.uint8)
    s = np.ones((2, 1), np.float32)
    with pytest.raises(ValueError):
        oracle.gemv(4, 2, 5, 0, q, s, np.zeros(5, np.float32))   # odd K for int4
    with pytest.raises(ValueError):
        oracle.gemv(3, 2, 6, 0, q, s, np.zeros(6, np.float32))   # unknown format


# ---- MoE invariants ----------------------------------------------------------

def _moe_case(seed=20, fmt=4, gs=64, T=3, E=6, H=128, I=64, k=3):
    ex = synth.expert_set(seed, fmt, E, H, I, gs)
    g = np.random.default_rng([seed, 1])
    x = synth.activations(g, (T, H), "bf16")
    ids, w = synth.uniform_routing(g, T, E, k)
    return ex, x, ids, w


def test_moe_zero_weights_give_zero(oracle):
    ex, x, ids, w = _moe_case()
    y, _, _ = oracle.moe_ffn(ex, x, ids, np.zeros_like(w))
    assert np.all(y == 0)


def test_moe_gate_all_eight_gives_zero(oracle):
    ex, x, ids, w = _moe_case()
    ex["gate_q"][:] = 0x88
    y, h, _ = oracle.moe_ffn(ex, x, ids, w, want_h=True)
    assert np.all(h == 0) and np.all(y == 0)


def test_moe_slot_permutation_and_linearity(oracle):
    ex, x, ids, w = _moe_case()
    y, _, nrm = oracle.moe_ffn(ex, x, ids, w)
    perm = [2, 0, 1]
    yp, _, _ = oracle.moe_ffn(ex, x, ids[:, perm], w[:, perm])
    assert np.all(np.abs(yp - y) <= 1e-14 * nrm)
    y2, _, _ = oracle.moe_ffn(ex, x, ids, (2 * w).astype(np.float32))
    assert np.all(np.abs(y2 - 2 * y) <= 1e-14 * nrm)


def test_moe_tokens_independent(oracle):
    ex, x, ids, w = _moe_case()
    y, _, nrm = oracle.moe_ffn(ex, x, ids, w)
    ids2 = ids.copy()
    ids2[1] = (ids2[1] + 1) % ex["n_experts"]
    y2, _, _ = oracle.moe_ffn(ex, x, ids2, w)
    assert np.array_equal(y2[0], y[0]) and np.array_equal(y2[2], y[2])
    assert not np.array_equal(y2[1], y[1])


def test_moe_single_expert_is_one_ffn(oracle):
    ex, x, ids, w = _moe_case(T=1, k=1)
    y, h, _ = oracle.moe_ffn(ex, x, ids, np.ones_like(w), want_h=True)
    e = int(ids[0, 0])
    sub = lambda name: (ex[name + "_q"][e], ex[name + "_s"][e])
    a, _ = oracle.gemv(4, 64, 128, 64, *sub("gate"), x[0])
    b, _ = oracle.gemv(4, 64, 128, 64, *sub("up"), x[0])
    hh = np.array([oracle.silu(v) for v in a]) * b
    assert np.allclose(h[0], hh, rtol=1e-15, atol=0)


def test_moe_duplicate_ids_sum(oracle):
    ex, x, ids, w = _moe_case(T=1, k=2)
    ids[0, 1] = ids[0, 0]
    y, _, nrm = oracle.moe_ffn(ex, x, ids, w)
    y1, _, _ = oracle.moe_ffn(ex, x, ids[:, :1], (w[:, :1] + w[:, 1:]).astype(np.float32))
    assert np.all(np.abs(y - y1) <= 1e-7 * nrm)  # w0 + w1 rounded to fp32 once


def test_moe_out_of_range_id_skipped(oracle):
    ex, x, ids, w = _moe_case(T=1, k=3)
    bad = ids.copy()
    bad[0, 1] = ex["n_experts"] + 5
    y, h, _ = oracle.moe_ffn(ex, x, bad, w, want_h=True)
    keep = [0, 2]
    y2, _, nrm = oracle.moe_ffn(ex, x, ids[:, keep], w[:, keep])
    assert np.all(np.abs(y - y2) <= 1e-14 * nrm) and np.all(h[1] == 0)


def test_moe_bf16_mode_rounds_h(oracle):
    ex, x, ids, w = _moe_case()
    xf = synth.bf16_bits_to_f32(x)
    y0, h0, _ = oracle.moe_ffn(ex, xf, ids, w, want_h=True)
    y1, h1, _ = oracle.moe_ffn(ex, xf, ids, w, flags=ref.BF16_ACT, want_h=True)
    assert np.array_equal(h1, np.vectorize(oracle.round_bf16)(h0))
    assert not np.array_equal(y0, y1)


# ---- the pins catch planted mistakes ----------------------------------------

MUTANTS = {1: "high nibble first", 2: "offset 7", 3: "wrong group index", 4: "silu sign",
           5: "gate/up swapped", 6: "routing list transposed", 7: "routing weight dropped",
           8: "bf16 truncation", 9: "int8 unsigned", 10: "rmsnorm sum for mean", 11: "int3 offset 3",
           12: "normaliser keeps the sign of the routing weight",
           13: "routing weight left out of the normaliser",
           14: "fp32 x not rounded in the bf16 activation mode"}


def test_real_oracle_passes_battery(oracle):
    run_battery(oracle)


@pytest.mark.parametrize("m", sorted(MUTANTS))
def test_mutants_are_caught(tmp_path, m):
    path = str(tmp_path / ("libqmref_m%d.so" % m))
    ref.build(path, mutant=m)
    o = ref.Oracle(path)
    with pytest.raises(AssertionError):
        run_battery(o)
