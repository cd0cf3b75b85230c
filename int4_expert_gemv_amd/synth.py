"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module draws random numbers and nothing else: it holds none of the
method's arithmetic (no decode, no dot products, no activation).  Packed int4
weights are drawn as uniform random bytes, which is the same as two
independent uniform nibbles per byte, so no packing is done here either.
bf16 activations are fp32 draws rounded by torch's own conversion.

Every tensor of an expert set comes from its own PCG64 stream keyed by
(seed, tensor, expert), so any single expert can be regenerated without
drawing the others, and a large stack can be drawn on several threads.
"""
import concurrent.futures

import numpy as np
import torch

FMT_INT8_ROW = 1
FMT_INT4 = 4
FMT_INT3 = 5

_T_GATE, _T_UP, _T_DOWN = 1, 2, 3
_T_Q, _T_S = 0, 1


def rng(*key):
    return np.random.default_rng(list(key))


def n_groups(k, gs):
    """Scale groups per row: gs 0 (or None) means one scale per row."""
    return 1 if not gs else -(-k // gs)


def quant_matrix(g, fmt, n, k, gs, scale_lo=0.005, scale_hi=0.02):
    """(q, scales) for an n x k matrix: int4 -> uint8 [n][k/2] uniform bytes;
    int8 -> int8 [n][k] uniform in [-127, 127].  Scales U(lo, hi) fp32."""
    if fmt == FMT_INT4:
        q = g.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
        s = uniform_f32(g, (n, n_groups(k, gs)), scale_lo, scale_hi)
    elif fmt == FMT_INT8_ROW:
        q = g.integers(-127, 128, size=(n, k), dtype=np.int8)
        s = uniform_f32(g, (n, 1), scale_lo, scale_hi)
    elif fmt == FMT_INT3:  # any bit pattern is a valid int3 group (24 bytes per 64 inputs)
        ng = (k + 63) // 64
        q = g.integers(0, 256, size=(n, ng * 24), dtype=np.uint8)
        s = uniform_f32(g, (n, ng), scale_lo, scale_hi)
    else:
        raise ValueError(fmt)
    return q, s


def uniform_f32(g, shape, lo, hi):
    """fp32 draws in [lo, hi)."""
    return g.random(size=shape, dtype=np.float32) * np.float32(hi - lo) + np.float32(lo)


def normal_f32(g, shape):
    return g.standard_normal(size=shape, dtype=np.float32)


def to_bf16_bits(a):
    """fp32 array -> uint16 bf16 bit patterns, rounded by torch's conversion."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(b):
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def activations(g, shape, dtype):
    """N(0,1) activations, as fp32 or as bf16 bits ('bf16')."""
    x = normal_f32(g, shape)
    return to_bf16_bits(x) if dtype == "bf16" else x


def small_int_activations(g, shape, dtype, lo=-4, hi=4):
    """Integer-valued activations in [lo, hi]: exact in fp32 and in bf16."""
    x = g.integers(lo, hi + 1, size=shape).astype(np.float32)
    return to_bf16_bits(x) if dtype == "bf16" else x


def pow2_scales(g, shape, lo_exp=-9, hi_exp=-5):
    """Power-of-two scales 2^e, e uniform in [lo_exp, hi_exp]."""
    e = g.integers(lo_exp, hi_exp + 1, size=shape)
    return np.ldexp(np.ones(shape, np.float32), e).astype(np.float32)


def uniform_routing(g, n_tokens, n_experts, top_k):
    """Per token: top_k distinct expert ids uniform without replacement, and
    gate weights = softmax of top_k N(0,1) logits (float32)."""
    ids = np.stack([g.choice(n_experts, size=top_k, replace=False) for _ in range(n_tokens)])
    logits = g.standard_normal(size=(n_tokens, top_k))
    w = np.exp(logits - logits.max(axis=1, keepdims=True))
    w = w / w.sum(axis=1, keepdims=True)
    return ids.astype(np.int32).reshape(n_tokens, top_k), w.astype(np.float32)


def zipf_routing(g, n_tokens, n_experts, top_k, alpha=1.1):
    """Per token: top_k distinct experts drawn with probability proportional to
    (id + 1)^-alpha, without replacement (Gumbel-top-k), and softmax gate
    weights of N(0,1) logits.  Expert id equals popularity rank."""
    logp = -alpha * np.log(np.arange(1, n_experts + 1, dtype=np.float64))
    gumbel = g.gumbel(size=(n_tokens, n_experts))
    ids = np.argsort(-(logp[None, :] + gumbel), axis=1, kind="stable")[:, :top_k]
    logits = g.standard_normal(size=(n_tokens, top_k))
    w = np.exp(logits - logits.max(axis=1, keepdims=True))
    w = w / w.sum(axis=1, keepdims=True)
    return ids.astype(np.int32), w.astype(np.float32)


# standard deviation of a uniformly drawn code, as the dequantized value
# (code - offset): int4 nibble - 8, int8 in [-127, 127], int3 code - 4
_CODE_STD = {FMT_INT4: float(np.sqrt((16 * 16 - 1) / 12.0)), FMT_INT8_ROW: float(np.sqrt((255 * 255 - 1) / 12.0)),
             FMT_INT3: float(np.sqrt((8 * 8 - 1) / 12.0))}


def scale_range(fmt, k, scales):
    """Scale draw range of an n x k matrix.  "wide": U(0.005, 0.02) whatever
    the shape (with N(0, 1) activations the gate/up pre-activations then have
    a standard deviation of about 4.7 at k = 6144, and SiLU's negative tail
    spreads h over many binades); "unit": U(0.5, 1.5) / (code std sqrt(k)),
    so that a product with N(0, 1) inputs has about unit variance, as the
    normalised layers of a trained model keep them."""
    if scales == "wide":
        return 0.005, 0.02
    if scales == "unit":
        c = 1.0 / (_CODE_STD[fmt] * np.sqrt(k))
        return 0.5 * c, 1.5 * c
    raise ValueError(scales)


def expert_set(seed, fmt, n_experts, hidden, inter, gs, experts=None, threads=1, scales="wide"):
    """Stacked expert weights as a dict (the layout the library and the oracle
    both take).  `experts` limits generation to a subset of ids; the other
    experts' slots are left zero (only valid when routing avoids them).
    `scales`: the scale draw range, see scale_range."""
    if fmt == FMT_INT3:  # 24 bytes and one scale per 64 inputs (gs is 64)
        gs = 64
        G_h, G_i = (hidden + 63) // 64, (inter + 63) // 64
        rb_h, rb_i = G_h * 24, G_i * 24
    else:
        G_h = n_groups(hidden, gs) if fmt == FMT_INT4 else 1
        G_i = n_groups(inter, gs) if fmt == FMT_INT4 else 1
        rb_h = hidden // 2 if fmt == FMT_INT4 else hidden
        rb_i = inter // 2 if fmt == FMT_INT4 else inter
    qdt = np.int8 if fmt == FMT_INT8_ROW else np.uint8
    out = {
        "n_experts": n_experts, "hidden": hidden, "inter": inter, "fmt": fmt,
        "gs": int(gs or 0) if fmt in (FMT_INT4, FMT_INT3) else 0,
        "gate_q": np.zeros((n_experts, inter, rb_h), qdt),
        "up_q": np.zeros((n_experts, inter, rb_h), qdt),
        "down_q": np.zeros((n_experts, hidden, rb_i), qdt),
        "gate_s": np.zeros((n_experts, inter, G_h), np.float32),
        "up_s": np.zeros((n_experts, inter, G_h), np.float32),
        "down_s": np.zeros((n_experts, hidden, G_i), np.float32),
    }
    ids = range(n_experts) if experts is None else sorted(set(int(i) for i in experts if 0 <= i < n_experts))

    def fill(e):
        for tag, name, n, k in ((_T_GATE, "gate", inter, hidden), (_T_UP, "up", inter, hidden),
                                (_T_DOWN, "down", hidden, inter)):
            q, s = quant_matrix(rng(seed, tag, e), fmt, n, k, gs, *scale_range(fmt, k, scales))
            out[name + "_q"][e] = q
            out[name + "_s"][e] = s.reshape(out[name + "_s"][e].shape)

    if threads > 1 and len(ids) > 1:
        with concurrent.futures.ThreadPoolExecutor(threads) as pool:
            list(pool.map(fill, ids))
    else:
        for e in ids:
            fill(e)
    return out
