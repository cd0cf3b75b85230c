"""Independent dense float64 re-statement of the format, used to pin the
oracle (and nothing else).  Written with vectorised numpy and BLAS rather
than the oracle's element loops: weights are expanded to a dense float64
matrix and multiplied with numpy's matmul.

Format (colibri page "Vulkan backend: expert tier + dense + MLA attention on
any Vulkan 1.2 GPU", commit notes on qmatmul.comp and "fmt=4 grouped
scales"): int4 value = nibble - 8, two per byte with the low nibble first,
one fp32 scale per gs consecutive inputs of a row (gs 0 = one per row);
int8 per-row = two's complement with one fp32 scale per row; int3-g64 as
in dense_int3.
"""
import numpy as np


def pack_nibbles(nib):
    """[n][k] nibble values 0..15 -> [n][k/2] bytes, element 2j in the low
    nibble of byte j (the encoding direction of the format)."""
    nib = np.asarray(nib, dtype=np.uint8)
    return (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)


def dense_int4(q, scales, k, gs):
    q = np.asarray(q, dtype=np.uint8)
    n = q.shape[0]
    nib = np.empty((n, k), dtype=np.int64)
    nib[:, 0::2] = q & 0x0F
    nib[:, 1::2] = q >> 4
    vals = nib.astype(np.float64) - 8.0
    s = np.asarray(scales, dtype=np.float32).astype(np.float64).reshape(n, -1)
    if gs:
        cols = np.minimum(np.arange(k) // gs, s.shape[1] - 1)
        smat = s[:, cols]
    else:
        smat = np.repeat(s[:, :1], k, axis=1)
    return vals, smat


def dense_int8(q, scales, k):
    vals = np.asarray(q).view(np.int8).astype(np.float64)
    s = np.asarray(scales, dtype=np.float32).astype(np.float64).reshape(-1, 1)
    return vals, np.repeat(s, k, axis=1)


def dense_int3(q, scales, k):
    """int3-g64 (int3 commit notes of the same page): per 64-group 24 bytes,
    four little-endian 32-bit words of 2-bit low parts (value i at bits
    2 (i % 16) of word i // 16), then a little-endian 64-bit word of high
    bits (value i at bit i); element = value - 4; one scale per group."""
    q = np.asarray(q, dtype=np.uint8)
    n = q.shape[0]
    G = (k + 63) // 64
    b = q.reshape(n, G, 24)
    words = np.ascontiguousarray(b[:, :, :16]).view("<u4").astype(np.uint64)   # [n][G][4]
    high = np.ascontiguousarray(b[:, :, 16:]).view("<u8")[:, :, 0]             # [n][G]
    i = np.arange(64, dtype=np.uint64)
    low = (words[:, :, i // 16] >> (2 * (i % 16))) & 3
    hb = (high[:, :, None] >> i) & 1
    vals = (low | (hb << 2)).astype(np.int64).reshape(n, G * 64)[:, :k] - 4
    s = np.asarray(scales, dtype=np.float32).astype(np.float64).reshape(n, G)
    return vals.astype(np.float64), s[:, np.arange(k) // 64]


def dense(fmt, q, scales, k, gs):
    """(values, per-element scales) as float64 [n][k]."""
    if fmt == 4:
        return dense_int4(q, scales, k, gs)
    if fmt == 5:
        return dense_int3(q, scales, k)
    return dense_int8(q, scales, k)


def gemv(fmt, q, scales, k, gs, x):
    v, s = dense(fmt, q, scales, k, gs)
    W = v * s
    x = np.asarray(x, dtype=np.float64)
    return W @ x, np.abs(W) @ np.abs(x)


def silu(z):
    return z / (1.0 + np.exp(-z))


def moe(ex, x, ids, w, round_h=None):
    """Dense float64 MoE: y_t = sum_j w_tj * D_e (silu(G_e x_t) * (U_e x_t)).

    Returns (y, norm) with norm[t][i] = sum_j |w_tj| * sum_m |D_e[i][m] h_m|,
    the per-output sum of absolute terms of the final contraction (the
    scale the parity bar is measured against).  round_h, when given, is
    applied to each hidden vector before the down projection."""
    H, I, fmt, gs = ex["hidden"], ex["inter"], ex["fmt"], ex["gs"]
    x = np.asarray(x, dtype=np.float64)
    T, k = ids.shape
    y = np.zeros((T, H))
    nrm = np.zeros((T, H))
    for t in range(T):
        for j in range(k):
            e = int(ids[t, j])
            if e < 0 or e >= ex["n_experts"]:
                continue
            G = np.prod(dense(fmt, ex["gate_q"][e], ex["gate_s"][e], H, gs), axis=0)
            U = np.prod(dense(fmt, ex["up_q"][e], ex["up_s"][e], H, gs), axis=0)
            D = np.prod(dense(fmt, ex["down_q"][e], ex["down_s"][e], I, gs), axis=0)
            h = silu(G @ x[t]) * (U @ x[t])
            if round_h is not None:
                h = round_h(h)
            y[t] += float(w[t, j]) * (D @ h)
            nrm[t] += abs(float(w[t, j])) * (np.abs(D) @ np.abs(h))
    return y, nrm
