/*
 * qmoe.h -- C ABI of libqmoe.so: int4/int8 quantized GEMV, small-batch GEMV
 * and the routed MoE expert FFN on an MI355X (gfx950) GPU.
 *
 * Sources (colibri pull-request pages):
 *  [V] "Vulkan backend: expert tier + dense + MLA attention on any Vulkan 1.2
 *      GPU (successor to #84)" -- commit notes "backend_vulkan.c/.h +
 *      shaders/qmatmul.comp" (int4 nibble-8 and int8 per-row GEMV with an
 *      S-token batch), "qmatmul_gate_up.comp" (fused silu(gate x) * up x),
 *      the K-expert group note (gate_up for K experts, one barrier, down,
 *      hidden kept on the device), "fmt=4 grouped scales" (one scale per gs
 *      inputs of a row), and the PR summary (batch-union prefill touches
 *      nearly every expert; a cooperative-matrix prefill is future work).
 *  [Q] "qwen36: Vulkan expert tier, and staged device-local uploads" --
 *      int4-gs64 as fmt 4 / group 64, int8 experts as fmt 1, and the
 *      issue/take path accumulating expert outputs with their routing weights.
 *
 * Conventions shared by every entry point
 *  - Pointers marked "device" are HIP device pointers; the caller owns every
 *    buffer (weights, activations, outputs, workspace).  The library keeps no
 *    pointer after a call returns and allocates nothing.  Its only global
 *    state is, per device, the compute-unit count (looked up once, kept in
 *    an atomic) and the address of moe_expert_ffn_noalloc's scratch array
 *    (looked up once under a mutex), so calls are reentrant.  Two calls must
 *    not share one workspace while both are in flight (on different
 *    streams), as for any scratch buffer.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Calls only enqueue work and return; results are ready when the stream
 *    reaches them.  Time them with events on that stream.
 *  - Arguments are validated on the host before any HIP call.  A negative
 *    status means nothing was enqueued and no output byte was written.
 *    QM_ERR_LAUNCH means a HIP launch failed after validation; outputs are
 *    then unspecified.
 *  - Outputs are overwritten, never accumulated into.
 *
 * Weight formats (the layouts the kernels read directly; no repacking)
 *  - QM_FMT_INT4: element (r, c) of an n x k matrix is nibble(r, c) - 8 with
 *    nibble(r, c) = (q[r*k/2 + c/2] >> (4*(c&1))) & 15, i.e. two per byte,
 *    low nibble first [V: qmatmul.comp note; reading: low nibble = even
 *    element].  Scales are fp32 [n][k/gs] row-major, one per gs consecutive
 *    inputs of a row [V: fmt=4 note]; group_size 0 (or k) means one scale per
 *    row ([n] floats).  gs must be a multiple of 32 that divides k.
 *  - QM_FMT_INT8_ROW: element (r, c) = (int8_t)q[r*k + c] times scale[r]
 *    (two's complement, no zero point) [V: qmatmul.comp note, Q: fmt 1].
 *    group_size must be 0.
 *  - QM_FMT_INT3 (int3-g64, two bit planes): each 64 inputs of a row take 24
 *    bytes -- four 32-bit words of 2-bit low parts (16 values per word), then
 *    a 64-bit word of high bits -- with one fp32 scale per group, [n][ceil(k/64)]
 *    [V: the int3 commit notes, 24 bytes per 64-group].  Reading of the bit
 *    order: value i of a group at bits 2 (i % 16) of little-endian low word
 *    i / 16 and at bit i of the little-endian high word; element = value - 4.
 *    Rows are ceil(k/64) * 24 bytes (a ragged last group is padded).
 *    group_size must be 64; k a multiple of 32, k <= 16384.  qgemv,
 *    qgemv_pair, qgemm_small (any batch) and the expert FFN take it: the
 *    kernels are the int4 ones, each value turned into a signed nibble
 *    (element = lo + 4 hb - 4) as it is loaded, so int3 has the int4
 *    arithmetic and limits.  The expert FFN runs it on its decode kernels
 *    for any number of tokens; it has no prefill kernels (QM_PATH_PREFILL
 *    gives QM_ERR_UNSUPPORTED) [V: int3 commit notes, int3 expert matmuls
 *    and fused gate_up].
 *  Value = element * its scale.
 *
 * Arithmetic.  The int4, int3 and int8 kernels apply the weights with integer dot
 * products (eight int4 or four int8 products per instruction) to activations
 * written as stacked 15-bit integer "digit planes": each group of 32 (int4) or
 * 16 (int8) activations shares a power-of-two exponent, and a call uses as
 * many planes as its widest group needs so that every activation is exact
 * (bf16 input) or within 2^-15 of itself (fp32 input, and the expert FFN's
 * fp32 hidden vector, in groups of 16).  The error of an output is therefore
 * at most 2^-15 * sum_k |w_k x_k| plus fp32 accumulation, for any finite
 * input: a large activation beside small ones costs more planes (more
 * work), not accuracy.  Typical activations need two planes.  The prefill
 * kernels (bf16 MFMA) use floating-point products instead (see
 * moe_expert_ffn).
 *
 * Shape limits of the GPU path (QM_ERR_UNSUPPORTED otherwise): int4 needs
 * k % 32 == 0, int8 needs k % 16 == 0; 1 <= k <= QM_K_MAX; q and x must be
 * 16-byte aligned, scales/y 4-byte aligned.  n == 0 is a no-op.
 */
#ifndef QMOE_H
#define QMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define QM_API __attribute__((visibility("default")))
#else
#define QM_API
#endif

typedef enum {
  QM_OK = 0,
  QM_ERR_INVALID = -1,     /* malformed argument: null pointer, negative size, bad enum */
  QM_ERR_UNSUPPORTED = -2, /* well-formed but outside what the GPU path implements */
  QM_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required */
  QM_ERR_LAUNCH = -4,      /* a HIP launch failed */
  QM_ERR_TOO_LARGE = -5    /* needs more scratch than moe_expert_ffn_noalloc holds */
} qm_status;

typedef enum { QM_FMT_INT8_ROW = 1, QM_FMT_INT4 = 4, QM_FMT_INT3 = 5 } qm_fmt;
typedef enum { QM_F32 = 0, QM_BF16 = 1 } qm_dtype;

enum {
  QM_SMALL_MAX = 8,           /* largest batch of qgemm_small                       */
  QM_TOPK_MAX = 32,           /* largest top_k of moe_expert_ffn                    */
  QM_DECODE_MAX_TOKENS = 8,   /* moe_expert_ffn runs the decode kernels up to this  */
  QM_K_MAX = 1 << 20,         /* largest reduction length                           */
  QM_NOALLOC_SCRATCH_BYTES = 32 << 20  /* fixed scratch of moe_expert_ffn_noalloc, per GPU */
};

/* which kernels moe_expert_ffn_path runs */
enum { QM_PATH_AUTO = 0, QM_PATH_DECODE = 1, QM_PATH_PREFILL = 2 };

/* A quantized n x k matrix resident on the device. */
typedef struct {
  int32_t fmt;        /* qm_fmt                                                */
  int32_t n, k;       /* outputs (rows), inputs per row                        */
  int32_t group_size; /* int4: 0 (= per row), k, or a multiple of 32 dividing k */
  const void *q;      /* device: int4 n*k/2 bytes, int8 n*k bytes, row-major   */
  const float *scales;/* device: int4 n*(k/gs) (or n) fp32, int8 n fp32       */
} qm_qmat;

/* E experts stacked expert-major, all in one format and group size.
 *   gate_q, up_q: [E][inter][hidden] elements (int4: hidden/2 bytes per row)
 *   down_q:       [E][hidden][inter] elements (int4: inter/2 bytes per row)
 *   gate_s, up_s: [E][inter][hidden/gs] fp32 (gs 0: [E][inter])
 *   down_s:       [E][hidden][inter/gs] fp32 (gs 0: [E][hidden])           */
typedef struct {
  int32_t n_experts, hidden, inter, fmt, group_size;
  const void *gate_q, *up_q, *down_q;  /* device */
  const float *gate_s, *up_s, *down_s; /* device */
} qm_experts;

/* y[r] = sum_c W[r][c] * x[c], r < w->n.
 * [V: qmatmul.comp note -- the dense quantized GEMV, one token]
 * x: device, k elements of x_dtype.  y: device, n fp32 (overwritten).    */
QM_API int qgemv(const qm_qmat *w, const void *x, int32_t x_dtype, float *y, void *stream);

/* Two projections of one x: y1 = W1 x and y2 = W2 x (W1, W2 with the same k).
 * [V: PR summary, dense tier -- the two attention-input projections of one
 * x share a submission (the matmul_pair path)]  With the same format and
 * grouping (int4 or int8) both run in one launch (x staged once per
 * workgroup); otherwise as two launches on the stream.  x: device, k
 * elements.
 * y1, y2: device, w1->n and w2->n fp32 (overwritten, must not overlap).
 * Both matrices are validated before anything is enqueued.                  */
QM_API int qgemv_pair(const qm_qmat *w1, const qm_qmat *w2, const void *x, int32_t x_dtype, float *y1, float *y2,
                      void *stream);

/* The q-prep chain: u = W_a x and kv = W_kv x (one qgemv_pair launch), then
 * u is RMS-normalised in place, u[i] <- u[i] / sqrt(mean u^2 + eps) * g[i],
 * then q = W_b u -- three launches on the stream and no host
 * synchronisation.  [V: the q-prep chain commit note -- q_a + kv_a, the
 * latent norm and q_b recorded as one GPU sequence]
 * w_kv->k == w_a->k, w_b->k == w_a->n >= 1.  x: device, w_a->k elements of
 * x_dtype.  u: device fp32 [w_a->n], 16-byte aligned (receives the
 * normalised latent; it is also q_b's input).  kv: device fp32 [w_kv->n].
 * q: device fp32 [w_b->n].  norm_w: device fp32 [w_a->n], or NULL for ones.
 * eps >= 0.  All three matrices are validated before anything is enqueued. */
QM_API int qgemv_norm_chain(const qm_qmat *w_a, const qm_qmat *w_kv, const float *norm_w, float eps,
                            const qm_qmat *w_b, const void *x, int32_t x_dtype, float *u, float *kv, float *q,
                            void *stream);

/* Y[t][r] = sum_c W[r][c] * X[t][c] for t < batch, reading W once for all
 * t (int4, int3 and int8).
 * [V: qmatmul.comp note -- the S-token batch of the same GEMV]
 * x: device [batch][ldx] (ldx >= k, ldx*elemsize a multiple of 16 bytes).
 * y: device [batch][ldy] fp32 (ldy >= n).  1 <= batch <= QM_SMALL_MAX.     */
QM_API int qgemm_small(const qm_qmat *w, const void *x, int32_t x_dtype, int32_t batch, int64_t ldx,
                float *y, int64_t ldy, void *stream);

/* Bytes of device workspace moe_expert_ffn needs for these sizes (covers
 * every kernel path moe_expert_ffn_path may take for them).  0 on invalid
 * arguments. */
QM_API size_t moe_expert_ffn_workspace(const qm_experts *ex, int32_t n_tokens, int32_t top_k);

/* Routed expert FFN.  For each token t and slot j < top_k, with
 * e = topk_ids[t][j]:  h = silu(G_e x_t) * (U_e x_t)  and
 *   y_t = sum_j topk_w[t][j] * (D_e h),  summed in slot order.
 * [V: qmatmul_gate_up.comp note and the K-expert group note; Q: weighted
 *  accumulation of the expert outputs; silu(z) = z / (1 + e^-z)]
 * Gate weights are used as given (no renormalisation).  Decode: within one
 * pass of tokens (all of a decode batch whose activations fit the kernels'
 * LDS: up to 8 tokens at hidden 4608, 5 at 6144) each routed expert's gate
 * and up rows are read once for all tokens routed to it, and its down rows
 * are streamed by adjacent waves so that the second token's read hits the
 * cache.
 * Ids outside [0, n_experts) are skipped (the pair contributes nothing);
 * the same id twice in one token is summed.
 * x:         device [n_tokens][hidden] of x_dtype (16-byte aligned rows)
 * topk_ids:  device int32 [n_tokens][top_k];  topk_w: device fp32 [n_tokens][top_k]
 * y:         device fp32 [n_tokens][hidden] (overwritten)
 * workspace: device, >= moe_expert_ffn_workspace(ex, n_tokens, top_k) bytes,
 *            256-byte aligned; its contents are scratch (not preserved).
 * n_tokens <= QM_DECODE_MAX_TOKENS runs the decode kernels (fp32 hidden
 * vector as digit planes) in passes of as many tokens as fit their LDS;
 * larger batches run the expert-grouped prefill kernels (bf16 MFMA, hidden
 * vector and fp32 activations rounded to bf16) when the experts qualify --
 * int4 with a group size (or, per row, a row length) that is a multiple of
 * 64 (grouped: a multiple of 4 groups per row, with 16-byte aligned scale
 * arrays), hidden % 512 == 0, inter % 256 == 0, n_experts <= 8192 -- and
 * otherwise the decode kernels pass by pass.  The decode kernels take
 * hidden up to 16384 (int4; 8192 int8) and inter up to 4096 (int4; 2048
 * int8; int3 as int4); other shapes return QM_ERR_UNSUPPORTED.  int3-g64
 * experts always run the decode kernels (pass by pass for large batches).  */
QM_API int moe_expert_ffn(const qm_experts *ex, const void *x, int32_t x_dtype, int32_t n_tokens,
                   const int32_t *topk_ids, const float *topk_w, int32_t top_k,
                   float *y, void *workspace, size_t workspace_bytes, void *stream);

/* moe_expert_ffn with the kernel path chosen by the caller: QM_PATH_AUTO,
 * QM_PATH_DECODE (any n_tokens, in passes of a few tokens) or
 * QM_PATH_PREFILL (any n_tokens; QM_ERR_UNSUPPORTED for experts the
 * prefill kernels do not take, see moe_expert_ffn).                        */
QM_API int moe_expert_ffn_path(const qm_experts *ex, const void *x, int32_t x_dtype, int32_t n_tokens,
                        const int32_t *topk_ids, const float *topk_w, int32_t top_k,
                        float *y, void *workspace, size_t workspace_bytes, void *stream,
                        int32_t path);

/* Stage 1 of the decode path on its own (the fused gate+up dispatch of the
 * "qmatmul_gate_up.comp" commit note [V]): for every pair p = t*top_k + j
 * with a valid id e, h[p][:] = silu(G_e x_t) * (U_e x_t).  Rows of pairs with
 * an invalid id are not written.  Any n_tokens, in the decode passes
 * moe_expert_ffn uses (a few tokens per launch; each expert's weights are
 * read once per pass for all of that pass's tokens routed to it).
 * h: device fp32 [n_tokens*top_k][inter], 4-byte aligned.
 * workspace as for moe_expert_ffn (scratch for activations that need more
 * than two digit planes).                                                   */
QM_API int moe_gate_up(const qm_experts *ex, const void *x, int32_t x_dtype, int32_t n_tokens,
                       const int32_t *topk_ids, int32_t top_k, float *h, void *workspace, size_t workspace_bytes,
                       void *stream);

/* Stage 2 of the decode path on its own: y_t = sum_j topk_w[t][j] *
 * (D_e h[t*top_k + j]) in slot order, from the hidden rows that moe_gate_up
 * wrote.  h: device fp32 [n_tokens*top_k][inter], 16-byte aligned;
 * workspace as for moe_expert_ffn.  moe_gate_up followed by moe_down on one
 * stream computes exactly what moe_expert_ffn computes for these sizes.    */
QM_API int moe_down(const qm_experts *ex, const float *h, int32_t n_tokens, const int32_t *topk_ids,
                    const float *topk_w, int32_t top_k, float *y, void *workspace, size_t workspace_bytes,
                    void *stream);

/* moe_expert_ffn for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments and results as moe_expert_ffn without the workspace: the
 * scratch it needs comes from a fixed device array of
 * QM_NOALLOC_SCRATCH_BYTES inside the library, one copy per GPU, held until
 * the process ends.  Nothing is allocated by the call (no hipMalloc, no
 * allocating library routine); the array's device address is looked up once
 * per GPU on the first call made with that GPU current.  A call that needs
 * more scratch than that (moe_expert_ffn_workspace() > the limit: large
 * prefill batches) returns QM_ERR_TOO_LARGE before anything is enqueued.
 * Every call on a GPU uses that GPU's one array, whose contents carry over
 * from the previous call: calls that can overlap on one GPU (several
 * streams, several host threads) race on it and must be serialised by the
 * caller.  Nothing in the array needs to start at zero.                    */
QM_API int moe_expert_ffn_noalloc(const qm_experts *ex, const void *x, int32_t x_dtype, int32_t n_tokens,
                                  const int32_t *topk_ids, const float *topk_w, int32_t top_k, float *y,
                                  void *stream);

/* Static text for a qm_status value. */
QM_API const char *qm_strerror(int status);

/* ---- packing, validation and quantization (host memory, no GPU) ----------
 * Weights in the layouts above, made on the host before the upload [Q:
 * int4-gs64 arriving as fmt 4 / group 64 at half a byte per element; V:
 * fmt=4 grouped scales].  All buffers are host memory owned by the caller;
 * nothing is allocated; QM_ERR_INVALID (nothing written) for a null pointer,
 * n < 0, k <= 0 or a value the format cannot hold.
 *
 * qm_pack_int4: v [n][k] int8 values in [-8, 7] (row-major) -> q [n][k/2]
 *   bytes, nibble = v + 8, even element in the low nibble.  k must be even.
 * qm_pack_int8: v [n][k] -> q [n][k] (the values themselves; q may be v).
 * qm_validate: checks a format's shape rules and that its scales
 *   ([n][groups] fp32, groups as in "Weight formats") are all finite; any
 *   int4/int8/int3 code byte is valid, so the codes are not read.
 * qm_quantize_int4: fp32 w [n][k] -> q [n][k/2] and scales [n][k/gs]
 *   (group_size 0 or k: [n]): per group s = max|w| / 7, code = clamp(
 *   round-half-even(w / s), -8, 7) (all codes 0 where s = 0).  w must be finite.
 * qm_quantize_int8: fp32 w [n][k] -> q [n][k], scales [n]: per row s =
 *   max|w| / 127, code = clamp(round-half-even(w / s), -127, 127).
 * (The quantizers are one plain rounding scheme; the kernels take any codes
 * and scales.) */
QM_API int qm_pack_int4(const int8_t *v, int64_t n, int64_t k, uint8_t *q);
QM_API int qm_pack_int8(const int8_t *v, int64_t n, int64_t k, int8_t *q);
QM_API int qm_validate(int32_t fmt, int64_t n, int64_t k, int32_t group_size, const float *scales);
QM_API int qm_quantize_int4(const float *w, int64_t n, int64_t k, int32_t group_size, uint8_t *q, float *scales);
QM_API int qm_quantize_int8(const float *w, int64_t n, int64_t k, int8_t *q, float *scales);

#ifdef __cplusplus
}
#endif
#endif
