/*
 * qmref.h -- plain fp64 CPU oracle for the quantized expert GEMV path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, calls or
 * loads this code; only the tests, the package's smoke check and the bench's
 * CPU-baseline leg do.  It shares no code, header, table or constant with the
 * HIP kernels.
 *
 * Every routine evaluates the plain definition of the operation in double
 * precision, in a fixed order, with no blocking or fusion:
 *
 *  - weight decode follows the int4 "nibble - 8 (offset-binary)" decode of the
 *    colibri page "Vulkan backend: expert tier + dense + MLA attention on any
 *    Vulkan 1.2 GPU" (commit note "backend_vulkan.c/.h + shaders/qmatmul.comp")
 *    and its "fmt=4 grouped scales" commit note (one scale per gs consecutive
 *    inputs of a row);
 *  - int8 per-row ("fmt 1") follows the same page's per-row int4/int8 GEMV and
 *    the colibri page "qwen36: Vulkan expert tier, and staged device-local
 *    uploads" (uploads "as fmt 1");
 *  - the fused expert FFN follows the "qmatmul_gate_up.comp" commit note
 *    (hidden = silu(gate(x)) * up(x)) and the K-expert group commit note
 *    (gate_up for K experts, then down, combined by weighted accumulation).
 *
 * All pointers are host pointers.  Return value 0 = ok, -1 = invalid argument
 * (nothing written).
 */
#ifndef QMREF_H
#define QMREF_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* weight formats */
#define QMREF_FMT_INT8_ROW 1 /* int8 two's complement, one fp32 scale per row */
#define QMREF_FMT_INT4 4     /* int4 nibble-8, one fp32 scale per gs inputs   */
#define QMREF_FMT_INT3 5     /* int3 in two bit planes per 64 inputs (24 bytes:
                                four 32-bit words of 2-bit low parts, 16 values
                                each, then one 64-bit word of high bits), value
                                - 4, one fp32 scale per 64 inputs (gs = 64)   */

/* activation dtypes */
#define QMREF_F32 0  /* IEEE binary32                                         */
#define QMREF_BF16 1 /* bfloat16 stored as uint16 (upper half of a binary32)  */
#define QMREF_F64 2  /* IEEE binary64 (gemv / gemm_small only: the input of a
                        projection that follows another step of the chain)  */

/* moe flags */
#define QMREF_BF16_ACT 1 /* prefill-precision mode: round x (if fp32) and the
                            hidden vector h to bf16 (RNE) before use        */

/* Decoded weight value and its scale for element (row, col) of a matrix with
 * `k` inputs per row.  gs == 0 means one group per row (per-row scales).  */
double qmref_weight(int fmt, int k, int gs, const uint8_t *q, const float *scales,
                    int64_t row, int64_t col, double *scale_out);

/* y[n] = sum_g s[n][g] * sum_{k in g} v[n][k] * x[k]   (double)
 * norm[n] = sum_k |v[n][k] * s[n][g(k)] * x[k]|          (double, may be NULL) */
int qmref_gemv(int fmt, int n, int k, int gs, const uint8_t *q, const float *scales,
               const void *x, int x_dtype, double *y, double *norm);

/* Column-batched form: Y[t][:] = W x_t for t < batch; x_t at x + t*ldx elements,
 * y_t at y + t*ldy.                                                           */
int qmref_gemm_small(int fmt, int n, int k, int gs, const uint8_t *q, const float *scales,
                     const void *x, int x_dtype, int batch, int64_t ldx,
                     double *y, int64_t ldy, double *norm);

typedef struct {
  int n_experts, hidden, inter, fmt, gs;
  const uint8_t *gate_q, *up_q, *down_q; /* [E][inter][hidden], [E][inter][hidden], [E][hidden][inter] */
  const float *gate_s, *up_s, *down_s;
} qmref_experts;

/* For every token t and slot j (in order), e = ids[t][j]:
 *   a = G_e x_t ; b = U_e x_t ; h = silu(a) * b ; y_t += w[t][j] * (D_e h).
 * Ids outside [0, n_experts) contribute nothing (the pair is skipped).
 * y:    [n_tokens][hidden]           (overwritten)
 * h:    [n_tokens*top_k][inter] or NULL (the hidden vector actually fed to D)
 * norm: [n_tokens][hidden] or NULL: sum_j |w_tj| * sum_m |d_{e,i,m} h_{tj,m}|   */
int qmref_moe_ffn(const qmref_experts *ex, const void *x, int x_dtype, int n_tokens,
                  const int32_t *ids, const float *w, int top_k, int flags,
                  double *y, double *h, double *norm);

double qmref_silu(double z);

/* RMS normalisation: out[i] = u[i] / sqrt(mean_j u[j]^2 + eps) * g[i], the
 * norm of the q latent between the q_a and q_b projections in the colibri
 * page "Vulkan backend: expert tier + dense + MLA attention on any Vulkan 1.2
 * GPU" (q-prep chain commit note).  The mean is taken over all n entries in
 * index order.  g may be NULL (all ones).  n >= 1, eps >= 0.               */
int qmref_rmsnorm(int n, const double *u, const float *g, double eps, double *out);

/* binary32 -> bfloat16, round to nearest, ties to even; NaN stays a quiet NaN */
uint16_t qmref_f32_to_bf16(float f);
float qmref_bf16_to_f32(uint16_t b);
/* double -> nearest bfloat16 value (ties to even, overflow to inf), as a double */
double qmref_round_bf16(double v);

/* OpenMP thread count for the row loops (results do not depend on it);
 * returns the count in effect.  n <= 0 leaves it unchanged.                 */
int qmref_set_threads(int n);

#ifdef __cplusplus
}
#endif
#endif
