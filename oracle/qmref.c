/*
 * qmref.c -- plain fp64 CPU oracle for the quantized expert GEMV path.
 *
 * TEST INFRASTRUCTURE ONLY: used by the tests, the package smoke check and
 * the bench's CPU-baseline leg, never by the product library.  It shares no
 * code with the HIP kernels.
 *
 * Sources (colibri pull-request pages):
 *  [V] "Vulkan backend: expert tier + dense + MLA attention on any Vulkan 1.2
 *      GPU (successor to #84)":
 *      - commit note "backend_vulkan.c/.h + shaders/qmatmul.comp": int4 is
 *        decoded as nibble - 8 (offset-binary), int8 is a per-row format;
 *      - commit note "qmatmul_gate_up.comp": hidden = silu(gate(x)) * up(x);
 *      - commit note on the K-expert group: gate_up for K experts, then the
 *        down projection, outputs combined by weighted accumulation;
 *      - commit note "fmt=4 grouped scales": one scale per gs consecutive
 *        inputs of a row, applied to the partial dot of that group; the
 *        per-row multiply is skipped;
 *      - the int3 commit notes ("fmt 5"): a 24-byte two-plane group per 64
 *        inputs, the low plane as 16-value words, the high plane shifted so a
 *        word's bits start at bit 0, one scale per group;
 *      - the q-prep chain commit note: an RMS norm of the q latent between
 *        the q_a and q_b projections.
 *  [Q] "qwen36: Vulkan expert tier, and staged device-local uploads": int4-gs64
 *      arrives as fmt 4 / group 64 at half a byte per element; int8 experts
 *      arrive as fmt 1; the take path accumulates each expert output with its
 *      routing weight.
 *
 * Readings where the pages are silent (each listed in the design notes):
 *  - the low nibble of byte j holds element 2j, the high nibble element 2j+1;
 *  - scales are fp32 laid out [row][group], groups run along the inputs and
 *    restart every row, the last group of a row may be shorter (ceil);
 *  - int8 is plain two's complement with no zero point;
 *  - int3: value i of a group sits at bits 2 (i % 16) of the little-endian
 *    low word i / 16 and at bit i of the little-endian high word; the
 *    decoded weight is value - 4 (offset-binary, as int4's nibble - 8);
 *  - the q-latent norm is u / sqrt(mean u^2 + eps) times a per-element
 *    weight;
 *  - the routing weight multiplies each expert's down output and the slots of
 *    a token are summed in slot order with no renormalisation;
 *  - silu(z) = z / (1 + exp(-z)).
 *
 * Accumulation is in double in a fixed order.  Row loops may run on OpenMP
 * threads; every row is computed by one thread in the same order, so results
 * do not depend on the thread count.
 *
 * QMREF_MUTANT (compile-time, tests only) plants one known mistake so the
 * pin tests can show that they catch it.  It is never set in the normal
 * build.
 */
#include "qmref.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#ifndef QMREF_MUTANT
#define QMREF_MUTANT 0
#endif

/* ---- bf16 helpers (IEEE round to nearest even) --------------------------- */

float qmref_bf16_to_f32(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

uint16_t qmref_f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  if ((u & 0x7fffffffu) > 0x7f800000u) /* NaN: keep sign and payload top, force quiet */
    return (uint16_t)((u >> 16) | 0x0040u);
#if QMREF_MUTANT == 8
  return (uint16_t)(u >> 16); /* mutant: truncation instead of rounding */
#else
  /* add half an ulp of the kept part, plus one if the kept lsb is odd (ties to even) */
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
#endif
}

/* double -> nearest bfloat16 value (ties to even), returned as a double.
 * bf16 keeps 8 significant bits; below 2^-126 the spacing is fixed at 2^-133. */
double qmref_round_bf16(double v) {
  if (v != v || v == 0.0 || isinf(v)) return v;
  double a = fabs(v);
  double r;
  if (a < ldexp(1.0, -126)) {
    r = nearbyint(ldexp(a, 133)) * ldexp(1.0, -133);
  } else {
    int e;
    double m = frexp(a, &e); /* a = m * 2^e, m in [0.5, 1) */
    r = ldexp(nearbyint(ldexp(m, 8)), e - 8);
    /* largest finite bf16 is (2 - 2^-7) * 2^127; anything that rounds past it is inf */
    if (r > ldexp(255.0, 120)) r = INFINITY;
  }
  return v < 0 ? -r : r;
}

double qmref_silu(double z) {
#if QMREF_MUTANT == 4
  return z / (1.0 + exp(z)); /* mutant: sign error in the sigmoid */
#else
  return z / (1.0 + exp(-z));
#endif
}

int qmref_rmsnorm(int n, const double *u, const float *g, double eps, double *out) {
  if (n < 1 || !u || !out || !(eps >= 0)) return -1;
  double ss = 0.0;
  for (int i = 0; i < n; ++i) ss += u[i] * u[i];
#if QMREF_MUTANT == 10
  const double r = 1.0 / sqrt(ss + eps); /* mutant: sum instead of mean */
#else
  const double r = 1.0 / sqrt(ss / n + eps);
#endif
  for (int i = 0; i < n; ++i) out[i] = u[i] * r * (g ? (double)g[i] : 1.0);
  return 0;
}

int qmref_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
  return omp_get_max_threads();
#else
  (void)n;
  return 1;
#endif
}

/* ---- weight decode -------------------------------------------------------- */

static int64_t row_bytes(int fmt, int k) {
  if (fmt == QMREF_FMT_INT3) return ((int64_t)k + 63) / 64 * 24;
  return fmt == QMREF_FMT_INT4 ? (int64_t)k / 2 : (int64_t)k;
}

static int64_t n_groups(int fmt, int k, int gs) {
  if (fmt == QMREF_FMT_INT3) return ((int64_t)k + 63) / 64;
  if (fmt != QMREF_FMT_INT4 || gs <= 0) return 1;
  return ((int64_t)k + gs - 1) / gs;
}

/* little-endian reads, independent of the host's byte order */
static uint64_t le_bytes(const uint8_t *p, int n) {
  uint64_t v = 0;
  for (int i = n - 1; i >= 0; --i) v = (v << 8) | p[i];
  return v;
}

double qmref_weight(int fmt, int k, int gs, const uint8_t *q, const float *scales,
                    int64_t row, int64_t col, double *scale_out) {
  const uint8_t *r = q + row * row_bytes(fmt, k);
  double v;
  int64_t g = 0;
  if (fmt == QMREF_FMT_INT3) {
    /* group g = col / 64 occupies bytes [24 g, 24 g + 24) of the row: low
     * parts of values 16 j .. 16 j + 15 in the 32-bit word j (value i at bits
     * 2 (i % 16), 2 (i % 16) + 1), high bits of values 0..63 in the 64-bit word
     * at byte 16 (value i at bit i) */
    const uint8_t *grp = r + (col / 64) * 24;
    const int i = (int)(col % 64);
    const int lo = (int)((le_bytes(grp + 4 * (i / 16), 4) >> (2 * (i % 16))) & 3u);
    const int hi = (int)((le_bytes(grp + 16, 8) >> i) & 1u);
#if QMREF_MUTANT == 11
    v = (double)((lo | (hi << 2)) - 3); /* mutant: wrong int3 offset */
#else
    v = (double)((lo | (hi << 2)) - 4);
#endif
    g = col / 64;
  } else if (fmt == QMREF_FMT_INT4) {
    uint8_t byte = r[col >> 1];
#if QMREF_MUTANT == 1
    int nib = (col & 1) ? (byte & 0xF) : (byte >> 4); /* mutant: high nibble first */
#else
    int nib = (col & 1) ? (byte >> 4) : (byte & 0xF); /* low nibble = even element */
#endif
#if QMREF_MUTANT == 2
    v = (double)(nib - 7); /* mutant: wrong offset */
#else
    v = (double)(nib - 8); /* offset-binary: nibble - 8 in [-8, 7] */
#endif
    if (gs > 0) g = col / gs;
#if QMREF_MUTANT == 3
    if (gs > 0) g = col % n_groups(fmt, k, gs); /* mutant: wrong group index */
#endif
  } else {
#if QMREF_MUTANT == 9
    v = (double)r[col]; /* mutant: int8 read as unsigned */
#else
    v = (double)(int8_t)r[col];
#endif
  }
  if (scale_out) *scale_out = (double)scales[row * n_groups(fmt, k, gs) + g];
  return v;
}

/* y[n] = sum over groups g of s[n][g] * (sum over k in g of v[n][k] * x[k]) */
static void gemv_d(int fmt, int n, int k, int gs, const uint8_t *q, const float *scales,
                   const double *x, double *y, double *norm) {
  int64_t G = n_groups(fmt, k, gs);
  int64_t glen = fmt == QMREF_FMT_INT3 ? 64 : ((fmt == QMREF_FMT_INT4 && gs > 0) ? gs : k);
#ifdef _OPENMP
#pragma omp parallel for schedule(static)
#endif
  for (int64_t row = 0; row < n; ++row) {
    double acc = 0.0, nrm = 0.0;
    for (int64_t g = 0; g < G; ++g) {
      int64_t k0 = g * glen, k1 = k0 + glen < k ? k0 + glen : k;
      double part = 0.0, s = 0.0;
      for (int64_t c = k0; c < k1; ++c) {
        double v = qmref_weight(fmt, k, gs, q, scales, row, c, &s);
        part += v * x[c];
        nrm += fabs(v * s * x[c]);
      }
      if (k1 > k0) acc += s * part;
    }
    y[row] = acc;
    if (norm) norm[row] = nrm;
  }
}

static int check_mat(int fmt, int n, int k, int gs, const void *q, const float *scales) {
  if (fmt != QMREF_FMT_INT4 && fmt != QMREF_FMT_INT8_ROW && fmt != QMREF_FMT_INT3) return -1;
  if (n < 0 || k < 0 || gs < 0) return -1;
  if (fmt == QMREF_FMT_INT3 && gs != 64) return -1;
  if (fmt == QMREF_FMT_INT4 && (k & 1)) return -1;
  if ((n > 0 && k > 0) && (!q || !scales)) return -1;
  return 0;
}

static double x_at(const void *x, int dt, int64_t i) {
  if (dt == QMREF_BF16) return (double)qmref_bf16_to_f32(((const uint16_t *)x)[i]);
  if (dt == QMREF_F64) return ((const double *)x)[i];
  return (double)((const float *)x)[i];
}

int qmref_gemm_small(int fmt, int n, int k, int gs, const uint8_t *q, const float *scales,
                     const void *x, int x_dtype, int batch, int64_t ldx,
                     double *y, int64_t ldy, double *norm) {
  if (check_mat(fmt, n, k, gs, q, scales)) return -1;
  if (x_dtype != QMREF_F32 && x_dtype != QMREF_BF16 && x_dtype != QMREF_F64) return -1;
  if (batch < 0 || ldx < k || ldy < n || !y || (k > 0 && batch > 0 && !x)) return -1;
  double *xd = (double *)malloc(sizeof(double) * (size_t)(k > 0 ? k : 1));
  if (!xd) return -1;
  for (int t = 0; t < batch; ++t) {
    for (int64_t c = 0; c < k; ++c) xd[c] = x_at(x, x_dtype, t * ldx + c);
    gemv_d(fmt, n, k, gs, q, scales, xd, y + t * ldy, norm ? norm + t * ldy : NULL);
  }
  free(xd);
  return 0;
}

int qmref_gemv(int fmt, int n, int k, int gs, const uint8_t *q, const float *scales,
               const void *x, int x_dtype, double *y, double *norm) {
  return qmref_gemm_small(fmt, n, k, gs, q, scales, x, x_dtype, 1, k, y, n, norm);
}

/* ---- fused expert FFN over the routed experts ----------------------------- */

int qmref_moe_ffn(const qmref_experts *ex, const void *x, int x_dtype, int n_tokens,
                  const int32_t *ids, const float *w, int top_k, int flags,
                  double *y, double *h, double *norm) {
  if (!ex || n_tokens < 0 || top_k < 1 || !y) return -1;
  int H = ex->hidden, I = ex->inter, E = ex->n_experts, fmt = ex->fmt, gs = ex->gs;
  if (E < 0 || check_mat(fmt, I, H, gs, ex->gate_q, ex->gate_s) ||
      check_mat(fmt, I, H, gs, ex->up_q, ex->up_s) ||
      check_mat(fmt, H, I, gs, ex->down_q, ex->down_s))
    return -1;
  if (x_dtype != QMREF_F32 && x_dtype != QMREF_BF16) return -1;
  if (n_tokens > 0 && (!x || !ids || !w)) return -1;

  int64_t gate_rows_bytes = (int64_t)I * row_bytes(fmt, H);
  int64_t down_rows_bytes = (int64_t)H * row_bytes(fmt, I);
  int64_t gate_scales = (int64_t)I * n_groups(fmt, H, gs);
  int64_t down_scales = (int64_t)H * n_groups(fmt, I, gs);

  double *xt = (double *)malloc(sizeof(double) * (size_t)(H > 0 ? H : 1));
  double *a = (double *)malloc(sizeof(double) * (size_t)(I > 0 ? I : 1));
  double *b = (double *)malloc(sizeof(double) * (size_t)(I > 0 ? I : 1));
  double *hv = (double *)malloc(sizeof(double) * (size_t)(I > 0 ? I : 1));
  double *o = (double *)malloc(sizeof(double) * (size_t)(H > 0 ? H : 1));
  double *on = (double *)malloc(sizeof(double) * (size_t)(H > 0 ? H : 1));
  if (!xt || !a || !b || !hv || !o || !on) {
    free(xt); free(a); free(b); free(hv); free(o); free(on);
    return -1;
  }

  for (int t = 0; t < n_tokens; ++t) {
    double *yt = y + (int64_t)t * H;
    double *nt = norm ? norm + (int64_t)t * H : NULL;
    for (int i = 0; i < H; ++i) {
      yt[i] = 0.0;
      if (nt) nt[i] = 0.0;
    }
    for (int c = 0; c < H; ++c) {
      double v = x_at(x, x_dtype, (int64_t)t * H + c);
#if QMREF_MUTANT != 14 /* mutant 14: fp32 x not rounded in the bf16 activation mode */
      if ((flags & QMREF_BF16_ACT) && x_dtype == QMREF_F32) v = qmref_round_bf16(v);
#endif
      xt[c] = v;
    }
    for (int j = 0; j < top_k; ++j) {
#if QMREF_MUTANT == 6
      int64_t p = (int64_t)j * n_tokens + t; /* mutant: routing list read transposed */
#else
      int64_t p = (int64_t)t * top_k + j;
#endif
      int e = ids[p];
      double wt = (double)w[p];
      double *hp = h ? h + p * I : NULL;
      if (e < 0 || e >= E) { /* out-of-range id: the pair contributes nothing */
        if (hp)
          for (int i = 0; i < I; ++i) hp[i] = 0.0;
        continue;
      }
      gemv_d(fmt, I, H, gs, ex->gate_q + e * gate_rows_bytes, ex->gate_s + e * gate_scales, xt, a, NULL);
      gemv_d(fmt, I, H, gs, ex->up_q + e * gate_rows_bytes, ex->up_s + e * gate_scales, xt, b, NULL);
      for (int i = 0; i < I; ++i) {
#if QMREF_MUTANT == 5
        double v = qmref_silu(b[i]) * a[i]; /* mutant: gate and up swapped */
#else
        double v = qmref_silu(a[i]) * b[i];
#endif
        if (flags & QMREF_BF16_ACT) v = qmref_round_bf16(v);
        hv[i] = v;
        if (hp) hp[i] = v;
      }
      gemv_d(fmt, H, I, gs, ex->down_q + e * down_rows_bytes, ex->down_s + e * down_scales, hv, o, on);
      for (int i = 0; i < H; ++i) {
#if QMREF_MUTANT == 7
        yt[i] += o[i]; /* mutant: routing weight dropped */
#else
        yt[i] += wt * o[i];
#endif
#if QMREF_MUTANT == 12
        if (nt) nt[i] += wt * on[i]; /* mutant: sign of the routing weight kept */
#elif QMREF_MUTANT == 13
        if (nt) nt[i] += on[i]; /* mutant: routing weight left out of the normaliser */
#else
        if (nt) nt[i] += fabs(wt) * on[i];
#endif
      }
    }
  }
  free(xt); free(a); free(b); free(hv); free(o); free(on);
  return 0;
}
