// pack.cpp -- host-side packing, validation and quantization of weights into
// the layouts the kernels read (include/qmoe.h "Weight formats"): int4 with
// one fp32 scale per group of gs inputs of a row (the "fmt=4 grouped scales"
// note of the colibri page "Vulkan backend: expert tier + dense + MLA
// attention on any Vulkan 1.2 GPU"; int4-gs64 as fmt 4 / group 64 at half a
// byte per element on the page "qwen36: Vulkan expert tier, and staged
// device-local uploads") and int8 with one scale per row (fmt 1 there).
// Plain C++ on host memory: no GPU is needed or touched.
#include <cmath>
#include <cstdint>
#include <cstring>

#include "qmoe.h"

namespace {

// group size checks shared with the GPU entry points: 0 (or k) is one scale
// per row; otherwise a multiple of 32 dividing k
bool int4_groups(int64_t k, int32_t gs, int64_t* groups) {
  if (gs == 0 || gs == k) {
    *groups = 1;
    return true;
  }
  if (gs < 32 || gs % 32 != 0 || k % gs != 0) return false;
  *groups = k / gs;
  return true;
}

bool finite_all(const float* s, int64_t count) {
  for (int64_t i = 0; i < count; ++i)
    if (!std::isfinite(s[i])) return false;
  return true;
}

}  // namespace

extern "C" {

QM_API int qm_pack_int4(const int8_t* v, int64_t n, int64_t k, uint8_t* q) {
  if (!v || !q || n < 0 || k <= 0 || (k & 1)) return QM_ERR_INVALID;
  for (int64_t i = 0; i < n * k; ++i)
    if (v[i] < -8 || v[i] > 7) return QM_ERR_INVALID;
  for (int64_t r = 0; r < n; ++r) {
    const int8_t* vr = v + r * k;
    uint8_t* qr = q + r * (k / 2);
    for (int64_t c = 0; c < k; c += 2)
      qr[c / 2] = (uint8_t)((unsigned)(vr[c] + 8) | ((unsigned)(vr[c + 1] + 8) << 4));
  }
  return QM_OK;
}

QM_API int qm_pack_int8(const int8_t* v, int64_t n, int64_t k, int8_t* q) {
  if (!v || !q || n < 0 || k <= 0) return QM_ERR_INVALID;
  // every int8 value is an element (two's complement, no zero point): the
  // layout is the values themselves, row-major
  if (q != v) std::memmove(q, v, (size_t)(n * k));
  return QM_OK;
}

QM_API int qm_validate(int32_t fmt, int64_t n, int64_t k, int32_t group_size, const float* scales) {
  if (n < 0 || k <= 0 || (n > 0 && !scales)) return QM_ERR_INVALID;
  int64_t groups = 1;
  if (fmt == QM_FMT_INT4) {
    if ((k & 1) || !int4_groups(k, group_size, &groups)) return QM_ERR_INVALID;
  } else if (fmt == QM_FMT_INT8_ROW) {
    if (group_size != 0) return QM_ERR_INVALID;
  } else if (fmt == QM_FMT_INT3) {
    if (group_size != 64) return QM_ERR_INVALID;
    groups = (k + 63) / 64;
  } else {
    return QM_ERR_INVALID;
  }
  return finite_all(scales, n * groups) ? QM_OK : QM_ERR_INVALID;
}

QM_API int qm_quantize_int4(const float* w, int64_t n, int64_t k, int32_t group_size, uint8_t* q, float* scales) {
  int64_t groups = 1;
  if (!w || !q || !scales || n < 0 || k <= 0 || (k & 1) || !int4_groups(k, group_size, &groups))
    return QM_ERR_INVALID;
  if (!finite_all(w, n * k)) return QM_ERR_INVALID;
  const int64_t gs = k / groups;
  for (int64_t r = 0; r < n; ++r) {
    for (int64_t g = 0; g < groups; ++g) {
      const float* wg = w + r * k + g * gs;
      float amax = 0.f;
      for (int64_t c = 0; c < gs; ++c) amax = std::fmax(amax, std::fabs(wg[c]));
      // symmetric: the largest magnitude maps to 7 (codes -7 .. 7 result)
      const float s = amax / 7.f;
      scales[r * groups + g] = s;
      for (int64_t c = 0; c < gs; c += 2) {
        int a = 0, b = 0;
        if (s > 0.f) {
          a = (int)std::nearbyint(wg[c] / s);
          b = (int)std::nearbyint(wg[c + 1] / s);
        }
        a = a < -8 ? -8 : (a > 7 ? 7 : a);
        b = b < -8 ? -8 : (b > 7 ? 7 : b);
        q[r * (k / 2) + (g * gs + c) / 2] = (uint8_t)((unsigned)(a + 8) | ((unsigned)(b + 8) << 4));
      }
    }
  }
  return QM_OK;
}

QM_API int qm_quantize_int8(const float* w, int64_t n, int64_t k, int8_t* q, float* scales) {
  if (!w || !q || !scales || n < 0 || k <= 0) return QM_ERR_INVALID;
  if (!finite_all(w, n * k)) return QM_ERR_INVALID;
  for (int64_t r = 0; r < n; ++r) {
    const float* wr = w + r * k;
    float amax = 0.f;
    for (int64_t c = 0; c < k; ++c) amax = std::fmax(amax, std::fabs(wr[c]));
    const float s = amax / 127.f;
    scales[r] = s;
    for (int64_t c = 0; c < k; ++c) {
      int a = s > 0.f ? (int)std::nearbyint(wr[c] / s) : 0;
      a = a < -127 ? -127 : (a > 127 ? 127 : a);
      q[r * k + c] = (int8_t)a;
    }
  }
  return QM_OK;
}

}  // extern "C"
