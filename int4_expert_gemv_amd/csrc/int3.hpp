// int3.hpp -- the int3-g64 two-plane format (fmt 5) on the GPU: activation
// staging in LDS and the dot of one 24-byte weight group with it.  Used by
// the dense GEMV (qgemv_i3.hip) and the expert FFN (moe_int3.hip).
//
// Format (the colibri page "Vulkan backend: expert tier + dense + MLA
// attention on any Vulkan 1.2 GPU", int3 commit notes): 64 inputs of a row
// in 24 bytes -- four 32-bit words holding the 2-bit low parts of 16 values
// each, then 64 high bits -- and one fp32 scale per group.  Bit order
// (reading): value i of a group at bits 2 (i % 16) of low word i / 16 and at
// bit i of the little-endian high word; weight = value - 4.
//
// Decode: for low word j and pair p < 8, the values p and p + 8 of the word
// become one bf16 pair 0x4300 | v, i.e. (128 + v_p, 128 + v_{p+8}):
//   ((lo_j >> 2p) & 0x00030003) | ((t_j >> p) & 0x00040004) | 0x43004300
// where t_j carries the word's 16 high bits spread to bits 2..9 and 18..25.
// One v_dot2 (bf16 x bf16, fp32 accumulate) takes the pair against the
// activations staged as the bf16 pair (x_p, x_{p+8}); the offset 128 + 4 =
// 132 is removed by starting each group's dot at -132 * (sum of the group's
// staged activations).  fp32 activations are split into hi + lo bf16 halves
// (|x - hi - lo| <= 2^-17 |x|) and both halves are dotted.
#pragma once

#include "device.hpp"

namespace qm {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// LDS image of nq staged "units" (a unit is one 64-wide group of one
// activation vector; unit q = v * G + g for vector v, group g):
//   hi[kUnitV q + 2 w + h]  u32x4: bf16 pairs (x_{16w+4h+c}, x_{16w+4h+c+8}),
//                           c = 0..3, of the unit's word w (16 values)
//   lo[...]                 the same for x - hi (fp32 activations only)
//   wsum[w * nq + q]        sum of word w's staged values
//   corr[q]                 -132 * sum of the unit's staged values
// A unit's eight slots are padded to nine (144 bytes, 9 coprime with the 16
// slots of a bank cycle), so 16 lanes that take consecutive units read 16
// distinct bank groups, and a slot's offset within its unit is a constant.
constexpr int kUnitV = 9;
struct I3Lds {
  u32x4* hi;
  u32x4* lo;
  float* wsum;
  float* corr;
  int nq;
};

__host__ __device__ constexpr size_t i3_lds_bytes(int nq, bool split) {
  return (size_t)nq * (16u * kUnitV * (split ? 2u : 1u) + 16u + 4u);
}

__device__ __forceinline__ I3Lds i3_carve(void* base, int nq, bool split) {
  I3Lds L;
  L.hi = reinterpret_cast<u32x4*>(base);
  L.lo = L.hi + kUnitV * nq;
  L.wsum = reinterpret_cast<float*>(L.hi + (split ? 2 : 1) * kUnitV * nq);
  L.corr = L.wsum + 4 * nq;
  L.nq = nq;
  return L;
}

// Stage nv activation vectors of k values each (G = ceil(k / 64) groups;
// k % 16 == 0, so a 16-value word lies wholly inside or wholly past the
// vector and the latter is staged as zeros).  src(v) is vector v's first
// value (bf16 bits when bf16x, else fp32; 16-byte aligned).  Threads tid,
// tid + nthr, ... take one word each; the caller synchronises, then calls
// i3_corr, then synchronises again.
template <bool SPLIT, typename SrcF>
__device__ __forceinline__ void i3_stage(const I3Lds& L, int G, int k, bool bf16x, SrcF src, int tid, int nthr) {
  const int nq = L.nq;
  for (int i = tid; i < 4 * nq; i += nthr) {
    const int q = i >> 2, w = i & 3;  // consecutive threads read consecutive words of x
    const int v = q / G, g = q - v * G;
    const int c0 = 64 * g + 16 * w;
    float val[16];
    if (c0 < k) {
      if (bf16x) {
        const u32x4* p = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(src(v)) + c0);
        const u32x4 a0 = p[0], a1 = p[1];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          val[2 * t] = bf16_bits_to_f32(a0[t] & 0xFFFFu);
          val[2 * t + 1] = bf16_bits_to_f32(a0[t] >> 16);
          val[8 + 2 * t] = bf16_bits_to_f32(a1[t] & 0xFFFFu);
          val[8 + 2 * t + 1] = bf16_bits_to_f32(a1[t] >> 16);
        }
      } else {
        const f32x4* p = reinterpret_cast<const f32x4*>(static_cast<const float*>(src(v)) + c0);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const f32x4 a = p[t];
#pragma unroll
          for (int u = 0; u < 4; ++u) val[4 * t + u] = a[u];
        }
      }
    } else {
#pragma unroll
      for (int t = 0; t < 16; ++t) val[t] = 0.f;
    }
    float sum = 0.f;
    u32x4 hp[2], lp[2];
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const uint32_t ha = f32_to_bf16_bits(val[p]), hb = f32_to_bf16_bits(val[p + 8]);
      hp[p >> 2][p & 3] = ha | (hb << 16);
      // the values the dots see: hi (+ lo)
      sum += bf16_bits_to_f32(ha) + bf16_bits_to_f32(hb);
      if constexpr (SPLIT) {
        const uint32_t la = f32_to_bf16_bits(val[p] - bf16_bits_to_f32(ha));
        const uint32_t lb = f32_to_bf16_bits(val[p + 8] - bf16_bits_to_f32(hb));
        lp[p >> 2][p & 3] = la | (lb << 16);
        sum += bf16_bits_to_f32(la) + bf16_bits_to_f32(lb);
      }
    }
    L.hi[kUnitV * q + 2 * w] = hp[0];
    L.hi[kUnitV * q + 2 * w + 1] = hp[1];
    if constexpr (SPLIT) {
      L.lo[kUnitV * q + 2 * w] = lp[0];
      L.lo[kUnitV * q + 2 * w + 1] = lp[1];
    }
    L.wsum[w * nq + q] = sum;
  }
}

__device__ __forceinline__ void i3_corr(const I3Lds& L, int tid, int nthr) {
  const int nq = L.nq;
  for (int q = tid; q < nq; q += nthr)
    L.corr[q] = -132.f * (((L.wsum[q] + L.wsum[nq + q]) + L.wsum[2 * nq + q]) + L.wsum[3 * nq + q]);
}

// The 24 bytes of one weight group, as three 8-byte loads (groups are 8-byte
// aligned: rows are whole groups of 24 bytes).
struct I3Group {
  u32x2 w[3];
};

__device__ __forceinline__ I3Group i3_load(const uint8_t* p) {
  const u32x2* g = reinterpret_cast<const u32x2*>(p);
  I3Group r;
#pragma unroll
  for (int t = 0; t < 3; ++t) r.w[t] = __builtin_nontemporal_load(g + t);
  return r;
}

// sum over the group's 64 inputs of (value - 4) * staged x for unit q, with
// one independent dot chain per low word
template <bool SPLIT>
__device__ __forceinline__ float i3_group_dot(const I3Group& wg, const I3Lds& L, int q) {
  const u32x4* xh = L.hi + kUnitV * q;
  const u32x4* xl = L.lo + kUnitV * q;
  const uint32_t lo[4] = {wg.w[0][0], wg.w[0][1], wg.w[1][0], wg.w[1][1]};
  float part[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t h16 = (wg.w[2][j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
    const uint32_t t = ((h16 & 0xFFu) | ((h16 & 0xFF00u) << 8)) << 2;
    const u32x4 x0 = xh[2 * j], x1 = xh[2 * j + 1];
    u32x4 l0, l1;
    if constexpr (SPLIT) {
      l0 = xl[2 * j];
      l1 = xl[2 * j + 1];
    }
    float c = j == 0 ? L.corr[q] : 0.f;
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const uint32_t pr = ((lo[j] >> (2 * p)) & 0x00030003u) | ((t >> p) & 0x00040004u) | 0x43004300u;
      c = dot2(pr, p < 4 ? x0[p] : x1[p - 4], c);
      if constexpr (SPLIT) c = dot2(pr, p < 4 ? l0[p] : l1[p - 4], c);
    }
    part[j] = c;
  }
  return (part[0] + part[1]) + (part[2] + part[3]);
}

}  // namespace qm
