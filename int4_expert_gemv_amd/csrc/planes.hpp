// planes.hpp -- activations as stacked integer "digit planes", so that the
// quantized weights can be applied with the integer dot-product instructions
// (v_dot8_i32_i4: eight int4 x int4 products per instruction; v_dot4_i32_i8:
// four int8 x int8) while every activation keeps an error bounded by its own
// magnitude.
//
// The operation is the quantized GEMV of the colibri page "Vulkan backend:
// expert tier + dense + MLA attention on any Vulkan 1.2 GPU" (commit notes
// "backend_vulkan.c/.h + shaders/qmatmul.comp" and "fmt=4 grouped scales"):
// y_n = sum_g s_ng * sum_{k in g} (nibble - 8) x_k for int4, and
// y_n = s_n * sum_k q_nk x_k for int8.  Only the encoding of x below is ours.
//
// Encoding.  Activations are taken in groups of N consecutive values v_i (N =
// 32 against int4 weights: one 16-byte weight chunk; N = 16 against int8).
// E is the group's exponent: the smallest integer with max|v_i| < 2^E.  With
// r0_i = v_i * 2^(14-E) (|r0| < 2^14, exact: a power-of-two scaling), plane p
// holds the integers X_pi = rint(r_pi) and passes on r_(p+1)i = (r_pi - X_pi)
// * 2^15 (exact in fp32: the rounding residual of rint is representable), so
//      v_i = 2^(E-14) * (X_0i + 2^-15 X_1i + ... + 2^(-15(P-1)) X_(P-1)i)
//            + 2^(E-14-15P) r_Pi,      |X_pi| <= 2^14,  |r_Pi| <= 2^14.
// With e_i = floor(log2 |v_i|) and e the smallest e_i of the group's non-zero
// values, P planes make every element
//  - exact when the activations are bf16 (8 significant bits, lowest bit
//    2^(e_i-7) >= the last plane's unit 2^(E-14-15(P-1))):
//    P = 1 + ceil(max(0, E - e - 7) / 15);
//  - off by at most 2^(E-15P) <= 2^-15 |v_i| for fp32 activations:
//    P = 1 + ceil((E - e) / 15).
// The plane count of a call is the largest over its groups (typically 2).
// A dot product's error is then at most 2^-15 * sum |w v| plus fp32
// accumulation: relative to each output's sum of absolute terms, for any
// input -- a large activation beside small ones costs planes, not accuracy.
//
// Integer form of a plane.  int4 weights: X (|X| <= 16384) is written with
// four balanced base-16 digits dig_d in [-8, 7]: U = X + 0x8888 is in
// [0, 0xFFFF] and dig_d = nibble_d(U) - 8, whose 4-bit two's complement is
// nibble_d(U) ^ 8.  Digit d of the activations 8j..8j+7 packed as nibbles
// (activation 8j+i at bits 4i, the weights' own nibble order) is one word; a
// 32-group's plane is 16 words, index 4j + d.  A weight word XOR 0x88888888
// holds the signed values nibble - 8, so sum_d 16^d v_dot8(w ^ 0x88888888,
// word_d) is the exact integer sum (nibble - 8) X (|.| <= 2^22 per group).
// int8 weights: X = lo + 256 hi with lo the signed low byte and hi in
// [-64, 64]; activations 4k..4k+3 give word 2k (their lo bytes) and word
// 2k+1 (their hi bytes); sum_k v_dot4(w_k, lo_k) + 256 v_dot4(w_k, hi_k) is
// exact.  Either way a plane costs 2 bytes per activation.
#pragma once

#include "device.hpp"

namespace qm {

constexpr int kPlaneMax = 20;  // planes cover any fp32 spread (2^-149 .. 2^128)

__device__ __forceinline__ int fexp(float a) { return __builtin_amdgcn_frexp_expf(a); }

// Exponent summary of a group: E with max|v| < 2^E, and the plane count its
// values need (see the header); an all-zero group gives (0, 1).
template <int N, int XT>
__device__ __forceinline__ int group_planes(const float (&v)[N], int* E_out) {
  float amax = 0.f, amin = __builtin_huge_valf();
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const float a = fabsf(v[i]);
    amax = fmaxf(amax, a);
    amin = fminf(amin, a > 0.f ? a : __builtin_huge_valf());
  }
  if (!(amax > 0.f)) {
    *E_out = 0;
    return 1;
  }
  const int E = fexp(amax);
  const int e = fexp(amin) - 1;  // floor(log2) of the smallest non-zero value
  *E_out = E;
  const int span = XT == kBF16 ? E - e - 7 : E - e;
  const int P = span <= 0 ? 1 : 1 + (span + 14) / 15;
  return P < kPlaneMax ? P : kPlaneMax;
}

// r <- the residual after `p` planes (r starts as v * 2^(14-E))
template <int N>
__device__ __forceinline__ void skip_planes(float (&r)[N], int p) {
  for (int q = 0; q < p; ++q) {
#pragma unroll
    for (int i = 0; i < N; ++i) r[i] = (r[i] - __builtin_rintf(r[i])) * 32768.f;
  }
}

// The 4 words (digits d = 0..3) of the current plane of 8 activations r[0..7]
// (int4 weights), r advanced to the next plane.
__device__ __forceinline__ void plane_words8_i4(float (&r)[8], uint32_t (&wd)[4]) {
  uint32_t pr[4];  // U of activations (i, 4 + i) in the two halves
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float a = __builtin_rintf(r[i]), b = __builtin_rintf(r[4 + i]);
    r[i] = (r[i] - a) * 32768.f;
    r[4 + i] = (r[4 + i] - b) * 32768.f;
    pr[i] = (uint32_t)((int)a + 0x8888) | ((uint32_t)((int)b + 0x8888) << 16);
  }
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    uint32_t w = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) w |= ((pr[i] >> (4 * d)) & 0x000F000Fu) << (4 * i);
    wd[d] = w ^ 0x88888888u;
  }
}

// int3-g64 weights (the colibri page "Vulkan backend: expert tier + dense +
// MLA attention on any Vulkan 1.2 GPU", int3 commit notes: 64 inputs in 24
// bytes, four 32-bit words of 2-bit low parts, then 64 high bits; reading:
// value i at bits 2 (i % 16) of low word i / 16 and at bit i of the high
// word; weight = value - 4) are the int4 case with signed nibbles:
// w = lo + 4 hb - 4 is lo (hb = 1) or lo - 4 (hb = 0), i.e. the 4-bit two's
// complement lo + 12 (1 - hb).  A 16-value low word gives two weight words
// without moving any 2-bit field: its even values (lo & 0x33333333: value
// 2k in nibble k) and its odd values ((lo >> 2) & 0x33333333), the 16 high
// bits spread once (bit i to bit 2 i) and masked for each.  The activations
// of those 16 inputs are staged in the same order: even ones, then odd ones.
// bit i of the 16-bit h -> bit 2 i (so value 2k's bit lands at 4k, value
// 2k + 1's at 4k + 2)
__device__ __forceinline__ uint32_t spread16(uint32_t h) {
  h = (h | (h << 8)) & 0x00FF00FFu;
  h = (h | (h << 4)) & 0x0F0F0F0Fu;
  h = (h | (h << 2)) & 0x33333333u;
  return (h | (h << 1)) & 0x55555555u;
}
// the two signed-nibble weight words (even, odd values) of one 16-value low
// word and its 16 high bits (bits 0..15 of h16)
__device__ __forceinline__ void i3_words(uint32_t lo, uint32_t h16, uint32_t& we, uint32_t& wo) {
  const uint32_t n = spread16(~h16 & 0xFFFFu);  // 1 - hb, at bit 4k (even) and 4k + 2 (odd)
  const uint32_t ne = n & 0x11111111u, no = n & 0x44444444u;
  we = (lo & 0x33333333u) | (ne << 2) | (ne << 3);
  wo = ((lo >> 2) & 0x33333333u) | no | (no << 1);
}
// the same as offset-binary nibbles (value + 4 = signed nibble + 8, the int4
// encoding): lo + 4 + 4 hb
__device__ __forceinline__ void i3_words_ob(uint32_t lo, uint32_t h16, uint32_t& we, uint32_t& wo) {
  const uint32_t b = spread16(h16 & 0xFFFFu);
  we = (lo & 0x33333333u) + 0x44444444u + ((b & 0x11111111u) << 2);
  wo = ((lo >> 2) & 0x33333333u) + 0x44444444u + ((b & 0x44444444u));
}

// The 2 words (low bytes, high bytes) of the current plane of 4 activations
// (int8 weights), r advanced to the next plane.
__device__ __forceinline__ void plane_words4_i8(float (&r)[4], uint32_t (&wd)[2]) {
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float a = __builtin_rintf(r[i]);
    r[i] = (r[i] - a) * 32768.f;
    const int X = (int)a;
    const int l = (int)(int8_t)(uint8_t)(X & 0xFF);
    const int h = (X - l) >> 8;
    lo |= ((uint32_t)l & 0xFFu) << (8 * i);
    hi |= ((uint32_t)h & 0xFFu) << (8 * i);
  }
  wd[0] = lo;
  wd[1] = hi;
}

__device__ __forceinline__ int sdot8(uint32_t a, uint32_t b, int c) {
  return __builtin_amdgcn_sdot8((int)a, (int)b, c, false);
}
__device__ __forceinline__ int sdot4(uint32_t a, uint32_t b, int c) {
  return __builtin_amdgcn_sdot4((int)a, (int)b, c, false);
}

// Exact integer sum over one 16-byte chunk of int4 weights (w, each word
// already XOR 0x88888888) against one plane of its 32-group (x[0..15]):
// sum_d 16^d T_d with T_d the digit-d products, accumulated from the top
// digit down (t <- 16 t + T_d), so that the accumulator of each dot
// instruction carries the running sum (|partial sums| stay below 2^22).
__device__ __forceinline__ int shl4(int t) { return (int)((uint32_t)t << 4); }
__device__ __forceinline__ int gdot_i4(const u32x4& w, const uint32_t* x) {
  int t = sdot8(w[3], x[12 + 3], sdot8(w[2], x[8 + 3], sdot8(w[1], x[4 + 3], sdot8(w[0], x[3], 0))));
#pragma unroll
  for (int d = 2; d >= 0; --d)
    t = sdot8(w[3], x[12 + d], sdot8(w[2], x[8 + d], sdot8(w[1], x[4 + d], sdot8(w[0], x[d], shl4(t)))));
  return t;
}

// The same for 16 int8 weights (words w[0..3]) against a 16-group's plane.
__device__ __forceinline__ int gdot_i8(const u32x4& w, const uint32_t* x) {
  int t = sdot4(w[0], x[1], sdot4(w[1], x[3], sdot4(w[2], x[5], sdot4(w[3], x[7], 0))));
  return sdot4(w[0], x[0], sdot4(w[1], x[2], sdot4(w[2], x[4], sdot4(w[3], x[6], t << 8))));
}

// Streaming loads through a buffer resource: one descriptor (scalar
// registers) for a whole region and per-lane byte offsets in vector
// registers, so that many rows in flight do not each hold a 64-bit scalar
// address.  Non-temporal (weights are read once per call).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t region_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 ld_region16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2);
}
__device__ __forceinline__ float ld_region4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 2));
}

// Load N (16 or 32) activations (bf16 or fp32) starting at element `e0` of `x`.
template <int XT, int N>
__device__ __forceinline__ void load_acts(const void* __restrict__ x, int64_t e0, float (&v)[N]) {
  if constexpr (XT == kBF16 && N == 4) {
    const uint2 d = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(x) + e0);
    v[0] = __uint_as_float(d.x << 16);
    v[1] = __uint_as_float(d.x & 0xFFFF0000u);
    v[2] = __uint_as_float(d.y << 16);
    v[3] = __uint_as_float(d.y & 0xFFFF0000u);
  } else if constexpr (XT == kBF16) {
    const u32x4* src = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(x) + e0);
#pragma unroll
    for (int r = 0; r < N / 8; ++r) {
      const u32x4 d = src[r];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[8 * r + 2 * i] = __uint_as_float(d[i] << 16);
        v[8 * r + 2 * i + 1] = __uint_as_float(d[i] & 0xFFFF0000u);
      }
    }
  } else {
    const f32x4* src = reinterpret_cast<const f32x4*>(static_cast<const float*>(x) + e0);
#pragma unroll
    for (int r = 0; r < N / 4; ++r) {
      const f32x4 d = src[r];
#pragma unroll
      for (int i = 0; i < 4; ++i) v[4 * r + i] = d[i];
    }
  }
}

// Planes [p0, p0 + np) (np <= 2) of one activation group of N = 32 (int4)
// or 16 (int8) values starting at element e0 of x, with the group's exponent
// E, written as words to dst[pp * pstride + k] (k < 16 or 8).  Works on 8 (4)
// values at a time to keep few registers live.
template <int FMT, int XT>
__device__ __forceinline__ void stage_group(const void* __restrict__ x, int64_t e0, int E, int p0, int np,
                                            uint32_t* __restrict__ dst, size_t pstride) {
  if constexpr (FMT == kFmtInt3) {
    // 32 activations as four sub-blocks of 8: the even and the odd ones of
    // each 16 (the order of the int3 weight words, i3_words)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      float v[16];
      load_acts<XT, 16>(x, e0 + 16 * hh, v);
#pragma unroll
      for (int par = 0; par < 2; ++par) {
        float r[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) r[i] = ldexpf(v[2 * i + par], 14 - E);
        skip_planes(r, p0);
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
          if (pp >= np) break;
          uint32_t wd[4];
          plane_words8_i4(r, wd);
#pragma unroll
          for (int k = 0; k < 4; ++k) dst[pp * pstride + (2 * hh + par) * 4 + k] = wd[k];
        }
      }
    }
    return;
  }
  constexpr int SB = FMT == kFmtInt4 ? 8 : 4;  // activations per sub-block
  constexpr int NSB = FMT == kFmtInt4 ? 4 : 4;  // sub-blocks per group
  constexpr int WPS = FMT == kFmtInt4 ? 4 : 2;  // words per sub-block and plane
#pragma unroll
  for (int j = 0; j < NSB; ++j) {
    float r[SB];
    load_acts<XT, SB>(x, e0 + j * SB, r);
#pragma unroll
    for (int i = 0; i < SB; ++i) r[i] = ldexpf(r[i], 14 - E);
    skip_planes(r, p0);
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) {
      if (pp >= np) break;
      uint32_t wd[WPS];
      if constexpr (FMT == kFmtInt4)
        plane_words8_i4(r, wd);
      else
        plane_words4_i8(r, wd);
#pragma unroll
      for (int k = 0; k < WPS; ++k) dst[pp * pstride + j * WPS + k] = wd[k];
    }
  }
}

// The same from the group's N values already in registers (planes p0 and
// p0 + 1); v is consumed.
template <int FMT, int N>
__device__ __forceinline__ void stage_group_vals(float (&v)[N], int E, int p0, uint32_t* __restrict__ dst,
                                                 size_t pstride) {
  constexpr int SB = FMT == kFmtInt8 ? 4 : 8;
  constexpr int WPS = FMT == kFmtInt8 ? 2 : 4;
#pragma unroll
  for (int j = 0; j < N / SB; ++j) {
    float r[SB];
    // sub-block j: 8 consecutive values, or for int3 the even (j even) or
    // odd (j odd) values of the 16 starting at 16 (j / 2)
#pragma unroll
    for (int i = 0; i < SB; ++i)
      r[i] = ldexpf(FMT == kFmtInt3 ? v[16 * (j >> 1) + 2 * i + (j & 1)] : v[j * SB + i], 14 - E);
    skip_planes(r, p0);
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) {
      uint32_t wd[WPS];
      if constexpr (FMT == kFmtInt8)
        plane_words4_i8(r, wd);
      else
        plane_words8_i4(r, wd);
#pragma unroll
      for (int k = 0; k < WPS; ++k) dst[pp * pstride + j * WPS + k] = wd[k];
    }
  }
}

// Block-wide maximum of a small non-negative int through one LDS word
// (*slot must be 0 before the first barrier; every thread calls this).
__device__ __forceinline__ int block_max_int(int v, int* slot) {
  // wave maximum first, then one LDS atomic per wave
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = max(v, __shfl_xor(v, o, 64));
  if ((threadIdx.x & 63) == 0) atomicMax(slot, v);
  __syncthreads();
  return *slot;
}

}  // namespace qm
