// qgemv_i3.hip -- GEMV for the int3-g64 two-plane format (fmt 5).
//
// The colibri page "Vulkan backend: expert tier + dense + MLA attention on
// any Vulkan 1.2 GPU" (int3 commit notes) stores 64 inputs of a row in 24
// bytes: four 32-bit words holding the 2-bit low parts of 16 values each,
// then 64 high bits; each group has one fp32 scale.  Bit order (reading):
// value i of a group at bits 2 (i % 16) of low word i / 16 and at bit i of
// the little-endian high word; weight = value - 4.
//
// Decode: for low word j and pair p < 8 the values p and p + 8 of the word
// become one bf16 pair 0x4300 | v, i.e. (128 + v_p, 128 + v_{p+8}):
//   ((lo_j >> 2p) & 0x00030003) | ((t_j >> p) & 0x00040004) | 0x43004300
// where t_j carries the word's 16 high bits spread to bits 2..9 and 18..25
// (formed once per word from the high plane shifted to bit 0).  One v_dot2
// consumes the pair against x staged as the bf16 pair (x_p, x_{p+8}); the
// offset 128 + 4 = 132 is removed by starting each group's dot at
// -132 * (sum of the group's x).  fp32 x is split into hi + lo bf16 halves
// and both are dotted, as in the int4 kernels.
//
// Work mapping: L lanes per row (a power of two up to 64, chosen from the
// group count), lanes stride over the row's 24-byte groups (consecutive
// lanes read consecutive groups; a lane's groups, at most four, are all
// loaded before any is decoded), 64 / L rows per wave, rows grid-strided.
// Each group's four low words are dotted as four independent chains.  x for
// the whole row length lives in LDS (k <= 16384), staged one 16-value word
// per thread with vector loads.
#include "device.hpp"
#include "launch.hpp"

namespace qm {

namespace {

constexpr int kI3Threads = 256;
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kI3GplMax = 4;  // groups per lane: G <= 256 and L = 64 once G >= 64

template <bool SPLIT>
__global__ __launch_bounds__(kI3Threads) void stage_and_gemv_i3(const uint8_t* __restrict__ q,
                                                                 const float* __restrict__ sc, const void* x,
                                                                 float* __restrict__ y, int n, int k, int G, int L,
                                                                 int bf16x) {
  extern __shared__ __attribute__((aligned(16))) uint32_t xs[];  // [G][4][8] hi pairs, lo pairs, word sums, corr
  uint32_t* xl = xs + G * 32;
  float* wsum = reinterpret_cast<float*>(xs + (SPLIT ? 2 : 1) * G * 32);
  float* corr = wsum + G * 4;
  const int tid = threadIdx.x;
  // x as bf16 pairs (x_{16w+p}, x_{16w+p+8}), one 16-value word per thread
  // step; with fp32 x, hi and lo halves.  k % 32 == 0, so a word is either
  // inside x or wholly past its end (staged as zeros).
  for (int w = tid; w < G * 4; w += kI3Threads) {
    float v[16];
    if (16 * w < k) {
      if (bf16x) {
        const u32x4* src = reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(x) + 16 * w);
        const u32x4 a0 = src[0], a1 = src[1];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[2 * i] = bf16_bits_to_f32(a0[i] & 0xFFFFu);
          v[2 * i + 1] = bf16_bits_to_f32(a0[i] >> 16);
          v[8 + 2 * i] = bf16_bits_to_f32(a1[i] & 0xFFFFu);
          v[8 + 2 * i + 1] = bf16_bits_to_f32(a1[i] >> 16);
        }
      } else {
        const f32x4* src = reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(x) + 16 * w);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const f32x4 t = src[i];
#pragma unroll
          for (int j = 0; j < 4; ++j) v[4 * i + j] = t[j];
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = 0.f;
    }
    float sum = 0.f;
    u32x4 hp[2], lp[2];
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const uint32_t ha = f32_to_bf16_bits(v[p]), hb = f32_to_bf16_bits(v[p + 8]);
      hp[p >> 2][p & 3] = ha | (hb << 16);
      const float ra = v[p] - bf16_bits_to_f32(ha), rb = v[p + 8] - bf16_bits_to_f32(hb);
      const uint32_t la = f32_to_bf16_bits(ra), lb = f32_to_bf16_bits(rb);
      lp[p >> 2][p & 3] = la | (lb << 16);
      // the values the dots see: hi (+ lo)
      sum += bf16_bits_to_f32(ha) + bf16_bits_to_f32(hb);
      if constexpr (SPLIT) sum += bf16_bits_to_f32(la) + bf16_bits_to_f32(lb);
    }
    reinterpret_cast<u32x4*>(xs)[2 * w] = hp[0];
    reinterpret_cast<u32x4*>(xs)[2 * w + 1] = hp[1];
    if constexpr (SPLIT) {
      reinterpret_cast<u32x4*>(xl)[2 * w] = lp[0];
      reinterpret_cast<u32x4*>(xl)[2 * w + 1] = lp[1];
    }
    wsum[w] = sum;
  }
  __syncthreads();
  // per-group offset: -132 * (sum of the group's staged x), words in order
  for (int g = tid; g < G; g += kI3Threads)
    corr[g] = -132.f * (((wsum[4 * g] + wsum[4 * g + 1]) + wsum[4 * g + 2]) + wsum[4 * g + 3]);
  __syncthreads();

  const int wave = tid >> 6, lane = tid & 63;
  const int li = lane & (L - 1), rsub = lane / L, rpw = 64 / L;
  const int64_t rb = (int64_t)G * 24;
  const int rstride = gridDim.x * (kI3Threads / 64) * rpw;
  // A lane's groups of one row, loaded as one unit: the next row's unit is
  // in flight while the current one is decoded.
  struct Unit {
    u32x2 w[kI3GplMax][3];
    float s[kI3GplMax];
  };
  auto load = [&](int r0, Unit& u) {
    const int r = r0 + rsub;
    const bool ok = r0 < n && r < n;
    const uint8_t* row = q + (int64_t)(ok ? r : 0) * rb;
    const float* srow = sc + (int64_t)(ok ? r : 0) * G;
#pragma unroll
    for (int i = 0; i < kI3GplMax; ++i) {
      const int g = li + L * i;
      const int gg = g < G ? g : 0;
      const u32x2* gp = reinterpret_cast<const u32x2*>(row + (int64_t)gg * 24);
#pragma unroll
      for (int t = 0; t < 3; ++t) u.w[i][t] = __builtin_nontemporal_load(gp + t);
      u.s[i] = g < G ? srow[gg] : 0.f;
    }
  };
  Unit cur, nxt;
  int r0 = (blockIdx.x * (kI3Threads / 64) + wave) * rpw;
  if (r0 < n) load(r0, cur);
  for (; r0 < n; r0 += rstride) {
    if (r0 + rstride < n) load(r0 + rstride, nxt);
    const int r = r0 + rsub;
    const bool ok = r < n;
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < kI3GplMax; ++i) {
      const int g = li + L * i;
      if (g >= G) break;
      const uint32_t lo[4] = {cur.w[i][0][0], cur.w[i][0][1], cur.w[i][1][0], cur.w[i][1][1]};
      float part[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {  // one independent dot chain per low word
        const uint32_t h16 = (cur.w[i][2][j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
        const uint32_t t = ((h16 & 0xFFu) | ((h16 & 0xFF00u) << 8)) << 2;
        const u32x4* xp = reinterpret_cast<const u32x4*>(xs + (g * 4 + j) * 8);
        const u32x4 x0 = xp[0], x1 = xp[1];
        float c = j == 0 ? corr[g] : 0.f;
#pragma unroll
        for (int p = 0; p < 8; ++p) {
          const uint32_t pr = ((lo[j] >> (2 * p)) & 0x00030003u) | ((t >> p) & 0x00040004u) | 0x43004300u;
          c = dot2(pr, p < 4 ? x0[p] : x1[p - 4], c);
          if constexpr (SPLIT) c = dot2(pr, xl[(g * 4 + j) * 8 + p], c);
        }
        part[j] = c;
      }
      acc = __builtin_fmaf(cur.s[i], (part[0] + part[1]) + (part[2] + part[3]), acc);
    }
    switch (L) {  // sum over the row's L lanes
      case 4: acc = group_sum<4>(acc); break;
      case 8: acc = group_sum<8>(acc); break;
      case 16: acc = group_sum<16>(acc); break;
      case 32: acc = group_sum<32>(acc); break;
      default: acc = group_sum<64>(acc); break;
    }
    if (ok && li == 0) y[r] = acc;
    cur = nxt;
  }
}

}  // namespace

size_t qgemv_i3_lds(int k, int xdt) {
  const int G = (k + 63) / 64;
  return (size_t)G * 32 * 4 * (xdt == kF32 ? 2 : 1) + (size_t)G * 4 * 4 + (size_t)G * 4;
}

hipError_t launch_qgemv_i3(const uint8_t* q, const float* sc, const void* x, int xdt, float* y, int n, int k,
                           hipStream_t st) {
  const int G = (k + 63) / 64;
  int L = 4;
  while (L < 64 && 2 * L <= G) L *= 2;
  const int rows_per_block = (kI3Threads / 64) * (64 / L);
  int blocks = (n + rows_per_block - 1) / rows_per_block;
  if (blocks > 1024) blocks = 1024;
  const size_t lds = qgemv_i3_lds(k, xdt);
  if (xdt == kF32)
    hipLaunchKernelGGL(stage_and_gemv_i3<true>, dim3(blocks), dim3(kI3Threads), lds, st, q, sc, x, y, n, k, G, L, 0);
  else
    hipLaunchKernelGGL(stage_and_gemv_i3<false>, dim3(blocks), dim3(kI3Threads), lds, st, q, sc, x, y, n, k, G, L, 1);
  return hipGetLastError();
}

}  // namespace qm
