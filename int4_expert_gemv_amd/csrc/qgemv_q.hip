// qgemv_q.hip -- single-token int4 GEMV on integer dot products: y = W x for
// one resident quantized tensor, the dense quantized GEMV of the colibri page
// "Vulkan backend: expert tier + dense + MLA attention on any Vulkan 1.2 GPU"
// (commit notes "backend_vulkan.c/.h + shaders/qmatmul.comp" and "fmt=4
// grouped scales"), with x turned into the digit words of moe_t1_q.hpp so
// that one v_dot8_i32_i4 handles eight weights.
//
// Two matrices of the same x (and k, format, grouping) can share one launch:
// workgroups [0, nba) work on the first, the rest on the second.
//
// Work split: workgroups of eight waves; wave w of workgroup b owns NU
// consecutive rows and a lane owns chunks lane + 64 cb (cb < CB, K = 2048 CB)
// of each of them.  A lane's share of a row is CB 16-byte chunks and their
// scales, so the wave issues the loads of all NU rows at once into registers
// (no staging: every byte of the call is in flight from the start, the grid
// is sized to one workgroup per CU).  x is fetched first (loads complete in
// order), turned into digits once per workgroup in LDS while the weights
// stream in, and read back per row (or kept in registers for short rows).
#include <type_traits>

#include "moe_t1_q.hpp"

namespace qm {

#ifndef QM_Q4_CAP
#define QM_Q4_CAP 8  // most rows per wave of the int4 GEMV
#endif
#ifndef QM_Q8_CAP16
#define QM_Q8_CAP16 1  // rows per wave for int8 rows of 16384: one (more, smaller workgroups)
#endif

constexpr int kQvWaves = 8;
constexpr int kQvThreads = 64 * kQvWaves;

template <int XT, int CB, int NU, bool GROUPED>
__global__ __launch_bounds__(kQvThreads) void qgemv_q_kernel(GemvArgs a0, GemvArgs b0, int nba) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  constexpr int K = 2048 * CB;
  constexpr bool XREG = CB <= 4;  // keep the lane's x digits in registers
  const bool first = (int)blockIdx.x < nba;
  const GemvArgs& a = first ? a0 : b0;
  const int blk = first ? (int)blockIdx.x : (int)blockIdx.x - nba;
  const int wave = uniform(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int rb = (blk * kQvWaves + wave) * NU;  // this wave's first row
  uint32_t* xq = reinterpret_cast<uint32_t*>(lds);          // [K/16][8]
  float* xsc = reinterpret_cast<float*>(lds + (size_t)K * 2);  // [K/16]

  // x first
  constexpr int NG = (K / 16 + kQvThreads - 1) / kQvThreads;
  constexpr int NR = XT == kBF16 ? 2 : 4;
  u32x4 raw[NG][NR];
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    const int g = threadIdx.x + gi * kQvThreads;
    if (g < K / 16) {
      const u32x4* src =
          reinterpret_cast<const u32x4*>(static_cast<const char*>(a.x) + (size_t)g * 16 * (XT == kBF16 ? 2 : 4));
#pragma unroll
      for (int r = 0; r < NR; ++r) raw[gi][r] = src[r];
    }
  }
  // then every row of this wave
  u32x4 wv[NU][CB];
  float sv[NU][CB];
  const bool won = rb < a.n;
  if (won) {  // chunk-major, the order the arithmetic consumes them
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const int c = lane + 64 * cb;
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const int r = min(rb + u, a.n - 1);
        wv[u][cb] = ld_stream(a.q + (int64_t)r * a.row_bytes + (int64_t)c * 16);
        sv[u][cb] = ld_stream(a.s + (int64_t)r * a.G + (GROUPED ? (c >> a.gshift) : 0));
      }
    }
  }
  // x digits, once per workgroup
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    const int g = threadIdx.x + gi * kQvThreads;
    if (g < K / 16) {
      float v[16];
      if constexpr (XT == kBF16) {
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            v[8 * r + 2 * i] = __uint_as_float(raw[gi][r][i] << 16);
            v[8 * r + 2 * i + 1] = __uint_as_float(raw[gi][r][i] & 0xFFFF0000u);
          }
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int i = 0; i < 4; ++i) v[4 * r + i] = __uint_as_float(raw[gi][r][i]);
      }
      uint32_t wd[8];
      xsc[g] = q_group16(v, wd);
      u32x4* dst = reinterpret_cast<u32x4*>(xq + (size_t)g * 8);
      dst[0] = u32x4{wd[0], wd[1], wd[2], wd[3]};
      dst[1] = u32x4{wd[4], wd[5], wd[6], wd[7]};
    }
  }
  lds_barrier();
  if (!won) return;
  u32x4 xr[XREG ? CB : 1][4];
  float xsr[XREG ? CB : 1][2];
  if constexpr (XREG) {
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const int c = lane + 64 * cb;
      const u32x4* src = reinterpret_cast<const u32x4*>(xq + (size_t)c * 16);
#pragma unroll
      for (int j = 0; j < 4; ++j) xr[cb][j] = src[j];
      xsr[cb][0] = xsc[2 * c];
      xsr[cb][1] = xsc[2 * c + 1];
    }
  }
  // a chunk's x digits are read once for all NU rows
  float acc[NU];
#pragma unroll
  for (int u = 0; u < NU; ++u) acc[u] = 0.f;
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    if constexpr (XREG) {
#pragma unroll
      for (int u = 0; u < NU; ++u) acc[u] = q_chunk(wv[u][cb], xr[cb], xsr[cb], sv[u][cb], acc[u]);
    } else {
      const int c = lane + 64 * cb;
      const u32x4* src = reinterpret_cast<const u32x4*>(xq + (size_t)c * 16);
      const u32x4 xd[4] = {src[0], src[1], src[2], src[3]};
      const float xs[2] = {xsc[2 * c], xsc[2 * c + 1]};
#pragma unroll
      for (int u = 0; u < NU; ++u) acc[u] = q_chunk(wv[u][cb], xd, xs, sv[u][cb], acc[u]);
    }
  }
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const float yv = group_sum<64>(acc[u]);
    if (lane == 0 && rb + u < a.n) a.y[rb + u] = yv;
  }
}

// ---- small batch (qgemm_small), int4: NB activation rows per weight read --------
// Same work split and register prefetch; x is staged once per workgroup as
// bf16 pairs (activations 8q+i and 8q+4+i of a chunk in one word, the order
// of the nibble pairs (w >> 4i) & 0x000F000F | 0x43004300 = bf16 (128+n)),
// with the chunk's -136 * sum in an offset (fp32 activations as bf16 hi + lo,
// |x - hi - lo| <= 2^-17 |x|).  A chunk's nibble pairs are built once per row
// and used for every activation row; a row's x words are read once per chunk
// for the wave's NU rows.  Rows of the batch past nb are skipped.
template <int XT, int CB, int NB, int NU, bool GROUPED>
__global__ __launch_bounds__(kQvThreads) void qgemv_b_kernel(GemvArgs a) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  constexpr bool SPLIT = XT == kF32;
  constexpr int KCH = 64 * CB;  // chunks per row
  const int wave = uniform(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int rb = (blockIdx.x * kQvWaves + wave) * NU;
  const int nb = a.nb;
  u32x4* xh = reinterpret_cast<u32x4*>(lds);                 // [NB][4][KCH]
  u32x4* xl = xh + (SPLIT ? NB * 4 * KCH : 0);                // [NB][4][KCH] (fp32 x)
  float* xo = reinterpret_cast<float*>(xh + (SPLIT ? 2 : 1) * NB * 4 * KCH);  // [NB][KCH]
  // x first: one (row, chunk) per thread and step
  for (int it = threadIdx.x; it < nb * KCH; it += kQvThreads) {
    const int t = it / KCH, c = it - t * KCH;
    float v[32];
    if constexpr (XT == kBF16) {
      const u32x4* src = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.x) + (size_t)t * a.ldx + c * 32);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const u32x4 q4 = src[r];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[8 * r + 2 * i] = __uint_as_float(q4[i] << 16);
          v[8 * r + 2 * i + 1] = __uint_as_float(q4[i] & 0xFFFF0000u);
        }
      }
    } else {
      const f32x4* src = reinterpret_cast<const f32x4*>(static_cast<const float*>(a.x) + (size_t)t * a.ldx + c * 32);
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const f32x4 q4 = src[r];
#pragma unroll
        for (int i = 0; i < 4; ++i) v[4 * r + i] = q4[i];
      }
    }
    float sum = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      u32x4 ph, pl;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float a0 = v[8 * q + i], a1 = v[8 * q + 4 + i];
        const uint32_t h0 = f32_to_bf16_bits(a0), h1 = f32_to_bf16_bits(a1);
        ph[i] = h0 | (h1 << 16);
        if constexpr (SPLIT) {
          const uint32_t l0 = f32_to_bf16_bits(a0 - bf16_bits_to_f32(h0)), l1 = f32_to_bf16_bits(a1 - bf16_bits_to_f32(h1));
          pl[i] = l0 | (l1 << 16);
          sum += (bf16_bits_to_f32(h0) + bf16_bits_to_f32(l0)) + (bf16_bits_to_f32(h1) + bf16_bits_to_f32(l1));
        } else {
          sum += bf16_bits_to_f32(h0) + bf16_bits_to_f32(h1);
        }
      }
      xh[(t * 4 + q) * KCH + c] = ph;
      if constexpr (SPLIT) xl[(t * 4 + q) * KCH + c] = pl;
    }
    xo[t * KCH + c] = -136.0f * sum;
  }
  // then every row of this wave, chunk-major
  u32x4 wv[NU][CB];
  float sv[NU][CB];
  const bool won = rb < a.n;
  if (won) {
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const int c = lane + 64 * cb;
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const int r = min(rb + u, a.n - 1);
        wv[u][cb] = ld_stream(a.q + (int64_t)r * a.row_bytes + (int64_t)c * 16);
        sv[u][cb] = ld_stream(a.s + (int64_t)r * a.G + (GROUPED ? (c >> a.gshift) : 0));
      }
    }
  }
  lds_barrier();
  if (!won) return;
  const NibConst nk = nib_const();
  float acc[NB][NU];
#pragma unroll
  for (int t = 0; t < NB; ++t)
#pragma unroll
    for (int u = 0; u < NU; ++u) acc[t][u] = 0.f;
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const int c = lane + 64 * cb;
    uint32_t pr[NU][16];
#pragma unroll
    for (int u = 0; u < NU; ++u)
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int i = 0; i < 4; ++i) pr[u][q * 4 + i] = nib_pair(wv[u][cb][q] >> (4 * i), nk);
#pragma unroll
    for (int t = 0; t < NB; ++t) {
      if (t < nb) {
        u32x4 hq[4], lq[SPLIT ? 4 : 1];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          hq[q] = xh[(t * 4 + q) * KCH + c];
          if constexpr (SPLIT) lq[q] = xl[(t * 4 + q) * KCH + c];
        }
        const float off = xo[t * KCH + c];
#pragma unroll
        for (int u = 0; u < NU; ++u) {
          float tt = off;
#pragma unroll
          for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              tt = dot2(pr[u][q * 4 + i], hq[q][i], tt);
              if constexpr (SPLIT) tt = dot2(pr[u][q * 4 + i], lq[q][i], tt);
            }
          acc[t][u] = __builtin_fmaf(sv[u][cb], tt, acc[t][u]);
        }
      }
    }
  }
#pragma unroll
  for (int t = 0; t < NB; ++t)
    if (t < nb) {
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const float yv = group_sum<64>(acc[t][u]);
        if (lane == 0 && rb + u < a.n) a.y[(int64_t)t * a.ldy + rb + u] = yv;
      }
    }
}

template <int XT, int CB, int NB, bool GROUPED>
hipError_t launch_qvb(const GemvArgs& a, hipStream_t st) {
  constexpr int KCH = 64 * CB;
  const size_t lds = (size_t)NB * KCH * (4 * 16 * (XT == kF32 ? 2 : 1) + 4);
  if (lds > (size_t)kLdsMax) return hipErrorNotSupported;
  constexpr int kCus = 256;
  const int need = (a.n + kCus * kQvWaves - 1) / (kCus * kQvWaves);
  auto go = [&](auto nu_tag) {
    constexpr int NU = decltype(nu_tag)::value;
    const int rows = kQvWaves * NU;
    hipLaunchKernelGGL((qgemv_b_kernel<XT, CB, NB, NU, GROUPED>), dim3((a.n + rows - 1) / rows), dim3(kQvThreads),
                       lds, st, a);
    return hipGetLastError();
  };
  if (need <= 1) return go(std::integral_constant<int, 1>{});
  if (need <= 2 || CB > 4) return go(std::integral_constant<int, 2>{});
  return go(std::integral_constant<int, 3>{});
}

template <int XT, int CB, bool GROUPED>
hipError_t launch_qvb_nb(const GemvArgs& a, hipStream_t st) {
  // activation rows one launch stages: the batch rounded up to 2, 4 or 8,
  // fewer when their staging would not fit in LDS -- then the batch runs as
  // several launches over row groups (each reads the weights again; at these
  // batch sizes the arithmetic, not the weight stream, is the bound)
  constexpr size_t per = (size_t)64 * CB * (4 * 16 * (XT == kF32 ? 2 : 1) + 4);  // LDS bytes per row
  int nbs = a.nb <= 2 ? 2 : (a.nb <= 4 ? 4 : 8);
  while (nbs > 2 && (size_t)nbs * per > (size_t)kLdsMax) nbs /= 2;
  if ((size_t)nbs * per > (size_t)kLdsMax) return hipErrorNotSupported;
  const size_t xsz = XT == kBF16 ? 2 : 4;
  for (int t0 = 0; t0 < a.nb; t0 += nbs) {
    GemvArgs b = a;
    b.x = static_cast<const char*>(a.x) + (size_t)t0 * a.ldx * xsz;
    b.y = a.y + (size_t)t0 * a.ldy;
    b.nb = a.nb - t0 < nbs ? a.nb - t0 : nbs;
    const hipError_t e = nbs == 2 ? launch_qvb<XT, CB, 2, GROUPED>(b, st)
                                  : (nbs == 4 ? launch_qvb<XT, CB, 4, GROUPED>(b, st)
                                              : launch_qvb<XT, CB, 8, GROUPED>(b, st));
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int XT, bool GROUPED>
hipError_t launch_qvb_cb(const GemvArgs& a, hipStream_t st) {
  switch (a.k / 2048) {
    case 1: return launch_qvb_nb<XT, 1, GROUPED>(a, st);
    case 2: return launch_qvb_nb<XT, 2, GROUPED>(a, st);
    case 3: return launch_qvb_nb<XT, 3, GROUPED>(a, st);
    case 4: return launch_qvb_nb<XT, 4, GROUPED>(a, st);
    case 6: return launch_qvb_nb<XT, 6, GROUPED>(a, st);
    case 8: return launch_qvb_nb<XT, 8, GROUPED>(a, st);
    default: return hipErrorNotSupported;
  }
}

// ---- int8 per-row weights ------------------------------------------------------
// The same scheme with v_dot4_i32_i8: the integers X of a group of 16
// activations (as above, |X| <= 30567) are written with two balanced base-256
// digits, byte pattern X & 255 and ((X + 128) >> 8) & 255 (range [-32896,
// 32639]); digit d of activations 4j..4j+3 is word j*2+d.  A 16-byte chunk
// holds 16 int8 weights = one group: eight dot4 give its two digit sums,
// recombined as a0 + 256 a1 (exact in int32), scaled by 2^(E-15); the row's
// scale multiplies the row sum.
__device__ __forceinline__ float q8_group16(const float (&v)[16], uint32_t (&wd)[8]) {
  const int E = q_exp(q_amax16(v));
  int X[16];
  q_ints16(v, E, X);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t w0 = 0, w1 = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      w0 |= ((uint32_t)X[4 * j + i] & 255u) << (8 * i);
      w1 |= ((uint32_t)((X[4 * j + i] + 128) >> 8) & 255u) << (8 * i);
    }
    wd[j * 2] = w0;
    wd[j * 2 + 1] = w1;
  }
  return ldexpf(1.f, E - 15);
}

__device__ __forceinline__ float q8_chunk(const u32x4& w, const u32x4 (&xd)[2], float xs, float acc) {
  int a0 = 0, a1 = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t lo = xd[j >> 1][(j & 1) * 2], hi = xd[j >> 1][(j & 1) * 2 + 1];
    a0 = __builtin_amdgcn_sdot4((int)w[j], (int)lo, a0, false);
    a1 = __builtin_amdgcn_sdot4((int)w[j], (int)hi, a1, false);
  }
  const int t = (int)((uint32_t)a0 + ((uint32_t)a1 << 8));
  return __builtin_fmaf((float)t, xs, acc);
}

// K = 1024 CB int8 values per row (a lane owns chunks lane + 64 cb)
template <int XT, int CB, int NU>
__global__ __launch_bounds__(kQvThreads) void qgemv_q8_kernel(GemvArgs a0, GemvArgs b0, int nba) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  constexpr int K = 1024 * CB;
  constexpr bool XREG = CB <= 6;
  const bool first = (int)blockIdx.x < nba;
  const GemvArgs& a = first ? a0 : b0;
  const int blk = first ? (int)blockIdx.x : (int)blockIdx.x - nba;
  const int wave = uniform(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int rb = (blk * kQvWaves + wave) * NU;
  uint32_t* xq = reinterpret_cast<uint32_t*>(lds);             // [K/16][8]
  float* xsc = reinterpret_cast<float*>(lds + (size_t)K * 2);  // [K/16]
  constexpr int NG = (K / 16 + kQvThreads - 1) / kQvThreads;
  constexpr int NR = XT == kBF16 ? 2 : 4;
  u32x4 raw[NG][NR];
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    const int g = threadIdx.x + gi * kQvThreads;
    if (g < K / 16) {
      const u32x4* src =
          reinterpret_cast<const u32x4*>(static_cast<const char*>(a.x) + (size_t)g * 16 * (XT == kBF16 ? 2 : 4));
#pragma unroll
      for (int r = 0; r < NR; ++r) raw[gi][r] = src[r];
    }
  }
  u32x4 wv[NU][CB];
  float sr[NU];
  const bool won = rb < a.n;
  if (won) {
#pragma unroll
    for (int u = 0; u < NU; ++u) sr[u] = a.s[min(rb + u, a.n - 1)];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const int c = lane + 64 * cb;
#pragma unroll
      for (int u = 0; u < NU; ++u)
        wv[u][cb] = ld_stream(a.q + (int64_t)min(rb + u, a.n - 1) * a.row_bytes + (int64_t)c * 16);
    }
  }
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    const int g = threadIdx.x + gi * kQvThreads;
    if (g < K / 16) {
      float v[16];
      if constexpr (XT == kBF16) {
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            v[8 * r + 2 * i] = __uint_as_float(raw[gi][r][i] << 16);
            v[8 * r + 2 * i + 1] = __uint_as_float(raw[gi][r][i] & 0xFFFF0000u);
          }
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int i = 0; i < 4; ++i) v[4 * r + i] = __uint_as_float(raw[gi][r][i]);
      }
      uint32_t wd[8];
      xsc[g] = q8_group16(v, wd);
      u32x4* dst = reinterpret_cast<u32x4*>(xq + (size_t)g * 8);
      dst[0] = u32x4{wd[0], wd[1], wd[2], wd[3]};
      dst[1] = u32x4{wd[4], wd[5], wd[6], wd[7]};
    }
  }
  lds_barrier();
  if (!won) return;
  u32x4 xr[XREG ? CB : 1][2];
  float xsr[XREG ? CB : 1];
  if constexpr (XREG) {
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const int c = lane + 64 * cb;
      const u32x4* src = reinterpret_cast<const u32x4*>(xq + (size_t)c * 8);
      xr[cb][0] = src[0];
      xr[cb][1] = src[1];
      xsr[cb] = xsc[c];
    }
  }
  float acc[NU];
#pragma unroll
  for (int u = 0; u < NU; ++u) acc[u] = 0.f;
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    if constexpr (XREG) {
#pragma unroll
      for (int u = 0; u < NU; ++u) acc[u] = q8_chunk(wv[u][cb], xr[cb], xsr[cb], acc[u]);
    } else {
      const int c = lane + 64 * cb;
      const u32x4* src = reinterpret_cast<const u32x4*>(xq + (size_t)c * 8);
      const u32x4 xd[2] = {src[0], src[1]};
      const float xs = xsc[c];
#pragma unroll
      for (int u = 0; u < NU; ++u) acc[u] = q8_chunk(wv[u][cb], xd, xs, acc[u]);
    }
  }
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const float yv = group_sum<64>(acc[u]);
    if (lane == 0 && rb + u < a.n) a.y[rb + u] = sr[u] * yv;
  }
}

template <int XT, int CB>
hipError_t launch_qv8(const GemvArgs& a, const GemvArgs& b, bool pair, hipStream_t st) {
  constexpr int kCus = 256;
  const int rows_all = a.n + (pair ? b.n : 0);
  const int need = (rows_all + kCus * kQvWaves - 1) / (kCus * kQvWaves);
  constexpr int cap = CB <= 4 ? 8 : (CB <= 8 ? 4 : QM_Q8_CAP16);
  const size_t lds = (size_t)1024 * CB * 2 + (size_t)1024 * CB / 4;
  auto go = [&](auto nu_tag) {
    constexpr int NU = decltype(nu_tag)::value;
    const int rows = kQvWaves * NU;
    const int nba = (a.n + rows - 1) / rows;
    const int nbb = pair ? (b.n + rows - 1) / rows : 0;
    hipLaunchKernelGGL((qgemv_q8_kernel<XT, CB, NU>), dim3(nba + nbb), dim3(kQvThreads), lds, st, a, pair ? b : a,
                       nba);
    return hipGetLastError();
  };
  if (need <= 1 || cap <= 1) return go(std::integral_constant<int, 1>{});
  if (need <= 2 || cap <= 2) return go(std::integral_constant<int, 2>{});
  if (need <= 3) return go(std::integral_constant<int, 3>{});
  if (need <= 4 || cap <= 4) return go(std::integral_constant<int, 4>{});
  return go(std::integral_constant<int, cap>{});
}

template <int XT>
hipError_t launch_qv8_cb(const GemvArgs& a, const GemvArgs& b, bool pair, hipStream_t st) {
  switch (a.k / 1024) {
    case 2: return launch_qv8<XT, 2>(a, b, pair, st);
    case 4: return launch_qv8<XT, 4>(a, b, pair, st);
    case 6: return launch_qv8<XT, 6>(a, b, pair, st);
    case 8: return launch_qv8<XT, 8>(a, b, pair, st);
    case 12: return launch_qv8<XT, 12>(a, b, pair, st);
    case 16: return launch_qv8<XT, 16>(a, b, pair, st);
    default: return hipErrorNotSupported;
  }
}

// rows per wave: enough that one workgroup per CU covers n, within the
// register budget of CB * NU 16-byte chunks per lane
template <int XT, int CB, bool GROUPED>
hipError_t launch_qv(const GemvArgs& a, const GemvArgs& b, bool pair, hipStream_t st) {
  constexpr int kCus = 256;
  const int rows_all = a.n + (pair ? b.n : 0);
  const int need = (rows_all + kCus * kQvWaves - 1) / (kCus * kQvWaves);
  constexpr int cap = CB <= 3 ? (QM_Q4_CAP < 8 ? QM_Q4_CAP : 8) : (CB <= 4 ? (QM_Q4_CAP < 6 ? QM_Q4_CAP : 6) : (QM_Q4_CAP < 4 ? QM_Q4_CAP : 4));
  const size_t lds = (size_t)2048 * CB * 2 + (size_t)2048 * CB / 4;
  auto go = [&](auto nu_tag) {
    constexpr int NU = decltype(nu_tag)::value;
    const int rows = kQvWaves * NU;
    const int nba = (a.n + rows - 1) / rows;
    const int nbb = pair ? (b.n + rows - 1) / rows : 0;
    hipLaunchKernelGGL((qgemv_q_kernel<XT, CB, NU, GROUPED>), dim3(nba + nbb), dim3(kQvThreads), lds, st, a,
                       pair ? b : a, nba);
    return hipGetLastError();
  };
  if (need <= 1 || cap <= 1) return go(std::integral_constant<int, 1>{});
  if (cap <= 2) return go(std::integral_constant<int, (cap < 2 ? 1 : 2)>{});
  if (need <= 2) return go(std::integral_constant<int, 2>{});
  if (need <= 3 || cap <= 3) return go(std::integral_constant<int, (cap < 3 ? cap : 3)>{});
  if (need <= 4 || cap <= 4) return go(std::integral_constant<int, 4>{});
  if (need <= 6 || cap <= 6) return go(std::integral_constant<int, (cap < 6 ? cap : 6)>{});
  return go(std::integral_constant<int, cap>{});
}

template <int XT, bool GROUPED>
hipError_t launch_qv_cb(const GemvArgs& a, const GemvArgs& b, bool pair, hipStream_t st) {
  switch (a.k / 2048) {
    case 1: return launch_qv<XT, 1, GROUPED>(a, b, pair, st);
    case 2: return launch_qv<XT, 2, GROUPED>(a, b, pair, st);
    case 3: return launch_qv<XT, 3, GROUPED>(a, b, pair, st);
    case 4: return launch_qv<XT, 4, GROUPED>(a, b, pair, st);
    case 6: return launch_qv<XT, 6, GROUPED>(a, b, pair, st);
    case 8: return launch_qv<XT, 8, GROUPED>(a, b, pair, st);
    default: return hipErrorNotSupported;
  }
}

#ifndef QM_QGEMV_Q
#define QM_QGEMV_Q 1
#endif

// int4 (grouped or per row), one token, k = 2048 * {1,2,3,4,6,8}, x 16-byte
// aligned; hipErrorNotSupported otherwise (the caller runs the other kernels)
hipError_t launch_qgemv_q(int xdt, bool grouped, const GemvArgs& a, hipStream_t st) {
  if (!QM_QGEMV_Q || a.n < 1 || a.k % 2048 || ((uintptr_t)a.x & 15) != 0) return hipErrorNotSupported;
  if (xdt == kBF16) return grouped ? launch_qv_cb<kBF16, true>(a, a, false, st) : launch_qv_cb<kBF16, false>(a, a, false, st);
  return grouped ? launch_qv_cb<kF32, true>(a, a, false, st) : launch_qv_cb<kF32, false>(a, a, false, st);
}

// int8 per row, one token, k = 1024 * {2,4,6,8,12,16}, x 16-byte aligned
hipError_t launch_qgemv_q8(int xdt, const GemvArgs& a, hipStream_t st) {
  if (!QM_QGEMV_Q || a.n < 1 || a.k % 1024 || ((uintptr_t)a.x & 15) != 0) return hipErrorNotSupported;
  return xdt == kBF16 ? launch_qv8_cb<kBF16>(a, a, false, st) : launch_qv8_cb<kF32>(a, a, false, st);
}

hipError_t launch_qgemv_q8_pair(int xdt, const GemvArgs& a, const GemvArgs& b, hipStream_t st) {
  if (!QM_QGEMV_Q || a.n < 1 || b.n < 1 || a.k != b.k || a.k % 1024 || ((uintptr_t)a.x & 15) != 0)
    return hipErrorNotSupported;
  return xdt == kBF16 ? launch_qv8_cb<kBF16>(a, b, true, st) : launch_qv8_cb<kF32>(a, b, true, st);
}

// int4, 2..8 activation rows (qgemm_small), k = 2048 * {1,2,3,4,6,8} with the
// staged rows fitting in LDS; hipErrorNotSupported otherwise
hipError_t launch_qgemv_qb(int xdt, bool grouped, const GemvArgs& a, hipStream_t st) {
  if (!QM_QGEMV_Q || a.n < 1 || a.nb < 2 || a.nb > 8 || a.k % 2048 || ((uintptr_t)a.x & 15) != 0)
    return hipErrorNotSupported;
  if (xdt == kBF16) return grouped ? launch_qvb_cb<kBF16, true>(a, st) : launch_qvb_cb<kBF16, false>(a, st);
  return grouped ? launch_qvb_cb<kF32, true>(a, st) : launch_qvb_cb<kF32, false>(a, st);
}

// two int4 matrices of one x in one launch (same k and grouping)
hipError_t launch_qgemv_q_pair(int xdt, bool grouped, const GemvArgs& a, const GemvArgs& b, hipStream_t st) {
  if (!QM_QGEMV_Q || a.n < 1 || b.n < 1 || a.k != b.k || a.k % 2048 || ((uintptr_t)a.x & 15) != 0)
    return hipErrorNotSupported;
  if (xdt == kBF16) return grouped ? launch_qv_cb<kBF16, true>(a, b, true, st) : launch_qv_cb<kBF16, false>(a, b, true, st);
  return grouped ? launch_qv_cb<kF32, true>(a, b, true, st) : launch_qv_cb<kF32, false>(a, b, true, st);
}

}  // namespace qm
