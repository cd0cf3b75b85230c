// moe_t1_q.hpp -- routed expert FFN decode (int4 experts, 1..8 tokens, every
// routed (token, slot) pair on its own) on integer dot products: the K-expert group of the colibri page "Vulkan backend:
// expert tier + dense + MLA attention on any Vulkan 1.2 GPU" (gate+up with
// SiLU, then the down projection combined with the routing weights), with the
// activations turned into small integers so that one v_dot8_i32_i4 handles
// eight weights.
//
// Activation digits.  A group of 16 consecutive activations v_i is scaled by
// a power of two, 2^(15-E) with max|v| * 1.072 < 2^E, and rounded to
// integers X_i (|X_i| <= 30567).  Every X_i is written with four balanced
// base-16 digits in [-8, 7] (X = sum_d 16^d dig_d; nibble d is
// ((X + c_d) >> 4d) & 15 with c_d = 0, 0x8, 0x88, 0x888), so the signed range
// [-34952, 30583] covers it.  Digit d of the activations 8j..8j+7 packed as
// two's complement nibbles (activation 8j+i at bits 4i, the weights' own
// nibble order) is word j*4+d.  A weight word XOR 0x88888888 holds the
// signed values n - 8, so v_dot8_i32_i4(w ^ 0x88888888, word) is the exact
// integer sum_i (n_i - 8) dig_d(X_i); the four digit sums recombine with
// shifts into sum_i (n_i - 8) X_i (|.| < 2^22, exact in fp32), which is
// scaled by the weight scale and 2^(E-15).  The only rounding beyond fp32
// accumulation is X_i itself: at most 2^-15 * 1.072 * max|v| per activation
// of the group (exact for activations that are small integers).
//
// gate+up: one workgroup per (routed pair p = token * top_k + slot, tile of
// RPB rows of the intermediate dimension); each wave streams its rows of gate and up through
// an LDS ring (global_load_lds DMA, as in moe_t1_lds.hpp).  The block's h
// values are kept in LDS and turned into digits in its epilogue, so the down
// kernel reads them ready-made.  Several tokens are served pair by pair: an
// expert routed by two tokens is read twice (with independent routing over
// hundreds of experts that is rare).  down: one row of workgroups per token,
// one wave per routed pair of that token, the pair's
// digits in registers, rows of the down matrix loaded straight into registers
// (all of a wave's rows in flight at once; an LDS-ring variant takes the
// shapes whose rows do not fit), lane partials combined in a fixed order as
// in the register-h kernel.
#pragma once
#include "moe_t1_lds.hpp"

namespace qm {

constexpr float kQGuard = 1.072f;  // keeps max|X| at 30567 <= 30583

// E with amax * 1.072 < 2^E (0 when amax == 0)
__device__ __forceinline__ int q_exp(float amax) {
  return amax > 0.f ? __builtin_amdgcn_frexp_expf(amax * kQGuard) : 0;
}

template <int D>
__device__ __forceinline__ uint32_t q_nib(int X) {
  constexpr int c = 0x888 >> (12 - 4 * D);
  return (uint32_t)((X + c) >> (4 * D)) & 15u;
}

// digit word d of the 8 integers X[0..7]
template <int D>
__device__ __forceinline__ uint32_t q_word(const int* X) {
  uint32_t w = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) w |= q_nib<D>(X[i]) << (4 * i);
  return w;
}

__device__ __forceinline__ void q_ints16(const float (&v)[16], int E, int (&X)[16]) {
#pragma unroll
  for (int i = 0; i < 16; ++i) X[i] = (int)__builtin_rintf(ldexpf(v[i], 15 - E));
}

__device__ __forceinline__ float q_amax16(const float (&v)[16]) {
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(v[i]));
  return m;
}

// 16 activations -> 8 digit words (index j*4 + d) and the factor 2^(E-15)
__device__ __forceinline__ float q_group16(const float (&v)[16], uint32_t (&wd)[8]) {
  const int E = q_exp(q_amax16(v));
  int X[16];
  q_ints16(v, E, X);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    wd[j * 4 + 0] = q_word<0>(X + 8 * j);
    wd[j * 4 + 1] = q_word<1>(X + 8 * j);
    wd[j * 4 + 2] = q_word<2>(X + 8 * j);
    wd[j * 4 + 3] = q_word<3>(X + 8 * j);
  }
  return ldexpf(1.f, E - 15);
}

// Workgroup barrier for LDS only: waits for this wave's LDS operations, not
// for its outstanding global loads (__syncthreads() would also wait for
// every load in flight, here the weight prefetch).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ int sdot8(uint32_t a, uint32_t b, int c) {
  return __builtin_amdgcn_sdot8((int)a, (int)b, c, false);
}

// sum over the 32 weights of one 16-byte chunk against the chunk's digits:
// xd[j] = the four digit words of activations 8j..8j+7, xs[g] the factors of
// the chunk's two groups; returns sum_g (sum_{i in g} v_i X_i) * s * xs[g].
__device__ __forceinline__ float q_chunk(const u32x4& w, const u32x4 (&xd)[4], const float (&xs)[2], float s,
                                         float acc) {
  int a[2][4];
#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int d = 0; d < 4; ++d) a[g][d] = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t ws = w[j] ^ 0x88888888u;
#pragma unroll
    for (int d = 0; d < 4; ++d) a[j >> 1][d] = sdot8(ws, xd[j][d], a[j >> 1][d]);
  }
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const int t = (int)((uint32_t)a[g][0] + ((uint32_t)a[g][1] << 4) + ((uint32_t)a[g][2] << 8) +
                        ((uint32_t)a[g][3] << 12));
    acc = __builtin_fmaf((float)t, s * xs[g], acc);
  }
  return acc;
}

// ---- gate + up ----------------------------------------------------------------
// One row of gate and one of up of a routed expert per unit, streamed through
// an LDS ring of D slots per wave.
template <int CB, bool PS>
__host__ __device__ constexpr int q_gu_slot() {
  return 2 * CB * 1024 + (PS ? 1024 : 2 * CB * 256);
}

// One gate+up tile: routed pair p, intermediate rows r0 .. r0+RPB-1 (h to
// a.h when set, its digits to a.hq when set; COHERENT: the digits go out as
// device-coherent stores, for readers in other workgroups of the same
// launch).  Returns false for a pair with an invalid expert id (nothing done).
template <int XT, int CB, int RPB, int D, bool GROUPED, bool PS, bool COHERENT>
__device__ __forceinline__ bool gu_tile(const MoeDecodeArgs& a, char* lds, float* s_h, int p, int r0) {
  constexpr int M = 2;
  constexpr int NW = M * CB;              // 1 KiB weight blocks per unit
  constexpr int U = NW + (PS ? 1 : NW);   // VMEM operations per unit
  constexpr int SLOT = q_gu_slot<CB, PS>();
  constexpr int NU = RPB / kWaves;        // units per wave
  static_assert(!PS || GROUPED, "packed scales need grouped scales");
  static_assert(RPB % 16 == 0 && RPB % kWaves == 0, "tile of whole digit groups");
  const ExpertArgs& ex = a.ex;
  const int id = a.ids[p];
  if (id < 0 || id >= ex.E) return false;  // the down kernel skips this slot
  const char* xt = static_cast<const char*>(a.x) + (size_t)(p / a.topk) * ex.H * (XT == kBF16 ? 2 : 4);
  const int e = uniform(id);
  const int wave = uniform(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int H = ex.H;
  uint32_t* xq = reinterpret_cast<uint32_t*>(lds);                          // [H/16][8]
  float* xsc = reinterpret_cast<float*>(lds + (size_t)H * 2);                // [H/16]
  char* ring = lds + align_lds((size_t)H * 2 + (size_t)H / 4) + (size_t)wave * D * SLOT;
  auto issue = [&](int u, int slot) {
    const int r = r0 + wave + kWaves * u;
    const int64_t er = (int64_t)e * ex.I + r;
    char* sd = ring + slot * SLOT;
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const uint8_t* qrow = (m == 0 ? ex.gq : ex.uq) + er * ex.rb_h;
      const float* srow = (m == 0 ? ex.gs : ex.us) + er * ex.G_h;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const int c = lane + 64 * cb;
        const int blk = m * CB + cb;
        dma16(qrow + (int64_t)c * 16, sd + blk * 1024);
        if constexpr (!PS) dma4(srow + (GROUPED ? (c >> ex.gshift) : 0), sd + NW * 1024 + blk * 256);
      }
    }
    if constexpr (PS) {
      // floats 4f .. 4f+3 of the unit's two scale rows [m][G]; lanes past the
      // last piece reload it
      const int G = ex.G_h;
      const int f = 4 * min(lane, 2 * G / 4 - 1);
      const int m = f / G, g = f - m * G;
      const float* srow = (m == 0 ? ex.gs : ex.us) + er * G + g;
      dma16(srow, sd + NW * 1024);
    }
  };
  // the token's activations, fetched before the weight DMA so that waiting for
  // them does not wait for the ring (VMEM operations complete in order)
  constexpr int NG = (128 * CB + kThreads - 1) / kThreads;  // groups of 16 per thread (H = 2048 CB)
  constexpr int NR = XT == kBF16 ? 2 : 4;                    // 16-byte pieces per group
  u32x4 raw[NG][NR];
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    const int g = threadIdx.x + gi * kThreads;
    if (g < H / 16) {
      const u32x4* src = reinterpret_cast<const u32x4*>(xt + (size_t)g * 16 * (XT == kBF16 ? 2 : 4));
#pragma unroll
      for (int r = 0; r < NR; ++r) raw[gi][r] = src[r];
    }
  }
#pragma unroll
  for (int u = 0; u < D; ++u)
    if (u < NU) issue(u, u);

  // ... as digit words in LDS, once per block
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    const int g = threadIdx.x + gi * kThreads;
    if (g < H / 16) {
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
  lds_barrier();  // the digits are in LDS; the weight DMA stays in flight
  u32x4 xd[CB][4];
  float xs[CB][2];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const int c = lane + 64 * cb;
    const u32x4* src = reinterpret_cast<const u32x4*>(xq + (size_t)c * 16);
#pragma unroll
    for (int j = 0; j < 4; ++j) xd[cb][j] = src[j];
    xs[cb][0] = xsc[2 * c];
    xs[cb][1] = xsc[2 * c + 1];
  }

  for (int u = 0; u < NU; ++u) {
    wait_units<U, D>(min(D - 1, NU - 1 - u));
    const char* sd = ring + (u % D) * SLOT;
    float acc[M] = {0.f, 0.f};
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const int c = lane + 64 * cb;
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const int blk = m * CB + cb;
        const u32x4 w = *reinterpret_cast<const u32x4*>(sd + blk * 1024 + lane * 16);
        const float s = PS ? *reinterpret_cast<const float*>(sd + NW * 1024 + (m * ex.G_h + (c >> ex.gshift)) * 4)
                           : *reinterpret_cast<const float*>(sd + NW * 1024 + blk * 256 + lane * 4);
        acc[m] = q_chunk(w, xd[cb], xs[cb], s, acc[m]);
      }
    }
    slot_release();
    if (u + D < NU) issue(u + D, u % D);
    const float g = group_sum<64>(acc[0]);
    const float v = group_sum<64>(acc[1]);
    if (lane == 0) {
      const float hv = silu(g) * v;
      const int rl = wave + kWaves * u;
      s_h[rl] = hv;
      if (a.h) a.h[(int64_t)p * ex.I + r0 + rl] = hv;
    }
  }
  if (!a.hq) return true;
  __syncthreads();
  // digits of the tile's h: eight threads per group of 16, one word each
  // (shift and carry constant of digit d computed, not branched on)
  if (threadIdx.x < RPB / 16 * 8) {
    const int g = threadIdx.x >> 3, j = (threadIdx.x >> 2) & 1, d = threadIdx.x & 3;
    const f32x4* hv = reinterpret_cast<const f32x4*>(s_h + g * 16);
    float amax = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const f32x4 t = hv[r];
      amax = fmaxf(fmaxf(amax, fmaxf(fabsf(t[0]), fabsf(t[1]))), fmaxf(fabsf(t[2]), fabsf(t[3])));
    }
    const int E = q_exp(amax);
    const int sh = 4 * d, c = 0x888 >> (12 - sh);
    uint32_t w = 0;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const f32x4 t = hv[2 * j + r];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int X = (int)__builtin_rintf(ldexpf(t[i], 15 - E));
        w |= ((uint32_t)((X + c) >> sh) & 15u) << (4 * (4 * r + i));
      }
    }
    const int64_t gi = (int64_t)p * (ex.I / 16) + r0 / 16 + g;  // global group index
    if constexpr (COHERENT) {
      __hip_atomic_store(a.hq + gi * 8 + j * 4 + d, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if ((threadIdx.x & 7) == 0)
        __hip_atomic_store(a.hqs + gi, ldexpf(1.f, E - 15), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      a.hq[gi * 8 + j * 4 + d] = w;
      if ((threadIdx.x & 7) == 0) a.hqs[gi] = ldexpf(1.f, E - 15);
    }
  }
  return true;
}

// H = 64 * CB * 32 (a lane owns chunks lane + 64 cb of every row).  Block b:
// routed pair b / ntile (pair p = token * topk + slot), rows
// [RPB * (b % ntile), +RPB); wave w takes rows w, w + kWaves, ... of the tile.
template <int XT, int CB, int RPB, int D, bool GROUPED, bool PS>
__global__ __launch_bounds__(kThreads) void moe_gate_up_t1q_kernel(MoeDecodeArgs a) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  __shared__ __attribute__((aligned(16))) float s_h[RPB];
  const int ntile = a.ex.I / RPB;
  const int p = blockIdx.x / ntile, r0 = (blockIdx.x - p * ntile) * RPB;
  gu_tile<XT, CB, RPB, D, GROUPED, PS, false>(a, lds, s_h, p, r0);
}

// h (fp32 [T*k][I]) -> digit words and factors, one thread per group of 16;
// used when the hidden vectors come from the caller rather than from the
// gate+up kernel above.
template <int NT>
__global__ __launch_bounds__(NT) void hq_digits_kernel(const float* __restrict__ h, uint32_t* __restrict__ hq,
                                                        float* __restrict__ hqs, int ngroups) {
  const int g = blockIdx.x * NT + threadIdx.x;
  if (g >= ngroups) return;
  float v[16];
  const f32x4* src = reinterpret_cast<const f32x4*>(h + (size_t)g * 16);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f32x4 t = src[i];
    v[4 * i] = t[0];
    v[4 * i + 1] = t[1];
    v[4 * i + 2] = t[2];
    v[4 * i + 3] = t[3];
  }
  uint32_t wd[8];
  hqs[g] = q_group16(v, wd);
  u32x4* dst = reinterpret_cast<u32x4*>(hq + (size_t)g * 8);
  dst[0] = u32x4{wd[0], wd[1], wd[2], wd[3]};
  dst[1] = u32x4{wd[4], wd[5], wd[6], wd[7]};
}

// ---- down + weighted combine ----------------------------------------------------
// As moe_down_t1r_kernel, with the pair's digits (CPL chunks per lane) in
// registers instead of bf16 hi/lo pairs.
template <int L, int CPL, int D, bool GROUPED>
__global__ __launch_bounds__(kDT) void moe_down_t1q_kernel(MoeDecodeArgs a) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  __shared__ int s_e[kTopkMax], s_p[kTopkMax], s_n;
  __shared__ float s_w[kTopkMax];
  constexpr int PPW = 64 / L;
  constexpr int U = 2 * CPL;  // VMEM operations per unit
  constexpr int SLOT = ring_slot_bytes<1, 1, CPL>();
  const ExpertArgs& ex = a.ex;
  routed_pairs(a.ids, a.w, a.topk, ex.E, s_e, s_p, s_w, &s_n);
  __syncthreads();
  const int np = s_n;
  const int npg = (np + PPW - 1) / PPW;
  int npg2 = 1;
  while (npg2 < npg) npg2 <<= 1;
  const int S = kDW / npg2;
  const int wave = uniform(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int pg = wave % npg2, sl = wave / npg2;
  const int qi = lane / L, sub = lane - qi * L;
  const int q = pg * PPW + qi;
  const bool qok = pg < npg && q < np;
  const int qq = qok ? q : 0;
  const int e = s_e[qq], prow = s_p[qq];
  const float wq = qok ? s_w[qq] : 0.f;
  const int R = (ex.H + gridDim.x - 1) / gridDim.x;
  const int r0 = blockIdx.x * R, r1 = min(ex.H, r0 + R);
  float* part = reinterpret_cast<float*>(lds + (size_t)kDW * D * SLOT);  // [R][kDW][64] lane partials
  char* ring = lds + (size_t)wave * D * SLOT;
  const int span = r1 - r0 - sl;
  const int nunits = (pg < npg && span > 0) ? (span + S - 1) / S : 0;  // wave-uniform
  auto issue = [&](int u, int slot) {
    const int r = r0 + sl + S * u;
    const int64_t er = (int64_t)e * ex.H + r;
    const uint8_t* qrow = ex.dq + er * ex.rb_i;
    const float* srow = ex.ds + er * ex.G_i;
    char* sd = ring + slot * SLOT;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int c = sub + L * i;
      dma16(qrow + (int64_t)c * 16, sd + i * 1024);
      dma4(srow + (GROUPED ? (c >> ex.gshift) : 0), sd + CPL * 1024 + i * 256);
    }
  };
#pragma unroll
  for (int u = 0; u < D - 1; ++u)
    if (u < nunits) issue(u, u);

  u32x4 hd[CPL][4];
  float hs[CPL][2];
  const uint32_t* hqrow = a.hq + (int64_t)prow * (ex.I / 16) * 8;
  const float* hsrow = a.hqs + (int64_t)prow * (ex.I / 16);
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const int c = sub + L * i;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      hd[i][j] = qok ? *reinterpret_cast<const u32x4*>(hqrow + (size_t)c * 16 + j * 4) : u32x4{0u, 0u, 0u, 0u};
    hs[i][0] = qok ? hsrow[2 * c] : 0.f;
    hs[i][1] = qok ? hsrow[2 * c + 1] : 0.f;
  }
  for (int u = 0; u < nunits; ++u) {
    wait_units_upto<U, D - 2>(min(D - 2, nunits - 1 - u));
    const char* sd = ring + (u % D) * SLOT;
    float t = 0.f;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(sd + i * 1024 + lane * 16);
      const float sc = *reinterpret_cast<const float*>(sd + CPL * 1024 + i * 256 + lane * 4);
      t = q_chunk(w, hd[i], hs[i], sc, t);
    }
    slot_release();
    if (u + D - 1 < nunits) issue(u + D - 1, (u + D - 1) % D);
    part[((sl + S * u) * kDW + pg) * 64 + lane] = wq * t;
  }
  __syncthreads();
  for (int i = wave; i < r1 - r0; i += kDW) {
    float v = 0.f;
    for (int g = 0; g < npg; ++g) v += part[(i * kDW + g) * 64 + lane];
    v = group_sum<64>(v);
    if (lane == 0) a.y[r0 + i] = v;
  }
}

// ---- down + weighted combine, weights prefetched into registers ----------------
// The same work split as moe_down_t1q_kernel, but a lane's share of one unit
// (CPL 16-byte chunks and their scales) is small enough that a wave issues
// the loads of all its NU units at once into registers: no LDS ring, every
// byte of the wave's rows in flight from the start.  Units past the wave's
// last row reload that row and are dropped.
template <int L, int CPL, int NU, bool GROUPED>
__global__ __launch_bounds__(kDT) void moe_down_t1qr_kernel(MoeDecodeArgs a) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  __shared__ int s_e[kTopkMax], s_p[kTopkMax], s_n;
  __shared__ float s_w[kTopkMax];
  constexpr int PPW = 64 / L;
  const ExpertArgs& ex = a.ex;
  const int tok = blockIdx.y;  // token; its routed pairs are rows tok * topk + slot of h
  routed_pairs(a.ids + tok * a.topk, a.w + tok * a.topk, a.topk, ex.E, s_e, s_p, s_w, &s_n);
  __syncthreads();
  const int np = s_n;
  const int npg = (np + PPW - 1) / PPW;
  int npg2 = 1;
  while (npg2 < npg) npg2 <<= 1;
  const int S = kDW / npg2;
  const int wave = uniform(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int pg = wave % npg2, sl = wave / npg2;
  const int qi = lane / L, sub = lane - qi * L;
  const int q = pg * PPW + qi;
  const bool qok = pg < npg && q < np;
  const int qq = qok ? q : 0;
  const int e = s_e[qq], prow = tok * a.topk + s_p[qq];
  const float wq = qok ? s_w[qq] : 0.f;
  const int R = (ex.H + gridDim.x - 1) / gridDim.x;
  const int r0 = blockIdx.x * R, r1 = min(ex.H, r0 + R);
  float* yt = a.y + (int64_t)tok * ex.H;
  float* part = reinterpret_cast<float*>(lds);  // [R][kDW][64] lane partials
  const int span = r1 - r0 - sl;
  const int nunits = (pg < npg && span > 0) ? (span + S - 1) / S : 0;  // wave-uniform, <= NU
  if (nunits > 0) {
    u32x4 hd[CPL][4];
    float hs[CPL][2];
    const uint32_t* hqrow = a.hq + (int64_t)prow * (ex.I / 16) * 8;
    const float* hsrow = a.hqs + (int64_t)prow * (ex.I / 16);
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int c = sub + L * i;
#pragma unroll
      for (int j = 0; j < 4; ++j) hd[i][j] = *reinterpret_cast<const u32x4*>(hqrow + (size_t)c * 16 + j * 4);
      hs[i][0] = hsrow[2 * c];
      hs[i][1] = hsrow[2 * c + 1];
    }
    u32x4 wv[NU][CPL];
    float sv[NU][CPL];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int r = r0 + sl + S * min(u, nunits - 1);
      const int64_t er = (int64_t)e * ex.H + r;
      const uint8_t* qrow = ex.dq + er * ex.rb_i;
      const float* srow = ex.ds + er * ex.G_i;
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        const int c = sub + L * i;
        wv[u][i] = ld_stream(qrow + (int64_t)c * 16);
        sv[u][i] = ld_stream(srow + (GROUPED ? (c >> ex.gshift) : 0));
      }
    }
    const float wz = qok ? wq : 0.f;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      float t = 0.f;
#pragma unroll
      for (int i = 0; i < CPL; ++i) t = q_chunk(wv[u][i], hd[i], hs[i], sv[u][i], t);
      if (u < nunits) part[((sl + S * u) * kDW + pg) * 64 + lane] = wz * t;
    }
  }
  __syncthreads();
  for (int i = wave; i < r1 - r0; i += kDW) {
    float v = 0.f;
    for (int g = 0; g < npg; ++g) v += part[(i * kDW + g) * 64 + lane];
    v = group_sum<64>(v);
    if (lane == 0) yt[r0 + i] = v;
  }
}

// ---- launch ---------------------------------------------------------------------

#ifndef QM_T1Q
#define QM_T1Q 1
#endif
constexpr int kQMaxTokens = 8;  // tokens per decode pass (one workgroup row of the grid per token in down)
#ifndef QM_T1Q_GU_MIN_CB
#define QM_T1Q_GU_MIN_CB 1
#endif
#ifndef QM_T1Q_DN_D
#define QM_T1Q_DN_D 4
#endif
#ifndef QM_T1Q_DN_BLOCKS
#define QM_T1Q_DN_BLOCKS 512
#endif

template <int CB>
constexpr int q_gu_depth() { return CB <= 2 ? 3 : 2; }

template <int CB, bool PS>
inline size_t q_gu_lds(int H) {
  return align_lds((size_t)H * 2 + (size_t)H / 4) + (size_t)kWaves * q_gu_depth<CB>() * q_gu_slot<CB, PS>();
}

// rows per gate+up tile: 32 when that still gives two workgroups per CU
inline int q_gu_rpb(const MoeDecodeArgs& a) { return (a.T * a.topk * (a.ex.I / 32) >= 512) ? 32 : 16; }

// Does the digit gate+up kernel take this call?  int4 experts, one token,
// H = 2048 * CB (CB <= 4), I a multiple of 32 and of the row tile.
inline bool q_gate_up_ok(const MoeDecodeArgs& a) {
  if (!QM_T1Q || a.T < 1 || a.T > kQMaxTokens || a.topk > kTopkMax) return false;
  if (a.ex.H % 2048 || a.ex.H / 2048 > 4 || a.ex.H / 2048 < QM_T1Q_GU_MIN_CB) return false;
  if (a.ex.I % 32 || a.ex.I % q_gu_rpb(a)) return false;
  if (((uintptr_t)a.x & 15) != 0) return false;
  return true;
}

// Does the digit down kernel take this call?  int4 experts, one token, a
// down row of 64 or 128 chunks (L = 64) or, for 9..16 slots, of 64 chunks
// with two pairs per wave; needs the digit buffers.
inline bool q_down_shape(const MoeDecodeArgs& a, int* L, int* cpl) {
  if (!QM_T1Q || a.T < 1 || a.T > kQMaxTokens || a.topk > kTopkMax || !a.hq) return false;
  const int kch = a.ex.I / 32;
  if (a.ex.I % 32) return false;
  if (kch % 64 == 0 && kch / 64 <= 2 && a.topk <= kDW) {
    *L = 64;
    *cpl = kch / 64;
  } else if (kch == 64 && (a.topk + 1) / 2 <= kDW) {
    *L = 32;
    *cpl = 2;
  } else {
    return false;
  }
  return true;
}

template <int XT, int CB, bool GROUPED, bool PS>
inline hipError_t launch_gu_t1q(const MoeDecodeArgs& a, hipStream_t st) {
  constexpr int D = q_gu_depth<CB>();
  const size_t lds = q_gu_lds<CB, PS>(a.ex.H);
  if (lds > (size_t)kLdsMax) return hipErrorNotSupported;
  const int rpb = q_gu_rpb(a);
  const int blocks = a.T * a.topk * (a.ex.I / rpb);
  if (rpb == 32)
    hipLaunchKernelGGL((moe_gate_up_t1q_kernel<XT, CB, 32, D, GROUPED, PS>), dim3(blocks), dim3(kThreads), lds, st,
                       a);
  else
    hipLaunchKernelGGL((moe_gate_up_t1q_kernel<XT, CB, 16, D, GROUPED, PS>), dim3(blocks), dim3(kThreads), lds, st,
                       a);
  return hipGetLastError();
}

template <int XT, int CB, bool GROUPED>
inline hipError_t launch_gu_t1q_ps(const MoeDecodeArgs& a, hipStream_t st) {
  if constexpr (GROUPED) {
    if (gu_packed_scales(a, 1)) return launch_gu_t1q<XT, CB, true, true>(a, st);
  }
  return launch_gu_t1q<XT, CB, GROUPED, false>(a, st);
}

// hipErrorNotSupported: not taken (the caller goes on to the other kernels)
template <int XT, bool GROUPED>
inline hipError_t try_gate_up_t1q(const MoeDecodeArgs& a, hipStream_t st) {
  if (!q_gate_up_ok(a)) return hipErrorNotSupported;
  switch (a.ex.H / 2048) {
    case 1: return launch_gu_t1q_ps<XT, 1, GROUPED>(a, st);
    case 2: return launch_gu_t1q_ps<XT, 2, GROUPED>(a, st);
    case 3: return launch_gu_t1q_ps<XT, 3, GROUPED>(a, st);
    default: return launch_gu_t1q_ps<XT, 4, GROUPED>(a, st);
  }
}

#ifndef QM_T1QR
#define QM_T1QR 1
#endif
#ifndef QM_T1QR_NU
#define QM_T1QR_NU 8
#endif

// register-prefetch down kernel: units per wave = rows per block / row slices
template <int L, int CPL, bool GROUPED>
inline hipError_t launch_dn_t1qr(const MoeDecodeArgs& a, hipStream_t st) {
  constexpr int NU = QM_T1QR_NU / CPL;
  constexpr int PPW = 64 / L;
  const int npg = (a.topk + PPW - 1) / PPW;
  int npg2 = 1;
  while (npg2 < npg) npg2 <<= 1;
  if (!QM_T1QR || npg2 > kDW) return hipErrorNotSupported;
  const int S = kDW / npg2;
  const int blocks = (a.ex.H + NU * S - 1) / (NU * S);  // R = ceil(H / blocks) <= NU * S rows
  const int R = (a.ex.H + blocks - 1) / blocks;
  if ((R + S - 1) / S > NU) return hipErrorNotSupported;
  const size_t lds = (size_t)R * kDW * 64 * 4;
  if (lds > (size_t)kLdsMax) return hipErrorNotSupported;
  hipLaunchKernelGGL((moe_down_t1qr_kernel<L, CPL, NU, GROUPED>), dim3(blocks, a.T), dim3(kDT), lds, st, a);
  return hipGetLastError();
}

template <int L, int CPL, bool GROUPED>
inline hipError_t launch_dn_t1q(const MoeDecodeArgs& a, hipStream_t st) {
  {
    const hipError_t er = launch_dn_t1qr<L, CPL, GROUPED>(a, st);
    if (er != hipErrorNotSupported || a.T != 1) return er;  // the ring kernel below takes one token
  }
  constexpr int D = (CPL == 1 || L == 32) ? QM_T1Q_DN_D : (QM_T1Q_DN_D + 1) / 2;
  constexpr int PPW = 64 / L;
  const int npg = (a.topk + PPW - 1) / PPW;
  int npg2 = 1;
  while (npg2 < npg) npg2 <<= 1;
  if (npg2 > kDW) return hipErrorNotSupported;
  const int S = kDW / npg2;
  int blocks = a.max_blocks > 0 ? a.max_blocks : (L == 32 ? QM_T1Q_DN_BLOCKS / 2 : QM_T1Q_DN_BLOCKS);
  if (blocks > (a.ex.H + S - 1) / S) blocks = (a.ex.H + S - 1) / S;
  const int R = (a.ex.H + blocks - 1) / blocks;
  const size_t lds = (size_t)kDW * D * ring_slot_bytes<1, 1, CPL>() + (size_t)R * kDW * 64 * 4;
  if (lds > (size_t)kLdsMax) return hipErrorNotSupported;
  hipLaunchKernelGGL((moe_down_t1q_kernel<L, CPL, D, GROUPED>), dim3(blocks), dim3(kDT), lds, st, a);
  return hipGetLastError();
}

// hq_ready: the digits of a.h are already in a.hq (written by the gate+up
// kernel above); otherwise they are made from a.h first.
template <bool GROUPED>
inline hipError_t try_down_t1q(const MoeDecodeArgs& a, bool hq_ready, hipStream_t st) {
  int L = 0, cpl = 0;
  if (!q_down_shape(a, &L, &cpl)) return hipErrorNotSupported;
  if (!hq_ready) {
    const int ngroups = a.T * a.topk * (a.ex.I / 16);
    hipLaunchKernelGGL(hq_digits_kernel<256>, dim3((ngroups + 255) / 256), dim3(256), 0, st, a.h, a.hq, a.hqs, ngroups);
    const hipError_t e0 = hipGetLastError();
    if (e0 != hipSuccess) return e0;
  }
  if (L == 32) return launch_dn_t1q<32, 2, GROUPED>(a, st);
  if (cpl == 1) return launch_dn_t1q<64, 1, GROUPED>(a, st);
  return launch_dn_t1q<64, 2, GROUPED>(a, st);
}

}  // namespace qm
