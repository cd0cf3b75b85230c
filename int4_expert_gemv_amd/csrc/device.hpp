// device.hpp -- building blocks shared by the quantized GEMV and the MoE
// decode kernels (gfx950, wave64).
//
// Weight formats (colibri page "Vulkan backend: expert tier + dense + MLA
// attention on any Vulkan 1.2 GPU", commit notes "backend_vulkan.c/.h +
// shaders/qmatmul.comp" and "fmt=4 grouped scales"): int4 value = nibble - 8,
// two nibbles per byte with element 2j in the low nibble of byte j, one fp32
// scale per gs consecutive inputs of a row (or one per row); int8 is two's
// complement with one fp32 scale per row.
//
// Work mapping.  A row's inputs are cut into 16-byte "chunks" (32 int4 or 16
// int8 weights); each lane streams whole chunks with one 128-bit load, so a
// wave reads 1 KiB of contiguous row bytes per load instruction.  L lanes
// (16, 32 or 64) share a row; a wave covers 64/L rows per load and RU such
// row sets per tile.  The activation vector is staged once per block in LDS,
// already in the layout the inner loop consumes, and reused for every row.
//
// int4 inner loop.  For a 32-bit word holding 8 nibbles n0..n7, the value
// (w >> 4i) & 0x000F000F | 0x43004300 is a pair of bf16 numbers
// (128 + n_i, 128 + n_{i+4}) -- exact, since bf16 128.0 = 0x4300 has seven
// free mantissa bits.  One v_dot2 (bf16 x bf16 -> fp32 accumulate) then
// consumes two weights.  x is staged as matching bf16 pairs (x_i, x_{i+4}),
// and the 128 + 8 = 136 offset is removed by starting each chunk's
// accumulator at -136 * (sum of the chunk's x).  Cost: 7 VALU ops to unpack
// and 4 dot2 per 8 weights.  fp32 activations are split into x = hi + lo with
// hi = bf16(x), lo = bf16(x - hi) and both halves are dotted (error bounded
// by 2^-17 |x| per element, far inside the fp32-accumulation tolerance).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qm {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kLdsBudget = 64 * 1024;  // bytes of activation staging per block
#ifndef QM_V2_MAX_BLOCKS
#define QM_V2_MAX_BLOCKS 1024
#endif
constexpr int kV2MaxBlocks = QM_V2_MAX_BLOCKS;  // grid cap of the pipelined kernels

constexpr int kTopkMax = 32;  // largest top_k accepted by the C ABI

constexpr int kFmtInt8 = 1;
constexpr int kFmtInt4 = 4;
constexpr int kFmtInt3 = 5;
constexpr int kF32 = 0;
constexpr int kBF16 = 1;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

template <int FMT> struct Fmt;
template <> struct Fmt<kFmtInt4> { static constexpr int kPerChunk = 32; };  // weights per 16 B
template <> struct Fmt<kFmtInt8> { static constexpr int kPerChunk = 16; };

// ---- scalar helpers -----------------------------------------------------------

__device__ __forceinline__ uint32_t nib_pair(uint32_t w) { return (w & 0x000F000Fu) | 0x43004300u; }

// The same pair built with one v_and_or_b32.  gfx9 VOP3 encodings take no
// literal constants and read at most one SGPR, so the mask comes in an SGPR
// and the bf16 128.0 pair in a VGPR (both loop-invariant, set up once).
struct NibConst {
  uint32_t mask;  // 0x000F000F, scalar register
  uint32_t base;  // 0x43004300, vector register
};

__device__ __forceinline__ NibConst nib_const() {
  NibConst k;
  k.mask = __builtin_amdgcn_readfirstlane(0x000F000Fu);
  asm volatile("v_mov_b32 %0, 0x43004300" : "=v"(k.base));
  return k;
}

__device__ __forceinline__ uint32_t nib_pair(uint32_t w, const NibConst& k) {
  uint32_t d;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(d) : "v"(w), "s"(k.mask), "v"(k.base));
  return d;
}

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c,
                                         false);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

// Weights and scales are read exactly once per call: stream them with
// non-temporal loads so they do not displace the activations, the hidden
// vectors and the other waves' data from the caches.
__device__ __forceinline__ u32x4 ld_stream(const uint8_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ float ld_stream(const float* p) { return __builtin_nontemporal_load(p); }

// fp32 -> bf16 bits, round to nearest even (v_cvt_pk_bf16_f32 on gfx950)
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}

// The token's valid routed pairs in slot order -- expert id, slot, routing
// weight -- compacted by wave 0 with the slots read in parallel (one load
// latency rather than one per slot); the caller's __syncthreads() publishes
// them.  topk <= kTopkMax <= 64.
__device__ __forceinline__ void routed_pairs(const int32_t* ids, const float* w, int topk, int E, int* s_e,
                                             int* s_p, float* s_w, int* s_n) {
  if (threadIdx.x < 64) {
    const int j = threadIdx.x;
    const int id = j < topk ? ids[j] : -1;
    const float wj = j < topk ? w[j] : 0.f;
    const bool ok = id >= 0 && id < E;
    const unsigned long long m = __ballot(ok);
    const int n = __popcll(m & ((1ull << j) - 1));
    if (ok) {
      s_e[n] = id;
      s_p[n] = j;
      s_w[n] = wj;
    }
    if (j == 0) *s_n = __popcll(m);
  }
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

// Sum over aligned groups of L lanes; every lane of a group ends with the sum.
template <int L>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (L >= 2)  // lane ^ 1
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
  if constexpr (L >= 4)  // lane ^ 2
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
  if constexpr (L >= 8)  // row_half_mirror: the other quad of the 8-lane half-row
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));
  if constexpr (L >= 16)  // row_mirror: the other half of the 16-lane row
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));
  if constexpr (L >= 32) v += __shfl_xor(v, 16, 64);
  if constexpr (L >= 64) v += __shfl_xor(v, 32, 64);
  return v;
}

// ---- activation staging ------------------------------------------------------
//
// LDS layout for one segment of `segc` chunks and NB tokens:
//  int4: hi pairs  [NB][4 words][segc] x 16 B  (word j: pairs (x_{8j+i}, x_{8j+4+i}), i<4)
//        lo pairs  [NB][4][segc] x 16 B       (fp32 activations only)
//        offsets   [NB][segc] fp32            (-136 * sum of the chunk's activations)
//  int8: values    [NB][4 quarters][segc] x 16 B (quarter j: fp32 x_{4j..4j+3})
// Consecutive lanes read consecutive 16-byte slots, so the reads are
// bank-conflict free.

template <int FMT, bool SPLIT>
__host__ __device__ constexpr int stage_bytes_per_chunk() {
  return FMT == kFmtInt4 ? (SPLIT ? 132 : 68) : 64;
}

// tok(b) gives the activation row of batch slot b (a callable, so that the
// caller's token list can live in registers or in LDS).
template <int FMT, int XT, int NB, typename TokF>
__device__ __forceinline__ void stage_x(char* __restrict__ lds, const void* __restrict__ x, int64_t ldx,
                                        TokF tok, int kc0, int segc) {
  constexpr bool SPLIT = (FMT == kFmtInt4 && XT == kF32);
  constexpr int PER = Fmt<FMT>::kPerChunk;
  u32x4* hi = reinterpret_cast<u32x4*>(lds);
  u32x4* lo = hi + NB * 4 * segc;
  float* off = reinterpret_cast<float*>(lds + (size_t)NB * 4 * segc * 16 * (SPLIT ? 2 : 1));
  for (int it = threadIdx.x; it < NB * segc; it += kThreads) {
    const int b = it / segc, c = it - b * segc;
    const int64_t e0 = (int64_t)tok(b) * ldx + (int64_t)(kc0 + c) * PER;
    float v[PER];
    if constexpr (XT == kBF16) {
      const u32x4* src = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(x) + e0);
#pragma unroll
      for (int m = 0; m < PER / 8; ++m) {
        u32x4 d = src[m];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          v[8 * m + 2 * t] = bf16_bits_to_f32(d[t] & 0xFFFFu);
          v[8 * m + 2 * t + 1] = bf16_bits_to_f32(d[t] >> 16);
        }
      }
    } else {
      const f32x4* src = reinterpret_cast<const f32x4*>(static_cast<const float*>(x) + e0);
#pragma unroll
      for (int m = 0; m < PER / 4; ++m) {
        f32x4 d = src[m];
#pragma unroll
        for (int t = 0; t < 4; ++t) v[4 * m + t] = d[t];
      }
    }
    if constexpr (FMT == kFmtInt4) {
      float sum = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u32x4 ph, pl;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float a = v[8 * j + i], bq = v[8 * j + 4 + i];
          const uint32_t ha = f32_to_bf16_bits(a), hb = f32_to_bf16_bits(bq);
          ph[i] = ha | (hb << 16);
          if constexpr (SPLIT) {
            const float ra = a - bf16_bits_to_f32(ha), rb = bq - bf16_bits_to_f32(hb);
            const uint32_t la = f32_to_bf16_bits(ra), lb = f32_to_bf16_bits(rb);
            pl[i] = la | (lb << 16);
            sum += (bf16_bits_to_f32(ha) + bf16_bits_to_f32(la)) + (bf16_bits_to_f32(hb) + bf16_bits_to_f32(lb));
          } else {
            sum += bf16_bits_to_f32(ha) + bf16_bits_to_f32(hb);
          }
        }
        hi[(b * 4 + j) * segc + c] = ph;
        if constexpr (SPLIT) lo[(b * 4 + j) * segc + c] = pl;
      }
      off[b * segc + c] = -136.0f * sum;
    } else {
      f32x4* q4 = reinterpret_cast<f32x4*>(lds);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f32x4 t4 = {v[4 * j], v[4 * j + 1], v[4 * j + 2], v[4 * j + 3]};
        q4[(b * 4 + j) * segc + c] = t4;
      }
    }
  }
}

// ---- per-tile partial dot products --------------------------------------------
//
// For each of M matrices (same shape, e.g. an expert's gate and up) adds to
// acc[m][j][b] this lane's share of  sum_c W_m[row_j][c] * x_b[c]  over the
// staged segment [kc0, kc0 + segc) chunks, with row_j = row0 + j * rstride.
// GROUPED (int4 only): each chunk's partial is multiplied by its group scale
// (chunk index >> gshift selects the group); otherwise the row scale is
// applied by the caller after the lane reduction.  All weight loads of a
// batch of CB chunks are issued before any of them is consumed.

template <int M>
struct Mats {
  const uint8_t* q[M];
  const float* s[M];
};

template <int FMT, bool SPLIT, int L, int M, int RU, int NB, bool GROUPED>
__device__ __forceinline__ void tile_partial(const Mats<M>& mt, int64_t row_bytes, int G, int gshift,
                                             int row0, int rstride, int nrows, int kc0, int segc,
                                             const char* __restrict__ lds, float (&acc)[M][RU][NB]) {
  constexpr int CB = (M * RU >= 4) ? 4 : 8;  // chunks in flight per lane per row
  const int li = (threadIdx.x & 63) % L;
  const u32x4* hi = reinterpret_cast<const u32x4*>(lds);
  const u32x4* lo = hi + NB * 4 * segc;
  const float* off = reinterpret_cast<const float*>(lds + (size_t)NB * 4 * segc * 16 * (SPLIT ? 2 : 1));
  const f32x4* xf = reinterpret_cast<const f32x4*>(lds);

  for (int c0 = li; c0 < segc; c0 += L * CB) {
    u32x4 w[CB][M][RU];
    float s[CB][M][RU];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const int c = c0 + cb * L;
#pragma unroll
      for (int m = 0; m < M; ++m)
#pragma unroll
        for (int j = 0; j < RU; ++j) {
          const int r = row0 + j * rstride;
          if (c < segc && r < nrows) {
            w[cb][m][j] =
                *reinterpret_cast<const u32x4*>(mt.q[m] + (int64_t)r * row_bytes + (int64_t)(kc0 + c) * 16);
            s[cb][m][j] = GROUPED ? mt.s[m][(int64_t)r * G + ((kc0 + c) >> gshift)] : 1.0f;
          } else {
            const uint32_t z = (FMT == kFmtInt4) ? 0x88888888u : 0u;  // weight value 0
            w[cb][m][j] = u32x4{z, z, z, z};
            s[cb][m][j] = 0.0f;
          }
        }
    }
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const int c = c0 + cb * L;
      if (c >= segc) break;
      if constexpr (FMT == kFmtInt4) {
        u32x4 xh[NB][4];
        u32x4 xl[SPLIT ? NB : 1][4];
        float xo[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            xh[b][t] = hi[(b * 4 + t) * segc + c];
            if constexpr (SPLIT) xl[b][t] = lo[(b * 4 + t) * segc + c];
          }
          xo[b] = off[b * segc + c];
        }
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
          for (int j = 0; j < RU; ++j) {
            uint32_t p[4][4];
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
              for (int i = 0; i < 4; ++i) p[t][i] = nib_pair(w[cb][m][j][t] >> (4 * i));
#pragma unroll
            for (int b = 0; b < NB; ++b) {
              float a = xo[b];
#pragma unroll
              for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) a = dot2(p[t][i], xh[b][t][i], a);
              if constexpr (SPLIT) {
#pragma unroll
                for (int t = 0; t < 4; ++t)
#pragma unroll
                  for (int i = 0; i < 4; ++i) a = dot2(p[t][i], xl[b][t][i], a);
              }
              if constexpr (GROUPED)
                acc[m][j][b] = __builtin_fmaf(s[cb][m][j], a, acc[m][j][b]);
              else
                acc[m][j][b] += a;
            }
          }
      } else {
        f32x4 xv[NB][4];
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int t = 0; t < 4; ++t) xv[b][t] = xf[(b * 4 + t) * segc + c];
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
          for (int j = 0; j < RU; ++j) {
#pragma unroll
            for (int b = 0; b < NB; ++b) {
              float a = acc[m][j][b];
#pragma unroll
              for (int t = 0; t < 4; ++t) {
                const uint32_t wt = w[cb][m][j][t];
#pragma unroll
                for (int i = 0; i < 4; ++i) a = __builtin_fmaf((float)(int8_t)(wt >> (8 * i)), xv[b][t][i], a);
              }
              acc[m][j][b] = a;
            }
          }
      }
    }
  }
}


// ---- pipelined tiles (whole reduction staged in LDS) ---------------------------
//
// A "unit" is one pass over one tile: CB chunks per lane (chunk
// li + L * (pass * CB + cb)) of RU row sets of M matrices.  TileW holds the
// weights of one unit in registers, so a wave can load unit i+1 while it
// computes unit i.  Rows beyond nrows and chunks beyond kchunks load as
// zero weights and are skipped by the compute.

template <int M, int RU, int CB>
struct TileW {
  u32x4 w[CB][M][RU];
  float s[CB][M][RU];
};

template <int FMT, int L, int M, int RU, int CB, bool GROUPED>
__device__ __forceinline__ void unit_load(TileW<M, RU, CB>& t, const Mats<M>& mt, int64_t row_bytes, int G,
                                          int gshift, int row0, int rstride, int nrows, int kchunks, int pass) {
  const int li = (threadIdx.x & 63) % L;
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const int c = li + L * (pass * CB + cb);
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
      for (int j = 0; j < RU; ++j) {
        const int r = row0 + j * rstride;
        if (c < kchunks && r < nrows) {
          t.w[cb][m][j] = ld_stream(mt.q[m] + (int64_t)r * row_bytes + (int64_t)c * 16);
          t.s[cb][m][j] = GROUPED ? ld_stream(mt.s[m] + (int64_t)r * G + (c >> gshift)) : 1.0f;
        } else {
          const uint32_t z = (FMT == kFmtInt4) ? 0x88888888u : 0u;
          t.w[cb][m][j] = u32x4{z, z, z, z};
          t.s[cb][m][j] = 0.0f;
        }
      }
  }
}

template <int FMT, bool SPLIT, int L, int M, int RU, int CB, int NB, bool GROUPED>
__device__ __forceinline__ void unit_compute(const TileW<M, RU, CB>& t, const char* __restrict__ lds, int kchunks,
                                             int pass, float (&acc)[M][RU][NB]) {
  const int li = (threadIdx.x & 63) % L;
  const int segc = kchunks;
  const u32x4* hi = reinterpret_cast<const u32x4*>(lds);
  const u32x4* lo = hi + NB * 4 * segc;
  const float* off = reinterpret_cast<const float*>(lds + (size_t)NB * 4 * segc * 16 * (SPLIT ? 2 : 1));
  const f32x4* xf = reinterpret_cast<const f32x4*>(lds);
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const int c = li + L * (pass * CB + cb);
    if (c >= kchunks) break;
    if constexpr (FMT == kFmtInt4) {
      u32x4 xh[NB][4];
      u32x4 xl[SPLIT ? NB : 1][4];
      float xo[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          xh[b][q] = hi[(b * 4 + q) * segc + c];
          if constexpr (SPLIT) xl[b][q] = lo[(b * 4 + q) * segc + c];
        }
        xo[b] = off[b * segc + c];
      }
#pragma unroll
      for (int m = 0; m < M; ++m)
#pragma unroll
        for (int j = 0; j < RU; ++j) {
          uint32_t p[4][4];
#pragma unroll
          for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int i = 0; i < 4; ++i) p[q][i] = nib_pair(t.w[cb][m][j][q] >> (4 * i));
#pragma unroll
          for (int b = 0; b < NB; ++b) {
            float a = xo[b];
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
              for (int i = 0; i < 4; ++i) a = dot2(p[q][i], xh[b][q][i], a);
            if constexpr (SPLIT) {
#pragma unroll
              for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int i = 0; i < 4; ++i) a = dot2(p[q][i], xl[b][q][i], a);
            }
            if constexpr (GROUPED)
              acc[m][j][b] = __builtin_fmaf(t.s[cb][m][j], a, acc[m][j][b]);
            else
              acc[m][j][b] += a;
          }
        }
    } else {
      f32x4 xv[NB][4];
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int q = 0; q < 4; ++q) xv[b][q] = xf[(b * 4 + q) * segc + c];
#pragma unroll
      for (int m = 0; m < M; ++m)
#pragma unroll
        for (int j = 0; j < RU; ++j)
#pragma unroll
          for (int b = 0; b < NB; ++b) {
            float a = acc[m][j][b];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const uint32_t wt = t.w[cb][m][j][q];
#pragma unroll
              for (int i = 0; i < 4; ++i) a = __builtin_fmaf((float)(int8_t)(wt >> (8 * i)), xv[b][q][i], a);
            }
            acc[m][j][b] = a;
          }
    }
  }
}

// Walks this wave's tiles tile0, tile0 + tstride, ... (< ntiles), each in
// npasses units, loading unit i+1 while computing unit i.  first_load() must
// have been issued for (tile0, pass 0) into `a` (before the caller's staging
// barrier); emit(tile, acc) is called once per tile with the lane partials.
template <int FMT, bool SPLIT, int L, int M, int RU, int CB, int NB, bool GROUPED, typename Emit>
__device__ __forceinline__ void pipeline_tiles(TileW<M, RU, CB>& a, TileW<M, RU, CB>& b, const Mats<M>& mt,
                                               int64_t row_bytes, int G, int gshift, int nrows, int kchunks,
                                               int tile0, int tstride, int ntiles, int npasses,
                                               const char* __restrict__ lds, Emit emit) {
  constexpr int RPW = 64 / L;
  constexpr int TILE = RPW * RU;
  const int lrow = (threadIdx.x & 63) / L;
  float acc[M][RU][NB];
  auto zero = [&]() {
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
      for (int j = 0; j < RU; ++j)
#pragma unroll
        for (int q = 0; q < NB; ++q) acc[m][j][q] = 0.f;
  };
  zero();
  int tile = tile0, pass = 0;
  auto step = [&](TileW<M, RU, CB>& cur, TileW<M, RU, CB>& nxt) {
    int ntile = tile, npass = pass + 1;
    if (npass == npasses) {
      npass = 0;
      ntile = tile + tstride;
    }
    if (ntile < ntiles)
      unit_load<FMT, L, M, RU, CB, GROUPED>(nxt, mt, row_bytes, G, gshift, ntile * TILE + lrow, RPW, nrows, kchunks,
                                            npass);
    unit_compute<FMT, SPLIT, L, M, RU, CB, NB, GROUPED>(cur, lds, kchunks, pass, acc);
    if (pass == npasses - 1) {
      emit(tile, acc);
      zero();
    }
    tile = ntile;
    pass = npass;
  };
  while (tile < ntiles) {
    step(a, b);
    if (tile >= ntiles) break;
    step(b, a);
  }
}

// ---- runtime row count staging and one-row compute ------------------------------
//
// Same LDS layout as stage_x, with the number of staged rows known only at
// run time; XRow points at one staged row of that layout.

// 16-byte slots of one staged row: 4 words x segc chunks, padded by 128 bytes
// so that consecutive rows start on different LDS banks.
__host__ __device__ constexpr int row_slots(int segc) { return 4 * segc + 8; }

// LDS bytes of stage_rows for nrows rows of kchunks chunks
template <int FMT, bool SPLIT>
__host__ __device__ constexpr size_t stage_rows_bytes(int nrows, int kchunks) {
  return (size_t)nrows * (FMT == kFmtInt4 ? (row_slots(kchunks) * 16 * (SPLIT ? 2 : 1) + kchunks * 4)
                                          : row_slots(kchunks) * 16);
}

template <int FMT, int XT, typename TokF>
__device__ __forceinline__ void stage_rows(char* __restrict__ lds, const void* __restrict__ x, int64_t ldx,
                                           TokF tok, int nrows, int kchunks) {
  // One thread per 32-bit word of the layout (8 int4 weights' activations, or
  // a quarter chunk of 4 for int8), so the staging holds few registers while
  // the caller's first weight tiles are already in flight; SB words per
  // thread are loaded before any is converted, so their latencies overlap.
  // The four words of a chunk sit in one lane quad, which sums the chunk
  // with two DPP steps.
  constexpr bool SPLIT = (FMT == kFmtInt4 && XT == kF32);
  constexpr int PER = Fmt<FMT>::kPerChunk;
  constexpr int WE = PER / 4;                       // activations per word
  constexpr int NV = (XT == kBF16) ? (WE + 7) / 8 : WE / 4;  // 16-byte loads per word (bf16 int8: half)
  constexpr int SB = 4;                             // words per thread in flight
  const int segc = kchunks;
  const int rs = row_slots(segc);  // 16-byte slots per staged row, padded
  u32x4* hi = reinterpret_cast<u32x4*>(lds);
  u32x4* lo = hi + nrows * rs;
  float* off = reinterpret_cast<float*>(lds + (size_t)nrows * rs * 16 * (SPLIT ? 2 : 1));
  const int total = nrows * segc * 4;
  for (int base = 0; base < total; base += kThreads * SB) {  // uniform trip count: DPP needs whole quads
    u32x4 raw[SB][NV];
#pragma unroll
    for (int sb = 0; sb < SB; ++sb) {
      const int it = base + sb * kThreads + (int)threadIdx.x;
      const int itc = it < total ? it : 0;
      const int j = itc & 3, bc = itc >> 2;
      const int b = bc / segc, c = bc - b * segc;
      const int64_t e0 = (int64_t)tok(b) * ldx + (int64_t)c * PER + j * WE;
      if constexpr (XT == kBF16) {
        if constexpr (WE == 8) {
          raw[sb][0] = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(x) + e0);
        } else {
          const uint2 d = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(x) + e0);
          raw[sb][0] = u32x4{d.x, d.y, 0u, 0u};
        }
      } else {
#pragma unroll
        for (int m = 0; m < NV; ++m)
          raw[sb][m] = __builtin_bit_cast(u32x4, reinterpret_cast<const f32x4*>(static_cast<const float*>(x) + e0)[m]);
      }
    }
#pragma unroll
    for (int sb = 0; sb < SB; ++sb) {
      const int it = base + sb * kThreads + (int)threadIdx.x;
      const bool ok = it < total;
      const int itc = ok ? it : 0;
      const int j = itc & 3, bc = itc >> 2;
      const int b = bc / segc, c = bc - b * segc;
      float v[WE];
      if constexpr (XT == kBF16) {
#pragma unroll
        for (int t = 0; t < WE / 2; ++t) {
          v[2 * t] = bf16_bits_to_f32(raw[sb][0][t] & 0xFFFFu);
          v[2 * t + 1] = bf16_bits_to_f32(raw[sb][0][t] >> 16);
        }
      } else {
#pragma unroll
        for (int t = 0; t < WE; ++t) v[t] = __uint_as_float(raw[sb][t / 4][t % 4]);
      }
      if constexpr (FMT == kFmtInt4) {
        float sum = 0.f;
        u32x4 ph, pl;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float a = v[i], bq = v[4 + i];
          const uint32_t ha = f32_to_bf16_bits(a), hb = f32_to_bf16_bits(bq);
          ph[i] = ha | (hb << 16);
          if constexpr (SPLIT) {
            const float ra = a - bf16_bits_to_f32(ha), rb = bq - bf16_bits_to_f32(hb);
            const uint32_t la = f32_to_bf16_bits(ra), lb = f32_to_bf16_bits(rb);
            pl[i] = la | (lb << 16);
            sum += (bf16_bits_to_f32(ha) + bf16_bits_to_f32(la)) + (bf16_bits_to_f32(hb) + bf16_bits_to_f32(lb));
          } else {
            sum += bf16_bits_to_f32(ha) + bf16_bits_to_f32(hb);
          }
        }
        sum = group_sum<4>(sum);  // the chunk's four words
        if (ok) {
          hi[b * rs + j * segc + c] = ph;
          if constexpr (SPLIT) lo[b * rs + j * segc + c] = pl;
          if (j == 0) off[b * segc + c] = -136.0f * sum;
        }
      } else {
        if (ok) {
          f32x4* q4 = reinterpret_cast<f32x4*>(lds);
          q4[b * rs + j * segc + c] = f32x4{v[0], v[1], v[2], v[3]};
        }
      }
    }
  }
}

struct XRow {
  const u32x4* hi;   // int4: [4][segc] pairs of this row
  const u32x4* lo;   // int4 + fp32 activations: [4][segc]
  const float* off;  // int4: [segc]
  int segc;
};

template <int FMT, bool SPLIT>
__device__ __forceinline__ XRow xrow(const char* lds, int nrows, int kchunks, int b) {
  XRow r;
  const int rs = row_slots(kchunks);
  const u32x4* hi = reinterpret_cast<const u32x4*>(lds);
  r.hi = hi + b * rs;
  r.lo = hi + nrows * rs + b * rs;
  r.off = reinterpret_cast<const float*>(lds + (size_t)nrows * rs * 16 * (SPLIT ? 2 : 1)) + b * kchunks;
  r.segc = kchunks;
  return r;
}

// acc[m][j] += this lane's share of  scale * sum_c W_m[row_j][c] x[c]  for the
// unit's chunks, with t.s holding the full multiplier of each chunk partial.
template <int FMT, bool SPLIT, int L, int M, int RU, int CB, bool FULL = false>
__device__ __forceinline__ void unit_compute_row(const TileW<M, RU, CB>& t, const XRow& xr, int kchunks, int pass,
                                                 float (&acc)[M][RU], const NibConst& nk) {
  const int li = (threadIdx.x & 63) % L;
  const int segc = xr.segc;
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const int c = li + L * (pass * CB + cb);
    if (!FULL && c >= kchunks) break;
    if constexpr (FMT == kFmtInt4) {
      u32x4 xh[4], xl[SPLIT ? 4 : 1];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        xh[q] = xr.hi[q * segc + c];
        if constexpr (SPLIT) xl[q] = xr.lo[q * segc + c];
      }
      const float xo = xr.off[c];
#pragma unroll
      for (int m = 0; m < M; ++m)
#pragma unroll
        for (int j = 0; j < RU; ++j) {
          float a = xo;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t w = t.w[cb][m][j][q];
            uint32_t pr[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) pr[i] = nib_pair(w >> (4 * i), nk);
#pragma unroll
            for (int i = 0; i < 4; ++i) a = dot2(pr[i], xh[q][i], a);
            if constexpr (SPLIT) {
#pragma unroll
              for (int i = 0; i < 4; ++i) a = dot2(pr[i], xl[q][i], a);
            }
          }
          acc[m][j] = __builtin_fmaf(t.s[cb][m][j], a, acc[m][j]);
        }
    } else {
      const f32x4* xf = reinterpret_cast<const f32x4*>(xr.hi);
      f32x4 xv[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) xv[q] = xf[q * segc + c];
#pragma unroll
      for (int m = 0; m < M; ++m)
#pragma unroll
        for (int j = 0; j < RU; ++j) {
          float a = 0.f;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t wt = t.w[cb][m][j][q];
#pragma unroll
            for (int i = 0; i < 4; ++i) a = __builtin_fmaf((float)(int8_t)(wt >> (8 * i)), xv[q][i], a);
          }
          acc[m][j] = __builtin_fmaf(t.s[cb][m][j], a, acc[m][j]);
        }
    }
  }
}

// Loads one unit with t.s = (group scale, or row scale) * mul for every chunk.
// FULL: every chunk index of the unit is below kchunks (no per-chunk test).
template <int FMT, int L, int M, int RU, int CB, bool GROUPED, bool FULL = false>
__device__ __forceinline__ void unit_load_scaled(TileW<M, RU, CB>& t, const Mats<M>& mt, int64_t row_bytes, int G,
                                                 int gshift, int row0, int rstride, int nrows, int kchunks, int pass,
                                                 float mul) {
  const int li = (threadIdx.x & 63) % L;
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const int c = li + L * (pass * CB + cb);
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
      for (int j = 0; j < RU; ++j) {
        const int r = row0 + j * rstride;
        if ((FULL || c < kchunks) && r < nrows) {
          t.w[cb][m][j] = ld_stream(mt.q[m] + (int64_t)r * row_bytes + (int64_t)c * 16);
          t.s[cb][m][j] = mul * ld_stream(mt.s[m] + (int64_t)r * G + (GROUPED ? (c >> gshift) : 0));
        } else {
          const uint32_t z = (FMT == kFmtInt4) ? 0x88888888u : 0u;
          t.w[cb][m][j] = u32x4{z, z, z, z};
          t.s[cb][m][j] = 0.0f;
        }
      }
  }
}

// Loader for wave-uniform rows (L = 64: one row per load instruction).  The
// row base is scalar, each lane adds its 16-byte slot and the CB chunks of a
// lane sit at fixed 1 KiB steps, so no per-load 64-bit vector arithmetic.
// qrow[m] points at row `row0` of matrix m, srow[m] at that row's scales;
// rows row0 + j (j < RU) at or beyond nrows load as zero.
template <int FMT, int M, int RU, int CB, bool GROUPED>
__device__ __forceinline__ void unit_load_row64(TileW<M, RU, CB>& t, const uint8_t* const (&qrow)[M],
                                                const float* const (&srow)[M], int64_t row_bytes, int G,
                                                int gshift, int row0, int nrows, float mul) {
  const int li = threadIdx.x & 63;
#pragma unroll
  for (int j = 0; j < RU; ++j) {
    if (row0 + j < nrows) {
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const int c = li + 64 * cb;
#pragma unroll
        for (int m = 0; m < M; ++m) {
          t.w[cb][m][j] = ld_stream(qrow[m] + j * row_bytes + (int64_t)c * 16);
          t.s[cb][m][j] = mul * ld_stream(srow[m] + j * G + (GROUPED ? (c >> gshift) : 0));
        }
      }
    } else {
      const uint32_t z = (FMT == kFmtInt4) ? 0x88888888u : 0u;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int m = 0; m < M; ++m) {
          t.w[cb][m][j] = u32x4{z, z, z, z};
          t.s[cb][m][j] = 0.0f;
        }
    }
  }
}

}  // namespace qm
