// moe_t1_lds.hpp -- single-token routed expert FFN with the weight stream
// prefetched into LDS (gfx950 global_load_lds_dwordx4 DMA).
//
// Computes what moe_t1_impl.hpp computes (the K-expert group of the colibri
// page "Vulkan backend: expert tier + dense + MLA attention on any Vulkan 1.2
// GPU": silu(gate x) * up x, then the down projection, outputs combined with
// the routing weights).  The difference is where the prefetched weights wait:
// every wave owns a ring of D slots in LDS; a slot holds one unit of work
// (RU rows x CB 16-byte chunks per lane of every matrix, plus the matching
// scales), filled by DMA loads that need no registers, and drained with one
// ds_read_b128 per chunk right before the chunk is consumed.  D - 1 units
// stay in flight while one is computed, at a register cost independent of D.
//
// vmcnt bookkeeping: a unit issues exactly U = 2 * (weight loads) VMEM
// operations; before unit k is read the wave waits until at most
// U * (units issued after k) VMEM operations are outstanding.  Anything else
// issued after k (hidden-vector or output stores, staging loads) only makes
// that wait stricter, never weaker.
#pragma once
#include "lds_ring.hpp"
#include "moe_t1_impl.hpp"

namespace qm {

constexpr size_t align_lds(size_t v) { return (v + 255) / 256 * 256; }

template <int RU, int M, int CB>
__host__ __device__ constexpr int ring_slot_bytes() {
  return RU * M * CB * (1024 + 256);
}

// ---- gate + up ----------------------------------------------------------------
// L = 64 lanes per row and exactly CB chunks per lane (H = 64 * CB * 32 for
// int4).  Unit = RU consecutive rows of gate and up of one routed expert.
// PS (packed scales): the unit's RU * 2 scale rows (G floats each, G a
// multiple of 4, at most 256 floats in all) arrive with one 16-byte DMA per
// lane instead of one 4-byte DMA per weight block, each lane fetching its own
// chunk's scale.
template <int RU, int M, int CB, bool PS>
__host__ __device__ constexpr int gu_slot_bytes() {
  return RU * M * CB * 1024 + (PS ? 1024 : RU * M * CB * 256);
}

template <int FMT, int XT, int CB, int RU, int D, bool GROUPED, bool PS>
__global__ __launch_bounds__(kThreads) void moe_gate_up_t1l_kernel(MoeDecodeArgs a) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  __shared__ int s_e[kTopkMax];
  constexpr bool SPLIT = (FMT == kFmtInt4 && XT == kF32);
  constexpr int M = 2;
  constexpr int NW = RU * M * CB;         // 1 KiB weight blocks per unit
  constexpr int U = NW + (PS ? 1 : NW);   // VMEM operations per unit
  constexpr int SLOT = gu_slot_bytes<RU, M, CB, PS>();
  static_assert(!PS || GROUPED, "packed scales need grouped scales");
  const ExpertArgs& ex = a.ex;
  const int k = a.topk;
  if ((int)threadIdx.x < k) {
    const int id = a.ids[threadIdx.x];
    s_e[threadIdx.x] = (id >= 0 && id < ex.E) ? id : -1;
  }
  __syncthreads();
  const int wave = uniform(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int kchunks = 64 * CB;
  const int ntiles = (ex.I + RU - 1) / RU;
  const int nitems = k * ntiles;
  const int istride = gridDim.x * kWaves;
  char* ring = lds + align_lds(stage_rows_bytes<FMT, SPLIT>(1, kchunks)) + (size_t)wave * D * SLOT;
  auto next_valid = [&](int it) {
    while (it < nitems && uniform(s_e[it / ntiles]) < 0) it += istride;
    return it;
  };
  auto issue = [&](int it, int slot) {
    const int p = it / ntiles;
    const int e = uniform(s_e[p]);
    const int row0 = (it - p * ntiles) * RU;
    char* sd = ring + slot * SLOT;
#pragma unroll
    for (int j = 0; j < RU; ++j) {
      const int r = min(row0 + j, ex.I - 1);  // a tail row past I reloads row I-1; its result is dropped
      const int64_t er = (int64_t)e * ex.I + r;
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const uint8_t* qrow = (m == 0 ? ex.gq : ex.uq) + er * ex.rb_h;
        const float* srow = (m == 0 ? ex.gs : ex.us) + er * ex.G_h;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
          const int c = lane + 64 * cb;
          const int blk = (j * M + m) * CB + cb;
          dma16(qrow + (int64_t)c * 16, sd + blk * 1024);
          if constexpr (!PS) dma4(srow + (GROUPED ? (c >> ex.gshift) : 0), sd + NW * 1024 + blk * 256);
        }
      }
    }
    if constexpr (PS) {
      // floats 4f .. 4f+3 of the unit's scale rows [j][m][G]; lanes past the
      // last piece reload it (no extra traffic)
      const int G = ex.G_h;
      const int f = 4 * min(lane, RU * M * G / 4 - 1);
      const int rm = f / G, g = f - rm * G;
      const int j = rm / M, m = rm - j * M;
      const int r = min(row0 + j, ex.I - 1);
      const float* srow = (m == 0 ? ex.gs : ex.us) + ((int64_t)e * ex.I + r) * G + g;
      dma16(srow, sd + NW * 1024);
    }
  };
  int head = next_valid(uniform(blockIdx.x * kWaves + wave));
  int tail = head, inflight = 0;
#pragma unroll
  for (int i = 0; i < D; ++i)
    if (tail < nitems) {
      issue(tail, i);
      ++inflight;
      tail = next_valid(tail + istride);
    }
  stage_rows<FMT, XT>(lds, a.x, ex.H, [](int) { return 0; }, 1, kchunks);
  __syncthreads();
  const XRow xr = xrow<FMT, SPLIT>(lds, 1, kchunks, 0);
  const NibConst nk = nib_const();
  int hs = 0;
  while (inflight > 0) {
    wait_units<U, D>(inflight - 1);
    const char* sd = ring + hs * SLOT;
    float acc[M][RU];
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
      for (int j = 0; j < RU; ++j) acc[m][j] = 0.f;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const int c = lane + 64 * cb;
      u32x4 xh[4], xl[SPLIT ? 4 : 1];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        xh[q] = xr.hi[q * kchunks + c];
        if constexpr (SPLIT) xl[q] = xr.lo[q * kchunks + c];
      }
      const float xo = FMT == kFmtInt4 ? xr.off[c] : 0.f;
#pragma unroll
      for (int j = 0; j < RU; ++j)
#pragma unroll
        for (int m = 0; m < M; ++m) {
          const int blk = (j * M + m) * CB + cb;
          const u32x4 w = *reinterpret_cast<const u32x4*>(sd + blk * 1024 + lane * 16);
          const float s = PS ? *reinterpret_cast<const float*>(sd + NW * 1024 + ((j * M + m) * ex.G_h +
                                                                                   (c >> ex.gshift)) * 4)
                             : *reinterpret_cast<const float*>(sd + NW * 1024 + blk * 256 + lane * 4);
          float t;
          if constexpr (FMT == kFmtInt4) {
            t = xo;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              uint32_t pr[4];
#pragma unroll
              for (int i = 0; i < 4; ++i) pr[i] = nib_pair(w[q] >> (4 * i), nk);
#pragma unroll
              for (int i = 0; i < 4; ++i) t = dot2(pr[i], xh[q][i], t);
              if constexpr (SPLIT) {
#pragma unroll
                for (int i = 0; i < 4; ++i) t = dot2(pr[i], xl[q][i], t);
              }
            }
          } else {
            const f32x4* xf = reinterpret_cast<const f32x4*>(xh);
            t = 0.f;
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
              for (int i = 0; i < 4; ++i) t = __builtin_fmaf((float)(int8_t)(w[q] >> (8 * i)), xf[q][i], t);
          }
          acc[m][j] = __builtin_fmaf(s, t, acc[m][j]);
        }
    }
    slot_release();
    const int it = head;
    if (tail < nitems) {
      issue(tail, hs);
      tail = next_valid(tail + istride);
    } else {
      --inflight;
    }
    head = next_valid(head + istride);
    hs = hs + 1 == D ? 0 : hs + 1;
    const int p = it / ntiles, row0 = (it - p * ntiles) * RU;
#pragma unroll
    for (int j = 0; j < RU; ++j) {
      const float g = group_sum<64>(acc[0][j]);
      const float v = group_sum<64>(acc[1][j]);
      if (lane == 0 && row0 + j < ex.I) a.h[(int64_t)p * ex.I + row0 + j] = silu(g) * v;
    }
  }
}

// ---- down + weighted combine ----------------------------------------------------
// Lanes are split into groups of LPP per routed pair (pair q = lane / LPP);
// each lane walks chunks sub + LPP * i of its pair's row, so its expert and
// routing weight stay fixed.  Unit = RU output rows x CB chunks per lane.
template <int FMT, int CB, int RU, int D, bool GROUPED>
__global__ __launch_bounds__(kThreads) void moe_down_t1l_kernel(MoeDecodeArgs a) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  __shared__ int s_e[kTopkMax], s_p[kTopkMax], s_n;
  __shared__ float s_w[kTopkMax];
  constexpr bool SPLIT = (FMT == kFmtInt4);  // h is fp32
  constexpr int M = 1;
  constexpr int NW = RU * CB;
  constexpr int U = 2 * NW;
  constexpr int SLOT = ring_slot_bytes<RU, M, CB>();
  const ExpertArgs& ex = a.ex;
  routed_pairs(a.ids, a.w, a.topk, ex.E, s_e, s_p, s_w, &s_n);  // valid pairs of the token, in slot order
  __syncthreads();
  const int np = s_n;
  if (np == 0) {
    for (int i = blockIdx.x * kThreads + threadIdx.x; i < ex.H; i += gridDim.x * kThreads) a.y[i] = 0.f;
    return;
  }
  const int wave = uniform(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int kchunks = ex.I / Fmt<FMT>::kPerChunk;
  int npp = 1;
  while (npp < np) npp <<= 1;
  const int lpp = 64 / npp;             // lanes per pair (np <= 32 keeps lpp >= 2)
  const int q = lane / lpp, sub = lane - q * lpp;
  const bool lane_ok = q < np;
  const int qq = lane_ok ? q : 0;
  const int e = s_e[qq];
  const float wq = lane_ok ? s_w[qq] : 0.f;
  const int cpl = (kchunks + lpp - 1) / lpp;  // chunks per lane per row
  const int npasses = (cpl + CB - 1) / CB;
  const int ntiles = (ex.H + RU - 1) / RU;
  const int nunits = ntiles * npasses;
  const int ustride_t = gridDim.x * kWaves;  // tile stride
  const size_t xbytes = align_lds(stage_rows_bytes<FMT, SPLIT>(a.topk, kchunks));
  char* ring = lds + xbytes + (size_t)wave * D * SLOT;
  auto next_unit = [&](int v) {
    const int t = v / npasses, ps = v - t * npasses;
    return ps + 1 < npasses ? v + 1 : (t + ustride_t) * npasses;
  };
  auto issue = [&](int v, int slot) {
    const int t = v / npasses, ps = v - t * npasses;
    char* sd = ring + slot * SLOT;
#pragma unroll
    for (int j = 0; j < RU; ++j) {
      const int r = min(t * RU + j, ex.H - 1);
      const int64_t er = (int64_t)e * ex.H + r;
      const uint8_t* qrow = ex.dq + er * ex.rb_i;
      const float* srow = ex.ds + er * ex.G_i;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        int c = sub + lpp * (ps * CB + cb);
        c = c < kchunks ? c : 0;  // past the row: reload chunk 0, weighted by zero below
        const int blk = j * CB + cb;
        dma16(qrow + (int64_t)c * 16, sd + blk * 1024);
        dma4(srow + (GROUPED ? (c >> ex.gshift) : 0), sd + NW * 1024 + blk * 256);
      }
    }
  };
  int head = uniform(blockIdx.x * kWaves + wave) * npasses;
  int tail = head, inflight = 0;
#pragma unroll
  for (int i = 0; i < D; ++i)
    if (tail < nunits) {
      issue(tail, i);
      ++inflight;
      tail = next_unit(tail);
    }
  stage_rows<FMT, kF32>(lds, a.h, ex.I, [&](int b) { return s_p[b]; }, np, kchunks);
  __syncthreads();
  const int rs = row_slots(kchunks);
  const u32x4* xhi = reinterpret_cast<const u32x4*>(lds);
  const u32x4* xlo = xhi + np * rs;
  const float* xoff = reinterpret_cast<const float*>(lds + (size_t)np * rs * 16 * (SPLIT ? 2 : 1));
  const f32x4* xf8 = reinterpret_cast<const f32x4*>(lds);
  const NibConst nk = nib_const();
  float acc[RU];
#pragma unroll
  for (int j = 0; j < RU; ++j) acc[j] = 0.f;
  int hs = 0;
  while (inflight > 0) {
    wait_units<U, D>(inflight - 1);
    const char* sd = ring + hs * SLOT;
    const int v = head, t = v / npasses, ps = v - t * npasses;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const int c0 = sub + lpp * (ps * CB + cb);
      const bool ok = lane_ok && c0 < kchunks;
      const int c = ok ? c0 : 0;
      const float mul = ok ? wq : 0.f;
      if constexpr (FMT == kFmtInt4) {
        u32x4 xh[4], xl[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          xh[r] = xhi[qq * rs + r * kchunks + c];
          xl[r] = xlo[qq * rs + r * kchunks + c];
        }
        const float xo = xoff[qq * kchunks + c];
#pragma unroll
        for (int j = 0; j < RU; ++j) {
          const int blk = j * CB + cb;
          const u32x4 w = *reinterpret_cast<const u32x4*>(sd + blk * 1024 + lane * 16);
          const float s = *reinterpret_cast<const float*>(sd + NW * 1024 + blk * 256 + lane * 4);
          float tt = xo;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            uint32_t pr[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) pr[i] = nib_pair(w[r] >> (4 * i), nk);
#pragma unroll
            for (int i = 0; i < 4; ++i) tt = dot2(pr[i], xh[r][i], tt);
#pragma unroll
            for (int i = 0; i < 4; ++i) tt = dot2(pr[i], xl[r][i], tt);
          }
          acc[j] = __builtin_fmaf(mul * s, tt, acc[j]);
        }
      } else {
        f32x4 xv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) xv[r] = xf8[qq * rs + r * kchunks + c];
#pragma unroll
        for (int j = 0; j < RU; ++j) {
          const int blk = j * CB + cb;
          const u32x4 w = *reinterpret_cast<const u32x4*>(sd + blk * 1024 + lane * 16);
          const float s = *reinterpret_cast<const float*>(sd + NW * 1024 + blk * 256 + lane * 4);
          float tt = 0.f;
#pragma unroll
          for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int i = 0; i < 4; ++i) tt = __builtin_fmaf((float)(int8_t)(w[r] >> (8 * i)), xv[r][i], tt);
          acc[j] = __builtin_fmaf(mul * s, tt, acc[j]);
        }
      }
    }
    slot_release();
    if (tail < nunits) {
      issue(tail, hs);
      tail = next_unit(tail);
    } else {
      --inflight;
    }
    head = next_unit(head);
    hs = hs + 1 == D ? 0 : hs + 1;
    if (ps == npasses - 1) {
#pragma unroll
      for (int j = 0; j < RU; ++j) {
        const float yv = group_sum<64>(acc[j]);
        if (lane == 0 && t * RU + j < ex.H) a.y[t * RU + j] = yv;
        acc[j] = 0.f;
      }
    }
  }
}


// ---- down + weighted combine, hidden vector in registers ----------------------
// One wave owns PPW = 64 / L routed pairs (L lanes each) and, for a slice of
// this block's output rows, reads every row of those pairs' down matrices:
// lane (pair, sub) holds chunks c = sub + L * i (i < CPL) of the row, and
// those chunks of h sit in its registers for the whole kernel (converted once
// to bf16 hi/lo pairs plus the chunk's -136 * sum offset), so the LDS holds
// only the weight ring.  Unit = one row of the wave's pairs; the ring keeps
// D - 1 units in flight per wave.  Each lane stores its weighted partial of a
// row in a per-wave LDS table (no cross-lane work inside the loop); at the
// end every row's 64 partials of every pair group are added in a fixed order
// (lane order within a group, then group order), so y is written once,
// deterministically.
constexpr int kDW = 8;           // waves per block of the register-h down kernel
constexpr int kDT = 64 * kDW;

template <int FMT, int L, int CPL, int D, bool GROUPED>
__global__ __launch_bounds__(kDT) void moe_down_t1r_kernel(MoeDecodeArgs a) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  __shared__ int s_e[kTopkMax], s_p[kTopkMax], s_n;
  __shared__ float s_w[kTopkMax];
  constexpr int PPW = 64 / L;
  constexpr int U = 2 * CPL;  // VMEM operations per unit
  constexpr int SLOT = ring_slot_bytes<1, 1, CPL>();
  constexpr int PER = Fmt<FMT>::kPerChunk;
  const ExpertArgs& ex = a.ex;
  routed_pairs(a.ids, a.w, a.topk, ex.E, s_e, s_p, s_w, &s_n);  // valid pairs of the token, in slot order
  __syncthreads();
  const int np = s_n;
  const int npg = (np + PPW - 1) / PPW;  // pair groups: waves per row slice
  int npg2 = 1;
  while (npg2 < npg) npg2 <<= 1;  // <= kDW (checked on the host for top_k)
  const int S = kDW / npg2;       // row slices per block
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

  // this lane's chunks of h, in registers
  const float* hrow = a.h + (int64_t)prow * ex.I;
  u32x4 hh[CPL][4], hl[CPL][4];
  float ho[CPL];
  f32x4 hf[CPL][4];
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const int c = sub + L * i;
    if constexpr (FMT == kFmtInt4) {
      float sum = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 va = *reinterpret_cast<const f32x4*>(hrow + c * 32 + 8 * j);
        const f32x4 vb = *reinterpret_cast<const f32x4*>(hrow + c * 32 + 8 * j + 4);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const float x0 = qok ? va[t] : 0.f, x1 = qok ? vb[t] : 0.f;
          const uint32_t h0 = f32_to_bf16_bits(x0), h1 = f32_to_bf16_bits(x1);
          const float r0f = x0 - bf16_bits_to_f32(h0), r1f = x1 - bf16_bits_to_f32(h1);
          const uint32_t l0 = f32_to_bf16_bits(r0f), l1 = f32_to_bf16_bits(r1f);
          hh[i][j][t] = h0 | (h1 << 16);
          hl[i][j][t] = l0 | (l1 << 16);
          sum += (bf16_bits_to_f32(h0) + bf16_bits_to_f32(l0)) + (bf16_bits_to_f32(h1) + bf16_bits_to_f32(l1));
        }
      }
      ho[i] = -136.0f * sum;
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(hrow + c * 16 + 4 * j);
        hf[i][j] = qok ? v : f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
  }
  const NibConst nk = nib_const();
  for (int u = 0; u < nunits; ++u) {
    wait_units_upto<U, D - 2>(min(D - 2, nunits - 1 - u));
    const char* sd = ring + (u % D) * SLOT;
    float t = 0.f;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(sd + i * 1024 + lane * 16);
      const float sc = *reinterpret_cast<const float*>(sd + CPL * 1024 + i * 256 + lane * 4);
      float tt;
      if constexpr (FMT == kFmtInt4) {
        tt = ho[i];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          uint32_t pr[4];
#pragma unroll
          for (int m = 0; m < 4; ++m) pr[m] = nib_pair(w[j] >> (4 * m), nk);
#pragma unroll
          for (int m = 0; m < 4; ++m) tt = dot2(pr[m], hh[i][j][m], tt);
#pragma unroll
          for (int m = 0; m < 4; ++m) tt = dot2(pr[m], hl[i][j][m], tt);
        }
      } else {
        tt = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int m = 0; m < 4; ++m) tt = __builtin_fmaf((float)(int8_t)(w[j] >> (8 * m)), hf[i][j][m], tt);
      }
      t = __builtin_fmaf(sc, tt, t);
    }
    slot_release();
    if (u + D - 1 < nunits) issue(u + D - 1, (u + D - 1) % D);
    part[((sl + S * u) * kDW + pg) * 64 + lane] = wq * t;
  }
  __syncthreads();
  // row i of this block: one wave per row, lanes add the pair groups' partials
  for (int i = wave; i < r1 - r0; i += kDW) {
    float v = 0.f;
    for (int g = 0; g < npg; ++g) v += part[(i * kDW + g) * 64 + lane];
    v = group_sum<64>(v);
    if (lane == 0) a.y[r0 + i] = v;
  }
  (void)PER;
}

// ---- launch ---------------------------------------------------------------------

#ifndef QM_LDS_GU_D
#define QM_LDS_GU_D 2
#endif
#ifndef QM_LDS_DN_D
#define QM_LDS_DN_D 2
#endif
#ifndef QM_LDS_GU_BLOCKS
#define QM_LDS_GU_BLOCKS 512
#endif
#ifndef QM_LDS_DN_BLOCKS
#define QM_LDS_DN_BLOCKS 256
#endif
constexpr int kLdsMax = 160 * 1024;  // LDS per workgroup on gfx950

template <int CB>
constexpr int gu_ru() { return CB >= 3 ? 1 : (CB == 2 ? 1 : 2); }

template <int FMT, int XT, int CB, bool GROUPED, bool PS = false>
inline size_t gu_lds_bytes() {
  return align_lds(stage_rows_bytes<FMT, FMT == kFmtInt4 && XT == kF32>(1, 64 * CB)) +
         (size_t)kWaves * QM_LDS_GU_D * gu_slot_bytes<gu_ru<CB>(), 2, CB, PS>();
}

// packed scales: grouped, G a multiple of 4 with all of a unit's scale rows in
// 1 KiB, and 16-byte aligned scale rows
inline bool gu_packed_scales(const MoeDecodeArgs& a, int RU) {
  const int G = a.ex.G_h;
  return G % 4 == 0 && RU * 2 * G <= 256 && ((uintptr_t)a.ex.gs & 15) == 0 && ((uintptr_t)a.ex.us & 15) == 0;
}

template <int FMT, int XT, int CB, bool GROUPED>
inline hipError_t launch_gu_t1l(const MoeDecodeArgs& a, hipStream_t st) {
  constexpr int RU = gu_ru<CB>();
  const int ntiles = (a.ex.I + RU - 1) / RU;
  int blocks = (a.topk * ntiles + kWaves - 1) / kWaves;
  const int cap = a.max_blocks > 0 ? a.max_blocks : QM_LDS_GU_BLOCKS;
  if (blocks > cap) blocks = cap;
  if constexpr (GROUPED) {
    if (gu_packed_scales(a, RU)) {
      const size_t lds = gu_lds_bytes<FMT, XT, CB, GROUPED, true>();
      hipLaunchKernelGGL((moe_gate_up_t1l_kernel<FMT, XT, CB, RU, QM_LDS_GU_D, GROUPED, true>), dim3(blocks),
                         dim3(kThreads), lds, st, a);
      return hipGetLastError();
    }
  }
  const size_t lds = gu_lds_bytes<FMT, XT, CB, GROUPED>();
  hipLaunchKernelGGL((moe_gate_up_t1l_kernel<FMT, XT, CB, RU, QM_LDS_GU_D, GROUPED, false>), dim3(blocks),
                     dim3(kThreads), lds, st, a);
  return hipGetLastError();
}

constexpr int kDnRU = 2;

template <int FMT, int CB>
inline size_t dn_lds_bytes(int topk, int kchunks) {
  return align_lds(stage_rows_bytes<FMT, FMT == kFmtInt4>(topk, kchunks)) +
         (size_t)kWaves * QM_LDS_DN_D * ring_slot_bytes<kDnRU, 1, CB>();
}

template <int FMT, int CB, bool GROUPED>
inline hipError_t launch_dn_t1l(const MoeDecodeArgs& a, hipStream_t st) {
  const int ntiles = (a.ex.H + kDnRU - 1) / kDnRU;
  int blocks = (ntiles + kWaves - 1) / kWaves;
  const int cap = a.max_blocks > 0 ? a.max_blocks : QM_LDS_DN_BLOCKS;
  if (blocks > cap) blocks = cap;
  const size_t lds = dn_lds_bytes<FMT, CB>(a.topk, a.ex.I / Fmt<FMT>::kPerChunk);
  hipLaunchKernelGGL((moe_down_t1l_kernel<FMT, CB, kDnRU, QM_LDS_DN_D, GROUPED>), dim3(blocks), dim3(kThreads), lds,
                     st, a);
  return hipGetLastError();
}

// The LDS-ring gate+up kernel needs H to be exactly 64 * CB chunks (CB <= 4);
// both need T = 1 and their LDS within the workgroup limit.
template <int FMT, int XT, bool GROUPED>
inline bool try_gate_up_t1l(const MoeDecodeArgs& a, hipStream_t st, hipError_t* err) {
  if (a.T != 1 || a.topk > kTopkMax) return false;
  const int kch = a.ex.H / Fmt<FMT>::kPerChunk;
  if (kch % 64 || kch / 64 > 4 || kch / 64 < 1) return false;
  switch (kch / 64) {
    case 1:
      if (gu_lds_bytes<FMT, XT, 1, GROUPED>() > (size_t)kLdsMax) return false;
      *err = launch_gu_t1l<FMT, XT, 1, GROUPED>(a, st);
      return true;
    case 2:
      if (gu_lds_bytes<FMT, XT, 2, GROUPED>() > (size_t)kLdsMax) return false;
      *err = launch_gu_t1l<FMT, XT, 2, GROUPED>(a, st);
      return true;
    case 3:
      if (gu_lds_bytes<FMT, XT, 3, GROUPED>() > (size_t)kLdsMax) return false;
      *err = launch_gu_t1l<FMT, XT, 3, GROUPED>(a, st);
      return true;
    default:
      if (gu_lds_bytes<FMT, XT, 4, GROUPED>() > (size_t)kLdsMax) return false;
      *err = launch_gu_t1l<FMT, XT, 4, GROUPED>(a, st);
      return true;
  }
}

// chunks per lane and pass: the chunks one lane owns in a row when every
// routed pair is valid (lanes per pair = 64 / next_pow2(top_k)), up to 4
template <int FMT, bool GROUPED>
inline bool try_down_t1l(const MoeDecodeArgs& a, hipStream_t st, hipError_t* err) {
  if (a.T != 1 || a.topk > kTopkMax) return false;
  const int kch = a.ex.I / Fmt<FMT>::kPerChunk;
  int npp = 1;
  while (npp < a.topk) npp <<= 1;
#ifndef QM_LDS_DN_CBMAX
#define QM_LDS_DN_CBMAX 4
#endif
  int cpl = (kch + 64 / npp - 1) / (64 / npp);
  if (cpl > QM_LDS_DN_CBMAX) cpl = QM_LDS_DN_CBMAX;
  if (cpl <= 1) {
    if (dn_lds_bytes<FMT, 1>(a.topk, kch) > (size_t)kLdsMax) return false;
    *err = launch_dn_t1l<FMT, 1, GROUPED>(a, st);
  } else if (cpl == 2) {
    if (dn_lds_bytes<FMT, 2>(a.topk, kch) > (size_t)kLdsMax) return false;
    *err = launch_dn_t1l<FMT, 2, GROUPED>(a, st);
  } else {
    if (dn_lds_bytes<FMT, 4>(a.topk, kch) > (size_t)kLdsMax) return false;
    *err = launch_dn_t1l<FMT, 4, GROUPED>(a, st);
  }
  return true;
}


#ifndef QM_DOWN_REG
#define QM_DOWN_REG 1
#endif
#ifndef QM_DOWN_REG_BLOCKS
#define QM_DOWN_REG_BLOCKS 512
#endif
#ifndef QM_DOWN_REG_D
#define QM_DOWN_REG_D 4
#endif

template <int FMT, int L, int CPL, bool GROUPED>
inline hipError_t launch_dn_t1r(const MoeDecodeArgs& a, hipStream_t st) {
  // two pairs per wave (L = 32): the full ring depth, one block per CU
  constexpr int D = (CPL == 1 || L == 32) ? QM_DOWN_REG_D : (QM_DOWN_REG_D + 1) / 2;
  constexpr int PPW = 64 / L;
  const int npg = (a.topk + PPW - 1) / PPW;
  int npg2 = 1;
  while (npg2 < npg) npg2 <<= 1;
  const int S = kDW / npg2;
  int blocks = a.max_blocks > 0 ? a.max_blocks : (L == 32 ? QM_DOWN_REG_BLOCKS / 2 : QM_DOWN_REG_BLOCKS);
  if (blocks > (a.ex.H + S - 1) / S) blocks = (a.ex.H + S - 1) / S;
  const int R = (a.ex.H + blocks - 1) / blocks;
  const size_t lds = (size_t)kDW * D * ring_slot_bytes<1, 1, CPL>() + (size_t)R * kDW * 64 * 4;
  if (lds > (size_t)kLdsMax) return hipErrorNotSupported;
  hipLaunchKernelGGL((moe_down_t1r_kernel<FMT, L, CPL, D, GROUPED>), dim3(blocks), dim3(kDT), lds, st, a);
  return hipGetLastError();
}

// Register-h down kernel: T = 1, each row's chunks over 64 lanes with one or
// two chunks per lane (one wave per routed pair, at most kDW pairs), or, for
// kDW < top_k <= 2 kDW (a shared expert folded in as a ninth slot), over 32
// lanes with two pairs per wave.
template <int FMT, bool GROUPED>
inline bool try_down_t1r(const MoeDecodeArgs& a, hipStream_t st, hipError_t* err) {
  if (!QM_DOWN_REG || a.T != 1 || a.topk > kTopkMax) return false;
  const int kch = a.ex.I / Fmt<FMT>::kPerChunk;
  int L = 0, cpl = 0;
  // Short rows (fewer than 64 chunks) finish faster in the shared-LDS kernel,
  // whose startup is shorter; the register-h kernel takes rows of 64 or 128
  // chunks (inter 2048 / 4096 for int4).
  if (kch % 64 == 0 && kch / 64 <= 2 && a.topk <= kDW) {
    L = 64;
    cpl = kch / 64;
  } else if (kch == 64 && (a.topk + 1) / 2 <= kDW) {
    L = 32;
    cpl = 2;
  } else {
    return false;
  }
  if ((a.topk + 64 / L - 1) / (64 / L) > kDW) return false;
  hipError_t e2;
  if (L == 32)
    e2 = launch_dn_t1r<FMT, 32, 2, GROUPED>(a, st);
  else if (cpl == 1)
    e2 = launch_dn_t1r<FMT, 64, 1, GROUPED>(a, st);
  else
    e2 = launch_dn_t1r<FMT, 64, 2, GROUPED>(a, st);
  if (e2 == hipErrorNotSupported) return false;
  *err = e2;
  return true;
}

// Stage entry points used by the C ABI: LDS-ring kernels first, then the
// register-pipelined single-token kernels, then the general decode kernels.
template <int FMT, int XT, bool GROUPED>
inline hipError_t stage_gate_up_any(const MoeDecodeArgs& a, hipStream_t st) {
  hipError_t err = hipSuccess;
  if (try_gate_up_t1l<FMT, XT, GROUPED>(a, st, &err)) return err;
  return stage_gate_up<FMT, XT, GROUPED>(a, st);
}

template <int FMT, bool GROUPED>
inline hipError_t stage_down_any(const MoeDecodeArgs& a, hipStream_t st) {
  hipError_t err = hipSuccess;
  if (try_down_t1r<FMT, GROUPED>(a, st, &err)) return err;
  if (try_down_t1l<FMT, GROUPED>(a, st, &err)) return err;
  return stage_down<FMT, GROUPED>(a, st);
}

}  // namespace qm
