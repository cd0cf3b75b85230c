// moe_t1_impl.hpp -- the routed expert FFN for a single token (decode, B = 1).
//
// Same computation as moe_decode_impl.hpp (the K-expert group of the colibri
// page "Vulkan backend: expert tier + dense + MLA attention on any Vulkan 1.2
// GPU": fused silu(gate x) * up x, then the down projection, outputs combined
// with the routing weights), laid out for one token:
//  - gate_up: the token's activations are staged once per block; the work
//    items are (routed pair, tile of rows) over all routed experts, walked by
//    every wave with three tiles of weights in registers (two in flight while
//    the third is consumed);
//  - down: y = sum_j w_j D_j h_j is one GEMV whose reduction axis is the
//    concatenation of the routed pairs' hidden vectors: every block stages
//    all of them, every lane walks chunks of that concatenated axis (rows of
//    different experts, each chunk partial pre-multiplied by its pair's
//    routing weight and scale), and one lane reduction per output row
//    finishes it -- the weighted combine needs no extra pass, buffer or
//    atomic, and the output rows give H-way parallelism.
#pragma once
#include "moe_decode_impl.hpp"

namespace qm {

#ifndef QM_T1_BUF
#define QM_T1_BUF 2
#endif
constexpr int kT1Buf = QM_T1_BUF;  // units of weights per wave held in registers
#ifndef QM_T1_WAVES
#define QM_T1_WAVES 2
#endif
// waves per SIMD the register allocation must allow (latency hiding)
#define QM_T1_OCC __attribute__((amdgpu_waves_per_eu(QM_T1_WAVES, 8)))

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

template <int FMT, int XT, int L, int CB, bool GROUPED, bool FULL>
__global__ __launch_bounds__(kThreads) QM_T1_OCC void moe_gate_up_t1_kernel(MoeDecodeArgs a) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  __shared__ int s_e[kTopkMax];
  constexpr bool SPLIT = (FMT == kFmtInt4 && XT == kF32);
  constexpr int M = 2;
  constexpr int RU = ru_for(M, CB);
  constexpr int RPW = 64 / L;
  constexpr int TILE = RPW * RU;
  const ExpertArgs& ex = a.ex;
  const int k = a.topk;
  if ((int)threadIdx.x < k) {
    const int id = a.ids[threadIdx.x];
    s_e[threadIdx.x] = (id >= 0 && id < ex.E) ? id : -1;
  }
  __syncthreads();
  const int wave = uniform(threadIdx.x >> 6), lane = threadIdx.x & 63, lrow = lane / L;
  const int kchunks = ex.H / Fmt<FMT>::kPerChunk;
  const int ntiles = (ex.I + TILE - 1) / TILE;
  const int nitems = k * ntiles;
  const int istride = gridDim.x * kWaves;
  const NibConst nk = nib_const();
  auto next_valid = [&](int it) {
    while (it < nitems && uniform(s_e[it / ntiles]) < 0) it += istride;
    return it;
  };
  auto load = [&](TileW<M, RU, CB>& t, int it) {
    const int p = it / ntiles;
    const int e = uniform(s_e[p]), tile = it - p * ntiles;
    const int64_t eoff = (int64_t)e * ex.I;
    if constexpr (L == 64 && FULL) {  // scalar row base; every chunk of the unit exists
      const int row0 = tile * TILE;
      const uint8_t* const qrow[M] = {ex.gq + (eoff + row0) * ex.rb_h, ex.uq + (eoff + row0) * ex.rb_h};
      const float* const srow[M] = {ex.gs + (eoff + row0) * ex.G_h, ex.us + (eoff + row0) * ex.G_h};
      unit_load_row64<FMT, M, RU, CB, GROUPED>(t, qrow, srow, ex.rb_h, ex.G_h, ex.gshift, row0, ex.I, 1.0f);
    } else {
      Mats<M> mt;
      mt.q[0] = ex.gq + eoff * ex.rb_h;
      mt.q[1] = ex.uq + eoff * ex.rb_h;
      mt.s[0] = ex.gs + eoff * ex.G_h;
      mt.s[1] = ex.us + eoff * ex.G_h;
      unit_load_scaled<FMT, L, M, RU, CB, GROUPED, FULL>(t, mt, ex.rb_h, ex.G_h, ex.gshift, tile * TILE + lrow, RPW,
                                                         ex.I, kchunks, 0, 1.0f);
    }
  };
  int u[kT1Buf];
  TileW<M, RU, CB> buf[kT1Buf];
  u[0] = next_valid(uniform(blockIdx.x * kWaves + wave));
#pragma unroll
  for (int i = 1; i < kT1Buf; ++i) u[i] = u[i - 1] < nitems ? next_valid(u[i - 1] + istride) : nitems;
#pragma unroll
  for (int i = 0; i < kT1Buf; ++i)
    if (u[i] < nitems) load(buf[i], u[i]);
  stage_rows<FMT, XT>(lds, a.x, ex.H, [](int) { return 0; }, 1, kchunks);
  __syncthreads();
  const XRow xr = xrow<FMT, SPLIT>(lds, 1, kchunks, 0);
  while (true) {
#pragma unroll
    for (int i = 0; i < kT1Buf; ++i) {
      const int it = u[i];
      if (it >= nitems) return;
      float acc[M][RU];
#pragma unroll
      for (int m = 0; m < M; ++m)
#pragma unroll
        for (int j = 0; j < RU; ++j) acc[m][j] = 0.f;
      unit_compute_row<FMT, SPLIT, L, M, RU, CB, FULL>(buf[i], xr, kchunks, 0, acc, nk);
      const int last = u[(i + kT1Buf - 1) % kT1Buf];
      const int nu = last < nitems ? next_valid(last + istride) : nitems;
      if (nu < nitems) load(buf[i], nu);
      u[i] = nu;
      const int p = it / ntiles, tile = it - p * ntiles;
#pragma unroll
      for (int j = 0; j < RU; ++j) {
        const int r = tile * TILE + lrow + j * RPW;
        const float g = group_sum<L>(acc[0][j]);
        const float v = group_sum<L>(acc[1][j]);
        if ((lane % L) == 0 && r < ex.I) a.h[(int64_t)p * ex.I + r] = silu(g) * v;
      }
    }
  }
}

// Down projection + weighted combine for one token.  Lanes (all 64 on one
// row) walk the concatenated reduction axis: chunk C of a row belongs to
// valid pair q = C / kchunks at chunk c = C % kchunks of expert e_q's row.
template <int FMT, int CB, bool GROUPED>
__global__ __launch_bounds__(kThreads) QM_T1_OCC void moe_down_t1_kernel(MoeDecodeArgs a) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  __shared__ int s_e[kTopkMax], s_p[kTopkMax], s_n;
  __shared__ float s_w[kTopkMax];
  constexpr bool SPLIT = (FMT == kFmtInt4);  // h is fp32
  constexpr int M = 1;
  constexpr int RU = ru_for(M, CB) > 4 ? 4 : ru_for(M, CB);
  const ExpertArgs& ex = a.ex;
  routed_pairs(a.ids, a.w, a.topk, ex.E, s_e, s_p, s_w, &s_n);  // valid pairs of the token, in slot order
  __syncthreads();
  const int np = s_n;
  const int wave = uniform(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int kchunks = ex.I / Fmt<FMT>::kPerChunk;
  const int ktot = np * kchunks;
  const int npasses = (ktot + 64 * CB - 1) / (64 * CB);
  const int ntiles = (ex.H + RU - 1) / RU;
  const int tstride = gridDim.x * kWaves;
  const NibConst nk = nib_const();
  if (np == 0) {  // no valid expert: the output is zero
    for (int i = blockIdx.x * kThreads + threadIdx.x; i < ex.H; i += gridDim.x * kThreads) a.y[i] = 0.f;
    return;
  }
  // unit v = tile * npasses + pass
  const int nunits = ntiles * npasses;
  auto load = [&](TileW<M, RU, CB>& t, int v) {
    const int tile = v / npasses, pass = v - tile * npasses;
    const int row0 = tile * RU;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const int C = lane + 64 * (pass * CB + cb);
      const bool okc = C < ktot;
      const int q = okc ? C / kchunks : 0, c = okc ? C - q * kchunks : 0;
      const int e = s_e[q];
      const float mul = okc ? s_w[q] : 0.f;
      const uint8_t* qb = ex.dq + ((int64_t)e * ex.H + row0) * ex.rb_i + (int64_t)c * 16;
      const float* sb = ex.ds + ((int64_t)e * ex.H + row0) * ex.G_i + (GROUPED ? (c >> ex.gshift) : 0);
#pragma unroll
      for (int j = 0; j < RU; ++j) {
        if (okc && row0 + j < ex.H) {
          t.w[cb][0][j] = ld_stream(qb + j * ex.rb_i);
          t.s[cb][0][j] = mul * ld_stream(sb + j * ex.G_i);
        } else {
          const uint32_t z = (FMT == kFmtInt4) ? 0x88888888u : 0u;
          t.w[cb][0][j] = u32x4{z, z, z, z};
          t.s[cb][0][j] = 0.0f;
        }
      }
    }
  };
  int u[kT1Buf];
  TileW<M, RU, CB> buf[kT1Buf];
  u[0] = uniform(blockIdx.x * kWaves + wave) * npasses;
  auto next_unit = [&](int v) {
    const int tile = v / npasses, pass = v - tile * npasses;
    return pass + 1 < npasses ? v + 1 : (tile + tstride) * npasses;
  };
#pragma unroll
  for (int i = 1; i < kT1Buf; ++i) u[i] = u[i - 1] < nunits ? next_unit(u[i - 1]) : nunits;
#pragma unroll
  for (int i = 0; i < kT1Buf; ++i)
    if (u[i] < nunits) load(buf[i], u[i]);
  stage_rows<FMT, kF32>(lds, a.h, ex.I, [&](int b) { return s_p[b]; }, np, kchunks);
  __syncthreads();
  const int rs = row_slots(kchunks);
  const u32x4* hi = reinterpret_cast<const u32x4*>(lds);
  const u32x4* lo = hi + np * rs;
  const float* off = reinterpret_cast<const float*>(lds + (size_t)np * rs * 16 * (SPLIT ? 2 : 1));
  float acc[RU];
#pragma unroll
  for (int j = 0; j < RU; ++j) acc[j] = 0.f;
  while (true) {
#pragma unroll
    for (int i = 0; i < kT1Buf; ++i) {
      const int v = u[i];
      if (v >= nunits) return;
      const int tile = v / npasses, pass = v - tile * npasses;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const int C = lane + 64 * (pass * CB + cb);
        if (C >= ktot) break;
        const int q = C / kchunks, c = C - q * kchunks;
        if constexpr (FMT == kFmtInt4) {
          u32x4 xh[4], xl[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            xh[r] = hi[q * rs + r * kchunks + c];
            xl[r] = lo[q * rs + r * kchunks + c];
          }
          const float xo = off[q * kchunks + c];
#pragma unroll
          for (int j = 0; j < RU; ++j) {
            float s = xo;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const uint32_t w = buf[i].w[cb][0][j][r];
              uint32_t pr[4];
#pragma unroll
              for (int b = 0; b < 4; ++b) pr[b] = nib_pair(w >> (4 * b), nk);
#pragma unroll
              for (int b = 0; b < 4; ++b) s = dot2(pr[b], xh[r][b], s);
#pragma unroll
              for (int b = 0; b < 4; ++b) s = dot2(pr[b], xl[r][b], s);
            }
            acc[j] = __builtin_fmaf(buf[i].s[cb][0][j], s, acc[j]);
          }
        } else {
          const f32x4* xf = reinterpret_cast<const f32x4*>(lds);
          f32x4 xv[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) xv[r] = xf[q * rs + r * kchunks + c];
#pragma unroll
          for (int j = 0; j < RU; ++j) {
            float s = 0.f;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const uint32_t wt = buf[i].w[cb][0][j][r];
#pragma unroll
              for (int b = 0; b < 4; ++b) s = __builtin_fmaf((float)(int8_t)(wt >> (8 * b)), xv[r][b], s);
            }
            acc[j] = __builtin_fmaf(buf[i].s[cb][0][j], s, acc[j]);
          }
        }
      }
      const int last = u[(i + kT1Buf - 1) % kT1Buf];
      const int nu = last < nunits ? next_unit(last) : nunits;
      if (nu < nunits) load(buf[i], nu);
      u[i] = nu;
      if (pass == npasses - 1) {
#pragma unroll
        for (int j = 0; j < RU; ++j) {
          const int r = tile * RU + j;
          const float yv = group_sum<64>(acc[j]);
          if (lane == 0 && r < ex.H) a.y[r] = yv;
          acc[j] = 0.f;
        }
      }
    }
  }
}

// ---- launch --------------------------------------------------------------------

// The single-token kernels need at least 16 lanes per row, gate/up rows that
// fit one unit per lane (at most 8 chunks per lane), and the staged
// activations (x, or the hidden vectors of all routed pairs) within budget.
constexpr int kT1LdsBudget = 80 * 1024;

inline bool t1_gate_up_ok(int T, int topk, int L, int kchunks, size_t stage) {
  return T == 1 && topk <= kTopkMax && L >= 16 && (kchunks + L - 1) / L <= 8 && stage <= (size_t)kT1LdsBudget;
}

inline bool t1_down_ok(int T, int topk, size_t stage) {
  return T == 1 && topk <= kTopkMax && stage <= (size_t)kT1LdsBudget;
}

template <int FMT, int XT, int L, int CB, bool GROUPED>
inline hipError_t launch_gu_t1(const MoeDecodeArgs& a, hipStream_t st) {
  constexpr int TILE = (64 / L) * ru_for(2, CB);
  const int kchunks = a.ex.H / Fmt<FMT>::kPerChunk;
  const int ntiles = (a.ex.I + TILE - 1) / TILE;
  int blocks = (a.topk * ntiles + kWaves - 1) / kWaves;
  const int cap = a.max_blocks > 0 ? a.max_blocks : kV2MaxBlocks;
  if (blocks > cap) blocks = cap;
  const size_t lds = stage_rows_bytes<FMT, FMT == kFmtInt4 && XT == kF32>(1, kchunks);
  if (kchunks == L * CB)
    hipLaunchKernelGGL((moe_gate_up_t1_kernel<FMT, XT, L, CB, GROUPED, true>), dim3(blocks), dim3(kThreads), lds,
                       st, a);
  else
    hipLaunchKernelGGL((moe_gate_up_t1_kernel<FMT, XT, L, CB, GROUPED, false>), dim3(blocks), dim3(kThreads), lds,
                       st, a);
  return hipGetLastError();
}

#ifndef QM_T1_DOWN_BLOCKS
#define QM_T1_DOWN_BLOCKS 512
#endif

template <int FMT, int CB, bool GROUPED>
inline hipError_t launch_dn_t1(const MoeDecodeArgs& a, hipStream_t st) {
  constexpr int RU = ru_for(1, CB) > 4 ? 4 : ru_for(1, CB);
  const int ntiles = (a.ex.H + RU - 1) / RU;
  int blocks = (ntiles + kWaves - 1) / kWaves;
  const int cap = a.max_blocks > 0 ? a.max_blocks : QM_T1_DOWN_BLOCKS;
  if (blocks > cap) blocks = cap;
  const size_t lds = stage_rows_bytes<FMT, FMT == kFmtInt4>(a.topk, a.ex.I / Fmt<FMT>::kPerChunk);
  hipLaunchKernelGGL((moe_down_t1_kernel<FMT, CB, GROUPED>), dim3(blocks), dim3(kThreads), lds, st, a);
  return hipGetLastError();
}

template <int FMT, int XT, bool GROUPED>
inline hipError_t dispatch_gate_up_t1(const MoeDecodeArgs& a, int L, int CB, hipStream_t st) {
#define QM_T1_CB(LL)                                                   \
  switch (CB) {                                                        \
    case 1: return launch_gu_t1<FMT, XT, LL, 1, GROUPED>(a, st);       \
    case 2: return launch_gu_t1<FMT, XT, LL, 2, GROUPED>(a, st);       \
    case 3: return launch_gu_t1<FMT, XT, LL, 3, GROUPED>(a, st);       \
    case 4: return launch_gu_t1<FMT, XT, LL, 4, GROUPED>(a, st);       \
    default: return launch_gu_t1<FMT, XT, LL, 8, GROUPED>(a, st);      \
  }
  switch (L) {
    case 16: QM_T1_CB(16)
    case 32: QM_T1_CB(32)
    default: QM_T1_CB(64)
  }
#undef QM_T1_CB
}

// chunks of the concatenated reduction per lane and pass: 4 (2 for short axes)
template <int FMT, bool GROUPED>
inline hipError_t dispatch_down_t1(const MoeDecodeArgs& a, hipStream_t st) {
  const int ktot = a.topk * (a.ex.I / Fmt<FMT>::kPerChunk);
  if (ktot <= 64) return launch_dn_t1<FMT, 1, GROUPED>(a, st);
  if (ktot <= 128) return launch_dn_t1<FMT, 2, GROUPED>(a, st);
  return launch_dn_t1<FMT, 4, GROUPED>(a, st);
}

// Stage entry points used by the C ABI: the single-token kernels where they
// apply, the general decode kernels otherwise.
template <int FMT, int XT, bool GROUPED>
inline hipError_t stage_gate_up(const MoeDecodeArgs& a, hipStream_t st) {
  const int kch = a.ex.H / Fmt<FMT>::kPerChunk;
  const int L = lanes_per_row(kch);
  if (t1_gate_up_ok(a.T, a.topk, L, kch, stage_rows_bytes<FMT, FMT == kFmtInt4 && XT == kF32>(1, kch)))
    return dispatch_gate_up_t1<FMT, XT, GROUPED>(a, L, v2_cb(kch, L), st);
  return dispatch_gate_up<FMT, XT, GROUPED>(a, st);
}

template <int FMT, bool GROUPED>
inline hipError_t stage_down(const MoeDecodeArgs& a, hipStream_t st) {
  const int kch = a.ex.I / Fmt<FMT>::kPerChunk;
  if (t1_down_ok(a.T, a.topk, stage_rows_bytes<FMT, FMT == kFmtInt4>(a.topk, kch)))
    return dispatch_down_t1<FMT, GROUPED>(a, st);
  return dispatch_down<FMT, GROUPED>(a, st);
}

}  // namespace qm
