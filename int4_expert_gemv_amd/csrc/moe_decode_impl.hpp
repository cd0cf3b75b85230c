// moe_decode_impl.hpp -- routed expert FFN for a handful of tokens (decode).
//
// Follows the K-expert group of the colibri page "Vulkan backend: expert
// tier + dense + MLA attention on any Vulkan 1.2 GPU" (commit notes
// "qmatmul_gate_up.comp" and the K-expert group note): for every routed
// expert, hidden = silu(gate x) * up x computed in one pass that reads x
// once for both projections; then the down projection; the hidden vector
// stays on the device; expert outputs are combined with their routing
// weights (page "qwen36: Vulkan expert tier, and staged device-local
// uploads": weighted accumulation of the take buffer).
//
// Three kernels on one stream, no host synchronisation:
//  1. gate_up: one block group per distinct routed expert (found by an
//     in-kernel scan of the routing list), each expert's gate and up rows read
//     once for all tokens routed to it -> h[pair][I] fp32 (workspace);
//  2. down: per distinct expert, D_e rows dotted with h of each of its pairs
//     -> pout[pair][H] fp32 (workspace);
//  3. combine: y[t] = sum_j w[t][j] * pout[t*k + j], slots in order, so the
//     result is deterministic without atomics.
#pragma once
#include "device.hpp"
#include "launch.hpp"

namespace qm {

constexpr int kMaxPairs = kThreads;  // T * top_k handled by the block-wide scan

// Block-wide scan of the routing list ids[0..P): the u-th distinct valid
// expert id in order of first occurrence, and the list of pairs routed to it
// (pair index p = t * top_k + j, ascending) in s_pairs.  Returns the expert id
// or -1 (uniform across the block).
__device__ inline int route_unique(const int32_t* __restrict__ ids, int P, int E, int u, int* s_ids, int* s_flag,
                            int* s_pairs, int* s_misc) {
  const int t = threadIdx.x;
  if (t < P) s_ids[t] = ids[t];
  if (t == 0) {
    s_misc[0] = -1;
    s_misc[1] = 0;
  }
  __syncthreads();
  if (t < P) {
    const int id = s_ids[t];
    int first = (id >= 0 && id < E);
    for (int p = 0; p < t && first; ++p) first = s_ids[p] != id;
    s_flag[t] = first;
  }
  __syncthreads();
  if (t < P && s_flag[t]) {
    int rank = 0;
    for (int p = 0; p < t; ++p) rank += s_flag[p];
    if (rank == u) s_misc[0] = s_ids[t];
  }
  __syncthreads();
  const int e = s_misc[0];
  if (e < 0) return -1;
  if (t < P && s_ids[t] == e) {
    int pos = 0;
    for (int p = 0; p < t; ++p) pos += (s_ids[p] == e);
    s_pairs[pos] = t;
    atomicAdd(&s_misc[1], 1);
  }
  __syncthreads();
  return e;
}

template <int FMT, int XT, int L, int RU, int NB, bool GROUPED>
__global__ __launch_bounds__(kThreads) void moe_gate_up_kernel(MoeDecodeArgs a) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  __shared__ int s_ids[kMaxPairs], s_flag[kMaxPairs], s_pairs[kMaxPairs], s_misc[2];
  constexpr bool SPLIT = (FMT == kFmtInt4 && XT == kF32);
  constexpr int RPW = 64 / L;
  constexpr int TILE = RPW * RU;
  const ExpertArgs& ex = a.ex;
  const int u = blockIdx.x / a.parts, part = blockIdx.x - u * a.parts;
  const int e = route_unique(a.ids, a.T * a.topk, ex.E, u, s_ids, s_flag, s_pairs, s_misc);
  if (e < 0) return;
  const int npairs = s_misc[1];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int kchunks = ex.H / Fmt<FMT>::kPerChunk;
  const int nseg = (kchunks + a.segc - 1) / a.segc;
  Mats<2> mt;
  mt.q[0] = ex.gq + (int64_t)e * ex.I * ex.rb_h;
  mt.q[1] = ex.uq + (int64_t)e * ex.I * ex.rb_h;
  mt.s[0] = ex.gs + (int64_t)e * ex.I * ex.G_h;
  mt.s[1] = ex.us + (int64_t)e * ex.I * ex.G_h;
  bool staged = false;

  for (int pb = 0; pb < npairs; pb += NB) {
    const int nb = min(NB, npairs - pb);
    auto tok = [&](int b) { return s_pairs[pb + (b < nb ? b : nb - 1)] / a.topk; };
    for (int round = 0; round < a.rounds; ++round) {
      const int tile = (part * a.rounds + round) * kWaves + wave;
      const int row0 = tile * TILE + lane / L;
      float acc[2][RU][NB];
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int j = 0; j < RU; ++j)
#pragma unroll
          for (int b = 0; b < NB; ++b) acc[m][j][b] = 0.f;
      for (int sg = 0; sg < nseg; ++sg) {
        const int kc0 = sg * a.segc;
        const int segc = min(a.segc, kchunks - kc0);
        if (nseg > 1 || round == 0) {
          if (staged) __syncthreads();
          stage_x<FMT, XT, NB>(lds, a.x, ex.H, tok, kc0, segc);
          __syncthreads();
          staged = true;
        }
        tile_partial<FMT, SPLIT, L, 2, RU, NB, GROUPED>(mt, ex.rb_h, ex.G_h, ex.gshift, row0, RPW, ex.I, kc0,
                                                         segc, lds, acc);
      }
#pragma unroll
      for (int j = 0; j < RU; ++j) {
        const int r = row0 + j * RPW;
        const bool ok = r < ex.I;
        const float gsr = (!GROUPED && ok) ? mt.s[0][r] : 1.0f;
        const float usr = (!GROUPED && ok) ? mt.s[1][r] : 1.0f;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const float g = group_sum<L>(acc[0][j][b]) * gsr;
          const float v = group_sum<L>(acc[1][j][b]) * usr;
          if ((lane % L) == 0 && ok && b < nb) a.h[(int64_t)s_pairs[pb + b] * ex.I + r] = silu(g) * v;
        }
      }
    }
  }
}

template <int FMT, int L, int RU, int NB, bool GROUPED>
__global__ __launch_bounds__(kThreads) void moe_down_kernel(MoeDecodeArgs a) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  __shared__ int s_ids[kMaxPairs], s_flag[kMaxPairs], s_pairs[kMaxPairs], s_misc[2];
  constexpr bool SPLIT = (FMT == kFmtInt4);  // h is fp32
  constexpr int RPW = 64 / L;
  constexpr int TILE = RPW * RU;
  const ExpertArgs& ex = a.ex;
  const int u = blockIdx.x / a.parts, part = blockIdx.x - u * a.parts;
  const int e = route_unique(a.ids, a.T * a.topk, ex.E, u, s_ids, s_flag, s_pairs, s_misc);
  if (e < 0) return;
  const int npairs = s_misc[1];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int kchunks = ex.I / Fmt<FMT>::kPerChunk;
  const int nseg = (kchunks + a.segc - 1) / a.segc;
  Mats<1> mt;
  mt.q[0] = ex.dq + (int64_t)e * ex.H * ex.rb_i;
  mt.s[0] = ex.ds + (int64_t)e * ex.H * ex.G_i;
  bool staged = false;

  for (int pb = 0; pb < npairs; pb += NB) {
    const int nb = min(NB, npairs - pb);
    auto tok = [&](int b) { return s_pairs[pb + (b < nb ? b : nb - 1)]; };
    for (int round = 0; round < a.rounds; ++round) {
      const int tile = (part * a.rounds + round) * kWaves + wave;
      const int row0 = tile * TILE + lane / L;
      float acc[1][RU][NB];
#pragma unroll
      for (int j = 0; j < RU; ++j)
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[0][j][b] = 0.f;
      for (int sg = 0; sg < nseg; ++sg) {
        const int kc0 = sg * a.segc;
        const int segc = min(a.segc, kchunks - kc0);
        if (nseg > 1 || round == 0) {
          if (staged) __syncthreads();
          stage_x<FMT, kF32, NB>(lds, a.h, ex.I, tok, kc0, segc);
          __syncthreads();
          staged = true;
        }
        tile_partial<FMT, SPLIT, L, 1, RU, NB, GROUPED>(mt, ex.rb_i, ex.G_i, ex.gshift, row0, RPW, ex.H, kc0,
                                                         segc, lds, acc);
      }
#pragma unroll
      for (int j = 0; j < RU; ++j) {
        const int r = row0 + j * RPW;
        const bool ok = r < ex.H;
        const float rs = (!GROUPED && ok) ? mt.s[0][r] : 1.0f;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const float v = group_sum<L>(acc[0][j][b]) * rs;
          if ((lane % L) == 0 && ok && b < nb) a.pout[(int64_t)s_pairs[pb + b] * ex.H + r] = v;
        }
      }
    }
  }
}

// y[t][n] = sum_j w[t][j] * pout[t*k + j][n] over valid ids, in slot order.
static __global__ __launch_bounds__(256) void moe_combine_kernel(MoeDecodeArgs a) {
  const int H = a.ex.H;
  const int64_t total = (int64_t)a.T * H;
  for (int64_t i = blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    const int t = (int)(i / H);
    const int n = (int)(i - (int64_t)t * H);
    float acc = 0.f;
    for (int j = 0; j < a.topk; ++j) {
      const int p = t * a.topk + j;
      const int id = a.ids[p];
      if (id >= 0 && id < a.ex.E) acc = __builtin_fmaf(a.w[p], a.pout[(int64_t)p * H + n], acc);
    }
    a.y[i] = acc;
  }
}

// ---- host-side dispatch --------------------------------------------------------

template <int FMT, int XT, int L, int NB, bool GROUPED>
inline hipError_t launch_dec(const MoeDecodeArgs& a0, hipStream_t st) {
  constexpr int RU_GU = NB == 1 ? 2 : 1;  // gate and up rows: 2 * RU_GU rows in flight per lane
  const int P = a0.T * a0.topk;
  const ExpertArgs& ex = a0.ex;
  // gate_up: K = H
  {
    MoeDecodeArgs a = a0;
    const int kchunks = ex.H / Fmt<FMT>::kPerChunk;
    a.segc = seg_chunks(FMT, XT, NB, kchunks);
    const int tiles = (ex.I + (64 / L) * RU_GU - 1) / ((64 / L) * RU_GU);
    a.rounds = a0.rounds > 0 ? a0.rounds : 1;
    a.parts = (tiles + kWaves * a.rounds - 1) / (kWaves * a.rounds);
    const size_t lds = stage_bytes(FMT, XT, NB, a.segc);
    hipLaunchKernelGGL((moe_gate_up_kernel<FMT, XT, L, RU_GU, NB, GROUPED>), dim3(P * a.parts), dim3(kThreads),
                       lds, st, a);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

template <int FMT, int L, int NB, bool GROUPED>
inline hipError_t launch_down(const MoeDecodeArgs& a0, hipStream_t st) {
  constexpr int RU_DN = NB == 1 ? 4 : (NB <= 4 ? 2 : 1);
  const int P = a0.T * a0.topk;
  const ExpertArgs& ex = a0.ex;
  MoeDecodeArgs a = a0;
  const int kchunks = ex.I / Fmt<FMT>::kPerChunk;
  a.segc = seg_chunks(FMT, kF32, NB, kchunks);
  const int tiles = (ex.H + (64 / L) * RU_DN - 1) / ((64 / L) * RU_DN);
  a.rounds = a0.rounds > 0 ? a0.rounds : 1;
  a.parts = (tiles + kWaves * a.rounds - 1) / (kWaves * a.rounds);
  const size_t lds = stage_bytes(FMT, kF32, NB, a.segc);
  hipLaunchKernelGGL((moe_down_kernel<FMT, L, RU_DN, NB, GROUPED>), dim3(P * a.parts), dim3(kThreads), lds, st,
                     a);
  return hipGetLastError();
}


// ---- pipelined single-token kernels --------------------------------------------
// One batch slot (NB = 1): every pair of a distinct expert is processed in
// turn with the whole activation row staged in LDS; each wave walks its tiles
// with the next unit's weights in flight (see pipeline_tiles).

constexpr int ru_for(int M, int CB) {
  return 8 / (M * CB) >= 8 ? 8 : (8 / (M * CB) >= 4 ? 4 : (8 / (M * CB) >= 2 ? 2 : 1));
}

template <int FMT, int XT, int L, int CB, bool GROUPED>
__global__ __launch_bounds__(kThreads) void moe_gate_up_v2_kernel(MoeDecodeArgs a) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  __shared__ int s_ids[kMaxPairs], s_flag[kMaxPairs], s_pairs[kMaxPairs], s_misc[2];
  constexpr bool SPLIT = (FMT == kFmtInt4 && XT == kF32);
  constexpr int RU = ru_for(2, CB);
  constexpr int RPW = 64 / L;
  constexpr int TILE = RPW * RU;
  const ExpertArgs& ex = a.ex;
  const int u = blockIdx.x / a.parts, part = blockIdx.x - u * a.parts;
  const int e = route_unique(a.ids, a.T * a.topk, ex.E, u, s_ids, s_flag, s_pairs, s_misc);
  if (e < 0) return;
  const int npairs = s_misc[1];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int lrow = lane / L;
  const int kchunks = ex.H / Fmt<FMT>::kPerChunk;
  const int ntiles = (ex.I + TILE - 1) / TILE;
  const int npasses = (kchunks + L * CB - 1) / (L * CB);
  const int tile0 = part * kWaves + wave, tstride = a.parts * kWaves;
  Mats<2> mt;
  mt.q[0] = ex.gq + (int64_t)e * ex.I * ex.rb_h;
  mt.q[1] = ex.uq + (int64_t)e * ex.I * ex.rb_h;
  mt.s[0] = ex.gs + (int64_t)e * ex.I * ex.G_h;
  mt.s[1] = ex.us + (int64_t)e * ex.I * ex.G_h;
  for (int pb = 0; pb < npairs; ++pb) {
    const int pair = s_pairs[pb];
    const int tok = pair / a.topk;
    TileW<2, RU, CB> A, B;
    if (tile0 < ntiles)
      unit_load<FMT, L, 2, RU, CB, GROUPED>(A, mt, ex.rb_h, ex.G_h, ex.gshift, tile0 * TILE + lrow, RPW, ex.I,
                                            kchunks, 0);
    if (pb > 0) __syncthreads();
    stage_x<FMT, XT, 1>(lds, a.x, ex.H, [tok](int) { return tok; }, 0, kchunks);
    __syncthreads();
    pipeline_tiles<FMT, SPLIT, L, 2, RU, CB, 1, GROUPED>(
        A, B, mt, ex.rb_h, ex.G_h, ex.gshift, ex.I, kchunks, tile0, tstride, ntiles, npasses, lds,
        [&](int tile, float (&acc)[2][RU][1]) {
#pragma unroll
          for (int j = 0; j < RU; ++j) {
            const int r = tile * TILE + lrow + j * RPW;
            const bool ok = r < ex.I;
            const float gsr = (!GROUPED && ok) ? mt.s[0][r] : 1.0f;
            const float usr = (!GROUPED && ok) ? mt.s[1][r] : 1.0f;
            const float g = group_sum<L>(acc[0][j][0]) * gsr;
            const float v = group_sum<L>(acc[1][j][0]) * usr;
            if ((lane % L) == 0 && ok) a.h[(int64_t)pair * ex.I + r] = silu(g) * v;
          }
        });
  }
}

template <int FMT, int L, int CB, bool GROUPED>
__global__ __launch_bounds__(kThreads) void moe_down_v2_kernel(MoeDecodeArgs a) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  __shared__ int s_ids[kMaxPairs], s_flag[kMaxPairs], s_pairs[kMaxPairs], s_misc[2];
  constexpr bool SPLIT = (FMT == kFmtInt4);
  constexpr int RU = ru_for(1, CB);
  constexpr int RPW = 64 / L;
  constexpr int TILE = RPW * RU;
  const ExpertArgs& ex = a.ex;
  const int u = blockIdx.x / a.parts, part = blockIdx.x - u * a.parts;
  const int e = route_unique(a.ids, a.T * a.topk, ex.E, u, s_ids, s_flag, s_pairs, s_misc);
  if (e < 0) return;
  const int npairs = s_misc[1];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int lrow = lane / L;
  const int kchunks = ex.I / Fmt<FMT>::kPerChunk;
  const int ntiles = (ex.H + TILE - 1) / TILE;
  const int npasses = (kchunks + L * CB - 1) / (L * CB);
  const int tile0 = part * kWaves + wave, tstride = a.parts * kWaves;
  Mats<1> mt;
  mt.q[0] = ex.dq + (int64_t)e * ex.H * ex.rb_i;
  mt.s[0] = ex.ds + (int64_t)e * ex.H * ex.G_i;
  for (int pb = 0; pb < npairs; ++pb) {
    const int pair = s_pairs[pb];
    TileW<1, RU, CB> A, B;
    if (tile0 < ntiles)
      unit_load<FMT, L, 1, RU, CB, GROUPED>(A, mt, ex.rb_i, ex.G_i, ex.gshift, tile0 * TILE + lrow, RPW, ex.H,
                                            kchunks, 0);
    if (pb > 0) __syncthreads();
    stage_x<FMT, kF32, 1>(lds, a.h, ex.I, [pair](int) { return pair; }, 0, kchunks);
    __syncthreads();
    pipeline_tiles<FMT, SPLIT, L, 1, RU, CB, 1, GROUPED>(
        A, B, mt, ex.rb_i, ex.G_i, ex.gshift, ex.H, kchunks, tile0, tstride, ntiles, npasses, lds,
        [&](int tile, float (&acc)[1][RU][1]) {
#pragma unroll
          for (int j = 0; j < RU; ++j) {
            const int r = tile * TILE + lrow + j * RPW;
            const bool ok = r < ex.H;
            const float rs = (!GROUPED && ok) ? mt.s[0][r] : 1.0f;
            const float v = group_sum<L>(acc[0][j][0]) * rs;
            if ((lane % L) == 0 && ok) a.pout[(int64_t)pair * ex.H + r] = v;
          }
        });
  }
}

// blocks per distinct expert for the pipelined kernels
inline int v2_parts(int ntiles, int P, int max_blocks) {
  const int cap = (max_blocks > 0 ? max_blocks : kV2MaxBlocks) / (P > 0 ? P : 1);
  int parts = (ntiles + kWaves - 1) / kWaves;
  if (parts > cap) parts = cap;
  return parts < 1 ? 1 : parts;
}

template <int FMT, int XT, int L, int CB, bool GROUPED>
inline hipError_t launch_gu_v2(const MoeDecodeArgs& a0, hipStream_t st) {
  MoeDecodeArgs a = a0;
  constexpr int RU = ru_for(2, CB);
  const int P = a.T * a.topk;
  const int kchunks = a.ex.H / Fmt<FMT>::kPerChunk;
  const int ntiles = (a.ex.I + (64 / L) * RU - 1) / ((64 / L) * RU);
  a.parts = v2_parts(ntiles, P, a.max_blocks);
  a.segc = kchunks;
  const size_t lds = stage_bytes(FMT, XT, 1, kchunks);
  hipLaunchKernelGGL((moe_gate_up_v2_kernel<FMT, XT, L, CB, GROUPED>), dim3(P * a.parts), dim3(kThreads), lds, st,
                     a);
  return hipGetLastError();
}

template <int FMT, int L, int CB, bool GROUPED>
inline hipError_t launch_dn_v2(const MoeDecodeArgs& a0, hipStream_t st) {
  MoeDecodeArgs a = a0;
  constexpr int RU = ru_for(1, CB);
  const int P = a.T * a.topk;
  const int kchunks = a.ex.I / Fmt<FMT>::kPerChunk;
  const int ntiles = (a.ex.H + (64 / L) * RU - 1) / ((64 / L) * RU);
  a.parts = v2_parts(ntiles, P, a.max_blocks);
  a.segc = kchunks;
  const size_t lds = stage_bytes(FMT, kF32, 1, kchunks);
  hipLaunchKernelGGL((moe_down_v2_kernel<FMT, L, CB, GROUPED>), dim3(P * a.parts), dim3(kThreads), lds, st, a);
  return hipGetLastError();
}

#define QM_V2_SWITCH(LAUNCH, ...)                     \
  switch (L) {                                        \
    case 16: QM_V2_CB(LAUNCH, 16, __VA_ARGS__) break; \
    case 32: QM_V2_CB(LAUNCH, 32, __VA_ARGS__) break; \
    default: QM_V2_CB(LAUNCH, 64, __VA_ARGS__) break; \
  }

// true when the single-token pipelined kernels apply: one token, at least 16
// lanes per row and the whole activation row fits the staging budget
inline bool v2_ok(int T, int L, size_t stage) { return T == 1 && L >= 16 && stage <= (size_t)kLdsBudget; }

template <int FMT, int XT, bool GROUPED>
inline hipError_t dispatch_gate_up_v2(const MoeDecodeArgs& a, int L, int CB, hipStream_t st) {
#define QM_V2_CB(LAUNCH, LL, ...)                                   \
  switch (CB) {                                                     \
    case 1: return LAUNCH<FMT, __VA_ARGS__ LL, 1, GROUPED>(a, st);  \
    case 2: return LAUNCH<FMT, __VA_ARGS__ LL, 2, GROUPED>(a, st);  \
    case 3: return LAUNCH<FMT, __VA_ARGS__ LL, 3, GROUPED>(a, st);  \
    case 4: return LAUNCH<FMT, __VA_ARGS__ LL, 4, GROUPED>(a, st);  \
    default: return LAUNCH<FMT, __VA_ARGS__ LL, 8, GROUPED>(a, st); \
  }
  QM_V2_SWITCH(launch_gu_v2, XT, )
  return hipErrorInvalidValue;
}

template <int FMT, bool GROUPED>
inline hipError_t dispatch_down_v2(const MoeDecodeArgs& a, int L, int CB, hipStream_t st) {
  QM_V2_SWITCH(launch_dn_v2, )
  return hipErrorInvalidValue;
#undef QM_V2_CB
}

inline int decode_nb(int T) { return T <= 1 ? 1 : (T <= 2 ? 2 : (T <= 4 ? 4 : 8)); }

// Stage 1: h for every valid pair.  Batch slots per pass over an expert's
// weights = the token count rounded up to 1, 2, 4 or 8.
template <int FMT, int XT, bool GROUPED>
inline hipError_t dispatch_gate_up(const MoeDecodeArgs& a, hipStream_t st) {
  const int Lg = lanes_per_row(a.ex.H / Fmt<FMT>::kPerChunk);
  if (v2_ok(a.T, Lg, stage_bytes(FMT, XT, 1, a.ex.H / Fmt<FMT>::kPerChunk)))
    return dispatch_gate_up_v2<FMT, XT, GROUPED>(a, Lg, v2_cb(a.ex.H / Fmt<FMT>::kPerChunk, Lg), st);
#define QM_GU(NB)                                                      \
  switch (Lg) {                                                        \
    case 8: return launch_dec<FMT, XT, 8, NB, GROUPED>(a, st);         \
    case 16: return launch_dec<FMT, XT, 16, NB, GROUPED>(a, st);       \
    case 32: return launch_dec<FMT, XT, 32, NB, GROUPED>(a, st);       \
    default: return launch_dec<FMT, XT, 64, NB, GROUPED>(a, st);       \
  }
  switch (decode_nb(a.T)) {
    case 1: QM_GU(1)
    case 2: QM_GU(2)
    case 4: QM_GU(4)
    default: QM_GU(8)
  }
#undef QM_GU
}

// Stage 2: per-pair down projections, then the slot-ordered weighted combine.
template <int FMT, bool GROUPED>
inline hipError_t dispatch_down(const MoeDecodeArgs& a, hipStream_t st) {
  const int Ld = lanes_per_row(a.ex.I / Fmt<FMT>::kPerChunk);
  hipError_t err;
  if (v2_ok(a.T, Ld, stage_bytes(FMT, kF32, 1, a.ex.I / Fmt<FMT>::kPerChunk))) {
    err = dispatch_down_v2<FMT, GROUPED>(a, Ld, v2_cb(a.ex.I / Fmt<FMT>::kPerChunk, Ld), st);
    if (err != hipSuccess) return err;
    const int64_t total = (int64_t)a.T * a.ex.H;
    int blocks = (int)((total + 255) / 256);
    if (blocks > 2048) blocks = 2048;
    hipLaunchKernelGGL(moe_combine_kernel, dim3(blocks), dim3(256), 0, st, a);
    return hipGetLastError();
  }
#define QM_DN(NB)                                                      \
  switch (Ld) {                                                        \
    case 8: err = launch_down<FMT, 8, NB, GROUPED>(a, st); break;      \
    case 16: err = launch_down<FMT, 16, NB, GROUPED>(a, st); break;    \
    case 32: err = launch_down<FMT, 32, NB, GROUPED>(a, st); break;    \
    default: err = launch_down<FMT, 64, NB, GROUPED>(a, st); break;    \
  }
  switch (decode_nb(a.T)) {
    case 1: QM_DN(1) break;
    case 2: QM_DN(2) break;
    case 4: QM_DN(4) break;
    default: QM_DN(8) break;
  }
#undef QM_DN
  if (err != hipSuccess) return err;
  const int64_t total = (int64_t)a.T * a.ex.H;
  int blocks = (int)((total + 255) / 256);
  if (blocks > 2048) blocks = 2048;
  hipLaunchKernelGGL(moe_combine_kernel, dim3(blocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace qm
