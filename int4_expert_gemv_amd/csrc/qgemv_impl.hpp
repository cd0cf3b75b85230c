// qgemv_impl.hpp -- the quantized GEMV kernel template and its launch
// helpers; instantiated per (format, activation type) in qgemv_*.hip so the
// instantiations compile in parallel.
#pragma once
#include "device.hpp"
#include "launch.hpp"

namespace qm {

template <int FMT, int XT, int L, int RU, int NB, bool GROUPED>
__global__ __launch_bounds__(kThreads) void qgemv_kernel(GemvArgs a) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  constexpr bool SPLIT = (FMT == kFmtInt4 && XT == kF32);
  constexpr int RPW = 64 / L;
  constexpr int TILE = RPW * RU;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int kchunks = a.k / Fmt<FMT>::kPerChunk;
  const int nseg = (kchunks + a.segc - 1) / a.segc;
  const int nb = a.nb;
  auto tok = [nb](int b) { return b < nb ? b : nb - 1; };  // padding slots repeat the last token

  for (int round = 0; round < a.rounds; ++round) {
    const int tile = (blockIdx.x * a.rounds + round) * kWaves + wave;
    const int row0 = tile * TILE + lane / L;
    float acc[1][RU][NB];
#pragma unroll
    for (int j = 0; j < RU; ++j)
#pragma unroll
      for (int b = 0; b < NB; ++b) acc[0][j][b] = 0.f;
    const Mats<1> mt = {{a.q}, {a.s}};

    for (int sg = 0; sg < nseg; ++sg) {
      const int kc0 = sg * a.segc;
      const int segc = min(a.segc, kchunks - kc0);
      if (nseg > 1 || round == 0) {
        if (nseg > 1 && (round > 0 || sg > 0)) __syncthreads();
        stage_x<FMT, XT, NB>(lds, a.x, a.ldx, tok, kc0, segc);
        __syncthreads();
      }
      tile_partial<FMT, SPLIT, L, 1, RU, NB, GROUPED>(mt, a.row_bytes, a.G, a.gshift, row0, RPW, a.n, kc0,
                                                       segc, lds, acc);
    }

#pragma unroll
    for (int j = 0; j < RU; ++j) {
      const int r = row0 + j * RPW;
      const float rs = (!GROUPED && r < a.n) ? a.s[r] : 1.0f;
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const float v = group_sum<L>(acc[0][j][b]);
        if ((lane % L) == 0 && r < a.n && b < a.nb) a.y[(int64_t)b * a.ldy + r] = GROUPED ? v : v * rs;
      }
    }
  }
}

// ---- host-side dispatch --------------------------------------------------------

template <int FMT, int XT, int L, int RU, int NB, bool GROUPED>
inline hipError_t launch_t(const GemvArgs& a, int blocks, size_t lds, hipStream_t st) {
  hipLaunchKernelGGL((qgemv_kernel<FMT, XT, L, RU, NB, GROUPED>), dim3(blocks), dim3(kThreads), lds, st, a);
  return hipGetLastError();
}

template <int FMT, int XT, int L, int NB, bool GROUPED>
inline hipError_t launch_nb(const GemvArgs& a, int blocks, size_t lds, hipStream_t st) {
  constexpr int RU = NB == 1 ? 4 : (NB <= 4 ? 2 : 1);
  return launch_t<FMT, XT, L, RU, NB, GROUPED>(a, blocks, lds, st);
}

template <int FMT, int XT, int L, bool GROUPED>
inline hipError_t launch_l(const GemvArgs& a, int NB, int blocks, size_t lds, hipStream_t st) {
  switch (NB) {
    case 1: return launch_nb<FMT, XT, L, 1, GROUPED>(a, blocks, lds, st);
    case 2: return launch_nb<FMT, XT, L, 2, GROUPED>(a, blocks, lds, st);
    case 4: return launch_nb<FMT, XT, L, 4, GROUPED>(a, blocks, lds, st);
    default: return launch_nb<FMT, XT, L, 8, GROUPED>(a, blocks, lds, st);
  }
}

template <int FMT, int XT, bool GROUPED>
inline hipError_t launch_g(const GemvArgs& a, int L, int NB, int blocks, size_t lds, hipStream_t st) {
  switch (L) {
    case 8: return launch_l<FMT, XT, 8, GROUPED>(a, NB, blocks, lds, st);
    case 16: return launch_l<FMT, XT, 16, GROUPED>(a, NB, blocks, lds, st);
    case 32: return launch_l<FMT, XT, 32, GROUPED>(a, NB, blocks, lds, st);
    default: return launch_l<FMT, XT, 64, GROUPED>(a, NB, blocks, lds, st);
  }
}


// Pipelined single-token GEMV: the whole x is staged once per block, each
// wave walks its tiles (grid stride) with unit i+1's weights in flight while
// unit i is computed, and the first unit's loads are issued before staging.
// Blocks [0, na) compute matrix `a0`, the others matrix `b0` (a pair of
// projections of one x in one launch; b0 = a0 and na = gridDim.x for one).
template <int FMT, int XT, int L, int RU, int CB, bool GROUPED>
__global__ __launch_bounds__(kThreads) void qgemv_v2_kernel(GemvArgs a0, GemvArgs b0, int na) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const bool first = (int)blockIdx.x < na;
  const GemvArgs a = first ? a0 : b0;
  const int bid = first ? (int)blockIdx.x : (int)blockIdx.x - na;
  const int nblk = first ? na : (int)gridDim.x - na;
  constexpr bool SPLIT = (FMT == kFmtInt4 && XT == kF32);
  constexpr int RPW = 64 / L;
  constexpr int TILE = RPW * RU;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int lrow = lane / L;
  const int kchunks = a.k / Fmt<FMT>::kPerChunk;
  const int ntiles = (a.n + TILE - 1) / TILE;
  const int npasses = (kchunks + L * CB - 1) / (L * CB);
  const int tstride = nblk * kWaves;
  const int tile0 = bid * kWaves + wave;
  const Mats<1> mt = {{a.q}, {a.s}};
  TileW<1, RU, CB> A, B;
  if (tile0 < ntiles)
    unit_load<FMT, L, 1, RU, CB, GROUPED>(A, mt, a.row_bytes, a.G, a.gshift, tile0 * TILE + lrow, RPW, a.n, kchunks,
                                          0);
  stage_x<FMT, XT, 1>(lds, a.x, a.ldx, [](int) { return 0; }, 0, kchunks);
  __syncthreads();
  pipeline_tiles<FMT, SPLIT, L, 1, RU, CB, 1, GROUPED>(
      A, B, mt, a.row_bytes, a.G, a.gshift, a.n, kchunks, tile0, tstride, ntiles, npasses, lds,
      [&](int tile, float (&acc)[1][RU][1]) {
#pragma unroll
        for (int j = 0; j < RU; ++j) {
          const int r = tile * TILE + lrow + j * RPW;
          const float rs = (!GROUPED && r < a.n) ? a.s[r] : 1.0f;
          const float v = group_sum<L>(acc[0][j][0]);
          if ((lane % L) == 0 && r < a.n) a.y[r] = GROUPED ? v : v * rs;
        }
      });
}

template <int FMT, int XT, int L, int CB, bool GROUPED>
inline hipError_t launch_v2_cb(const GemvArgs& a, const GemvArgs& b, int na, int blocks, size_t lds, hipStream_t st) {
  constexpr int RU = (8 / CB) >= 1 ? (8 / CB >= 8 ? 8 : (8 / CB >= 4 ? 4 : (8 / CB >= 2 ? 2 : 1))) : 1;
  hipLaunchKernelGGL((qgemv_v2_kernel<FMT, XT, L, RU, CB, GROUPED>), dim3(blocks), dim3(kThreads), lds, st, a, b, na);
  return hipGetLastError();
}

template <int FMT, int XT, bool GROUPED>
inline hipError_t launch_v2(const GemvArgs& a, const GemvArgs& b, int na, int L, int CB, int blocks, size_t lds,
                            hipStream_t st) {
#define QM_V2L(LL)                                                                     \
  switch (CB) {                                                                        \
    case 1: return launch_v2_cb<FMT, XT, LL, 1, GROUPED>(a, b, na, blocks, lds, st);   \
    case 2: return launch_v2_cb<FMT, XT, LL, 2, GROUPED>(a, b, na, blocks, lds, st);   \
    case 3: return launch_v2_cb<FMT, XT, LL, 3, GROUPED>(a, b, na, blocks, lds, st);   \
    case 4: return launch_v2_cb<FMT, XT, LL, 4, GROUPED>(a, b, na, blocks, lds, st);   \
    default: return launch_v2_cb<FMT, XT, LL, 8, GROUPED>(a, b, na, blocks, lds, st);  \
  }
  switch (L) {
    case 16: QM_V2L(16)
    case 32: QM_V2L(32)
    default: QM_V2L(64)
  }
#undef QM_V2L
}

}  // namespace qm
