// gemv.hip -- y = W x for one resident quantized matrix (qgemv), two matrices
// sharing x (qgemv_pair) and up to 8 activation rows per weight read
// (qgemm_small): the quantized GEMV of the colibri page "Vulkan backend:
// expert tier + dense + MLA attention on any Vulkan 1.2 GPU" (commit notes
// "backend_vulkan.c/.h + shaders/qmatmul.comp", the S-token batch of the same
// shader, and "fmt=4 grouped scales"), int4 (grouped or per row) and int8 per
// row, and int3-g64 (the int3 commit notes of the same page; as signed
// nibbles, planes.hpp), on the activation digit planes of planes.hpp.
//
// Work split.  A persistent grid of as many workgroups (eight waves each) as
// the CUs hold at once (one or two per CU, by the kernel's registers).
// A row's inputs are cut into chunks of 32 int4 (16 bytes), 16 int8 (16
// bytes) or 32 int3 weights (12 bytes: half a 24-byte group -- two low-part
// words and their 32 high bits -- turned into four signed-nibble words when
// used);
// lane l takes chunks l + 64 i of every row.  The reduction runs over
// segments of 64 * CPL chunks (one segment covers a row when the digit planes
// of all its activations fit the LDS budget).  Per segment the workgroup
// turns the segment's activations into digit planes in LDS -- once per
// workgroup, for all its rows; their loads go first, so that they do not
// wait behind weight requests -- and then every wave walks its row tiles
// (NU rows; tiles wave, wave + all waves, ...) with the next tile's weights
// loaded into a second register buffer while the current one is computed.  A plane's
// digits are read from LDS once per chunk for all NU rows of the tile.  The
// rows of a second matrix of the same x (qgemv_pair) continue the row index
// space of the first.  Per-lane partial sums are reduced across the wave in
// a fixed order, so results do not depend on timing.
#include <atomic>

#include "launch.hpp"
#include "planes.hpp"

namespace qm {

namespace {

constexpr int kGvWaves = 8;
constexpr int kGvThreads = 64 * kGvWaves;
constexpr int kGvItems = 1024;  // activation groups staged per segment (two per thread)

__device__ __forceinline__ int wave_uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

template <int FMT> constexpr int per_chunk() { return FMT == kFmtInt8 ? 16 : 32; }
template <int FMT> constexpr int words_per_group() { return FMT == kFmtInt8 ? 8 : 16; }

// LDS: two planes of digit words [2][NB][SEGC][W] plus factors [NB][SEGC] and
// the plane-count slot.  (One group per chunk: 32 activations against int4,
// 16 against int8.)
template <int FMT, int NB, int CPL>
constexpr size_t gv_lds() {
  return (size_t)2 * NB * 64 * CPL * words_per_group<FMT>() * 4 + (size_t)NB * 64 * CPL * 4 + 16;
}

struct RowRef {
  const uint8_t* q;
  const float* s;
  float* y;
  int64_t ldy;
};

template <int FMT, int XT, int NB, int CPL, int NU, bool GROUPED>
__global__ __launch_bounds__(kGvThreads) void gemv_kernel(GemvArgs a0, GemvArgs a1, int nrows1) {
  constexpr int PER = per_chunk<FMT>();
  constexpr int W = words_per_group<FMT>();
  constexpr int SEGC = 64 * CPL;  // chunks (= activation groups) per segment and token
  constexpr int MI = (NB * SEGC + kGvThreads - 1) / kGvThreads;  // staged groups per thread
  static_assert(NB * SEGC <= kGvItems, "segment too large for the staging loop");
  extern __shared__ __attribute__((aligned(16))) char lds[];
  uint32_t* xd = reinterpret_cast<uint32_t*>(lds);                            // [2][NB][SEGC][W]
  float* xf = reinterpret_cast<float*>(lds + (size_t)2 * NB * SEGC * W * 4);  // [NB][SEGC]
  int* pslot = reinterpret_cast<int*>(xf + NB * SEGC);

  const int wave = wave_uniform(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int n0 = a0.n;
  const int nrows = n0 + nrows1;  // rows of both matrices
  const int ntiles = (nrows + NU - 1) / NU;
  const int wstep = gridDim.x * kGvWaves;
  const int w0 = blockIdx.x * kGvWaves + wave;  // this wave's first tile
  const int kch = a0.k / PER;
  const int nseg = (kch + SEGC - 1) / SEGC;
  const int nb = a0.nb;

  auto row_ref = [&](int r) -> RowRef {
    r = min(r, nrows - 1);
    if (r < n0) return RowRef{a0.q + (int64_t)r * a0.row_bytes, a0.s + (int64_t)r * a0.G, a0.y + r, a0.ldy};
    r -= n0;
    return RowRef{a1.q + (int64_t)r * a1.row_bytes, a1.s + (int64_t)r * a1.G, a1.y + r, a1.ldy};
  };
  const int gshift = a0.gshift;

  u32x4 wa[NU][CPL], wb[NU][CPL];
  float sa[NU][CPL], sb[NU][CPL];
  auto load_tile = [&](u32x4 (&wv)[NU][CPL], float (&sv)[NU][CPL], int tile, int c0) {
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const RowRef rr = row_ref(tile * NU + u);
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        const int c = c0 + lane + 64 * i;
        if (c < kch) {
          if constexpr (FMT == kFmtInt3) {  // group c / 2: low words 2 (c & 1), +1 and their 32 high bits
            const uint8_t* gp = rr.q + (int64_t)(c >> 1) * 24;
            const u32x2 lw = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(gp + 8 * (c & 1)));
            const uint32_t hw = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(gp + 16 + 4 * (c & 1)));
            wv[u][i] = u32x4{lw[0], lw[1], hw, 0u};
          } else {
            wv[u][i] = ld_stream(rr.q + (int64_t)c * 16);
          }
          if constexpr (GROUPED) sv[u][i] = ld_stream(rr.s + (c >> gshift));
        }
      }
    }
  };

  // partial sums of one tile over one segment, reduced and written (first
  // segment) or added (later segments) to y
  auto compute_tile = [&](const u32x4 (&wv)[NU][CPL], const float (&sv)[NU][CPL], int tile, int c0, int P,
                          bool first_seg) {
    float acc[NU][NB];
#pragma unroll
    for (int u = 0; u < NU; ++u)
#pragma unroll
      for (int t = 0; t < NB; ++t) acc[u][t] = 0.f;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int cl = lane + 64 * i;  // chunk within the segment
      if (c0 + cl >= kch) continue;
      u32x4 w[NU];
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        w[u] = wv[u][i];
        if constexpr (FMT == kFmtInt4) w[u] ^= 0x88888888u;
        if constexpr (FMT == kFmtInt3) {
          uint32_t e0, o0, e1, o1;
          i3_words(wv[u][i][0], wv[u][i][2] & 0xFFFFu, e0, o0);
          i3_words(wv[u][i][1], wv[u][i][2] >> 16, e1, o1);
          w[u] = u32x4{e0, o0, e1, o1};
        }
      }
#pragma unroll
      for (int t = 0; t < NB; ++t) {
        if (t >= nb) break;
        float ta[NU];
#pragma unroll
        for (int u = 0; u < NU; ++u) ta[u] = 0.f;
        for (int pp = 0; pp < P; ++pp) {
          const float ps = ldexpf(1.f, -15 * pp);
          const u32x4* src = reinterpret_cast<const u32x4*>(xd + ((size_t)(pp * NB + t) * SEGC + cl) * W);
          uint32_t xw[W];
#pragma unroll
          for (int q = 0; q < W / 4; ++q) {
            const u32x4 v4 = src[q];
            xw[4 * q] = v4[0];
            xw[4 * q + 1] = v4[1];
            xw[4 * q + 2] = v4[2];
            xw[4 * q + 3] = v4[3];
          }
#pragma unroll
          for (int u = 0; u < NU; ++u) {
            const int S = FMT == kFmtInt8 ? gdot_i8(w[u], xw) : gdot_i4(w[u], xw);
            ta[u] = __builtin_fmaf((float)S, ps, ta[u]);
          }
        }
        const float f = xf[t * SEGC + cl];
#pragma unroll
        for (int u = 0; u < NU; ++u) acc[u][t] = __builtin_fmaf(ta[u], GROUPED ? f * sv[u][i] : f, acc[u][t]);
      }
    }
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int r = tile * NU + u;
      const RowRef rr = row_ref(r);
      const float srow = GROUPED ? 1.f : *rr.s;
#pragma unroll
      for (int t = 0; t < NB; ++t) {
        if (t >= nb) break;
        const float yv = group_sum<64>(acc[u][t]) * srow;
        if (lane == 0 && r < nrows) {
          float* dst = rr.y + (int64_t)t * rr.ldy;
          *dst = first_seg ? yv : *dst + yv;
        }
      }
    }
  };

  for (int seg = 0; seg < nseg; ++seg) {
    const int c0 = seg * SEGC;
    // 1. the segment's activations as digit planes in LDS (all planes the
    //    segment needs; the plane count is the largest over its groups)
    if (seg > 0) __syncthreads();  // every wave is done with the previous segment's planes
    if (threadIdx.x == 0) *pslot = 0;
    const int ng = min(SEGC, kch - c0);  // groups of this segment per token
    int E[MI];
    int pneed = 1;
#pragma unroll
    for (int m = 0; m < MI; ++m) {
      const int it = threadIdx.x + kGvThreads * m;
      const int t = it / SEGC, g = it - t * SEGC;
      E[m] = 0;
      if (t < nb && g < ng) {
        float v[PER];
        load_acts<XT, PER>(a0.x, (int64_t)t * a0.ldx + (int64_t)(c0 + g) * PER, v);
        pneed = max(pneed, group_planes<PER, XT>(v, &E[m]));
      }
    }
    __syncthreads();  // *pslot reset before any atomic
    const int P = block_max_int(pneed, pslot);
    // LDS holds two planes; more (rare, very wide activation ranges) are
    // consumed two at a time below
    for (int p0 = 0; p0 < P; p0 += 2) {
      if (p0 > 0) __syncthreads();
      const int np = min(2, P - p0);
#pragma unroll
      for (int m = 0; m < MI; ++m) {
        const int it = threadIdx.x + kGvThreads * m;
        const int t = it / SEGC, g = it - t * SEGC;
        if (t < nb && g < ng) {
          stage_group<FMT, XT>(a0.x, (int64_t)t * a0.ldx + (int64_t)(c0 + g) * PER, E[m], p0, np,
                               xd + ((size_t)t * SEGC + g) * W, (size_t)NB * SEGC * W);
          xf[t * SEGC + g] = ldexpf(1.f, E[m] - 14 - 15 * p0);
        }
      }
      __syncthreads();
      // 2. the wave's tiles (the first one's weights requested now), the next
      //    one's weights loading while one is computed
      const bool first = seg == 0 && p0 == 0;
      int tile = w0;
      if (tile < ntiles) load_tile(wa, sa, tile, c0);
      for (; tile < ntiles; tile += 2 * wstep) {
        const int t1 = tile + wstep, t2 = tile + 2 * wstep;
        if (t1 < ntiles) load_tile(wb, sb, t1, c0);
        compute_tile(wa, sa, tile, c0, np, first);
        if (t1 >= ntiles) break;
        if (t2 < ntiles) load_tile(wa, sa, t2, c0);
        compute_tile(wb, sb, t1, c0, np, first);
      }
    }
  }
}

template <int FMT, int XT, int NB, int CPL, bool GROUPED>
hipError_t launch_cpl(const GemvArgs& a, const GemvArgs* b, int cus, hipStream_t st) {
  // rows per tile: enough registers for two tiles of weights; grouped rows
  // of 3-4 chunks per lane take one row per tile, which leaves room for two
  // workgroups per CU (measured faster than two rows and one workgroup);
  // 4-bit weights at batch 8 take two rows, which share each read of the
  // activation digits (int8 rows measured slower so)
  constexpr int NU = NB == 1   ? (CPL <= 2 ? 4 : (CPL <= 4 ? (GROUPED ? 1 : 2) : 1))
                     : NB == 2 ? (CPL <= 2 ? 2 : 1)
                     : NB == 8 ? (CPL <= 2 && FMT != kFmtInt8 ? 2 : 1)
                               : 1;
  const int nrows = a.n + (b ? b->n : 0);
  const int ntiles = (nrows + NU - 1) / NU;
  constexpr size_t lds = gv_lds<FMT, NB, CPL>();
  const void* f = reinterpret_cast<const void*>(&gemv_kernel<FMT, XT, NB, CPL, NU, GROUPED>);
  // as many workgroups as the compute units hold at once (two per CU for the
  // kernels with few registers, e.g. int8 rows of 6144: more loads in
  // flight; one for the others, whose extra workgroups would only queue);
  // looked up once per kernel (racing first calls store the same value)
  static std::atomic<int> per_cu{0};
  int occ = per_cu.load(std::memory_order_relaxed);
  if (occ <= 0) {
    occ = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, f, kGvThreads, lds) != hipSuccess || occ < 1) {
      (void)hipGetLastError();
      occ = 1;
    }
    occ = occ > 2 ? 2 : occ;
    per_cu.store(occ, std::memory_order_relaxed);
  }
  int blocks = (ntiles + kGvWaves - 1) / kGvWaves;
  if (blocks > occ * cus) blocks = occ * cus;
  hipLaunchKernelGGL((gemv_kernel<FMT, XT, NB, CPL, NU, GROUPED>), dim3(blocks), dim3(kGvThreads), lds, st, a,
                     b ? *b : a, b ? b->n : 0);
  return hipGetLastError();
}

// chunks per lane per segment: the whole row when it fits the staging limit
// (NB * 64 * CPL <= kGvItems)
template <int FMT, int XT, int NB, bool GROUPED>
hipError_t launch_nb(const GemvArgs& a, const GemvArgs* b, int cus, hipStream_t st) {
  constexpr int CAP = kGvItems / (NB * 64) < 8 ? kGvItems / (NB * 64) : 8;  // more would spill registers
  const int kch = a.k / per_chunk<FMT>();
  const int need = (kch + 63) / 64;
  if (need <= 1 || CAP == 1) return launch_cpl<FMT, XT, NB, 1, GROUPED>(a, b, cus, st);
  if constexpr (CAP >= 2) {
    if (need <= 2 || CAP == 2) return launch_cpl<FMT, XT, NB, 2, GROUPED>(a, b, cus, st);
  }
  if constexpr (CAP >= 4) {
    if (need == 3) return launch_cpl<FMT, XT, NB, 3, GROUPED>(a, b, cus, st);
    if (need <= 4 || CAP == 4) return launch_cpl<FMT, XT, NB, 4, GROUPED>(a, b, cus, st);
  }
  if constexpr (CAP >= 8) {
    if (need <= 6) return launch_cpl<FMT, XT, NB, 6, GROUPED>(a, b, cus, st);
    if (need <= 8 || CAP == 8) return launch_cpl<FMT, XT, NB, 8, GROUPED>(a, b, cus, st);
  }
  if constexpr (CAP >= 16) return launch_cpl<FMT, XT, NB, 16, GROUPED>(a, b, cus, st);
  return hipErrorNotSupported;
}

template <int FMT, int XT, bool GROUPED>
hipError_t launch_fx(const GemvArgs& a, const GemvArgs* b, int cus, hipStream_t st) {
  if (a.nb <= 1) return launch_nb<FMT, XT, 1, GROUPED>(a, b, cus, st);
  if (a.nb <= 2) return launch_nb<FMT, XT, 2, GROUPED>(a, b, cus, st);
  if (a.nb <= 4) return launch_nb<FMT, XT, 4, GROUPED>(a, b, cus, st);
  return launch_nb<FMT, XT, 8, GROUPED>(a, b, cus, st);
}

}  // namespace

// Compute units of the current device, looked up once per device
// (thread-safe: an atomic per device; racing first calls store the same value).
hipError_t device_cus(int* cus) {
  constexpr int kMaxDev = 64;
  static std::atomic<int> cache[kMaxDev];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDev) return hipErrorInvalidDevice;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v <= 0) {
    e = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if (v <= 0) return hipErrorInvalidDevice;
    cache[dev].store(v, std::memory_order_relaxed);
  }
  *cus = v;
  return hipSuccess;
}

hipError_t launch_gemv_planes(int fmt, int xdt, bool grouped, const GemvArgs& a, const GemvArgs* b, hipStream_t st) {
  if (b && (b->k != a.k || b->nb != 1 || a.nb != 1 || b->G != a.G || b->gshift != a.gshift))
    return hipErrorNotSupported;
  int cus = 0;
  const hipError_t e = device_cus(&cus);
  if (e != hipSuccess) return e;
  if (fmt == kFmtInt4) {
    if (xdt == kBF16)
      return grouped ? launch_fx<kFmtInt4, kBF16, true>(a, b, cus, st) : launch_fx<kFmtInt4, kBF16, false>(a, b, cus, st);
    return grouped ? launch_fx<kFmtInt4, kF32, true>(a, b, cus, st) : launch_fx<kFmtInt4, kF32, false>(a, b, cus, st);
  }
  if (fmt == kFmtInt8 && !grouped)
    return xdt == kBF16 ? launch_fx<kFmtInt8, kBF16, false>(a, b, cus, st) : launch_fx<kFmtInt8, kF32, false>(a, b, cus, st);
  if (fmt == kFmtInt3 && grouped)
    return xdt == kBF16 ? launch_fx<kFmtInt3, kBF16, true>(a, b, cus, st) : launch_fx<kFmtInt3, kF32, true>(a, b, cus, st);
  return hipErrorNotSupported;
}

}  // namespace qm
