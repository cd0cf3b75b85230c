// moe_t1_s.hpp -- the single-token routed expert FFN layer in one launch, for
// small experts (inter 512): the K-expert group of the colibri page "Vulkan
// backend: expert tier + dense + MLA attention on any Vulkan 1.2 GPU" (gate+up
// with SiLU, then the down projection weighted by the routing weights and
// summed) on the integer dot products of moe_t1_q.hpp.
//
// At these sizes (about 14 MB of weights per layer) two launches cost more
// than the weights take to stream.  Here every workgroup computes one gate+up
// tile (routed pair, 16 rows of h), writes the tile's digits with
// device-coherent stores, waits for them to complete and sets the tile's
// 64-bit flag to the call's nonce (a fresh value per call, so flags left by
// earlier calls never match).  It then loads its share of the down weights
// into registers -- they do not depend on h -- and polls the flags of the
// tiles its pairs need (device-coherent loads, bounded: kSpinMax polls with a
// sleep), reads their digits the same way, and combines.  The launcher only
// uses this kernel when the occupancy query says all workgroups are resident
// at once, so every awaited tile is in progress; the bound makes the kernel
// end even if that did not hold.
//
// Down split: workgroup b owns output rows [R b, R b + R); wave w takes the
// compacted routed pairs 4 (w & 1) .. +3 (16 lanes each: a down row of inter
// 512 is 16 chunks) and the rows of slice w >> 1 (every other row).  Lane
// partials go to LDS; each row is summed over the two waves of its slice in
// a fixed order, then over the lanes, so y is deterministic.
#pragma once
#include "moe_t1_q.hpp"

namespace qm {

constexpr int kSTile = 16;         // rows of h per gate+up tile (one digit group, one flag)
constexpr int kSNUD = 8;           // down rows per wave held in registers
constexpr int kSpinMax = 1 << 20;  // flag polls before giving up (each with s_sleep)

template <int XT, int CB, bool GROUPED, bool PS>
__global__ __launch_bounds__(kThreads) void moe_ffn_t1s_kernel(MoeDecodeArgs a) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  __shared__ __attribute__((aligned(16))) float s_h[kSTile];
  __shared__ int s_e[kTopkMax], s_p[kTopkMax], s_n;
  __shared__ float s_w[kTopkMax];
  constexpr int D = kSTile / kWaves;  // every unit of a wave in flight at once
  const ExpertArgs& ex = a.ex;
  const int H = ex.H;
  const int ntile = ex.I / kSTile;
  const int wave = uniform(threadIdx.x >> 6), lane = threadIdx.x & 63;
  routed_pairs(a.ids, a.w, a.topk, ex.E, s_e, s_p, s_w, &s_n);
  __syncthreads();

  // down-phase bookkeeping
  const int np = s_n;
  const int pg = wave & 1, sl = wave >> 1;
  const int qi = lane >> 4, sub = lane & 15;
  const int q = 4 * pg + qi;
  const bool qok = q < np;
  const int qq = qok ? q : 0;
  const int eD = s_e[qq];
  const float wz = qok ? s_w[qq] : 0.f;
  const bool won = 4 * pg < np;  // wave-uniform: this wave has a routed pair
  const int R = (H + gridDim.x - 1) / gridDim.x;
  const int rb0 = blockIdx.x * R;
  const int nr = min(H, rb0 + R) - rb0;          // rows of this workgroup
  const int nu = nr > sl ? (nr - sl + 1) / 2 : 0;  // rows of this wave's slice (<= kSNUD)
  u32x4 wv[kSNUD];
  float sv[kSNUD];
  auto prefetch_down = [&]() {
    if (!won || nu <= 0) return;
#pragma unroll
    for (int u = 0; u < kSNUD; ++u) {
      const int r = rb0 + sl + 2 * min(u, nu - 1);
      const int64_t er = (int64_t)eD * H + r;
      wv[u] = ld_stream(ex.dq + er * ex.rb_i + (int64_t)sub * 16);
      sv[u] = ld_stream(ex.ds + er * ex.G_i + (GROUPED ? (sub >> ex.gshift) : 0));
    }
  };

  // gate+up tile
  const int p = blockIdx.x / ntile, r0 = (blockIdx.x - p * ntile) * kSTile;
  const bool tile = gu_tile<XT, CB, kSTile, D, GROUPED, PS, true>(a, lds, s_h, p, r0);
  if (tile && wave == 0) {
    wait_vmcnt<0>();  // the tile's digits (device-coherent stores) are complete
    if (lane == 0)
      __hip_atomic_store(a.flags + (int64_t)p * ntile + r0 / kSTile, a.nonce, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  }
  prefetch_down();

  // down
  float* part = reinterpret_cast<float*>(lds);  // [R][kWaves][64]; the tile's LDS is no longer used
  lds_barrier();                                // every wave is past the tile before part is written
  if (won && nu > 0) {
    for (int it = 0; it < kSpinMax; ++it) {
      bool ok = true;
      for (int i = lane; i < 4 * ntile; i += 64) {
        const int j = i / ntile, t = i - j * ntile;
        if (4 * pg + j < np)
          ok = ok && __hip_atomic_load(a.flags + (int64_t)s_p[4 * pg + j] * ntile + t, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT) == a.nonce;
      }
      if (__ballot(!ok) == 0) break;
      __builtin_amdgcn_s_sleep(4);
    }
    // this lane's chunk of its pair's digits, read device-coherently
    const int prow = s_p[qq];
    const uint64_t* hqrow = reinterpret_cast<const uint64_t*>(a.hq + (int64_t)prow * (ex.I / 16) * 8);
    const uint64_t* hsrow = reinterpret_cast<const uint64_t*>(a.hqs + (int64_t)prow * (ex.I / 16));
    u32x4 hd[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint64_t lo = __hip_atomic_load(hqrow + (size_t)sub * 8 + j * 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const uint64_t hi = __hip_atomic_load(hqrow + (size_t)sub * 8 + j * 2 + 1, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT);
      hd[j] = u32x4{(uint32_t)lo, (uint32_t)(lo >> 32), (uint32_t)hi, (uint32_t)(hi >> 32)};
    }
    const uint64_t sp = __hip_atomic_load(hsrow + sub, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const float hs[2] = {__uint_as_float((uint32_t)sp), __uint_as_float((uint32_t)(sp >> 32))};
#pragma unroll
    for (int u = 0; u < kSNUD; ++u) {
      const float t = q_chunk(wv[u], hd, hs, sv[u], 0.f);
      if (u < nu) part[((sl + 2 * u) * kWaves + wave) * 64 + lane] = wz * t;
    }
  } else {
    for (int u = 0; u < nu; ++u) part[((sl + 2 * u) * kWaves + wave) * 64 + lane] = 0.f;
  }
  lds_barrier();
  for (int i = wave; i < nr; i += kWaves) {
    const int w0 = 2 * (i & 1);  // the two waves of row i's slice
    float v = part[(i * kWaves + w0) * 64 + lane] + part[(i * kWaves + w0 + 1) * 64 + lane];
    v = group_sum<64>(v);
    if (lane == 0) a.y[rb0 + i] = v;
  }
}

#ifndef QM_T1S
#define QM_T1S 1
#endif

// int4 experts, one token, at most 8 routed slots, inter 512, hidden 2048 or
// 4096, at most 2 kSNUD down rows per workgroup
inline bool s_layer_ok(const MoeDecodeArgs& a) {
  if (!QM_T1S || a.T != 1 || a.topk > 8 || !a.hq || !a.flags) return false;
  if (a.ex.I != 512 || (a.ex.H != 2048 && a.ex.H != 4096)) return false;
  if (((uintptr_t)a.x & 15) != 0) return false;
  const int blocks = a.topk * (a.ex.I / kSTile);
  return (a.ex.H + blocks - 1) / blocks <= 2 * kSNUD;
}

template <int XT, int CB, bool GROUPED, bool PS>
inline hipError_t launch_s_layer(const MoeDecodeArgs& a, hipStream_t st) {
  constexpr int D = kSTile / kWaves;
  const auto kern = moe_ffn_t1s_kernel<XT, CB, GROUPED, PS>;
  const int blocks = a.topk * (a.ex.I / kSTile);
  const int R = (a.ex.H + blocks - 1) / blocks;
  size_t lds = align_lds((size_t)a.ex.H * 2 + (size_t)a.ex.H / 4) + (size_t)kWaves * D * q_gu_slot<CB, PS>();
  const size_t part = (size_t)R * kWaves * 64 * 4;
  if (part > lds) lds = part;
  if (lds > (size_t)kLdsMax) return hipErrorNotSupported;
  // every workgroup must be resident at once (the down rows wait on all tiles)
  static int cached_dev = -1, cached_fit = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return hipErrorNotSupported;
  if (dev != cached_dev) {
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(kern), kThreads, lds) !=
            hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return hipErrorNotSupported;
    cached_fit = per_cu * cus;
    cached_dev = dev;
  }
  if (blocks > cached_fit) return hipErrorNotSupported;
  hipLaunchKernelGGL(kern, dim3(blocks), dim3(kThreads), lds, st, a);
  return hipGetLastError();
}

// hipErrorNotSupported: not taken (the caller runs the two stages)
template <int XT, bool GROUPED>
inline hipError_t try_s_layer(const MoeDecodeArgs& a, hipStream_t st) {
  if (!s_layer_ok(a)) return hipErrorNotSupported;
  const bool ps = GROUPED && gu_packed_scales(a, 1);
  if (a.ex.H == 2048)
    return ps ? launch_s_layer<XT, 1, GROUPED, GROUPED>(a, st) : launch_s_layer<XT, 1, GROUPED, false>(a, st);
  return ps ? launch_s_layer<XT, 2, GROUPED, GROUPED>(a, st) : launch_s_layer<XT, 2, GROUPED, false>(a, st);
}

}  // namespace qm
