// moe_decode.hip -- the routed expert FFN for a few tokens (decode): the
// K-expert group of the colibri page "Vulkan backend: expert tier + dense +
// MLA attention on any Vulkan 1.2 GPU" (the qmatmul_gate_up.comp note: fused
// silu(gate x) * (up x) reading x once; the K-expert group note: gate+up for
// the routed experts, one barrier, then the down projections, the hidden
// vectors staying on the device) with the weighted accumulation of expert
// outputs of the page "qwen36: Vulkan expert tier, and staged device-local
// uploads".  Arithmetic on the activation digit planes of planes.hpp.
//
// Two launches on one stream:
//  1. gate+up (moe_gu_kernel): the routed experts of the call are made
//     unique (first-appearance order); a unit is (unique expert, 16 rows of
//     the intermediate dimension) and reads those gate and up rows once for
//     every (token, slot) pair routed to the expert.  Persistent workgroups
//     (about one per CU) stage the tokens' x as digit planes in LDS once and
//     walk the units; each wave takes two rows of a unit (a gate and an up
//     row each), the next unit's weights loading into a second register
//     buffer while the current one is computed.  The unit's 16 values of
//     h = silu(a) * b per pair are turned into h's own digit planes (one
//     exponent per 16 values, as many planes as those values need) and
//     written to the workspace.
//  2. down + combine (moe_down_kernel): each workgroup owns a block of output
//     rows; its waves take the routed pairs (pairs of one expert on adjacent
//     waves, so a shared expert's rows are fetched from HBM once and then hit
//     the cache), keep the pair's h digits in registers and stream the pair's
//     down rows; per-(row, pair) results meet in LDS and every output is
//     y_t = sum_j w_tj o_tj in slot order, so y does not depend on timing.
// Activations needing more than two planes (very wide value ranges) are
// consumed two planes per pass; weights are then read once per pass.
#include "launch.hpp"
#include "planes.hpp"

namespace qm {

namespace {

constexpr int kMW = 8;          // waves per workgroup (down)
constexpr int kMT = 64 * kMW;   // threads per workgroup (down)
constexpr int kGR = 1;          // intermediate rows per wave and gate+up unit
constexpr int kGW = 16 / kGR;   // waves per workgroup (gate+up)
constexpr int kGT = 64 * kGW;
constexpr int kHT = 16;         // rows of the intermediate dimension per gate+up unit (one h group)
constexpr int kMaxPairs = 128;  // (token, slot) pairs per pass (passes are sized to fit)

__device__ __forceinline__ int wuni(int v) { return __builtin_amdgcn_readfirstlane(v); }

template <int FMT> constexpr int per_chunk() { return FMT == kFmtInt4 ? 32 : 16; }
template <int FMT> constexpr int x_words() { return FMT == kFmtInt4 ? 16 : 8; }  // digit words per chunk and plane

// ---- routing table ---------------------------------------------------------------
// The valid pairs of the call grouped by expert: experts in order of first
// appearance, each expert's pairs in pair order.  Built by the whole
// workgroup in LDS.
struct Route {
  int np, nu;                   // pairs, unique experts
  int uexp[kMaxPairs];          // expert id of unique u
  int ustart[kMaxPairs + 1];    // pairs of u: upair[ustart[u] .. ustart[u+1])
  int upair[kMaxPairs];
  int tmp_id[kMaxPairs];        // expert id of every pair (as given)
  float wgt[kMaxPairs];         // routing weight of every pair (down only)
  int tmp_first[kMaxPairs];
  int tmp_rank[kMaxPairs];
  int tmp_u[kMaxPairs];
  int cnt[kMaxPairs];
};

__device__ void build_route(const int32_t* __restrict__ ids, int np, int E, Route& R,
                            const float* __restrict__ w = nullptr) {
  const int tid = threadIdx.x;
  if (tid < np) {
    R.tmp_id[tid] = ids[tid];
    if (w) R.wgt[tid] = w[tid];
  }
  if (tid < kMaxPairs) R.cnt[tid] = 0;
  __syncthreads();
  if (tid < np) {
    const int id = R.tmp_id[tid];
    int first = -1, rank = 0;
    if (id >= 0 && id < E) {
      first = tid;
      for (int q = 0; q < tid; ++q)
        if (R.tmp_id[q] == id) {
          if (first == tid) first = q;
          ++rank;
        }
    }
    R.tmp_first[tid] = first;
    R.tmp_rank[tid] = rank;
  }
  __syncthreads();
  if (tid < 64) {  // unique index of each first occurrence, in pair order
    int base = 0;
    for (int p0 = 0; p0 < np; p0 += 64) {
      const int p = p0 + tid;
      const bool f = p < np && R.tmp_first[p] == p;
      const unsigned long long m = __ballot(f);
      if (f) {
        const int u = base + __popcll(m & ((1ull << tid) - 1));
        R.tmp_u[p] = u;
        R.uexp[u] = R.tmp_id[p];
      }
      base += __popcll(m);
    }
    if (tid == 0) R.nu = base;
    if (tid == 0) R.np = np;
  }
  __syncthreads();
  if (tid < np && R.tmp_first[tid] >= 0) atomicAdd(&R.cnt[R.tmp_u[R.tmp_first[tid]]], 1);
  __syncthreads();
  if (tid == 0) {
    int s = 0;
    for (int u = 0; u < R.nu; ++u) {
      R.ustart[u] = s;
      s += R.cnt[u];
    }
    R.ustart[R.nu] = s;
  }
  __syncthreads();
  if (tid < np && R.tmp_first[tid] >= 0) {
    const int u = R.tmp_u[R.tmp_first[tid]];
    R.upair[R.ustart[u] + R.tmp_rank[tid]] = tid;
  }
  __syncthreads();
}

// Reductions over aligned groups of G (4, 8 or 16) lanes with DPP row
// operations; every lane of a group ends with the result.
template <int G>
__device__ __forceinline__ uint32_t group_or(uint32_t v) {
  v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);   // lane ^ 1
  v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false);   // lane ^ 2
  if constexpr (G >= 8) v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false);  // other quad
  return v;
}
template <int G, bool MAX>
__device__ __forceinline__ float group_minmax(float v) {
  auto step = [&](float a, float b) { return MAX ? fmaxf(a, b) : fminf(a, b); };
  v = step(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false)));
  v = step(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false)));
  if constexpr (G >= 8) v = step(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false)));
  if constexpr (G >= 16) v = step(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false)));
  return v;
}

// Digit planes of 16 fp32 values held one per lane by lanes 0..15 of a wave
// (lanes 16..63 pass anything, write nothing): factor 2^(E-14), plane count
// and the planes' words, to hq[kPlaneMax][8].  Same encoding as planes.hpp
// (fp32 rule for the plane count).  Called by a whole wave.
template <int FMT>
__device__ __forceinline__ void wave_h_planes(float v, uint32_t* __restrict__ hq, float* __restrict__ hf,
                                              int* __restrict__ hp) {
  const int lane = threadIdx.x & 63;
  const bool act = lane < 16;
  const float av = act ? fabsf(v) : 0.f;
  const float amax = group_minmax<16, true>(av);
  const float amin = group_minmax<16, false>(act && av > 0.f ? av : __builtin_huge_valf());
  int E = 0, P = 1;
  if (amax > 0.f) {
    E = fexp(amax);
    const int span = E - (fexp(amin) - 1);
    P = span <= 0 ? 1 : min(kPlaneMax, 1 + (span + 14) / 15);
  }
  float r = act ? ldexpf(v, 14 - E) : 0.f;
  for (int p = 0; p < P; ++p) {
    const float X = __builtin_rintf(r);
    r = (r - X) * 32768.f;
    const int xi = (int)X;
    uint32_t word[4];
    if constexpr (FMT == kFmtInt4) {
      // word (j, d) collects digit d of elements 8j .. 8j+7 as nibbles
      const uint32_t U = (uint32_t)(xi + 0x8888);
#pragma unroll
      for (int d = 0; d < 4; ++d) word[d] = group_or<8>(((U >> (4 * d)) & 15u) << (4 * (lane & 7)));
      if (act && (lane & 7) == 0) {
        const int j = lane >> 3;
        uint32_t* dst = hq + p * 8 + 4 * j;
#pragma unroll
        for (int d = 0; d < 4; ++d) dst[d] = word[d] ^ 0x88888888u;
      }
    } else {
      // word (k, 0) = low bytes, (k, 1) = high bytes of elements 4k .. 4k+3
      const int lo = (int)(int8_t)(uint8_t)(xi & 0xFF);
      const int hi = (xi - lo) >> 8;
      word[0] = group_or<4>(((uint32_t)lo & 0xFFu) << (8 * (lane & 3)));
      word[1] = group_or<4>(((uint32_t)hi & 0xFFu) << (8 * (lane & 3)));
      if (act && (lane & 3) == 0) {
        const int k = lane >> 2;
        hq[p * 8 + 2 * k] = word[0];
        hq[p * 8 + 2 * k + 1] = word[1];
      }
    }
  }
  if (lane == 0) {
    *hf = ldexpf(1.f, E - 14);
    *hp = P;
  }
}

// ---- gate + up ---------------------------------------------------------------------
// One 16-byte chunk of a gate or up row per lane and chunk position; wave w
// of a unit takes intermediate rows 16 * tile + kGR w + (0 .. kGR-1): their
// gate and up rows.
template <int FMT, int XT, bool GROUPED, int CPL>
__global__ __launch_bounds__(kGT) void moe_gu_kernel(MoeDecArgs a) {
  constexpr int PER = per_chunk<FMT>();
  constexpr int W = x_words<FMT>();
  extern __shared__ __attribute__((aligned(16))) char lds[];
  __shared__ Route R;
  // h of the units in progress: kSlots units at a time, each slot counting
  // the waves that have written their row (the last one turns the unit's h
  // into digit planes) and the epilogues it has completed
  constexpr int kSlots = 2;
  __shared__ float h_tile[kSlots][kMaxPairs][kHT];
  __shared__ int s_arrive[kSlots], s_done[kSlots];
  __shared__ int s_pmax;
  const ExpertArgs& ex = a.ex;
  const int H = ex.H, I = ex.I, T = a.T;
  const int KCH = H / PER;  // chunks per gate/up row
  const int wave = wuni(threadIdx.x >> 6), lane = threadIdx.x & 63;
  uint32_t* xd = reinterpret_cast<uint32_t*>(lds);                          // [2][T][KCH][W]
  float* xf = reinterpret_cast<float*>(lds + (size_t)2 * T * KCH * W * 4);  // [T][KCH]

  build_route(a.ids, T * a.topk, ex.E, R);
  const int nu = R.nu;
  const int ntile = (I + kHT - 1) / kHT;
  const int nunits = nu * ntile;

  // x: group exponents and the plane count (largest over all tokens' groups)
  if (threadIdx.x == 0) s_pmax = 0;
  if (threadIdx.x < kSlots) {
    s_arrive[threadIdx.x] = 0;
    s_done[threadIdx.x] = 0;
  }
  int pneed = 1;
  for (int it = threadIdx.x; it < T * KCH; it += kGT) {
    const int t = it / KCH, c = it - t * KCH;
    float v[PER];
    load_acts<XT, PER>(a.x, (int64_t)t * H + (int64_t)c * PER, v);
    int E;
    pneed = max(pneed, group_planes<PER, XT>(v, &E));
  }
  __syncthreads();
  const int P = block_max_int(pneed, &s_pmax);

  constexpr int NQ = 2 * kGR;  // weight rows per wave and unit: (gate, up) of each of its rows
  u32x4 wa[NQ][CPL];
  float sa[NQ][CPL];
  auto load_unit = [&](u32x4 (&wv)[NQ][CPL], float (&sv)[NQ][CPL], int unit) {
    const int u = unit / ntile, tile = unit - u * ntile;
    const int64_t e = R.uexp[u];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int r = min(tile * kHT + kGR * wave + (q >> 1), I - 1);
      const int64_t er = e * I + r;
      const uint8_t* qrow = ((q & 1) ? ex.uq : ex.gq) + er * ex.rb_h;
      const float* srow = ((q & 1) ? ex.us : ex.gs) + er * ex.G_h;
      if constexpr (!GROUPED) sv[q][0] = ld_stream(srow);  // the row's one scale
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        const int c = lane + 64 * i;
        if (c < KCH) {
          wv[q][i] = ld_stream(qrow + (int64_t)c * 16);
          if constexpr (GROUPED) sv[q][i] = ld_stream(srow + (c >> ex.gshift));
        }
      }
    }
  };

  // one unit against planes [p0, p0 + np) of x: a and b of the wave's row for
  // every pair of the unit; last pass: h into h_tile (and a.h), else the
  // partial sums to a.ab
  auto compute_unit = [&](const u32x4 (&wv)[NQ][CPL], const float (&sv)[NQ][CPL], int unit, int p0, int np,
                          bool last, int slot) {
    const int u = unit / ntile, tile = unit - u * ntile;
    const int pb = R.ustart[u], pe = R.ustart[u + 1];
    for (int pi = pb; pi < pe; ++pi) {
      const int pair = R.upair[pi];
      const int t = pair / a.topk;
      float acc[NQ];
#pragma unroll
      for (int q = 0; q < NQ; ++q) acc[q] = 0.f;
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        const int c = lane + 64 * i;
        if (c >= KCH) continue;
        float ta[NQ];
#pragma unroll
        for (int q = 0; q < NQ; ++q) ta[q] = 0.f;
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
          if (pp >= np) break;
          const float ps = pp ? 1.f / 32768.f : 1.f;
          const u32x4* src = reinterpret_cast<const u32x4*>(xd + ((size_t)(pp * T + t) * KCH + c) * W);
          uint32_t xw[W];
#pragma unroll
          for (int k4 = 0; k4 < W / 4; ++k4) {
            const u32x4 v4 = src[k4];
            xw[4 * k4] = v4[0];
            xw[4 * k4 + 1] = v4[1];
            xw[4 * k4 + 2] = v4[2];
            xw[4 * k4 + 3] = v4[3];
          }
#pragma unroll
          for (int q = 0; q < NQ; ++q) {
            const int S = FMT == kFmtInt4 ? gdot_i4(wv[q][i] ^ 0x88888888u, xw) : gdot_i8(wv[q][i], xw);
            ta[q] = __builtin_fmaf((float)S, ps, ta[q]);
          }
        }
        const float f = xf[t * KCH + c];
#pragma unroll
        for (int q = 0; q < NQ; ++q) acc[q] = __builtin_fmaf(ta[q], GROUPED ? f * sv[q][i] : f, acc[q]);
      }
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        acc[q] = group_sum<64>(acc[q]);
        if (!GROUPED) acc[q] *= sv[q][0];  // the row's one scale
      }
      if (lane < kGR) {  // lane hr finishes the wave's row hr
        const int hr = lane;
        const int r = tile * kHT + kGR * wave + hr;
        float av = acc[0], bv = acc[1];
#pragma unroll
        for (int q = 1; q < kGR; ++q)
          if (hr == q) {
            av = acc[2 * q];
            bv = acc[2 * q + 1];
          }
        if (r < I) {
          float* abp = a.ab + ((int64_t)pair * I + r) * 2;
          if (p0 > 0) {
            av += abp[0];
            bv += abp[1];
          }
          if (last) {
            const float hv = silu(av) * bv;
            h_tile[slot][pi - pb][kGR * wave + hr] = hv;
            if (a.h) a.h[(int64_t)pair * I + r] = hv;
          } else {
            abp[0] = av;
            abp[1] = bv;
          }
        }
      }
    }
  };

  for (int p0 = 0; p0 < P; p0 += 2) {
    const int np = min(2, P - p0);
    const bool last = p0 + 2 >= P;
    int unit = blockIdx.x;
    if (unit < nunits) load_unit(wa, sa, unit);  // first unit in flight during the staging
    if (p0 > 0) __syncthreads();
    // planes [p0, p0 + np) of every token's x
    for (int it = threadIdx.x; it < T * KCH; it += kGT) {
      const int t = it / KCH, c = it - t * KCH;
      int E;
      {
        float v[PER];
        load_acts<XT, PER>(a.x, (int64_t)t * H + (int64_t)c * PER, v);
        group_planes<PER, XT>(v, &E);
      }
      stage_group<FMT, XT>(a.x, (int64_t)t * H + (int64_t)c * PER, E, p0, np, xd + ((size_t)t * KCH + c) * W,
                           (size_t)T * KCH * W);
      xf[t * KCH + c] = ldexpf(1.f, E - 14 - 15 * p0);
    }
    __syncthreads();
    // the next unit's weights are requested as soon as the current unit's
    // registers are consumed; no workgroup barrier per unit: the last wave to
    // write its row of a unit builds the unit's h digit planes, the others go
    // on to their next unit
    for (int j = 0; unit < nunits; unit += gridDim.x, ++j) {
      const int cur = unit;
      const int slot = j % kSlots;
      const bool epi = last && a.hq;
      if (epi && j >= kSlots) {
        // the slot's previous unit must have had its epilogue
        while (__hip_atomic_load(&s_done[slot], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) < j / kSlots)
          __builtin_amdgcn_s_sleep(1);
      }
      compute_unit(wa, sa, cur, p0, np, last, slot);
      if (cur + (int)gridDim.x < nunits) load_unit(wa, sa, cur + gridDim.x);
      if (!epi) continue;  // h only (stage call) or a partial pass: no digit planes
      int old = 0;
      if (lane == 0) old = __hip_atomic_fetch_add(&s_arrive[slot], 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_WORKGROUP);
      old = __shfl(old, 0, 64);
      if (old != kGW - 1) continue;
      // this wave wrote the unit's last row: digit planes of every pair's h
      const int uu = cur / ntile, tile = cur - uu * ntile;
      const int pb = R.ustart[uu], pe = R.ustart[uu + 1];
      for (int pi = pb; pi < pe; ++pi) {
        const int pair = R.upair[pi];
        const int r = tile * kHT + lane;
        const float hv = (lane < kHT && r < I) ? h_tile[slot][pi - pb][lane] : 0.f;
        const int64_t g = (int64_t)pair * ((I + 15) / 16) + tile;
        wave_h_planes<FMT>(hv, a.hq + g * (kPlaneMax * 8), a.hf + g, a.hp + g);
      }
      if (lane == 0) {
        __hip_atomic_store(&s_arrive[slot], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        __hip_atomic_fetch_add(&s_done[slot], 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
      }
    }
  }
}

// ---- down + weighted combine -----------------------------------------------------
// L lanes per down row (RW = 64 / L rows per wave pass); a lane holds CPL
// chunk positions c = sub + L i of its pair's h digits (two planes).  A wave
// issues the loads of NB row passes (all of the workgroup's rows at the
// shapes it is sized for) before it reads the pair's h digits, so the whole
// row block is in flight at once.
template <int FMT, bool GROUPED, int L, int CPL, int NB>
__global__ __launch_bounds__(kMT) void moe_down_kernel(MoeDecArgs a) {
  constexpr int RW = 64 / L;
  constexpr int GPC = FMT == kFmtInt4 ? 2 : 1;  // h groups of 16 per chunk
  extern __shared__ __attribute__((aligned(16))) char lds[];
  __shared__ Route R;
  const ExpertArgs& ex = a.ex;
  const int H = ex.H, I = ex.I;
  const int np = a.T * a.topk;
  const int KCH = I / per_chunk<FMT>();  // chunks per down row
  const int NG = (I + 15) / 16;          // h groups per pair
  const int wave = wuni(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int sub = lane % L, rs = lane / L;
  const int Rb = (H + gridDim.x - 1) / gridDim.x;
  const int r0 = blockIdx.x * Rb, nr = min(Rb, H - r0);
  const int npass = (nr + RW - 1) / RW;
  float* part = reinterpret_cast<float*>(lds);  // [Rb][np]
  build_route(a.ids, np, ex.E, R, a.w);
  const int nvalid = R.ustart[R.nu];

  u32x4 wv[NB][CPL];
  float sv[NB][CPL];
  // the pair's expert's rows [r0, r0 + nr) as two buffer regions (weights,
  // scales); byte offsets in vector registers
  auto issue = [&](int e, int b0) {
    const int64_t er0 = (int64_t)e * H + r0;
    const __amdgpu_buffer_rsrc_t rq = region_rsrc(ex.dq + er0 * ex.rb_i, (uint32_t)(nr * ex.rb_i));
    const __amdgpu_buffer_rsrc_t rsc = region_rsrc(ex.ds + er0 * ex.G_i, (uint32_t)(nr * ex.G_i * 4));
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int rl = min((b0 + j) * RW + rs, nr - 1);
      const uint32_t qo = (uint32_t)(rl * ex.rb_i), so = (uint32_t)(rl * ex.G_i * 4);
      if constexpr (!GROUPED) sv[j][0] = ld_region4(rsc, so);  // the row's one scale
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        const int c = sub + L * i;
        if (b0 + j < npass && c < KCH) {
          wv[j][i] = ld_region16(rq, qo + (uint32_t)c * 16);
          if constexpr (GROUPED) sv[j][i] = ld_region4(rsc, so + (uint32_t)(c >> ex.gshift) * 4);
        }
      }
    }
  };

  for (int li = wave; li < nvalid; li += kMW) {
    const int pair = R.upair[li];
    const int e = R.tmp_id[pair];
    issue(e, 0);
    // the pair's plane count over the groups this wave touches
    int pw = 1;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int c = sub + L * i;
      if (c < KCH)
#pragma unroll
        for (int gg = 0; gg < GPC; ++gg) pw = max(pw, a.hp[(int64_t)pair * NG + c * GPC + gg]);
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) pw = max(pw, __shfl_xor(pw, o, 64));
    pw = wuni(pw);
    for (int p0 = 0; p0 < pw; p0 += 2) {
      // h digits of planes p0, p0 + 1 (zero past a group's own plane count)
      uint32_t hd[2][CPL][GPC * 8];
      float hfac[CPL][GPC];
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        const int c = sub + L * i;
#pragma unroll
        for (int gg = 0; gg < GPC; ++gg) {
          const int64_t g = (int64_t)pair * NG + (c < KCH ? c * GPC + gg : 0);
          const int pg = c < KCH ? a.hp[g] : 0;
          hfac[i][gg] = c < KCH ? a.hf[g] * ldexpf(1.f, -15 * p0) : 0.f;
#pragma unroll
          for (int pp = 0; pp < 2; ++pp) {
            // read whether or not the group has this plane (its slot exists),
            // then zero it: the loads do not wait for the plane count
            const bool on = p0 + pp < pg;
            const u32x4* src = reinterpret_cast<const u32x4*>(a.hq + g * (kPlaneMax * 8) + min(p0 + pp, kPlaneMax - 1) * 8);
            const u32x4 r0 = src[0], r1 = src[1];
            const u32x4 q0 = on ? r0 : u32x4{0u, 0u, 0u, 0u};
            const u32x4 q1 = on ? r1 : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              hd[pp][i][gg * 8 + k] = q0[k];
              hd[pp][i][gg * 8 + 4 + k] = q1[k];
            }
          }
        }
      }
      const int npl = min(2, pw - p0);
      for (int b0 = 0; b0 < npass; b0 += NB) {
        if (b0 > 0 || p0 > 0) issue(e, b0);
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          if (b0 + j >= npass) break;
          float acc = 0.f;
#pragma unroll
          for (int i = 0; i < CPL; ++i) {
            const int c = sub + L * i;
            if (c >= KCH) continue;
            u32x4 w = wv[j][i];
            float ta[GPC];
#pragma unroll
            for (int gg = 0; gg < GPC; ++gg) ta[gg] = 0.f;
            if constexpr (FMT == kFmtInt4) {
              w ^= 0x88888888u;
#pragma unroll
              for (int pp = 0; pp < 2; ++pp) {
                if (pp >= npl) break;
                const float ps = pp ? 1.f / 32768.f : 1.f;
                ta[0] = __builtin_fmaf((float)gdot16_i4(w[0], w[1], hd[pp][i]), ps, ta[0]);
                ta[GPC - 1] = __builtin_fmaf((float)gdot16_i4(w[2], w[3], hd[pp][i] + 8), ps, ta[GPC - 1]);
              }
            } else {
#pragma unroll
              for (int pp = 0; pp < 2; ++pp) {
                if (pp >= npl) break;
                const float ps = pp ? 1.f / 32768.f : 1.f;
                ta[0] = __builtin_fmaf((float)gdot_i8(w, hd[pp][i]), ps, ta[0]);
              }
            }
            float part_c = ta[0] * hfac[i][0];
            if constexpr (GPC == 2) part_c = __builtin_fmaf(ta[1], hfac[i][1], part_c);
            acc = __builtin_fmaf(part_c, GROUPED ? sv[j][i] : 1.f, acc);
          }
          acc = group_sum<L>(acc);
          const int rl = (b0 + j) * RW + rs;
          if (sub == 0 && rl < nr) {
            const float v = GROUPED ? acc : acc * sv[j][0];
            float* dst = part + (size_t)rl * np + pair;
            *dst = p0 == 0 ? v : *dst + v;
          }
        }
      }
    }
  }
  __syncthreads();
  // y_t[r] = sum over valid slots j, in order, of w_tj * part[r][t k + j]
  for (int it = threadIdx.x; it < nr * a.T; it += kMT) {
    const int rl = it % nr, t = it / nr;
    float v = 0.f;
    for (int j = 0; j < a.topk; ++j) {
      const int pair = t * a.topk + j;
      if (R.tmp_first[pair] >= 0) v = __builtin_fmaf(R.wgt[pair], part[(size_t)rl * np + pair], v);
    }
    a.y[(int64_t)t * H + r0 + rl] = v;
  }
}

// caller-supplied fp32 h [T*k][I] -> digit planes, one wave per (pair, group)
template <int FMT>
__global__ __launch_bounds__(256) void h_planes_kernel(MoeDecArgs a, int ngroups_total) {
  const int g = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (g >= ngroups_total) return;
  const int NG = (a.ex.I + 15) / 16;
  const int pair = g / NG, gi = g - pair * NG;
  const int lane = threadIdx.x & 63;
  const int r = gi * 16 + lane;
  const float v = (lane < 16 && r < a.ex.I) ? a.h[(int64_t)pair * a.ex.I + r] : 0.f;
  wave_h_planes<FMT>(v, a.hq + (int64_t)g * (kPlaneMax * 8), a.hf + g, a.hp + g);
}

// ---- launchers ------------------------------------------------------------------------

template <int FMT, int XT, bool GROUPED>
hipError_t launch_gu(const MoeDecArgs& a, int cus, hipStream_t st) {
  constexpr int PER = per_chunk<FMT>();
  const int KCH = a.ex.H / PER;
  const size_t lds = (size_t)2 * a.T * KCH * x_words<FMT>() * 4 + (size_t)a.T * KCH * 4;
  if (lds > kDecLdsMax) return hipErrorNotSupported;
  const int nunits_max = a.T * a.topk * ((a.ex.I + kHT - 1) / kHT);
  const int blocks = max(1, min(cus, nunits_max));
  const int cpl = (KCH + 63) / 64;
#define QM_GU(C)                                                                                         \
  hipLaunchKernelGGL((moe_gu_kernel<FMT, XT, GROUPED, C>), dim3(blocks), dim3(kGT), lds, st, a); \
  return hipGetLastError();
  switch (cpl) {
    case 1: { QM_GU(1) }
    case 2: { QM_GU(2) }
    case 3: { QM_GU(3) }
    case 4: { QM_GU(4) }
    default: break;
  }
  if (cpl <= 6) { QM_GU(6) }
  if (cpl <= 8) { QM_GU(8) }
#undef QM_GU
  return hipErrorNotSupported;
}

template <int FMT, bool GROUPED>
hipError_t launch_down(const MoeDecArgs& a, int cus, hipStream_t st) {
  const int KCH = a.ex.I / per_chunk<FMT>();
  const int Rb = (a.ex.H + cus - 1) / cus;      // rows per workgroup
  const int blocks = (a.ex.H + Rb - 1) / Rb;    // every workgroup has rows
  const size_t lds = (size_t)Rb * a.T * a.topk * 4;
  if (lds > kDecLdsMax) return hipErrorNotSupported;
#define QM_DN(L_, C, NB_)                                                                                    \
  hipLaunchKernelGGL((moe_down_kernel<FMT, GROUPED, L_, C, NB_>), dim3(blocks), dim3(kMT), lds, st, a); \
  return hipGetLastError();
  // NB row passes in flight per wave: the whole row block when it fits
  const int npass16 = (Rb + 3) / 4, npass32 = (Rb + 1) / 2;
  if (KCH <= 16) {
    if (npass16 <= 8) { QM_DN(16, 1, 8) }
    QM_DN(16, 1, 16)
  }
  if (KCH <= 32) {
    if (npass32 <= 12) { QM_DN(32, 1, 12) }
    QM_DN(32, 1, 16)
  }
  if (KCH <= 64) {
    if (Rb <= 12) { QM_DN(64, 1, 12) }
    QM_DN(64, 1, 24)
  }
  if (KCH <= 128) { QM_DN(64, 2, 8) }
#undef QM_DN
  return hipErrorNotSupported;
}

}  // namespace

size_t moe_decode_ws_bytes(int T, int topk, int H, int I) {
  const size_t P = (size_t)T * topk;
  const size_t NG = (size_t)(I + 15) / 16;
  auto al = [](size_t v) { return (v + 255) / 256 * 256; };
  return al(P * NG * kPlaneMax * 32) + al(P * NG * 4) + al(P * NG * 4) + al(P * (size_t)I * 8);
}

void moe_decode_ws_split(MoeDecArgs& a, void* ws) {
  const size_t P = (size_t)a.T * a.topk;
  const size_t NG = (size_t)(a.ex.I + 15) / 16;
  auto al = [](size_t v) { return (v + 255) / 256 * 256; };
  char* p = static_cast<char*>(ws);
  a.hq = reinterpret_cast<uint32_t*>(p);
  p += al(P * NG * kPlaneMax * 32);
  a.hf = reinterpret_cast<float*>(p);
  p += al(P * NG * 4);
  a.hp = reinterpret_cast<int*>(p);
  p += al(P * NG * 4);
  a.ab = reinterpret_cast<float*>(p);
}

bool moe_decode_supported(int fmt, int T, int topk, const ExpertArgs& e) {
  if (T < 1 || T * topk > kMaxPairs) return false;
  const int per = fmt == kFmtInt4 ? 32 : 16;
  const int kh = e.H / per, ki = e.I / per;
  if ((kh + 63) / 64 > 8 || ki > 128) return false;
  if ((size_t)2 * T * kh * (fmt == kFmtInt4 ? 16 : 8) * 4 + (size_t)T * kh * 4 > (size_t)kDecLdsMax) return false;
  return true;
}

// largest token count per pass whose x digit planes fit the LDS budget
int moe_decode_tokens_per_pass(int fmt, int topk, const ExpertArgs& e) {
  const int per = fmt == kFmtInt4 ? 32 : 16;
  const int kh = e.H / per;
  const size_t per_tok = (size_t)2 * kh * (fmt == kFmtInt4 ? 16 : 8) * 4 + (size_t)kh * 4;
  int t = (int)(kDecLdsMax / per_tok);
  t = min(t, kDecMaxTokens);
  t = min(t, kMaxPairs / topk);
  return max(t, 0);
}

hipError_t launch_moe_gate_up2(int fmt, int xdt, bool grouped, const MoeDecArgs& a, hipStream_t st) {
  int cus = 0;
  const hipError_t e = device_cus(&cus);
  if (e != hipSuccess) return e;
  if (fmt == kFmtInt4) {
    if (xdt == kBF16) return grouped ? launch_gu<kFmtInt4, kBF16, true>(a, cus, st) : launch_gu<kFmtInt4, kBF16, false>(a, cus, st);
    return grouped ? launch_gu<kFmtInt4, kF32, true>(a, cus, st) : launch_gu<kFmtInt4, kF32, false>(a, cus, st);
  }
  if (grouped) return hipErrorNotSupported;
  return xdt == kBF16 ? launch_gu<kFmtInt8, kBF16, false>(a, cus, st) : launch_gu<kFmtInt8, kF32, false>(a, cus, st);
}

hipError_t launch_moe_down2(int fmt, bool grouped, const MoeDecArgs& a, bool h_from_caller, hipStream_t st) {
  int cus = 0;
  hipError_t e = device_cus(&cus);
  if (e != hipSuccess) return e;
  if (h_from_caller) {
    const int ng = a.T * a.topk * ((a.ex.I + 15) / 16);
    if (fmt == kFmtInt4)
      hipLaunchKernelGGL(h_planes_kernel<kFmtInt4>, dim3((ng + 3) / 4), dim3(256), 0, st, a, ng);
    else
      hipLaunchKernelGGL(h_planes_kernel<kFmtInt8>, dim3((ng + 3) / 4), dim3(256), 0, st, a, ng);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (fmt == kFmtInt4) return grouped ? launch_down<kFmtInt4, true>(a, cus, st) : launch_down<kFmtInt4, false>(a, cus, st);
  if (grouped) return hipErrorNotSupported;
  return launch_down<kFmtInt8, false>(a, cus, st);
}

}  // namespace qm
