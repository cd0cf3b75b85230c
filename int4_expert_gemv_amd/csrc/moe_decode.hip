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
#include <algorithm>

#include "launch.hpp"
#include "planes.hpp"

namespace qm {

namespace {

constexpr int kMW = 8;          // waves per workgroup (down)
constexpr int kMT = 64 * kMW;   // threads per workgroup (down)
constexpr int kGR = 2;          // intermediate rows per wave and gate+up unit
constexpr int kGW = 16 / kGR;   // waves per workgroup (gate+up)
constexpr int kGT = 64 * kGW;
constexpr int kHT = 16;         // rows of the intermediate dimension per gate+up unit (one h group)
constexpr int kMaxPairs = 128;  // (token, slot) pairs per pass (passes are sized to fit)

__device__ __forceinline__ int wuni(int v) { return __builtin_amdgcn_readfirstlane(v); }

// int3-g64 experts run as int4 (planes.hpp: the values become signed
// nibbles when used; a 32-input chunk is 12 bytes of a 24-byte group)
template <int FMT> constexpr int per_chunk() { return FMT == kFmtInt8 ? 16 : 32; }
template <int FMT> constexpr int x_words() { return FMT == kFmtInt8 ? 8 : 16; }  // digit words per chunk and plane

// ---- routing table ---------------------------------------------------------------
// The valid pairs of the call grouped by expert: experts in order of first
// appearance, each expert's pairs in pair order.  Built in LDS (by one wave
// for up to 64 pairs, else by the whole workgroup).
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

// (id, w: this thread's pair's expert id and routing weight, threads < np;
// loaded by the caller, so that other loads can be in flight meanwhile)
__device__ void build_route(int id_t, float w_t, int np, int E, Route& R) {
  const int tid = threadIdx.x;
  if (np <= 64) {
    // up to 64 pairs: wave 0 builds the table in registers (lane j = pair
    // j), one barrier publishes it
    if (tid < 64) {
      const int lane = tid;
      const bool in = lane < np;
      const int id = in ? id_t : -1;
      const bool valid = in && id >= 0 && id < E;
      // first pair with this expert, pairs before this one with it, and all
      // pairs with it
      int first = valid ? lane : -1, rank = 0, total = 0;
      for (int i = 0; i < np; ++i) {
        const int xi = __builtin_amdgcn_readlane(id, i);
        if (valid && xi == id) {
          first = min(first, i);
          rank += i < lane ? 1 : 0;
          ++total;
        }
      }
      const bool is_first = valid && first == lane;
      const unsigned long long fm = __ballot(is_first);
      const int u = __popcll(fm & ((1ull << lane) - 1));  // unique index of a first pair
      // pair offsets of the experts: exclusive prefix of the first pairs' counts
      const int v = is_first ? total : 0;
      int incl = v;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(incl, o, 64);
        if (lane >= o) incl += t;
      }
      const int start = __shfl(incl - v, valid ? first : 0, 64);
      if (in) {
        R.tmp_id[lane] = id_t;
        R.wgt[lane] = w_t;
        R.tmp_first[lane] = valid ? first : -1;
      }
      if (is_first) {
        R.uexp[u] = id;
        R.ustart[u] = incl - v;
      }
      if (valid) R.upair[start + rank] = lane;
      const int nvalid = __shfl(incl, 63, 64);
      if (lane == 0) {
        const int nu = __popcll(fm);
        R.nu = nu;
        R.np = np;
        R.ustart[nu] = nvalid;
      }
    }
    __syncthreads();
    return;
  }
  if (tid < np) {
    R.tmp_id[tid] = id_t;
    R.wgt[tid] = w_t;
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

// Min or max over aligned groups of G (4, 8 or 16) lanes with DPP row
// operations; every lane of a group ends with the result.
template <int G, bool MAX>
__device__ __forceinline__ float group_minmax(float v) {
  auto step = [&](float a, float b) __attribute__((always_inline)) { return MAX ? fmaxf(a, b) : fminf(a, b); };
  v = step(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false)));
  v = step(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false)));
  if constexpr (G >= 8) v = step(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false)));
  if constexpr (G >= 16) v = step(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false)));
  return v;
}

// Sum over aligned groups of L (16, 32 or 64) lanes, complete in the
// group's last lane (L - 1 of the group; other lanes hold partial sums):
// rows of 16 lanes by DPP, then row broadcasts 15 and 31 carry row sums
// into the following rows.
template <int L>
__device__ __forceinline__ float sum_to_last(float v) {
  v = group_sum<16>(v);
  if constexpr (L >= 32)  // row_bcast:15 into rows 1 and 3
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xA, 0xF, false));
  if constexpr (L >= 64)  // row_bcast:31 into rows 2 and 3
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x143, 0xC, 0xF, false));
  return v;
}

// ---- h records ---------------------------------------------------------------------
// h (the intermediate activations) is taken in groups of 16 values (group G:
// elements 16 G .. 16 G + 15) and turned into digit planes (planes.hpp
// encoding, fp32 rule for the plane count P), written as records of two
// planes each ("plane pair" q: planes 2q and 2q + 1), 96 bytes:
//   bytes  0..63  for column c = 2 (plane - 2q) + b, 16 int8 digits: the
//                 plane's value X split as X = lo + 256 hi (lo its signed low
//                 byte; b = 0: lo, 1: hi); digit j is element dn_elem(j),
//                 the order in which the down kernel unpacks weights;
//   bytes 64..79  per column, int32: -8 x (sum of its digits) for int4
//                 weights (the matrix instruction takes the nibbles u as
//                 unsigned bytes, and sum (u - 8) d = sum u d - 8 sum d), 0
//                 for int8 weights;
//   bytes 80..83  the factor 2^(E - 14 - 30 q);
//   bytes 84..87  the group's plane count P (bits 8 and up: free for the
//                 down kernel's own use);
// so that the group's sum_k w_k h_k is, exactly up to fp32 rounding,
// factor x sum_c 2^(-15 p) 256^b (sum_j w_j d_cj + Cin_c) over its records.
// A pair's records: plane pair q, group G at
// hrec + ((pair * kRecPairs + q) * NGP + G) * kRecBytes, NGP = 8 ceil(I / 128)
// (groups past I / 16 are never written and never read).
constexpr int kRecBytes = 96;
constexpr int kRecPairs = kPlaneMax / 2;

__host__ __device__ constexpr int dn_ngp(int I) { return 8 * ((I + 127) / 128); }

// element of digit j of a group's column (the weights' unpacking order: an
// int4 word w gives bytes (w & 0x0F0F0F0F) = nibbles 0, 2, 4, 6 and
// (w >> 4) & 0x0F0F0F0F = nibbles 1, 3, 5, 7; int3 unpacks the words of its
// even and of its odd values (i3_words) the same way)
template <int FMT>
__device__ __forceinline__ int dn_elem(int j) {
  const int v = j >> 2, jj = j & 3;
  if constexpr (FMT == kFmtInt4) {
    return ((v & 2) ? 8 : 0) + 2 * jj + (v & 1);
  } else if constexpr (FMT == kFmtInt3) {
    return 4 * jj + ((v & 1) ? 2 : 0) + ((v & 2) ? 1 : 0);
  } else {
    return j;
  }
}

__device__ __forceinline__ int group_isum16(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false);
  return v;
}

// The records of one group of 16 fp32 values held one per lane by lanes
// 0..15 of a wave (lanes 16..63 pass anything, write nothing); rec: its plane
// pair 0 record, qstride: bytes between its plane pairs' records.  At least
// plane pair 0 is written (with zero digits past P).  Called by a whole wave.
template <int FMT>
__device__ __forceinline__ void wave_h_records(float v, uint8_t* __restrict__ rec, size_t qstride) {
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
  const int nq = (P + 1) / 2;
  const int t = lane & 15, c = t >> 2, vv = t & 3;  // this lane's output word: column c, word vv
  for (int q = 0; q < nq; ++q) {
    uint32_t packed = 0;  // the four column digits of this lane's element
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) {
      const float X = __builtin_rintf(r);
      r = (r - X) * 32768.f;
      const int xi = (int)X;
      const int lo = (int)(int8_t)(uint8_t)(xi & 0xFF);
      const int hi = (xi - lo) >> 8;
      packed |= (((uint32_t)lo & 0xFFu) << (16 * pp)) | (((uint32_t)hi & 0xFFu) << (16 * pp + 8));
    }
    if (!act) packed = 0u;
    int sum[4];
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) sum[cc] = group_isum16((int)(int8_t)(uint8_t)(packed >> (8 * cc)));
    uint32_t word = 0;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const uint32_t src = (uint32_t)__shfl((int)packed, dn_elem<FMT>(4 * vv + jj), 64);
      word |= ((src >> (8 * c)) & 0xFFu) << (8 * jj);
    }
    uint8_t* rq = rec + (size_t)q * qstride;
    if (act) reinterpret_cast<uint32_t*>(rq)[t] = word;
    if (lane == 0) {
      int* ci = reinterpret_cast<int*>(rq + 64);
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) ci[cc] = FMT == kFmtInt8 ? 0 : -8 * sum[cc];
      *reinterpret_cast<float*>(rq + 80) = ldexpf(1.f, E - 14 - 30 * q);
      *reinterpret_cast<int*>(rq + 84) = P;
    }
  }
}

// ---- gate + up ---------------------------------------------------------------------
// Wave w of a unit owns intermediate rows 16 * tile + kGR w + (0 .. kGR-1):
// their gate and up rows (weight row q: row q / 2, gate for even q, up for
// odd).  Lane l holds the 16-byte chunks c = l + 64 i (i < CPL) of each.
// Every row is read through a buffer resource spanning exactly that row, so
// chunks past its end (c >= KCH, or a row past I) load as zero without a
// branch; in LDS those chunk positions hold zero digits and a zero factor.
template <int CPL, bool GROUPED>
struct GuRegs {
  u32x4 w[2 * kGR][CPL];
  float s[2 * kGR][GROUPED ? CPL : 1];
};

template <int FMT, int XT, bool GROUPED, int CPL, int NBUF>
__global__ __launch_bounds__(kGT) void moe_gu_kernel(MoeDecArgs a) {
  constexpr int PER = per_chunk<FMT>();
  constexpr int W = x_words<FMT>();
  constexpr int KCHP = 64 * CPL;  // chunk positions of an x row in LDS
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
  const int NGP = dn_ngp(I);
  const int wave = wuni(threadIdx.x >> 6), lane = threadIdx.x & 63;
  uint32_t* xd = reinterpret_cast<uint32_t*>(lds);                           // [2][T][KCHP][W]
  float* xf = reinterpret_cast<float*>(lds + (size_t)2 * T * KCHP * W * 4);  // [T][KCHP]
  const size_t xps = (size_t)T * KCHP * W;                                   // words per plane

  if (threadIdx.x == 0) s_pmax = 0;
  if (threadIdx.x < kSlots) {
    s_arrive[threadIdx.x] = 0;
    s_done[threadIdx.x] = 0;
  }
  // the routing ids, then this thread's x groups (at most two: the launcher
  // keeps T * KCHP <= twice the block size), requested together ahead of
  // any weights (loads complete in order: staging x then waits for x alone)
  const int id_t = threadIdx.x < T * a.topk ? a.ids[threadIdx.x] : -1;
  constexpr int NV = XT == kBF16 ? PER / 8 : PER / 4;  // 16-byte words of a group
  // (buffer loads: a generic load would make its first use wait for every
  // load issued after it, the weights included)
  u32x4 raw[2][NV];
  {
    const __amdgpu_buffer_rsrc_t rx = region_rsrc(a.x, (uint32_t)((size_t)T * H * (XT == kBF16 ? 2 : 4)));
#pragma unroll
    for (int q2 = 0; q2 < 2; ++q2) {
      const int it = threadIdx.x + q2 * kGT;
      const int t = min(it / KCHP, T - 1), c = it - (it / KCHP) * KCHP;
      const bool real = it < T * KCHP && c < KCH;
      const uint32_t off = (uint32_t)(((int64_t)t * H + (int64_t)(real ? c : 0) * PER) * (XT == kBF16 ? 2 : 4));
#pragma unroll
      for (int q = 0; q < NV; ++q) raw[q2][q] = __builtin_amdgcn_raw_buffer_load_b128(rx, off + 16u * q, 0, 0);
    }
  }
  build_route(id_t, 0.f, T * a.topk, ex.E, R);
  const int nu = R.nu;
  const int ntile = (I + kHT - 1) / kHT;
  const int nunits = nu * ntile;
  const int G = gridDim.x;

  // a unit's weights; a unit past the end (or a row past I) loads zeros
  // without touching memory (empty buffer resources), so that callers issue
  // loads unconditionally (no branch, hence exact wait counts after it)
  auto load = [&](GuRegs<CPL, GROUPED>& g, int unit) __attribute__((always_inline)) {
    const bool uok = unit < nunits;
    const int uc = uok ? unit : 0;
    const int u = uc / ntile, tile = uc - u * ntile;
    const int64_t e = uok ? wuni(R.uexp[u]) : 0;
#pragma unroll
    for (int q = 0; q < 2 * kGR; ++q) {
      const int r = tile * kHT + kGR * wave + (q >> 1);
      const int64_t er = e * I + min(r, I - 1);
      const bool ok = uok && r < I;
      const __amdgpu_buffer_rsrc_t rq =
          region_rsrc(((q & 1) ? ex.uq : ex.gq) + er * ex.rb_h, ok ? (uint32_t)ex.rb_h : 0u);
      const __amdgpu_buffer_rsrc_t rs =
          region_rsrc(((q & 1) ? ex.us : ex.gs) + er * ex.G_h, ok ? (uint32_t)ex.G_h * 4u : 0u);
      if constexpr (!GROUPED) g.s[q][0] = ld_region4(rs, 0);  // the row's one scale
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        const uint32_t c = (uint32_t)(lane + 64 * i);
        if constexpr (FMT == kFmtInt3) {  // low words 2 (c & 1), +1 of group c / 2 and their 32 high bits
          const uint32_t gb = (c >> 1) * 24u;
          const u32x2 lw = __builtin_amdgcn_raw_buffer_load_b64(rq, gb + 8u * (c & 1u), 0, 2);
          const uint32_t hw = __builtin_amdgcn_raw_buffer_load_b32(rq, gb + 16u + 4u * (c & 1u), 0, 2);
          g.w[q][i] = u32x4{lw[0], lw[1], hw, 0u};
        } else {
          g.w[q][i] = ld_region16(rq, c * 16u);
        }
        if constexpr (GROUPED) g.s[q][i] = ld_region4(rs, (c >> ex.gshift) * 4u);
      }
    }
  };

  // planes [p0, p0 + 2) of every token's x into LDS (zero past the row);
  // returns the plane count this thread's groups need
  auto stage = [&](int p0) __attribute__((always_inline)) {
    int pneed = 1;
    for (int it = threadIdx.x; it < T * KCHP; it += kGT) {
      const int t = it / KCHP, c = it - t * KCHP;
      uint32_t* dst = xd + ((size_t)t * KCHP + c) * W;
      if (c < KCH) {
        int E;
        {
          float v[PER];
          load_acts<XT, PER>(a.x, (int64_t)t * H + (int64_t)c * PER, v);
          pneed = max(pneed, group_planes<PER, XT>(v, &E));
        }
        stage_group<FMT, XT>(a.x, (int64_t)t * H + (int64_t)c * PER, E, p0, 2, dst, xps);
        xf[t * KCHP + c] = ldexpf(1.f, E - 14 - 15 * p0);
      } else {
#pragma unroll
        for (int k = 0; k < W; ++k) {
          dst[k] = 0u;
          dst[xps + k] = 0u;
        }
        xf[t * KCHP + c] = 0.f;
      }
    }
    return pneed;
  };

  // one unit against planes [p0, p0 + np) of x: a and b of the wave's row for
  // every pair of the unit; last pass: h into h_tile (and a.h), else the
  // partial sums to a.ab
  auto compute = [&](const GuRegs<CPL, GROUPED>& g, int unit, int p0, int np, bool last, int slot)
                     __attribute__((always_inline)) {
    const int u = unit / ntile, tile = unit - u * ntile;
    const int pb = wuni(R.ustart[u]), pe = wuni(R.ustart[u + 1]);
    for (int pi = pb; pi < pe; ++pi) {
      const int pair = wuni(R.upair[pi]);
      const int t = pair / a.topk;
      float acc[2 * kGR];
#pragma unroll
      for (int q = 0; q < 2 * kGR; ++q) acc[q] = 0.f;
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        const int c = lane + 64 * i;
        float ta[2 * kGR];
#pragma unroll
        for (int q = 0; q < 2 * kGR; ++q) ta[q] = 0.f;
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
          if (pp >= np) break;
          const float ps = pp ? 1.f / 32768.f : 1.f;
          const u32x4* src = reinterpret_cast<const u32x4*>(xd + pp * xps + ((size_t)t * KCHP + c) * W);
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
          for (int q = 0; q < 2 * kGR; ++q) {
            int S;
            if constexpr (FMT == kFmtInt4) {
              S = gdot_i4(g.w[q][i] ^ 0x88888888u, xw);
            } else if constexpr (FMT == kFmtInt3) {
              uint32_t e0, o0, e1, o1;
              i3_words(g.w[q][i][0], g.w[q][i][2] & 0xFFFFu, e0, o0);
              i3_words(g.w[q][i][1], g.w[q][i][2] >> 16, e1, o1);
              S = gdot_i4(u32x4{e0, o0, e1, o1}, xw);
            } else {
              S = gdot_i8(g.w[q][i], xw);
            }
            ta[q] = __builtin_fmaf((float)S, ps, ta[q]);
          }
        }
        const float f = xf[t * KCHP + c];
#pragma unroll
        for (int q = 0; q < 2 * kGR; ++q) acc[q] = __builtin_fmaf(ta[q], GROUPED ? f * g.s[q][i] : f, acc[q]);
      }
#pragma unroll
      for (int q = 0; q < 2 * kGR; ++q) {
        acc[q] = sum_to_last<64>(acc[q]);
        if constexpr (!GROUPED) acc[q] *= g.s[q][0];  // the row's one scale
      }
      if (lane == 63) {  // the lane holding the sums
#pragma unroll
        for (int hr = 0; hr < kGR; ++hr) {
          const int r = tile * kHT + kGR * wave + hr;
          if (r >= I) continue;
          float av = acc[2 * hr], bv = acc[2 * hr + 1];
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

  // after a unit's rows are written: the last wave to arrive turns the
  // unit's h into digit planes (no workgroup barrier per unit)
  auto epilogue = [&](int unit, int slot) __attribute__((always_inline)) {
    int old = 0;
    if (lane == 0) old = __hip_atomic_fetch_add(&s_arrive[slot], 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_WORKGROUP);
    old = __shfl(old, 0, 64);
    if (old != kGW - 1) return;
    const int uu = unit / ntile, tile = unit - uu * ntile;
    const int pb = wuni(R.ustart[uu]), pe = wuni(R.ustart[uu + 1]);
    for (int pi = pb; pi < pe; ++pi) {
      const int pair = wuni(R.upair[pi]);
      const int r = tile * kHT + lane;
      const float hv = (lane < kHT && r < I) ? h_tile[slot][pi - pb][lane] : 0.f;
      wave_h_records<FMT>(hv, a.hrec + (((int64_t)pair * kRecPairs) * NGP + tile) * kRecBytes,
                          (size_t)NGP * kRecBytes);
    }
    if (lane == 0) {
      __hip_atomic_store(&s_arrive[slot], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      __hip_atomic_fetch_add(&s_done[slot], 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
  };

  // all units of this workgroup against planes [p0, p0 + np) of x, weights
  // of its first two units already requested into A and B
  GuRegs<CPL, GROUPED> A, B;
  auto run = [&](int p0, int np, bool last) __attribute__((always_inline)) {
    const bool epi = last && a.hrec;
    int unit = blockIdx.x, j = 0;
    auto step = [&](GuRegs<CPL, GROUPED>& g) __attribute__((always_inline)) {
      const int slot = j % kSlots;
      if (epi && j >= kSlots) {
        // the slot's previous unit must have had its epilogue
        while (__hip_atomic_load(&s_done[slot], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) < j / kSlots)
          __builtin_amdgcn_s_sleep(1);
      }
      compute(g, unit, p0, np, last, slot);
      load(g, unit + NBUF * G);
      if (epi) epilogue(unit, slot);
      unit += G;
      ++j;
    };
    while (unit < nunits) {
      step(A);
      if constexpr (NBUF == 2) {
        if (unit >= nunits) break;
        step(B);
      }
    }
  };
  auto load_first = [&]() __attribute__((always_inline)) {
    load(A, blockIdx.x);
    if constexpr (NBUF == 2) load(B, blockIdx.x + G);
  };

  int P;
  {
    const int unit = blockIdx.x;
    load(A, unit);
    int pneed = 1;
#pragma unroll
    for (int q2 = 0; q2 < 2; ++q2) {
      const int it = threadIdx.x + q2 * kGT;
      if (it >= T * KCHP) break;
      const int t = it / KCHP, c = it - t * KCHP;
      uint32_t* dst = xd + ((size_t)t * KCHP + c) * W;
      if (c < KCH) {
        float xv[PER];
#pragma unroll
        for (int q = 0; q < NV; ++q)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if constexpr (XT == kBF16) {
              xv[8 * q + 2 * i] = __uint_as_float(raw[q2][q][i] << 16);
              xv[8 * q + 2 * i + 1] = __uint_as_float(raw[q2][q][i] & 0xFFFF0000u);
            } else {
              xv[4 * q + i] = __uint_as_float(raw[q2][q][i]);
            }
          }
        int E;
        pneed = max(pneed, group_planes<PER, XT>(xv, &E));
        stage_group_vals<FMT, PER>(xv, E, 0, dst, xps);
        xf[t * KCHP + c] = ldexpf(1.f, E - 14);
      } else {
#pragma unroll
        for (int k = 0; k < W; ++k) {
          dst[k] = 0u;
          dst[xps + k] = 0u;
        }
        xf[t * KCHP + c] = 0.f;
      }
    }
    if constexpr (NBUF == 2) load(B, unit + G);
    P = block_max_int(pneed, &s_pmax);  // (its barrier publishes the staging)
  }
  run(0, min(2, P), P <= 2);
  // activations needing more planes (rare): planes two at a time, the
  // partial sums carried in the workspace
  for (int p0 = 2; p0 < P; p0 += 2) {
    __syncthreads();  // the previous pass's LDS reads are done
    stage(p0);
    load_first();
    __syncthreads();
    run(p0, min(2, P - p0), p0 + 2 >= P);
  }
}

// ---- down + weighted combine (matrix instructions) ------------------------------
// y_t = sum_j w_tj D_e(tj) h_tj on v_mfma_i32_16x16x64_i8: C[m][n] = C_in[m][n]
// + sum_k A[m][k] B[k][n] over 64 k, lane l holding row / column l % 16 and
// k-slot l / 16 (16 bytes) of A and B, and C[4 (l / 16) + i][l % 16], i < 4.
// B is 16 rows of D (a "tile"): lane (n, s) = (l % 16, l / 16) loads 16
// bytes of row n, covering k in [128 kb2 + 32 s, +32) of the 128-wide k
// block kb2 (int4: 32 nibbles; int8 weights: two loads), which feed the
// k-slot s of two instructions ("steps" hh = 0, 1): in step hh, slot s is h
// group G = 8 kb2 + 2 s + hh (16 k).  A row m = 4 g + c is column c of the
// record of group 8 kb2 + 2 g + hh, zero outside slot g, so that every C
// column sums over one group: one weight scale and one h factor.  Lane l's
// four outputs are the columns of its own group (g = l / 16), the record's
// Cin is the accumulator input, so each output is an exact integer, and
//   o[n] += scale x factor x (C0 + 256 C1 + 2^-15 (C2 + 256 C3))
// summed over the lane's k blocks and the four lanes of the row.
//
// A workgroup owns output rows [r0, r0 + nr) (tiles of 16).  A task is (a
// routed pair, a tile); waves take the tasks in turn, their k blocks in
// chunks of CK2, kNB chunks in flight per wave (a ring of register
// buffers).  The records (plane pair 0) of the pairs are staged in LDS, zero
// past the pair's groups up to whole chunks; with one round for all pairs
// (the usual case) a pair's LDS slot is its index and its records are
// requested at the start with the routing ids.  Each step's LDS reads sit at
// fixed offsets from a per-lane base (lanes off the diagonal read a zero
// block), issued one step ahead of the matrix instruction.
//
// Groups with more than two planes: the thread that stages such a group's
// record also requests its plane pair 1 record (before any weights), gets a
// slot in item order (a prefix count over the waves), writes it there and
// enters the slot in a per-(pair, chunk, k-slot) table of the chunk's eight
// steps (others point at a zero record).  A chunk with such groups runs
// every step with a second instruction on its plane pair 1 records, their
// addresses read from that table at the chunk's start.  Planes beyond those
// (and groups past the slots) are added after the wave's chunks, reloading
// the few weights they need.  Per-(row, pair) results meet in LDS and every
// output is y_t = sum_j w_tj o_tj in slot order, so y does not depend on
// timing.
constexpr int kMaxTasksPerWave = 64;            // tasks of a wave in one round (one per lane)
constexpr int kNB = 2;                          // chunks in flight per wave
constexpr uint32_t kOutside = 0x80000000u;      // a buffer offset past every record: loads zeros
constexpr size_t kDnLdsMax = 144 * 1024;        // dynamic LDS of the down kernel

__host__ __device__ constexpr int dn_ck2(int fmt) { return fmt == kFmtInt8 ? 2 : 4; }
// record slots per pair in LDS: whole chunks of k blocks
__host__ __device__ constexpr int dn_ngl(int fmt, int I) {
  return 8 * dn_ck2(fmt) * (((I + 127) / 128 + dn_ck2(fmt) - 1) / dn_ck2(fmt));
}
// zero block read by the lanes off the diagonal: the largest step offset + 16
__host__ __device__ constexpr int dn_zblock(int fmt) { return ((8 * (dn_ck2(fmt) - 1) + 1) * kRecBytes + 16 + 15) / 16 * 16; }

// Flags of 64 consecutive groups (bit i: group g0 + i, g0 a multiple of 64)
// to flags of their 16 steps: bit 2 b + h is set when a group 8 b + 2 s + h
// (s < 4) of k block g0 / 8 + b is flagged.
__device__ __forceinline__ uint32_t step_bits(uint64_t m) {
  uint64_t e = m & 0x5555555555555555ull, o = (m >> 1) & 0x5555555555555555ull;
  e |= e >> 2;
  e |= e >> 4;  // bit 8 b: any even group of byte b
  o |= o >> 2;
  o |= o >> 4;
  uint64_t z = (e & 0x0101010101010101ull) | ((o & 0x0101010101010101ull) << 1);  // 2 bits at 8 b
  z = (z | (z >> 6)) & 0x000F000F000F000Full;   // 4 bits at 16 c
  z = (z | (z >> 12)) & 0x000000FF000000FFull;  // 8 bits at 32 d
  return (uint32_t)(z | (z >> 24)) & 0xFFFFu;
}

// SM: weight scales.  0: one per row; 1: per group (any size); 2: groups of 64.
template <int FMT, int SM>
__global__ __launch_bounds__(kMT) void moe_down_kernel(MoeDecArgs a, int PR, int xcap) {
  constexpr int CK2 = dn_ck2(FMT);
  constexpr int NS = 2 * CK2;                  // steps per chunk
  constexpr int WV = FMT == kFmtInt8 ? 2 : 1;  // 16-byte weight loads per lane and k block (int3: 12 bytes)
  extern __shared__ __attribute__((aligned(16))) char lds[];
  __shared__ Route R;
  __shared__ int s_xready, s_cnt[2][kMW];
  const ExpertArgs& ex = a.ex;
  const int H = ex.H, I = ex.I;
  const int np = a.T * a.topk;
  const int NK2 = (I + 127) / 128, NGP = dn_ngp(I), NG = (I + 15) / 16, NGL = dn_ngl(FMT, I);
  const int CPT = (NK2 + CK2 - 1) / CK2;  // chunks per task
  const int wave = wuni(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int n = lane & 15, s = lane >> 4;
  const bool diag = (n >> 2) == s;
  const int Rb = (H + gridDim.x - 1) / gridDim.x;
  const int r0 = blockIdx.x * Rb, nr = min(Rb, H - r0);
  const int ntile = (nr + 15) / 16;
  // LDS: part [Rb][np] | records [PR][NGL] | zero block | step table
  // [PR][CPT][4] of 8 slot numbers | slots [xcap + 1] (the last: zeros)
  float* part = reinterpret_cast<float*>(lds);
  uint8_t* rec = reinterpret_cast<uint8_t*>(lds + ((size_t)Rb * np * 4 + 15) / 16 * 16);
  uint8_t* zblk = rec + (size_t)PR * NGL * kRecBytes;
  uint16_t* xtab = reinterpret_cast<uint16_t*>(zblk + dn_zblock(FMT));
  uint8_t* xrec = reinterpret_cast<uint8_t*>(xtab + (size_t)PR * CPT * 4 * 8);
  // the records of every pair: plane pairs q of pair p at (p kRecPairs + q) NGP
  const uint32_t rec_bytes = (uint32_t)((size_t)np * kRecPairs * NGP * kRecBytes);
  const __amdgpu_buffer_rsrc_t rall = region_rsrc(a.hrec, rec_bytes);

  // staged items: (pair slot, group) records, 96 bytes (zero past I / 16)
  const bool one = np <= PR;
  // (buffer loads: a generic load would make its first use wait for every
  // load issued after it)
  u32x4 st[2][6];
  auto stage_load = [&](int nit, int pb_, bool routed) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int it = min((int)threadIdx.x + kMT * j, max(nit, 1) - 1);
      const int pr = it / NGL, g = it - pr * NGL;
      const int pair = (one || !routed) ? pr : R.upair[pb_ + pr];
      const uint32_t off = (uint32_t)(((int64_t)pair * kRecPairs * NGP + min(g, NG - 1)) * kRecBytes);
#pragma unroll
      for (int k = 0; k < 6; ++k) st[j][k] = __builtin_amdgcn_raw_buffer_load_b128(rall, off + 16u * k, 0, 0);
    }
  };
  auto put = [&](int it, const u32x4* v6) __attribute__((always_inline)) {
    const int g = it % NGL;
    u32x4* dst = reinterpret_cast<u32x4*>(rec + (size_t)it * kRecBytes);
#pragma unroll
    for (int k = 0; k < 6; ++k) dst[k] = g < NG ? v6[k] : u32x4{0u, 0u, 0u, 0u};
  };
  {
    const int id_t = threadIdx.x < np ? a.ids[threadIdx.x] : -1;
    const float w_t = threadIdx.x < np ? a.w[threadIdx.x] : 0.f;
    stage_load(one ? np * NGL : 0, 0, false);
    build_route(id_t, w_t, np, ex.E, R);
  }
  const int nu = R.nu, nvalid = R.ustart[nu];
  // the zero block and the zero slot record
  for (int i = threadIdx.x; i < dn_zblock(FMT) / 4; i += kMT) reinterpret_cast<uint32_t*>(zblk)[i] = 0u;
  if (threadIdx.x < kRecBytes / 4) reinterpret_cast<uint32_t*>(xrec + (size_t)xcap * kRecBytes)[threadIdx.x] = 0u;

  struct Chunk {
    u32x4 sc4[SM == 2 ? (CK2 + 1) / 2 : 1];  // groups of 64: whole 16-byte loads
    float sc[SM == 2 ? 1 : CK2];
    u32x4 w[CK2][WV];
  };
  Chunk ring[kNB];
  typedef int v4i __attribute__((ext_vector_type(4)));

  auto bconv = [&](const u32x4 (&w)[WV], int hh) __attribute__((always_inline)) {
    if constexpr (FMT == kFmtInt4) {
      const uint32_t w0 = w[0][2 * hh], w1 = w[0][2 * hh + 1];
      return u32x4{w0 & 0x0F0F0F0Fu, (w0 >> 4) & 0x0F0F0F0Fu, w1 & 0x0F0F0F0Fu, (w1 >> 4) & 0x0F0F0F0Fu};
    } else if constexpr (FMT == kFmtInt3) {
      // the half's 16 values as offset-binary nibbles (signed nibble ^ 8 = value + 4), even then odd
      uint32_t we, wo;
      i3_words_ob(w[0][hh], (w[0][2] >> (16 * hh)) & 0xFFFFu, we, wo);
      return u32x4{we & 0x0F0F0F0Fu, (we >> 4) & 0x0F0F0F0Fu, wo & 0x0F0F0F0Fu, (wo >> 4) & 0x0F0F0F0Fu};
    } else {
      return w[hh];
    }
  };
  auto mfma = [&](const u32x4& av, const u32x4& bw, const u32x4& cin) __attribute__((always_inline)) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(v4i, av), __builtin_bit_cast(v4i, bw),
                                                 __builtin_bit_cast(v4i, cin), 0, 0, 0);
  };
  // a step's four integer columns into the lane's two accumulators: plane
  // 2q (C0 + 256 C1, exact: below 2^23) and plane 2q + 1 (C2 + 256 C3)
  float a01 = 0.f, a23 = 0.f;
  auto accum = [&](const v4i& c, float f) __attribute__((always_inline)) {
    a01 = __builtin_fmaf((float)(c[0] + (c[1] << 8)), f, a01);
    a23 = __builtin_fmaf((float)(c[2] + (c[3] << 8)), f, a23);
  };
  // o[n] of a task from the lane's accumulators, the four lanes of the row
  // (k-slots) summed
  auto row_value = [&](float p01, float p23) __attribute__((always_inline)) {
    float v = __builtin_fmaf(p23, 1.f / 32768.f, p01);
    v += __shfl_xor(v, 16, 64);
    v += __shfl_xor(v, 32, 64);
    return v;
  };

  int pb = 0, ub = 0;  // first pair and its unique expert of the round
  bool first = true;
  while (pb < nvalid) {
    // the round: pairs [pb, pe), ending at an expert boundary when one fits
    int pe = min(nvalid, pb + PR);
    int ue = ub;
    while (ue < nu && R.ustart[ue + 1] <= pe) ++ue;  // experts wholly inside
    if (ue > ub) pe = R.ustart[ue];
    else ue = ub + 1;                                // one expert split over rounds
    const int nit = one ? np * NGL : (pe - pb) * NGL;  // items staged for the round
    auto pair_of_slot = [&](int pr) __attribute__((always_inline)) { return one ? pr : R.upair[pb + pr]; };
    // tasks: t = (place in the routing table - pb) ntile + tile; wave w takes
    // t = w, w + kMW, ...: lane i of the wave holds its task i (expert id;
    // pair, LDS slot and tile packed)
    const int ntasks = (pe - pb) * ntile;
    const int myt = wave < ntasks ? (ntasks - 1 - wave) / kMW + 1 : 0;
    const int nj = myt * CPT;  // this wave's chunks
    int tk_e = 0, tk_p = 0;
    if (lane < myt) {
      const int t = wave + kMW * lane;
      const int pi = pb + t / ntile, tile = t % ntile;
      const int pair = R.upair[pi];
      tk_e = R.tmp_id[pair];
      tk_p = (pair << 24) | ((one ? pair : pi - pb) << 16) | tile;
    }

    if (!first) __syncthreads();  // the previous round's LDS reads are done
    if (threadIdx.x == 0) s_xready = 0;
    if (!one) stage_load(nit, pb, true);
    // the thread's first two items with more than two planes: their plane
    // pair 1 records requested (before any weights; others: zeros, no access)
    u32x4 xr[2][6];
    uint64_t xb[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int it = threadIdx.x + kMT * j;
      const int pr = it / NGL, g = it - pr * NGL;
      const bool f = it < nit && g < NG && (int)(st[j][5][1] & 0xFFu) > 2;
      xb[j] = __ballot(f);
      const uint32_t off =
          f ? (uint32_t)(((int64_t)pair_of_slot(f ? pr : 0) * kRecPairs + 1) * NGP + g) * kRecBytes : kOutside;
#pragma unroll
      for (int k = 0; k < 6; ++k) xr[j][k] = __builtin_amdgcn_raw_buffer_load_b128(rall, off + 16u * k, 0, 0);
      if (lane == 0) s_cnt[j][wave] = __popcll(xb[j]);
    }
    // every step table entry at the zero slot
    for (int i = threadIdx.x; i < (one ? np : pe - pb) * CPT * 4 * 8 / 2; i += kMT)
      reinterpret_cast<uint32_t*>(xtab)[i] = (uint32_t)xcap * 0x10001u;

    // weights of the wave's chunk j: task j / CPT, k blocks from CK2 (j %
    // CPT); the load cursor (lt, lp) walks j; past the end: empty resources
    // (loads of zeros)
    int lt = 0, lp = 0;
    __amdgpu_buffer_rsrc_t rq = region_rsrc(ex.dq, 0u), rsc = region_rsrc(ex.ds, 0u);
    auto task_rsrc = [&](int ti) __attribute__((always_inline)) {
      const bool ok = ti < myt;
      const int e = __builtin_amdgcn_readlane(tk_e, min(ti, 63));
      const int tile = __builtin_amdgcn_readlane(tk_p, min(ti, 63)) & 0xFFFF;
      const int rows = min(16, nr - 16 * tile);
      const int64_t er0 = (int64_t)e * H + r0 + 16 * tile;
      rq = region_rsrc(ex.dq + er0 * ex.rb_i, ok ? (uint32_t)(rows * ex.rb_i) : 0u);
      rsc = region_rsrc(ex.ds + er0 * ex.G_i, ok ? (uint32_t)(rows * ex.G_i * 4) : 0u);
    };
    // lane (n, s): row n, k in [128 kb2 + 32 s, +32) -- int3: half s & 1 of
    // group 2 kb2 + s / 2, its two low words and their 32 high bits
    const uint32_t qo = (uint32_t)n * (uint32_t)ex.rb_i +
                        (FMT == kFmtInt4   ? (uint32_t)s * 16u
                         : FMT == kFmtInt3 ? (uint32_t)(s >> 1) * 24u + 8u * (uint32_t)(s & 1)
                                           : (uint32_t)s * 32u);
    const uint32_t so = (uint32_t)n * (uint32_t)ex.G_i * 4u;
    // (cached loads: the 16 rows x 64 bytes of one k block are half of each
    // row's 128-byte line, whose other half the next k block reads at once)
    auto wload = [&](uint32_t kb2, u32x4 (&w)[WV]) __attribute__((always_inline)) {
      if constexpr (FMT == kFmtInt3) {
        const u32x2 lw = __builtin_amdgcn_raw_buffer_load_b64(rq, qo, 48u * kb2, 0);
        const uint32_t hw = __builtin_amdgcn_raw_buffer_load_b32(rq, qo + 16u - 4u * (uint32_t)(s & 1), 48u * kb2, 0);
        w[0] = u32x4{lw[0], lw[1], hw, 0u};
      } else {
#pragma unroll
        for (int v = 0; v < WV; ++v)
          w[v] = __builtin_amdgcn_raw_buffer_load_b128(rq, qo + 16u * v, (FMT == kFmtInt4 ? 64u : 128u) * kb2, 0);
      }
    };
    auto load = [&](Chunk& ch) __attribute__((always_inline)) {
      if (lp == 0) task_rsrc(lt);
      const int k0 = lp * CK2;
      if constexpr (SM == 0) {
        ch.sc[0] = ld_region4(rsc, so);  // the row's one scale
      } else if constexpr (SM == 1) {
#pragma unroll
        for (int kk = 0; kk < CK2; ++kk)
          ch.sc[kk] = ld_region4(rsc, so + (((uint32_t)(k0 + kk) * 128u + (uint32_t)s * 32u) >> (ex.gshift + 5)) * 4u);
      } else {  // groups of 64: scale 2 kb2 + s / 2; a 16-byte load from
                // 2 k0 + 4 v + s / 2 holds those of kb2 = k0 + 2v, k0 + 2v + 1
                // in its words 0 and 2
#pragma unroll
        for (int v = 0; v < (CK2 + 1) / 2; ++v)
          ch.sc4[v] = __builtin_amdgcn_raw_buffer_load_b128(rsc, so + (uint32_t)(s >> 1) * 4u, (uint32_t)(2 * k0 + 4 * v) * 4u, 0);
      }
#pragma unroll
      for (int kk = 0; kk < CK2; ++kk) wload((uint32_t)(k0 + kk), ch.w[kk]);
      if (++lp == CPT) {
        lp = 0;
        ++lt;
      }
    };

    // the round's records into LDS
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int it = threadIdx.x + kMT * j;
      if (it < nit) put(it, st[j]);
    }
    for (int it = threadIdx.x + 2 * kMT; it < nit; it += kMT) {  // items past two per thread
      const int pr = it / NGL, g = it - pr * NGL;
      const u32x4* src = reinterpret_cast<const u32x4*>(
          a.hrec + ((int64_t)pair_of_slot(pr) * kRecPairs * NGP + min(g, NG - 1)) * kRecBytes);
      u32x4 v6[6];
#pragma unroll
      for (int k = 0; k < 6; ++k) v6[k] = src[k];
      put(it, v6);
    }
    // the first kNB chunks of weights requested
#pragma unroll
    for (int b = 0; b < kNB; ++b) load(ring[b]);
    __syncthreads();
    // slots of the thread's items with more planes: their rank in item order;
    // the record marked, the step table entry and the slot written
    {
      int base = 0;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        for (int w = 0; w < kMW; ++w) base += (w < wave) ? s_cnt[j][w] : 0;
        int slot = base + __popcll(xb[j] & ((1ull << lane) - 1));
        for (int w = wave; w < kMW; ++w) base += s_cnt[j][w];
        if (((xb[j] >> lane) & 1) != 0 && slot < xcap) {
          const int it = threadIdx.x + kMT * j;
          const int pr = it / NGL, g = it - pr * NGL;
          int* pf = reinterpret_cast<int*>(rec + (size_t)it * kRecBytes + 84);
          *pf = (*pf & 0xFF) | ((slot + 1) << 8);
          const int kb2 = g >> 3, gs = (g >> 1) & 3, step = 2 * (kb2 % CK2) + (g & 1);
          xtab[(((size_t)pr * CPT + kb2 / CK2) * 4 + gs) * 8 + step] = (uint16_t)slot;
#pragma unroll
          for (int k = 0; k < 6; ++k) reinterpret_cast<u32x4*>(xrec + (size_t)slot * kRecBytes)[k] = xr[j][k];
        }
      }
    }
    // this wave's slots are written
    if (lane == 0) __hip_atomic_fetch_add(&s_xready, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);

    bool xseen = false;  // every wave's slots are written
    auto wait_slots = [&]() __attribute__((always_inline)) {
      if (!xseen) {
        while (__hip_atomic_load(&s_xready, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) < kMW)
          __builtin_amdgcn_s_sleep(1);
        xseen = true;
      }
    };
    uint64_t tmore = 0;  // this wave's tasks (by index) with groups of more than two planes

    // the compute cursor (ct, cp) walks the chunks in the same order
    int ct = 0, cp = 0;
    const uint8_t* rp = rec;
    uint32_t xm0 = 0, xm1 = 0;  // the task's steps with further planes (bit 2 kb2 + hh)
    auto compute = [&](Chunk& ch) __attribute__((always_inline)) {
      const int k0 = cp * CK2;
      const int tp = __builtin_amdgcn_readlane(tk_p, ct);
      const int slot = (tp >> 16) & 0xFF;
      if (cp == 0) {
        rp = rec + (size_t)slot * NGL * kRecBytes;
        a01 = a23 = 0.f;
        // steps of this task with further planes: bit 2 kb2 + hh for a
        // group G = 8 kb2 + 2 s + hh with P > 2
        xm0 = xm1 = 0;
        for (int g0 = 0; g0 < NG; g0 += 64) {
          const int g = g0 + lane;
          const bool f = g < NG && (*reinterpret_cast<const int*>(rp + (size_t)g * kRecBytes + 84) & 0xFF) > 2;
          const uint32_t bits = step_bits(__ballot(f));
          if (g0 < 128) xm0 |= bits << (g0 / 4);
          else xm1 |= bits << (g0 / 4 - 32);
        }
        if ((xm0 | xm1) != 0) tmore |= 1ull << ct;
      }
      const uint32_t xm = (uint32_t)((((uint64_t)xm1 << 32) | xm0) >> (2 * k0)) & ((1u << NS) - 1u);
      // scales of the chunk taken here (all words of their loads in use)
      if constexpr (SM == 2)
#pragma unroll
        for (int v = 0; v < (CK2 + 1) / 2; ++v) asm volatile("" : "+v"(ch.sc4[v]));
      auto scale_of = [&](int kk) __attribute__((always_inline)) {
        return SM == 2 ? __uint_as_float(ch.sc4[kk / 2][2 * (kk & 1)]) : (SM == 0 ? 1.f : ch.sc[kk]);
      };
      // the lane's records: step st (k block k0 + st / 2, half st % 2) at
      // a fixed offset from lb; lanes off the diagonal read the zero block
      const uint8_t* lb = rp + (size_t)(8 * k0 + 2 * s) * kRecBytes;
      const uint8_t* ab = diag ? lb + 16 * (n & 3) : zblk;
      struct StepIn {
        u32x4 av, cin;
        float hf;
      };
      auto rd = [&](int st_) __attribute__((always_inline)) {
        const int off = (8 * (st_ >> 1) + (st_ & 1)) * kRecBytes;
        StepIn r;
        r.av = *reinterpret_cast<const u32x4*>(ab + off);
        r.cin = *reinterpret_cast<const u32x4*>(lb + off + 64);
        r.hf = *reinterpret_cast<const float*>(lb + off + 80);
        return r;
      };
      if (xm == 0) {
        // software pipeline: the LDS reads of step st + 1 are issued before
        // the matrix instruction of step st, whose result is taken after that
        // of step st + 1 is issued
        StepIn cur = rd(0);
        v4i cprev = {0, 0, 0, 0};
        float fprev = 0.f;
#pragma unroll
        for (int st_ = 0; st_ < NS; ++st_) {
          StepIn nx = cur;
          if (st_ + 1 < NS) nx = rd(st_ + 1);
          __builtin_amdgcn_sched_barrier(0);
          const v4i c = mfma(cur.av, bconv(ch.w[st_ >> 1], st_ & 1), cur.cin);
          const float f = scale_of(st_ >> 1) * cur.hf;
          if (st_ > 0) accum(cprev, fprev);
          __builtin_amdgcn_sched_barrier(0);
          cprev = c;
          fprev = f;
          cur = nx;
        }
        accum(cprev, fprev);
      } else {
        // with plane pair 1: each step's slot record (or the zero record)
        // from the step table, read with the step's own records
        wait_slots();
        const u32x4 xt = *reinterpret_cast<const u32x4*>(xtab + (((size_t)slot * CPT + cp) * 4 + s) * 8);
        struct XIn {
          u32x4 av, cin;
          float hf;
        };
        auto xrd = [&](int st_) __attribute__((always_inline)) {
          const uint32_t sl = (xt[st_ >> 1] >> (16 * (st_ & 1))) & 0xFFFFu;
          const uint8_t* xg = xrec + sl * (uint32_t)kRecBytes;
          XIn r;
          r.av = *reinterpret_cast<const u32x4*>(diag ? xg + 16 * (n & 3) : zblk);
          r.cin = *reinterpret_cast<const u32x4*>(xg + 64);
          r.hf = *reinterpret_cast<const float*>(xg + 80);
          return r;
        };
        StepIn cur = rd(0);
        XIn xcur = xrd(0);
        v4i cprev = {0, 0, 0, 0}, xprev = {0, 0, 0, 0};
        float fprev = 0.f, xfprev = 0.f;
        bool xhas = false;
#pragma unroll
        for (int st_ = 0; st_ < NS; ++st_) {
          StepIn nx = cur;
          XIn xnx = xcur;
          if (st_ + 1 < NS) {
            nx = rd(st_ + 1);
            xnx = xrd(st_ + 1);
          }
          __builtin_amdgcn_sched_barrier(0);
          const u32x4 bw = bconv(ch.w[st_ >> 1], st_ & 1);
          const float sc = scale_of(st_ >> 1);
          const v4i c = mfma(cur.av, bw, cur.cin);
          const bool xs = (xm >> st_) & 1;
          v4i cx = {0, 0, 0, 0};
          if (xs) cx = mfma(xcur.av, bw, xcur.cin);
          if (st_ > 0) accum(cprev, fprev);
          if (xhas) accum(xprev, xfprev);
          __builtin_amdgcn_sched_barrier(0);
          cprev = c;
          fprev = sc * cur.hf;
          xprev = cx;
          xfprev = sc * xcur.hf;
          xhas = xs;
          cur = nx;
          xcur = xnx;
        }
        accum(cprev, fprev);
        if (xhas) accum(xprev, xfprev);
      }
      if (cp == CPT - 1) {
        const float v = row_value(a01, a23);
        const int row = 16 * (tp & 0xFFFF) + n;
        if (s == 0 && row < nr) part[(size_t)row * np + (tp >> 24)] = SM == 0 ? v * ch.sc[0] : v;
      }
      if (++cp == CPT) {
        cp = 0;
        ++ct;
      }
    };

    for (int j = 0; j < nj; j += kNB) {
#pragma unroll
      for (int b = 0; b < kNB; ++b) {
        if (j + b >= nj) break;
        compute(ring[b]);
        load(ring[b]);
      }
    }

    // planes past the slots: plane pairs 2 and up, and plane pair 1 of groups
    // without a slot, added to the task's rows (rare)
    if (tmore != 0) {
      wait_slots();
      for (int ti = 0; ti < myt; ++ti) {
        if (((tmore >> ti) & 1) == 0) continue;
        const int tp = __builtin_amdgcn_readlane(tk_p, ti);
        const int pair = tp >> 24, tile = tp & 0xFFFF;
        const uint8_t* trp = rec + (size_t)((tp >> 16) & 0xFF) * NGL * kRecBytes;
        uint32_t tm0 = 0, tm1 = 0;
        for (int g0 = 0; g0 < NG; g0 += 64) {
          const int g = g0 + lane;
          const int pinfo = g < NG ? *reinterpret_cast<const int*>(trp + (size_t)g * kRecBytes + 84) : 0;
          const int pc = pinfo & 0xFF;
          const uint32_t bits = step_bits(__ballot(pc > 4 || (pc > 2 && (pinfo >> 8) == 0)));
          if (g0 < 128) tm0 |= bits << (g0 / 4);
          else tm1 |= bits << (g0 / 4 - 32);
        }
        uint64_t tm = ((uint64_t)tm1 << 32) | tm0;
        if (tm == 0) continue;
        task_rsrc(ti);
        float t01 = 0.f, t23 = 0.f;
        while (tm != 0) {
          const int b = __builtin_ctzll(tm);
          tm &= tm - 1;
          const uint32_t kb2 = (uint32_t)(b >> 1);
          const int hh = b & 1;
          u32x4 w[WV];
          wload(kb2, w);
          float sc = 1.f;
          if constexpr (SM == 1) sc = ld_region4(rsc, so + ((kb2 * 128u + (uint32_t)s * 32u) >> (ex.gshift + 5)) * 4u);
          if constexpr (SM == 2) sc = ld_region4(rsc, so + (2u * kb2 + (uint32_t)(s >> 1)) * 4u);
          const u32x4 bw = bconv(w, hh);
          const int G = 8 * (int)kb2 + 2 * s + hh;
          const int pinfo = *reinterpret_cast<const int*>(trp + (size_t)G * kRecBytes + 84);
          const int pc = pinfo & 0xFF;
          const int qlo = (pinfo >> 8) != 0 ? 2 : 1;
          int nq = (pc + 1) / 2;
          nq = max(nq, __shfl_xor(nq, 16, 64));
          nq = wuni(max(nq, __shfl_xor(nq, 32, 64)));
          for (int q = 1; q < nq; ++q) {
            const bool act = q >= qlo && 2 * q < pc;
            const uint32_t ro = act ? (uint32_t)(((int64_t)pair * kRecPairs + q) * NGP + G) * kRecBytes : kOutside;
            const u32x4 xa = __builtin_amdgcn_raw_buffer_load_b128(rall, diag ? ro + 16u * (uint32_t)(n & 3) : kOutside, 0, 0);
            const u32x4 xc = __builtin_amdgcn_raw_buffer_load_b128(rall, ro + 64u, 0, 0);
            const float xh = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rall, ro + 80u, 0, 0));
            const v4i c2 = mfma(xa, bw, xc);
            t01 = __builtin_fmaf((float)(c2[0] + (c2[1] << 8)), sc * xh, t01);
            t23 = __builtin_fmaf((float)(c2[2] + (c2[3] << 8)), sc * xh, t23);
          }
        }
        float v = row_value(t01, t23);
        if constexpr (SM == 0) v *= ld_region4(rsc, so);
        const int row = 16 * tile + n;
        if (s == 0 && row < nr) part[(size_t)row * np + pair] += v;
      }
    }
    pb = pe;
    ub = ue;
    if (pb < nvalid && ub < nu && R.ustart[ub] > pb) --ub;  // an expert split over rounds continues
    first = false;
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

// caller-supplied fp32 h [T*k][I] -> records, one wave per (pair, group)
template <int FMT>
__global__ __launch_bounds__(256) void h_records_kernel(MoeDecArgs a, int ngroups_total) {
  const int g = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (g >= ngroups_total) return;
  const int NG = (a.ex.I + 15) / 16, NGP = dn_ngp(a.ex.I);
  const int pair = g / NG, gi = g - pair * NG;
  const int lane = threadIdx.x & 63;
  const int r = gi * 16 + lane;
  const float v = (lane < 16 && r < a.ex.I) ? a.h[(int64_t)pair * a.ex.I + r] : 0.f;
  wave_h_records<FMT>(v, a.hrec + (((int64_t)pair * kRecPairs) * NGP + gi) * kRecBytes, (size_t)NGP * kRecBytes);
}

// ---- launchers ------------------------------------------------------------------------

// chunk positions per lane of the gate+up kernel instantiated for rows of
// kch chunks (0: none)
int gu_cpl(int kch) {
  const int c = (kch + 63) / 64;
  if (c <= 4) return c;
  if (c <= 6) return 6;
  if (c <= 8) return 8;
  return 0;
}

// LDS bytes of the gate+up kernel: two planes of digit words and a factor per
// chunk position, for T tokens
size_t gu_lds(int fmt, int T, int H) {
  const int per = fmt == kFmtInt8 ? 16 : 32;
  const size_t kchp = (size_t)64 * gu_cpl(H / per);
  return (size_t)2 * T * kchp * (fmt == kFmtInt8 ? 8 : 16) * 4 + (size_t)T * kchp * 4;
}

template <int FMT, int XT, bool GROUPED>
hipError_t launch_gu(const MoeDecArgs& a, int cus, hipStream_t st) {
  constexpr int PER = per_chunk<FMT>();
  const int cpl = gu_cpl(a.ex.H / PER);
  const size_t lds = gu_lds(FMT, a.T, a.ex.H);
  if (cpl == 0 || lds > kDecLdsMax || a.T * 64 * cpl > 2 * kGT) return hipErrorNotSupported;
  const int nunits_max = a.T * a.topk * ((a.ex.I + kHT - 1) / kHT);
  const int blocks = max(1, min(cus, nunits_max));
  // two register buffers of weights (the next unit loading while one is
  // computed) where they fit the 256 registers of each of the 8 waves
#define QM_GU(C, NBUF)                                                                                         \
  hipLaunchKernelGGL((moe_gu_kernel<FMT, XT, GROUPED, C, NBUF>), dim3(blocks), dim3(kGT), lds, st, a); \
  return hipGetLastError();
  switch (cpl) {
    case 1: { QM_GU(1, 2) }
    case 2: { QM_GU(2, 2) }
    case 3: { QM_GU(3, 2) }
    case 4: { QM_GU(4, 1) }
    case 6: { QM_GU(6, 1) }
    case 8: { QM_GU(8, 1) }
    default: break;
  }
#undef QM_GU
  return hipErrorNotSupported;
}

// Down launch plan: rows per workgroup, pairs per round, slots for plane
// pair 1 records and the dynamic LDS bytes; false when the shape does not fit.
struct DnPlan {
  int Rb, blocks, PR, xcap;
  size_t lds;
};
bool dn_plan(int fmt, int T, int topk, int H, int I, int cus, DnPlan& p) {
  if (cus < 1 || H < 1 || I < 1) return false;
  p.Rb = (H + cus - 1) / cus;
  p.blocks = (H + p.Rb - 1) / p.Rb;  // every workgroup has rows
  const int np = T * topk;
  const int ntile = (p.Rb + 15) / 16;
  if (ntile > kMaxTasksPerWave * kMW || ntile > 0xFFFF || (I + 127) / 128 > 32) return false;  // bit masks, fields
  const int cpt = ((I + 127) / 128 + dn_ck2(fmt) - 1) / dn_ck2(fmt);
  const size_t fixed = ((size_t)p.Rb * np * 4 + 15) / 16 * 16 + dn_zblock(fmt) + kRecBytes;  // part, zeros
  const size_t per_pair = (size_t)dn_ngl(fmt, I) * kRecBytes + (size_t)cpt * 4 * 16;          // records, step table
  if (fixed + per_pair > kDnLdsMax) return false;
  p.PR = (int)std::min<size_t>((size_t)np, (kDnLdsMax - fixed) / per_pair);  // pairs per round
  p.PR = std::min(p.PR, kMaxTasksPerWave * kMW / ntile);                      // tasks per wave: one per lane
  const size_t used = fixed + (size_t)p.PR * per_pair;
  p.xcap = (int)std::min<size_t>(2 * kMT, (kDnLdsMax - used) / kRecBytes);
  p.lds = used + (size_t)p.xcap * kRecBytes;
  return true;
}

template <int FMT>
hipError_t launch_down(const MoeDecArgs& a, int gs, int cus, hipStream_t st) {
  DnPlan p;
  if (!dn_plan(FMT, a.T, a.topk, a.ex.H, a.ex.I, cus, p)) return hipErrorNotSupported;
#define QM_DN(SM_)                                                                                         \
  hipLaunchKernelGGL((moe_down_kernel<FMT, SM_>), dim3(p.blocks), dim3(kMT), p.lds, st, a, p.PR, p.xcap); \
  return hipGetLastError();
  if (gs == 0) { QM_DN(0) }
  if (gs == 64) { QM_DN(2) }
  QM_DN(1)
#undef QM_DN
}

}  // namespace

size_t moe_decode_ws_bytes(int T, int topk, int H, int I) {
  const size_t P = (size_t)T * topk;
  auto al = [](size_t v) { return (v + 255) / 256 * 256; };
  return al(P * kRecPairs * dn_ngp(I) * kRecBytes) + al(P * (size_t)I * 8);
}

void moe_decode_ws_split(MoeDecArgs& a, void* ws) {
  const size_t P = (size_t)a.T * a.topk;
  auto al = [](size_t v) { return (v + 255) / 256 * 256; };
  char* p = static_cast<char*>(ws);
  a.hrec = reinterpret_cast<uint8_t*>(p);
  p += al(P * kRecPairs * dn_ngp(a.ex.I) * kRecBytes);
  a.ab = reinterpret_cast<float*>(p);
}

bool moe_decode_supported(int fmt, int T, int topk, const ExpertArgs& e) {
  if (T < 1 || T * topk > kMaxPairs) return false;
  const int per = fmt == kFmtInt8 ? 16 : 32;
  const int kh = e.H / per, ki = e.I / per;
  (void)ki;
  if (gu_cpl(kh) == 0) return false;
  // the down plan on this device's compute units (without a device: checked
  // for 256, so that argument checks do not depend on one being present)
  int cus = 0;
  if (device_cus(&cus) != hipSuccess) cus = 256;
  DnPlan p;
  if (!dn_plan(fmt, T, topk, e.H, e.I, cus, p)) return false;
  return gu_lds(fmt, T, e.H) <= kDecLdsMax && T * 64 * gu_cpl(kh) <= 2 * kGT;
}

// largest token count per pass whose x digit planes fit the LDS budget
int moe_decode_tokens_per_pass(int fmt, int topk, const ExpertArgs& e) {
  const int per = fmt == kFmtInt8 ? 16 : 32;
  if (gu_cpl(e.H / per) == 0) return 0;
  int t = (int)(kDecLdsMax / gu_lds(fmt, 1, e.H));
  t = min(t, 2 * kGT / (64 * gu_cpl(e.H / per)));  // two x groups per thread when staging
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
  if (fmt == kFmtInt3) {
    if (!grouped) return hipErrorNotSupported;
    return xdt == kBF16 ? launch_gu<kFmtInt3, kBF16, true>(a, cus, st) : launch_gu<kFmtInt3, kF32, true>(a, cus, st);
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
      hipLaunchKernelGGL(h_records_kernel<kFmtInt4>, dim3((ng + 3) / 4), dim3(256), 0, st, a, ng);
    else if (fmt == kFmtInt3)
      hipLaunchKernelGGL(h_records_kernel<kFmtInt3>, dim3((ng + 3) / 4), dim3(256), 0, st, a, ng);
    else
      hipLaunchKernelGGL(h_records_kernel<kFmtInt8>, dim3((ng + 3) / 4), dim3(256), 0, st, a, ng);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // the down matrices' scale group size (0: one scale per row)
  const int gs = (grouped && a.ex.G_i > 1) ? (32 << a.ex.gshift) : 0;
  if (fmt == kFmtInt4) return launch_down<kFmtInt4>(a, gs, cus, st);
  if (fmt == kFmtInt3) return gs == 64 ? launch_down<kFmtInt3>(a, gs, cus, st) : hipErrorNotSupported;
  if (grouped) return hipErrorNotSupported;
  return launch_down<kFmtInt8>(a, 0, cus, st);
}

}  // namespace qm
