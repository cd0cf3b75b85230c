// moe_int3.hip -- the routed expert FFN for int3-g64 experts (fmt 5): for
// each token t and routed slot j with expert e = ids[t][j],
//   h_tj = silu(G_e x_t) * (U_e x_t),   y_t = sum_j w_tj * D_e h_tj
// (the colibri page "Vulkan backend: expert tier + dense + MLA attention on
// any Vulkan 1.2 GPU": the int3 commit notes give the expert matmuls and the
// fused gate_up this format; the K-expert group note gives gate+up for the
// routed experts, then the down projections and the weighted combine).  An
// expert id outside [0, E) makes its pair contribute nothing (its h row is
// not written and the down pass skips the slot).
//
// Two launches:
//  1. gate+up: workgroup (bx, t) stages x_t in LDS (int3.hpp layout); each
//     wave takes tasks (slot j, row i): the gate row and the up row of
//     expert e_j, 2 * G_h groups spread over the 64 lanes (lane l takes
//     units l, l + 64, ...: gate groups first, then up groups), two wave
//     sums, h = silu(gate) * up written as fp32 [T * topk][I].  The next
//     task's groups are in flight while the current ones are decoded.
//  2. down + combine: workgroup (bx, t) stages the topk hidden vectors of
//     token t (fp32, split into bf16 hi + lo); each wave takes output rows r
//     and reduces, in one pass over its 64 lanes, all topk * G_i groups of
//     row r of the routed down matrices (lane l: units l, l + 64, ...; unit
//     u is slot u / G_i, group u % G_i), each group's dot times its scale
//     times the slot's routing weight.  No atomics: every y element is
//     written once, by one lane.
// Every byte of the routed rows is read once per token that routes to the
// expert (tokens are independent; no union of the experts across tokens).
#include "int3.hpp"
#include "launch.hpp"

namespace qm {

namespace {

constexpr int kGuThreads = 256;
constexpr int kDnThreads = 512;
constexpr size_t kDnLdsMax = 144 * 1024;  // staged hidden vectors of one token

struct I3MoeArgs {
  ExpertArgs ex;
  const void* x;  // [T][H] activations (bf16 bits or fp32)
  int bf16x;
  const int32_t* ids;  // [T][topk]
  const float* w;      // [T][topk]
  float* h;            // [T * topk][I]
  float* y;            // [T][H]
  int topk;
};

template <bool SPLIT, int U>
__global__ __launch_bounds__(kGuThreads) void moe_i3_gate_up_kernel(I3MoeArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint32_t lds[];
  const ExpertArgs& ex = a.ex;
  const int t = blockIdx.y, G = ex.G_h, tid = threadIdx.x;
  const I3Lds X = i3_carve(lds, G, SPLIT);
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  // the token's expert ids, one per lane (top_k <= 64): a task reads its
  // expert from a register, so requesting the next task's weights never
  // waits for an id load (and with it for the loads already in flight)
  const int idv = lane < a.topk ? a.ids[(size_t)t * a.topk + lane] : -1;
  int ug[U];
  bool uup[U], uok[U];
#pragma unroll
  for (int i = 0; i < U; ++i) {
    const int u = lane + 64 * i;
    uok[i] = u < 2 * G;
    uup[i] = u >= G;
    ug[i] = uok[i] ? (uup[i] ? u - G : u) : 0;
  }
  struct Task {
    I3Group w[U];
    float s[U];
    int e;  // expert, or -1 for an id outside [0, E)
  };
  const int ntask = a.topk * ex.I;
  auto load = [&](int task, Task& k) {
    const int j = task / ex.I, i = task - j * ex.I;
    const int e = __builtin_amdgcn_readlane(idv, j);
    k.e = (e >= 0 && e < ex.E) ? e : -1;
    if (k.e < 0) return;
    const int64_t row = (int64_t)k.e * ex.I + i;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint8_t* base = uup[u] ? ex.uq : ex.gq;
      const float* sb = uup[u] ? ex.us : ex.gs;
      k.w[u] = i3_load(base + row * ex.rb_h + (int64_t)ug[u] * 24);
      k.s[u] = uok[u] ? ld_stream(sb + row * G + ug[u]) : 0.f;
    }
  };
  const int stride = gridDim.x * (kGuThreads / 64);
  int task = blockIdx.x * (kGuThreads / 64) + wave;
  Task cur, nxt;
  if (task < ntask) load(task, cur);  // in flight while x is staged
  const char* xt = static_cast<const char*>(a.x) + (size_t)t * ex.H * (a.bf16x ? 2 : 4);
  i3_stage<SPLIT>(X, G, ex.H, a.bf16x != 0, [&](int) { return static_cast<const void*>(xt); }, tid, kGuThreads);
  __syncthreads();
  i3_corr(X, tid, kGuThreads);
  __syncthreads();
  // the id load is long complete here (staging waited for every load): a
  // use of it here lets the loop read it without waiting on the weights
  asm volatile("" ::"v"(idv));
  for (; task < ntask; task += stride) {
    if (task + stride < ntask) load(task + stride, nxt);
    float hv = 0.f;
    if (cur.e >= 0) {
      float ag = 0.f, au = 0.f;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (!uok[u]) continue;
        const float d = i3_group_dot<SPLIT>(cur.w[u], X, ug[u]);
        if (uup[u])
          au = __builtin_fmaf(cur.s[u], d, au);
        else
          ag = __builtin_fmaf(cur.s[u], d, ag);
      }
      ag = group_sum<64>(ag);
      au = group_sum<64>(au);
      hv = silu(ag) * au;
    }
    if (lane == 0 && cur.e >= 0) {  // rows of pairs with an invalid id are not written
      const int j = task / ex.I, i = task - j * ex.I;
      a.h[((size_t)t * a.topk + j) * ex.I + i] = hv;
    }
    cur = nxt;
  }
}

template <int U>
__global__ __launch_bounds__(kDnThreads) void moe_i3_down_kernel(I3MoeArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint32_t lds[];
  const ExpertArgs& ex = a.ex;
  const int t = blockIdx.y, G = ex.G_i, K = a.topk, tid = threadIdx.x;
  const I3Lds Hs = i3_carve(lds, K * G, true);
  const int wave = tid >> 6, lane = tid & 63;
  // the lane's units: row-independent parts of their addresses
  int64_t woff[U], soff[U];
  float uw[U];
  bool uok[U];
#pragma unroll
  for (int i = 0; i < U; ++i) {
    const int u = lane + 64 * i;
    const bool in = u < K * G;
    const int j = in ? u / G : 0, g = u - j * G;
    const int e = a.ids[(size_t)t * K + j];
    uok[i] = in && e >= 0 && e < ex.E;
    uw[i] = uok[i] ? a.w[(size_t)t * K + j] : 0.f;
    woff[i] = uok[i] ? (int64_t)e * ex.H * ex.rb_i + (int64_t)g * 24 : 0;
    soff[i] = uok[i] ? (int64_t)e * ex.H * G + g : 0;
  }
  struct Row {
    I3Group w[U];
    float s[U];
  };
  auto load = [&](int r, Row& k) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      k.w[u] = i3_load(ex.dq + woff[u] + (int64_t)r * ex.rb_i);
      k.s[u] = uok[u] ? ld_stream(ex.ds + soff[u] + (int64_t)r * G) : 0.f;
    }
  };
  const int stride = gridDim.x * (kDnThreads / 64);
  int r = blockIdx.x * (kDnThreads / 64) + wave;
  Row cur, nxt;
  if (r < ex.H) load(r, cur);  // in flight while h is staged
  const float* ht = a.h + (size_t)t * K * ex.I;
  i3_stage<true>(Hs, G, ex.I, false, [&](int v) { return static_cast<const void*>(ht + (size_t)v * ex.I); }, tid,
                 kDnThreads);
  __syncthreads();
  i3_corr(Hs, tid, kDnThreads);
  __syncthreads();
  for (; r < ex.H; r += stride) {
    if (r + stride < ex.H) load(r + stride, nxt);
    float acc = 0.f;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (!uok[u]) continue;
      const float d = i3_group_dot<true>(cur.w[u], Hs, lane + 64 * u);
      acc = __builtin_fmaf(uw[u] * cur.s[u], d, acc);
    }
    acc = group_sum<64>(acc);
    if (lane == 0) a.y[(size_t)t * ex.H + r] = acc;
    cur = nxt;
  }
}

// smallest instantiated units-per-lane count >= need (0: none)
int pick_u(int need) {
  static const int us[] = {1, 2, 3, 4, 6, 8};
  for (int u : us)
    if (u >= need) return u;
  return 0;
}

template <bool SPLIT>
hipError_t launch_gu(int U, dim3 grid, size_t lds, hipStream_t st, const I3MoeArgs& a) {
  switch (U) {
    case 1: hipLaunchKernelGGL((moe_i3_gate_up_kernel<SPLIT, 1>), grid, dim3(kGuThreads), lds, st, a); break;
    case 2: hipLaunchKernelGGL((moe_i3_gate_up_kernel<SPLIT, 2>), grid, dim3(kGuThreads), lds, st, a); break;
    case 3: hipLaunchKernelGGL((moe_i3_gate_up_kernel<SPLIT, 3>), grid, dim3(kGuThreads), lds, st, a); break;
    case 4: hipLaunchKernelGGL((moe_i3_gate_up_kernel<SPLIT, 4>), grid, dim3(kGuThreads), lds, st, a); break;
    case 6: hipLaunchKernelGGL((moe_i3_gate_up_kernel<SPLIT, 6>), grid, dim3(kGuThreads), lds, st, a); break;
    case 8: hipLaunchKernelGGL((moe_i3_gate_up_kernel<SPLIT, 8>), grid, dim3(kGuThreads), lds, st, a); break;
    default: return hipErrorNotSupported;
  }
  return hipGetLastError();
}

hipError_t launch_dn(int U, dim3 grid, size_t lds, hipStream_t st, const I3MoeArgs& a) {
  switch (U) {
    case 1: hipLaunchKernelGGL(moe_i3_down_kernel<1>, grid, dim3(kDnThreads), lds, st, a); break;
    case 2: hipLaunchKernelGGL(moe_i3_down_kernel<2>, grid, dim3(kDnThreads), lds, st, a); break;
    case 3: hipLaunchKernelGGL(moe_i3_down_kernel<3>, grid, dim3(kDnThreads), lds, st, a); break;
    case 4: hipLaunchKernelGGL(moe_i3_down_kernel<4>, grid, dim3(kDnThreads), lds, st, a); break;
    case 6: hipLaunchKernelGGL(moe_i3_down_kernel<6>, grid, dim3(kDnThreads), lds, st, a); break;
    case 8: hipLaunchKernelGGL(moe_i3_down_kernel<8>, grid, dim3(kDnThreads), lds, st, a); break;
    default: return hipErrorNotSupported;
  }
  return hipGetLastError();
}

constexpr int kMaxGridY = 65535;  // tokens per launch

int cus_or_default() {
  int c = 0;
  return device_cus(&c) == hipSuccess && c > 0 ? c : 256;
}

}  // namespace

bool moe_i3_supported(int topk, const ExpertArgs& e) {
  if (e.H < 32 || e.I < 32 || e.H > kI3KMax || e.I > kI3KMax || e.H % 32 || e.I % 32) return false;
  if (topk < 1 || topk > kTopkMax) return false;
  if (!pick_u((2 * e.G_h + 63) / 64)) return false;
  return pick_u((topk * e.G_i + 63) / 64) && i3_lds_bytes(topk * e.G_i, true) <= kDnLdsMax;
}

size_t moe_i3_ws_bytes(int T, int topk, const ExpertArgs& e) { return (size_t)T * topk * e.I * sizeof(float); }

hipError_t launch_moe_i3_gate_up(int xdt, const ExpertArgs& e, const void* x, const int32_t* ids, int T, int topk,
                                 float* h, hipStream_t st) {
  if (!moe_i3_supported(topk, e)) return hipErrorNotSupported;
  const int U = pick_u((2 * e.G_h + 63) / 64);
  const bool split = xdt == kF32;
  const size_t lds = i3_lds_bytes(e.G_h, split);
  // about eight workgroups per compute unit in all, at least two tasks per wave
  const int tasks = topk * e.I;
  const int cus = cus_or_default();
  for (int t0 = 0; t0 < T; t0 += kMaxGridY) {
    const int nt = T - t0 < kMaxGridY ? T - t0 : kMaxGridY;
    int bx = (8 * cus + nt - 1) / nt;
    const int most = (tasks + 2 * (kGuThreads / 64) - 1) / (2 * (kGuThreads / 64));
    if (bx > most) bx = most;
    if (bx < 1) bx = 1;
    I3MoeArgs a{};
    a.ex = e;
    a.x = static_cast<const char*>(x) + (size_t)t0 * e.H * (split ? 4 : 2);
    a.bf16x = split ? 0 : 1;
    a.ids = ids + (size_t)t0 * topk;
    a.h = h + (size_t)t0 * topk * e.I;
    a.topk = topk;
    const hipError_t err = split ? launch_gu<true>(U, dim3(bx, nt), lds, st, a)
                                 : launch_gu<false>(U, dim3(bx, nt), lds, st, a);
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

hipError_t launch_moe_i3_down(const ExpertArgs& e, const float* h, const int32_t* ids, const float* w, int T,
                              int topk, float* y, hipStream_t st) {
  if (!moe_i3_supported(topk, e)) return hipErrorNotSupported;
  const int U = pick_u((topk * e.G_i + 63) / 64);
  const size_t lds = i3_lds_bytes(topk * e.G_i, true);
  // about one workgroup per compute unit in all (each stages its token's
  // hidden vectors), at least two rows per wave
  const int cus = cus_or_default();
  for (int t0 = 0; t0 < T; t0 += kMaxGridY) {
    const int nt = T - t0 < kMaxGridY ? T - t0 : kMaxGridY;
    int bx = (cus + nt - 1) / nt;
    const int most = (e.H + 2 * (kDnThreads / 64) - 1) / (2 * (kDnThreads / 64));
    if (bx > most) bx = most;
    if (bx < 1) bx = 1;
    I3MoeArgs a{};
    a.ex = e;
    a.ids = ids + (size_t)t0 * topk;
    a.w = w + (size_t)t0 * topk;
    a.h = const_cast<float*>(h) + (size_t)t0 * topk * e.I;
    a.y = y + (size_t)t0 * e.H;
    a.topk = topk;
    const hipError_t err = launch_dn(U, dim3(bx, nt), lds, st, a);
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

}  // namespace qm
