// qgemv_i3.hip -- GEMV for the int3-g64 two-plane format (fmt 5); the format,
// its decode and the activation staging are in int3.hpp.
//
// Work mapping: L lanes per row (a power of two up to 64, chosen from the
// group count), lanes stride over the row's 24-byte groups (consecutive
// lanes read consecutive groups; a lane's groups, at most four, are all
// loaded before any is decoded), 64 / L rows per wave, rows grid-strided.
// x for the whole row length lives in LDS (k <= 16384), one staged unit per
// group.
#include "int3.hpp"
#include "launch.hpp"

namespace qm {

namespace {

constexpr int kI3Threads = 256;
constexpr int kI3GplMax = 4;  // groups per lane: G <= 256 and L = 64 once G >= 64

template <bool SPLIT>
__global__ __launch_bounds__(kI3Threads) void stage_and_gemv_i3(const uint8_t* __restrict__ q,
                                                                 const float* __restrict__ sc, const void* x,
                                                                 float* __restrict__ y, int n, int k, int G, int L,
                                                                 int bf16x) {
  extern __shared__ __attribute__((aligned(16))) uint32_t xs[];
  const I3Lds X = i3_carve(xs, G, SPLIT);
  const int tid = threadIdx.x;
  i3_stage<SPLIT>(X, G, k, bf16x != 0, [&](int) { return x; }, tid, kI3Threads);
  __syncthreads();
  i3_corr(X, tid, kI3Threads);
  __syncthreads();

  const int wave = tid >> 6, lane = tid & 63;
  const int li = lane & (L - 1), rsub = lane / L, rpw = 64 / L;
  const int64_t rb = (int64_t)G * 24;
  const int rstride = gridDim.x * (kI3Threads / 64) * rpw;
  // A lane's groups of one row, loaded as one unit: the next row's unit is
  // in flight while the current one is decoded.
  struct Unit {
    I3Group w[kI3GplMax];
    float s[kI3GplMax];
  };
  auto load = [&](int r0, Unit& u) {
    const int r = r0 + rsub;
    const bool ok = r0 < n && r < n;
    const uint8_t* row = q + (int64_t)(ok ? r : 0) * rb;
    const float* srow = sc + (int64_t)(ok ? r : 0) * G;
#pragma unroll
    for (int i = 0; i < kI3GplMax; ++i) {
      const int g = li + L * i;
      const int gg = g < G ? g : 0;
      u.w[i] = i3_load(row + (int64_t)gg * 24);
      u.s[i] = g < G ? srow[gg] : 0.f;
    }
  };
  Unit cur, nxt;
  int r0 = (blockIdx.x * (kI3Threads / 64) + wave) * rpw;
  if (r0 < n) load(r0, cur);
  for (; r0 < n; r0 += rstride) {
    if (r0 + rstride < n) load(r0 + rstride, nxt);
    const int r = r0 + rsub;
    const bool ok = r < n;
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < kI3GplMax; ++i) {
      const int g = li + L * i;
      if (g >= G) break;
      acc = __builtin_fmaf(cur.s[i], i3_group_dot<SPLIT>(cur.w[i], X, g), acc);
    }
    switch (L) {  // sum over the row's L lanes
      case 4: acc = group_sum<4>(acc); break;
      case 8: acc = group_sum<8>(acc); break;
      case 16: acc = group_sum<16>(acc); break;
      case 32: acc = group_sum<32>(acc); break;
      default: acc = group_sum<64>(acc); break;
    }
    if (ok && li == 0) y[r] = acc;
    cur = nxt;
  }
}

}  // namespace

size_t qgemv_i3_lds(int k, int xdt) { return i3_lds_bytes((k + 63) / 64, xdt == kF32); }

hipError_t launch_qgemv_i3(const uint8_t* q, const float* sc, const void* x, int xdt, float* y, int n, int k,
                           hipStream_t st) {
  const int G = (k + 63) / 64;
  int L = 4;
  while (L < 64 && 2 * L <= G) L *= 2;
  const int rows_per_block = (kI3Threads / 64) * (64 / L);
  int blocks = (n + rows_per_block - 1) / rows_per_block;
  if (blocks > 1024) blocks = 1024;
  const size_t lds = qgemv_i3_lds(k, xdt);
  if (xdt == kF32)
    hipLaunchKernelGGL(stage_and_gemv_i3<true>, dim3(blocks), dim3(kI3Threads), lds, st, q, sc, x, y, n, k, G, L, 0);
  else
    hipLaunchKernelGGL(stage_and_gemv_i3<false>, dim3(blocks), dim3(kI3Threads), lds, st, q, sc, x, y, n, k, G, L, 1);
  return hipGetLastError();
}

}  // namespace qm
