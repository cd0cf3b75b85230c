// qchain.hip -- the RMS normalisation step of the q-prep chain.
//
// The colibri page "Vulkan backend: expert tier + dense + MLA attention on
// any Vulkan 1.2 GPU" (q-prep chain commit note) moves the q-latent norm
// between the q_a and q_b projections onto the GPU so that the chain
// [q_a + kv_a] -> norm -> q_b runs without a return to the host.  Here the
// chain is three launches on one stream (qgemv_pair, this kernel, qgemv);
// this kernel normalises the latent in place:
//   u[i] <- u[i] / sqrt(mean_j u[j]^2 + eps) * g[i]   (g == nullptr: ones).
// One workgroup: the sum of squares is reduced in a fixed order (per-thread
// strided partials, DPP within each wave, waves in index order), so the
// result is the same on every run.
#include "device.hpp"
#include "launch.hpp"

namespace qm {

namespace {

constexpr int kNormThreads = 1024;

__global__ __launch_bounds__(kNormThreads) void rmsnorm_kernel(float* __restrict__ u, const float* __restrict__ g,
                                                               int n, float eps) {
  __shared__ float part[kNormThreads / 64];
  __shared__ float s_r;
  const int tid = threadIdx.x;
  float ss = 0.f;
  for (int i = tid; i < n; i += kNormThreads) ss = __builtin_fmaf(u[i], u[i], ss);
  ss = group_sum<64>(ss);
  if ((tid & 63) == 0) part[tid >> 6] = ss;
  __syncthreads();
  if (tid == 0) {
    float t = 0.f;
    for (int w = 0; w < kNormThreads / 64; ++w) t += part[w];
    s_r = 1.0f / __builtin_sqrtf(t / (float)n + eps);
  }
  __syncthreads();
  const float r = s_r;
  for (int i = tid; i < n; i += kNormThreads) u[i] = u[i] * r * (g ? g[i] : 1.0f);
}

}  // namespace

hipError_t launch_rmsnorm(float* u, const float* g, int n, float eps, hipStream_t st) {
  hipLaunchKernelGGL(rmsnorm_kernel, dim3(1), dim3(kNormThreads), 0, st, u, g, n, eps);
  return hipGetLastError();
}

}  // namespace qm
