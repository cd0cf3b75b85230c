// qgemv.hip -- quantized GEMV / small-batch GEMV kernels (gfx950).
//
// Computes Y[t][r] = sum_c W[r][c] X[t][c] for the int4 (grouped or per-row)
// and int8 per-row formats, as the dense quantized GEMV with an S-token batch
// of the colibri page "Vulkan backend: expert tier + dense + MLA attention on
// any Vulkan 1.2 GPU" (commit notes "backend_vulkan.c/.h +
// shaders/qmatmul.comp" and "fmt=4 grouped scales").  The weight matrix is
// read from HBM exactly once per call whatever the batch.
#include "device.hpp"
#include "launch.hpp"

namespace qm {

__global__ void fill_zero_kernel(float* y, int64_t n, int64_t ld, int rows) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n * rows; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / n, c = i - r * n;
    y[r * ld + c] = 0.f;
  }
}

int lanes_per_row(int kchunks) {
  if (kchunks >= 64) return 64;
  if (kchunks >= 32) return 32;
  if (kchunks >= 16) return 16;
  return 8;
}

int rows_per_unit(int L, int NB) {
  const int RU = NB == 1 ? 4 : (NB <= 4 ? 2 : 1);
  return (64 / L) * RU;
}

int seg_chunks(int fmt, int xdt, int NB, int kchunks) {
  const bool split = fmt == kFmtInt4 && xdt == kF32;
  const int per = fmt == kFmtInt4 ? (split ? stage_bytes_per_chunk<kFmtInt4, true>()
                                           : stage_bytes_per_chunk<kFmtInt4, false>())
                                  : stage_bytes_per_chunk<kFmtInt8, false>();
  int segc = kLdsBudget / (NB * per);
  return segc < kchunks ? segc : kchunks;
}

size_t stage_bytes(int fmt, int xdt, int NB, int segc) {
  const bool split = fmt == kFmtInt4 && xdt == kF32;
  const int per = fmt == kFmtInt4 ? (split ? stage_bytes_per_chunk<kFmtInt4, true>()
                                           : stage_bytes_per_chunk<kFmtInt4, false>())
                                  : stage_bytes_per_chunk<kFmtInt8, false>();
  return (size_t)NB * segc * per;
}

hipError_t launch_qgemv(int fmt, int xdt, bool grouped, const GemvArgs& a0, int NB, hipStream_t st) {
  GemvArgs a = a0;
  const int kchunks = a.k / (fmt == kFmtInt4 ? 32 : 16);
  const int L = lanes_per_row(kchunks);
  a.segc = seg_chunks(fmt, xdt, NB, kchunks);
  const int tiles = (a.n + rows_per_unit(L, NB) - 1) / rows_per_unit(L, NB);
  if (a.rounds < 1) a.rounds = 1;
  const int blocks = (tiles + kWaves * a.rounds - 1) / (kWaves * a.rounds);
  const size_t lds = stage_bytes(fmt, xdt, NB, a.segc);
  if (fmt == kFmtInt4) {
    if (xdt == kBF16)
      return grouped ? qgemv_launch_i4_bf16_g(a, L, NB, blocks, lds, st)
                     : qgemv_launch_i4_bf16_r(a, L, NB, blocks, lds, st);
    return grouped ? qgemv_launch_i4_f32_g(a, L, NB, blocks, lds, st)
                   : qgemv_launch_i4_f32_r(a, L, NB, blocks, lds, st);
  }
  return xdt == kBF16 ? qgemv_launch_i8_bf16_r(a, L, NB, blocks, lds, st)
                      : qgemv_launch_i8_f32_r(a, L, NB, blocks, lds, st);
}

hipError_t launch_fill_zero(float* y, int64_t n, int64_t ld, int rows, hipStream_t st) {
  const int64_t total = n * rows;
  int blocks = (int)((total + 255) / 256);
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(fill_zero_kernel, dim3(blocks), dim3(256), 0, st, y, n, ld, rows);
  return hipGetLastError();
}

}  // namespace qm
