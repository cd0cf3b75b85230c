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

int v2_cb(int kchunks, int L) {
  const int c = (kchunks + L - 1) / L;
  return c <= 4 ? c : 8;
}

int v2_blocks(int ntiles, int max_blocks) {
  int b = (ntiles + kWaves - 1) / kWaves;
  const int cap = max_blocks > 0 ? max_blocks : kV2MaxBlocks;
  return b < cap ? b : cap;
}

hipError_t launch_qgemv(int fmt, int xdt, bool grouped, const GemvArgs& a0, int NB, hipStream_t st) {
  GemvArgs a = a0;
  const int kchunks = a.k / (fmt == kFmtInt4 ? 32 : 16);
  const int L = lanes_per_row(kchunks);
  // pipelined path: one bf16 token, whole x in LDS, at least 16 lanes per row
  if (NB == 1 && xdt == kBF16 && L >= 16 && stage_bytes(fmt, xdt, 1, kchunks) <= (size_t)kLdsBudget) {
    const int CB = v2_cb(kchunks, L);
    const int M = 1;
    const int RU = 8 / (M * CB) >= 8 ? 8 : (8 / (M * CB) >= 4 ? 4 : (8 / (M * CB) >= 2 ? 2 : 1));
    const int tile_rows = (64 / L) * RU;
    const int ntiles = (a.n + tile_rows - 1) / tile_rows;
    const int blocks = v2_blocks(ntiles, a.max_blocks);
    const size_t lds = stage_bytes(fmt, xdt, 1, kchunks);
    a.segc = kchunks;
    if (fmt == kFmtInt4)
      return grouped ? qgemv_v2_i4_bf16_g(a, a, blocks, L, CB, blocks, lds, st)
                     : qgemv_v2_i4_bf16_r(a, a, blocks, L, CB, blocks, lds, st);
    return qgemv_v2_i8_bf16_r(a, a, blocks, L, CB, blocks, lds, st);
  }
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

hipError_t launch_qgemv_pair(int fmt, int xdt, bool grouped, const GemvArgs& a0, const GemvArgs& b0, hipStream_t st) {
  GemvArgs a = a0, b = b0;
  if (fmt != kFmtInt4 && fmt != kFmtInt8) return hipErrorNotSupported;
  const int kchunks = a.k / (fmt == kFmtInt4 ? 32 : 16);
  const int L = lanes_per_row(kchunks);
  if (xdt != kBF16 || L < 16 || a.k != b.k || stage_bytes(fmt, xdt, 1, kchunks) > (size_t)kLdsBudget)
    return hipErrorNotSupported;
  const int CB = v2_cb(kchunks, L);
  const int RU = 8 / CB >= 8 ? 8 : (8 / CB >= 4 ? 4 : (8 / CB >= 2 ? 2 : 1));
  const int tile_rows = (64 / L) * RU;
  const int na = v2_blocks((a.n + tile_rows - 1) / tile_rows, a.max_blocks);
  const int nb = v2_blocks((b.n + tile_rows - 1) / tile_rows, b.max_blocks);
  const size_t lds = stage_bytes(fmt, xdt, 1, kchunks);
  a.segc = b.segc = kchunks;
  if (fmt == kFmtInt4)
    return grouped ? qgemv_v2_i4_bf16_g(a, b, na, L, CB, na + nb, lds, st)
                   : qgemv_v2_i4_bf16_r(a, b, na, L, CB, na + nb, lds, st);
  return qgemv_v2_i8_bf16_r(a, b, na, L, CB, na + nb, lds, st);
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
