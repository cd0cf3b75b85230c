// qgemv_i8_bf16.hip -- instantiations of the quantized GEMV kernel for one
// (format, activation type) pair.
#include "qgemv_impl.hpp"

namespace qm {

hipError_t qgemv_launch_i8_bf16_r(const GemvArgs& a, int L, int NB, int blocks, size_t lds, hipStream_t st) {
  return launch_g<kFmtInt8, kBF16, false>(a, L, NB, blocks, lds, st);
}

hipError_t qgemv_v2_i8_bf16_r(const GemvArgs& a, const GemvArgs& b, int na, int L, int CB, int blocks, size_t lds,
                  hipStream_t st) {
  return launch_v2<kFmtInt8, kBF16, false>(a, b, na, L, CB, blocks, lds, st);
}

}  // namespace qm
