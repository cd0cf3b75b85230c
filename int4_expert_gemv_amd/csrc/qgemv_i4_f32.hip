// qgemv_i4_f32.hip -- instantiations of the quantized GEMV kernel for one
// (format, activation type) pair.
#include "qgemv_impl.hpp"

namespace qm {

hipError_t qgemv_launch_i4_f32_g(const GemvArgs& a, int L, int NB, int blocks, size_t lds, hipStream_t st) {
  return launch_g<kFmtInt4, kF32, true>(a, L, NB, blocks, lds, st);
}

hipError_t qgemv_launch_i4_f32_r(const GemvArgs& a, int L, int NB, int blocks, size_t lds, hipStream_t st) {
  return launch_g<kFmtInt4, kF32, false>(a, L, NB, blocks, lds, st);
}

}  // namespace qm
