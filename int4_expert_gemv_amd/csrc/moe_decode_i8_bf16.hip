// moe_decode_i8_bf16.hip -- instantiations of the MoE decode kernels for one (format,
// activation type) pair.
#include "moe_t1_lds.hpp"

namespace qm {

hipError_t moe_gate_up_i8_bf16_r(const MoeDecodeArgs& a, hipStream_t st) {
  return stage_gate_up_any<kFmtInt8, kBF16, false>(a, st);
}

hipError_t moe_down_i8_r(const MoeDecodeArgs& a, hipStream_t st) {
  return stage_down_any<kFmtInt8, false>(a, st);
}

}  // namespace qm
