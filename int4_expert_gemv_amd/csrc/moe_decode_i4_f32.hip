// moe_decode_i4_f32.hip -- instantiations of the MoE decode kernels for one (format,
// activation type) pair.
#include "moe_t1_s.hpp"

namespace qm {

hipError_t moe_gate_up_i4_f32_g(const MoeDecodeArgs& a, hipStream_t st) {
  const hipError_t e = try_gate_up_t1q<kF32, true>(a, st);
  if (e != hipErrorNotSupported) return e;
  return stage_gate_up_any<kFmtInt4, kF32, true>(a, st);
}

hipError_t moe_gate_up_i4_f32_r(const MoeDecodeArgs& a, hipStream_t st) {
  const hipError_t e = try_gate_up_t1q<kF32, false>(a, st);
  if (e != hipErrorNotSupported) return e;
  return stage_gate_up_any<kFmtInt4, kF32, false>(a, st);
}

hipError_t moe_ffn_i4_f32_g(const MoeDecodeArgs& a, hipStream_t st) {
  return try_s_layer<kF32, true>(a, st);
}

hipError_t moe_ffn_i4_f32_r(const MoeDecodeArgs& a, hipStream_t st) {
  return try_s_layer<kF32, false>(a, st);
}

}  // namespace qm
