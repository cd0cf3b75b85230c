// moe_decode_i4_bf16.hip -- instantiations of the MoE decode kernels for one (format,
// activation type) pair.
#include "moe_t1_s.hpp"

namespace qm {

hipError_t moe_gate_up_i4_bf16_g(const MoeDecodeArgs& a, hipStream_t st) {
  const hipError_t e = try_gate_up_t1q<kBF16, true>(a, st);
  if (e != hipErrorNotSupported) return e;
  return stage_gate_up_any<kFmtInt4, kBF16, true>(a, st);
}

hipError_t moe_down_i4_g(const MoeDecodeArgs& a, hipStream_t st) {
  const hipError_t e = try_down_t1q<true>(a, a.hq_ready != 0, st);
  if (e != hipErrorNotSupported) return e;
  return stage_down_any<kFmtInt4, true>(a, st);
}

hipError_t moe_gate_up_i4_bf16_r(const MoeDecodeArgs& a, hipStream_t st) {
  const hipError_t e = try_gate_up_t1q<kBF16, false>(a, st);
  if (e != hipErrorNotSupported) return e;
  return stage_gate_up_any<kFmtInt4, kBF16, false>(a, st);
}

hipError_t moe_down_i4_r(const MoeDecodeArgs& a, hipStream_t st) {
  const hipError_t e = try_down_t1q<false>(a, a.hq_ready != 0, st);
  if (e != hipErrorNotSupported) return e;
  return stage_down_any<kFmtInt4, false>(a, st);
}

hipError_t moe_ffn_i4_bf16_g(const MoeDecodeArgs& a, hipStream_t st) {
  return try_s_layer<kBF16, true>(a, st);
}

hipError_t moe_ffn_i4_bf16_r(const MoeDecodeArgs& a, hipStream_t st) {
  return try_s_layer<kBF16, false>(a, st);
}

}  // namespace qm
