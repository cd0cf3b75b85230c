// moe_decode.hip -- dispatch of the routed expert FFN decode stages (the
// kernels themselves are in moe_decode_impl.hpp, instantiated per format and
// activation type in moe_decode_*.hip).
#include "launch.hpp"
#include "moe_t1_q.hpp"

namespace qm {

hipError_t launch_moe_gate_up(int fmt, int xdt, bool grouped, const MoeDecodeArgs& a, hipStream_t st) {
  if (fmt == 4) {
    if (xdt == 1) return grouped ? moe_gate_up_i4_bf16_g(a, st) : moe_gate_up_i4_bf16_r(a, st);
    return grouped ? moe_gate_up_i4_f32_g(a, st) : moe_gate_up_i4_f32_r(a, st);
  }
  return xdt == 1 ? moe_gate_up_i8_bf16_r(a, st) : moe_gate_up_i8_f32_r(a, st);
}

hipError_t launch_moe_down(int fmt, bool grouped, const MoeDecodeArgs& a, hipStream_t st) {
  if (fmt == 4) return grouped ? moe_down_i4_g(a, st) : moe_down_i4_r(a, st);
  return moe_down_i8_r(a, st);
}

hipError_t launch_moe_ffn_layer(int fmt, int xdt, bool grouped, const MoeDecodeArgs& a, hipStream_t st) {
  if (fmt != 4) return hipErrorNotSupported;
  if (xdt == 1) return grouped ? moe_ffn_i4_bf16_g(a, st) : moe_ffn_i4_bf16_r(a, st);
  return grouped ? moe_ffn_i4_f32_g(a, st) : moe_ffn_i4_f32_r(a, st);
}

bool moe_gate_up_writes_digits(int fmt, const MoeDecodeArgs& a) {
  return fmt == 4 && a.hq != nullptr && q_gate_up_ok(a);
}

}  // namespace qm
