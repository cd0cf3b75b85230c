// moe_prefill.hip -- expert-grouped batch-union FFN for many tokens (prefill).
#include "device.hpp"
#include "launch.hpp"

namespace qm {

size_t moe_prefill_workspace(int T, int topk, int E, int H, int I) {
  (void)T; (void)topk; (void)E; (void)H; (void)I;
  return 0;
}

hipError_t launch_moe_prefill(int fmt, int xdt, bool grouped, const ExpertArgs& ex, const void* x,
                              const int32_t* ids, const float* w, int T, int topk, float* y, void* ws,
                              hipStream_t st) {
  (void)fmt; (void)xdt; (void)grouped; (void)ex; (void)x; (void)ids; (void)w; (void)T; (void)topk; (void)y;
  (void)ws; (void)st;
  return hipErrorNotSupported;
}

}  // namespace qm
