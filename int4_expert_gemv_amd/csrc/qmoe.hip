// qmoe.hip -- the C ABI of libqmoe.so (declared in include/qmoe.h).
//
// Every entry point validates its arguments on the host before the first HIP
// call; a rejected call enqueues nothing and writes nothing (the colibri page
// "qwen36: Vulkan expert tier, and staged device-local uploads" keeps the
// caller's output untouched when the GPU path refuses a request).
#include "qmoe.h"
#include <atomic>
#include <chrono>
#include <mutex>

#include "launch.hpp"

#include <limits.h>

// Scratch of the allocation-free entry point: a fixed device array, one copy
// per GPU.  In host code `scratch` names a host-side stand-in, never the
// device memory; its device address is looked up per device (with that
// device current) and only that address is handed to kernels.
static __device__ __align__(256) char scratch[QM_NOALLOC_SCRATCH_BYTES];

namespace {

using namespace qm;

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

int ilog2(int v) {
  int r = 0;
  while ((1 << r) < v) ++r;
  return (1 << r) == v ? r : -1;
}

// Effective group size: 0 means one scale per row.
int eff_gs(int fmt, int gs, int k) {
  if (fmt == QM_FMT_INT3) return 64;
  return (fmt == QM_FMT_INT4 && gs > 0 && gs < k) ? gs : 0;
}

// Shape checks for one n x k matrix in (fmt, gs).  Returns a qm_status.
int check_shape(int fmt, int n, int k, int gs) {
  if (fmt != QM_FMT_INT4 && fmt != QM_FMT_INT8_ROW && fmt != QM_FMT_INT3) return QM_ERR_INVALID;
  if (fmt == QM_FMT_INT3) {  // int3-g64: group size 64 only
    if (n < 0 || k < 0 || gs != 64) return QM_ERR_INVALID;
    if (k == 0 || k > kI3KMax || k % 32) return QM_ERR_UNSUPPORTED;
    return QM_OK;
  }
  if (n < 0 || k < 0 || gs < 0) return QM_ERR_INVALID;
  if (fmt == QM_FMT_INT4 && (k & 1)) return QM_ERR_INVALID;
  if (fmt == QM_FMT_INT8_ROW && gs != 0) return QM_ERR_INVALID;
  if (k == 0 || k > QM_K_MAX) return QM_ERR_UNSUPPORTED;
  if (fmt == QM_FMT_INT4 && k % 32) return QM_ERR_UNSUPPORTED;
  if (fmt == QM_FMT_INT8_ROW && k % 16) return QM_ERR_UNSUPPORTED;
  const int g = eff_gs(fmt, gs, k);
  if (g) {
    if (g % 32 || k % g || ilog2(g / 32) < 0) return QM_ERR_UNSUPPORTED;
  } else if (fmt == QM_FMT_INT4 && gs > k) {
    return QM_ERR_UNSUPPORTED;
  }
  return QM_OK;
}

int64_t row_bytes(int fmt, int k) {
  if (fmt == QM_FMT_INT3) return ((int64_t)k + 63) / 64 * 24;
  return fmt == QM_FMT_INT4 ? (int64_t)k / 2 : (int64_t)k;
}

int groups(int fmt, int gs, int k) {
  if (fmt == QM_FMT_INT3) return (k + 63) / 64;
  const int g = eff_gs(fmt, gs, k);
  return g ? k / g : 1;
}

int xsize(int dt) { return dt == QM_BF16 ? 2 : 4; }

int check_gemm(const qm_qmat* w, const void* x, int32_t xdt, int32_t batch, int64_t ldx, const float* y,
               int64_t ldy) {
  if (!w) return QM_ERR_INVALID;
  if (xdt != QM_F32 && xdt != QM_BF16) return QM_ERR_INVALID;
  if (batch < 1) return QM_ERR_INVALID;
  int st = check_shape(w->fmt, w->n, w->k, w->group_size);
  if (st == QM_ERR_INVALID) return st;
  if (w->n == 0) return QM_OK;  // nothing to compute (pointers may be null)
  if (!w->q || !w->scales || !x || !y) return QM_ERR_INVALID;
  if (ldx < w->k || ldy < w->n) return QM_ERR_INVALID;
  if (st != QM_OK) return st;
  if (batch > QM_SMALL_MAX) return QM_ERR_UNSUPPORTED;
  if (!aligned(w->q, 16) || !aligned(x, 16) || !aligned(w->scales, 4) || !aligned(y, 4))
    return QM_ERR_UNSUPPORTED;
  if ((ldx * xsize(xdt)) % 16) return QM_ERR_UNSUPPORTED;
  return QM_OK;
}

GemvArgs gemv_args(const qm_qmat* w, const void* x, int32_t batch, int64_t ldx, float* y, int64_t ldy) {
  const int g = eff_gs(w->fmt, w->group_size, w->k);
  GemvArgs a{};
  a.q = static_cast<const uint8_t*>(w->q);
  a.s = w->scales;
  a.x = x;
  a.y = y;
  a.n = w->n;
  a.k = w->k;
  a.G = groups(w->fmt, w->group_size, w->k);
  a.gshift = g ? ilog2(g / 32) : 0;
  a.row_bytes = row_bytes(w->fmt, w->k);
  a.ldx = ldx;
  a.ldy = ldy;
  a.nb = batch;
  a.rounds = 1;
  return a;
}

int run_gemm(const qm_qmat* w, const void* x, int32_t xdt, int32_t batch, int64_t ldx, float* y, int64_t ldy,
             void* stream) {
  int st = check_gemm(w, x, xdt, batch, ldx, y, ldy);
  if (st != QM_OK || w->n == 0) return st;
  const GemvArgs a = gemv_args(w, x, batch, ldx, y, ldy);
  const hipError_t err = launch_gemv_planes(w->fmt, xdt, eff_gs(w->fmt, w->group_size, w->k) != 0, a, nullptr,
                                            static_cast<hipStream_t>(stream));
  if (err == hipErrorNotSupported) return QM_ERR_UNSUPPORTED;
  return err == hipSuccess ? QM_OK : QM_ERR_LAUNCH;
}

// ---- MoE -------------------------------------------------------------------------

// Shapes, format and group size only (no pointers).
bool moe_shape_ok(const qm_experts* ex) {
  if (ex->n_experts < 1 || ex->hidden < 1 || ex->inter < 1) return false;
  if (check_shape(ex->fmt, ex->inter, ex->hidden, ex->group_size) != QM_OK) return false;
  if (check_shape(ex->fmt, ex->hidden, ex->inter, ex->group_size) != QM_OK) return false;
  const int gh = eff_gs(ex->fmt, ex->group_size, ex->hidden);
  const int gi = eff_gs(ex->fmt, ex->group_size, ex->inter);
  return (gh == 0) == (gi == 0);
}
int check_experts(const qm_experts* ex) {
  if (!ex) return QM_ERR_INVALID;
  if (ex->n_experts < 1 || ex->hidden < 0 || ex->inter < 0) return QM_ERR_INVALID;
  int a = check_shape(ex->fmt, ex->inter, ex->hidden, ex->group_size);
  int b = check_shape(ex->fmt, ex->hidden, ex->inter, ex->group_size);
  if (a == QM_ERR_INVALID || b == QM_ERR_INVALID) return QM_ERR_INVALID;
  if (!ex->gate_q || !ex->up_q || !ex->down_q || !ex->gate_s || !ex->up_s || !ex->down_s) return QM_ERR_INVALID;
  if (a != QM_OK) return a;
  if (b != QM_OK) return b;
  if (ex->hidden < 1 || ex->inter < 1) return QM_ERR_UNSUPPORTED;
  const void* q[3] = {ex->gate_q, ex->up_q, ex->down_q};
  const void* s[3] = {ex->gate_s, ex->up_s, ex->down_s};
  for (int i = 0; i < 3; ++i)
    if (!aligned(q[i], 16) || !aligned(s[i], 4)) return QM_ERR_UNSUPPORTED;
  return QM_OK;
}

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

ExpertArgs expert_args(const qm_experts* ex) {
  ExpertArgs e{};
  e.gq = static_cast<const uint8_t*>(ex->gate_q);
  e.uq = static_cast<const uint8_t*>(ex->up_q);
  e.dq = static_cast<const uint8_t*>(ex->down_q);
  e.gs = ex->gate_s;
  e.us = ex->up_s;
  e.ds = ex->down_s;
  e.E = ex->n_experts;
  e.H = ex->hidden;
  e.I = ex->inter;
  e.G_h = groups(ex->fmt, ex->group_size, ex->hidden);
  e.G_i = groups(ex->fmt, ex->group_size, ex->inter);
  const int g = eff_gs(ex->fmt, ex->group_size, ex->hidden);
  e.gshift = g ? ilog2(g / 32) : 0;
  e.rb_h = row_bytes(ex->fmt, ex->hidden);
  e.rb_i = row_bytes(ex->fmt, ex->inter);
  return e;
}

// Decode pass arguments for tokens [t0, t0 + nt) of a call.
MoeDecArgs dec_args(const ExpertArgs& e, const void* x, int xdt, int t0, int nt, const int32_t* ids, const float* w,
                    int k, float* h, float* y, void* ws) {
  MoeDecArgs a{};
  a.ex = e;
  a.x = x ? static_cast<const char*>(x) + (size_t)t0 * e.H * xsize(xdt) : nullptr;
  a.ids = ids + (size_t)t0 * k;
  a.w = w ? w + (size_t)t0 * k : nullptr;
  a.h = h ? h + (size_t)t0 * k * e.I : nullptr;
  a.y = y ? y + (size_t)t0 * e.H : nullptr;
  a.T = nt;
  a.topk = k;
  if (ws) moe_decode_ws_split(a, ws);
  return a;
}

// tokens per decode pass for these experts (0: the decode kernels do not take them)
int dec_tokens(const qm_experts* ex, int top_k) {
  const ExpertArgs e = expert_args(ex);
  const int t = moe_decode_tokens_per_pass(ex->fmt, top_k, e);
  return (t >= 1 && moe_decode_supported(ex->fmt, t, top_k, e)) ? t : 0;
}

// grouped iff both projections' reduction lengths are split into groups
int moe_grouping(const qm_experts* ex, bool* grouped) {
  const int gh = eff_gs(ex->fmt, ex->group_size, ex->hidden);
  const int gi = eff_gs(ex->fmt, ex->group_size, ex->inter);
  if ((gh == 0) != (gi == 0)) return QM_ERR_UNSUPPORTED;  // grouped along one reduction only
  *grouped = gh != 0;
  return QM_OK;
}

constexpr int kMaxDevices = 64;

// Device address of `scratch` on the current device, looked up on the first
// call made with that device current; nullptr if HIP cannot give it.
void* scratch_ptr() {
  static std::atomic<void*> ptrs[kMaxDevices];
  static std::mutex mu;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = ptrs[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(mu);
  p = ptrs[dev].load(std::memory_order_relaxed);
  if (!p) {
    void* a = nullptr;
    if (hipGetSymbolAddress(&a, HIP_SYMBOL(scratch)) != hipSuccess || !a) return nullptr;
    ptrs[dev].store(a, std::memory_order_release);
    p = a;
  }
  return p;
}

}  // namespace

extern "C" {

const char* qm_strerror(int status) {
  switch (status) {
    case QM_OK: return "ok";
    case QM_ERR_INVALID: return "invalid argument";
    case QM_ERR_UNSUPPORTED: return "unsupported shape, format or alignment for the GPU path";
    case QM_ERR_WORKSPACE: return "workspace missing or too small";
    case QM_ERR_LAUNCH: return "HIP kernel launch failed";
    case QM_ERR_TOO_LARGE: return "needs more scratch than the allocation-free entry point holds";
    default: return "unknown status";
  }
}

int qgemv(const qm_qmat* w, const void* x, int32_t x_dtype, float* y, void* stream) {
  return run_gemm(w, x, x_dtype, 1, w ? w->k : 0, y, w ? w->n : 0, stream);
}

int qgemv_pair(const qm_qmat* w1, const qm_qmat* w2, const void* x, int32_t x_dtype, float* y1, float* y2,
               void* stream) {
  if (!w1 || !w2) return QM_ERR_INVALID;
  if (w1->k != w2->k) return QM_ERR_INVALID;
  const int s1 = check_gemm(w1, x, x_dtype, 1, w1->k, y1, w1->n);
  const int s2 = check_gemm(w2, x, x_dtype, 1, w2->k, y2, w2->n);
  if (s1 != QM_OK) return s1;
  if (s2 != QM_OK) return s2;
  if (w1->n == 0 || w2->n == 0) {
    const int r = run_gemm(w1, x, x_dtype, 1, w1->k, y1, w1->n, stream);
    return r != QM_OK ? r : run_gemm(w2, x, x_dtype, 1, w2->k, y2, w2->n, stream);
  }
  const int g1 = eff_gs(w1->fmt, w1->group_size, w1->k), g2 = eff_gs(w2->fmt, w2->group_size, w2->k);
  if (w1->fmt == w2->fmt && (g1 != 0) == (g2 != 0)) {
    // one launch: x staged once per workgroup for both matrices
    const GemvArgs a1 = gemv_args(w1, x, 1, w1->k, y1, w1->n), a2 = gemv_args(w2, x, 1, w2->k, y2, w2->n);
    const hipError_t err = launch_gemv_planes(w1->fmt, x_dtype, g1 != 0, a1, &a2, static_cast<hipStream_t>(stream));
    if (err == hipSuccess) return QM_OK;
    if (err != hipErrorNotSupported) return QM_ERR_LAUNCH;
  }
  const int r = run_gemm(w1, x, x_dtype, 1, w1->k, y1, w1->n, stream);
  return r != QM_OK ? r : run_gemm(w2, x, x_dtype, 1, w2->k, y2, w2->n, stream);
}

int qgemv_norm_chain(const qm_qmat* w_a, const qm_qmat* w_kv, const float* norm_w, float eps, const qm_qmat* w_b,
                     const void* x, int32_t x_dtype, float* u, float* kv, float* q, void* stream) {
  if (!w_a || !w_kv || !w_b) return QM_ERR_INVALID;
  if (w_a->k != w_kv->k || w_b->k != w_a->n || w_a->n < 1 || !(eps >= 0.f)) return QM_ERR_INVALID;
  int st = check_gemm(w_a, x, x_dtype, 1, w_a->k, u, w_a->n);
  if (st == QM_OK) st = check_gemm(w_kv, x, x_dtype, 1, w_kv->k, kv, w_kv->n);
  if (st == QM_OK) st = check_gemm(w_b, u, QM_F32, 1, w_b->k, q, w_b->n);
  if (st != QM_OK) return st;
  st = qgemv_pair(w_a, w_kv, x, x_dtype, u, kv, stream);
  if (st != QM_OK) return st;
  if (launch_rmsnorm(u, norm_w, w_a->n, eps, static_cast<hipStream_t>(stream)) != hipSuccess) return QM_ERR_LAUNCH;
  return run_gemm(w_b, u, QM_F32, 1, w_b->k, q, w_b->n, stream);
}

int qgemm_small(const qm_qmat* w, const void* x, int32_t x_dtype, int32_t batch, int64_t ldx, float* y,
                int64_t ldy, void* stream) {
  return run_gemm(w, x, x_dtype, batch, ldx, y, ldy, stream);
}

size_t moe_expert_ffn_workspace(const qm_experts* ex, int32_t n_tokens, int32_t top_k) {
  if (!ex || n_tokens < 0 || top_k < 1 || top_k > QM_TOPK_MAX) return 0;
  if (ex->hidden < 1 || ex->inter < 1 || ex->n_experts < 1) return 0;
  size_t need = 0;
  if (moe_shape_ok(ex)) {
    const int tpp = dec_tokens(ex, top_k);
    if (tpp > 0) {
      const int td = n_tokens < tpp ? n_tokens : tpp;
      need = moe_decode_ws_bytes(td > 0 ? td : 1, top_k, ex->hidden, ex->inter);
    }
    const ExpertArgs e = expert_args(ex);
    if (moe_prefill_supported(ex->fmt, top_k, e)) {
      const size_t p = moe_prefill_workspace(n_tokens, top_k, e);
      if (p > need) need = p;
    }
  }
  return need < 256 ? 256 : need;
}
int moe_expert_ffn_path(const qm_experts* ex, const void* x, int32_t x_dtype, int32_t n_tokens,
                        const int32_t* topk_ids, const float* topk_w, int32_t top_k, float* y, void* workspace,
                        size_t workspace_bytes, void* stream, int32_t path) {
  if (path != QM_PATH_AUTO && path != QM_PATH_DECODE && path != QM_PATH_PREFILL) return QM_ERR_INVALID;
  if (x_dtype != QM_F32 && x_dtype != QM_BF16) return QM_ERR_INVALID;
  if (n_tokens < 0 || top_k < 1) return QM_ERR_INVALID;
  int st = check_experts(ex);
  if (st == QM_ERR_INVALID) return st;
  if (n_tokens == 0) return QM_OK;
  if (!x || !topk_ids || !topk_w || !y) return QM_ERR_INVALID;
  if (st != QM_OK) return st;
  if (top_k > QM_TOPK_MAX) return QM_ERR_UNSUPPORTED;
  if (!aligned(x, 16) || !aligned(y, 4) || !aligned(topk_ids, 4) || !aligned(topk_w, 4)) return QM_ERR_UNSUPPORTED;
  bool grouped = false;
  st = moe_grouping(ex, &grouped);
  if (st != QM_OK) return st;
  const bool pre_ok = moe_prefill_supported(ex->fmt, top_k, expert_args(ex));
  const int tpp = dec_tokens(ex, top_k);
  if (path == QM_PATH_AUTO)
    path = (n_tokens > QM_DECODE_MAX_TOKENS && pre_ok) || tpp == 0 ? QM_PATH_PREFILL : QM_PATH_DECODE;
  if (path == QM_PATH_PREFILL && !pre_ok) return QM_ERR_UNSUPPORTED;
  if (path == QM_PATH_DECODE && tpp == 0) return QM_ERR_UNSUPPORTED;
  if (!workspace || !aligned(workspace, 256) ||
      workspace_bytes < moe_expert_ffn_workspace(ex, n_tokens, top_k))
    return QM_ERR_WORKSPACE;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const ExpertArgs e = expert_args(ex);
  hipError_t err = hipSuccess;
  if (path == QM_PATH_PREFILL) {
    err = launch_moe_prefill(ex->fmt, x_dtype, e, x, topk_ids, topk_w, n_tokens, top_k, y, workspace, s);
  } else {
    // decode kernels, up to tpp tokens per pass (one pass for a decode batch
    // whose activations' digit planes fit the LDS)
    for (int t0 = 0; t0 < n_tokens && err == hipSuccess; t0 += tpp) {
      const int nt = n_tokens - t0 < tpp ? n_tokens - t0 : tpp;
      const MoeDecArgs a = dec_args(e, x, x_dtype, t0, nt, topk_ids, topk_w, top_k, nullptr, y, workspace);
      err = launch_moe_gate_up2(ex->fmt, x_dtype, grouped, a, s);
      if (err == hipSuccess) err = launch_moe_down2(ex->fmt, grouped, a, false, s);
    }
  }
  if (err == hipErrorNotSupported) return QM_ERR_UNSUPPORTED;
  return err == hipSuccess ? QM_OK : QM_ERR_LAUNCH;
}
int moe_gate_up(const qm_experts* ex, const void* x, int32_t x_dtype, int32_t n_tokens, const int32_t* topk_ids,
                int32_t top_k, float* h, void* workspace, size_t workspace_bytes, void* stream) {
  if (x_dtype != QM_F32 && x_dtype != QM_BF16) return QM_ERR_INVALID;
  if (n_tokens < 0 || top_k < 1) return QM_ERR_INVALID;
  int st = check_experts(ex);
  if (st == QM_ERR_INVALID) return st;
  if (n_tokens == 0) return QM_OK;
  if (!x || !topk_ids || !h) return QM_ERR_INVALID;
  if (st != QM_OK) return st;
  if (top_k > QM_TOPK_MAX) return QM_ERR_UNSUPPORTED;
  if (!aligned(x, 16) || !aligned(h, 4) || !aligned(topk_ids, 4)) return QM_ERR_UNSUPPORTED;
  bool grouped = false;
  st = moe_grouping(ex, &grouped);
  if (st != QM_OK) return st;
  const int tpp = dec_tokens(ex, top_k);
  if (tpp == 0) return QM_ERR_UNSUPPORTED;
  if (!workspace || !aligned(workspace, 256) || workspace_bytes < moe_expert_ffn_workspace(ex, n_tokens, top_k))
    return QM_ERR_WORKSPACE;
  // decode passes of up to tpp tokens, as moe_expert_ffn runs them
  hipError_t err = hipSuccess;
  for (int t0 = 0; t0 < n_tokens && err == hipSuccess; t0 += tpp) {
    const int nt = n_tokens - t0 < tpp ? n_tokens - t0 : tpp;
    MoeDecArgs a = dec_args(expert_args(ex), x, x_dtype, t0, nt, topk_ids, nullptr, top_k, h, nullptr, workspace);
    a.hrec = nullptr;  // h only: no records for a down pass
    err = launch_moe_gate_up2(ex->fmt, x_dtype, grouped, a, static_cast<hipStream_t>(stream));
  }
  if (err == hipErrorNotSupported) return QM_ERR_UNSUPPORTED;
  return err == hipSuccess ? QM_OK : QM_ERR_LAUNCH;
}

int moe_down(const qm_experts* ex, const float* h, int32_t n_tokens, const int32_t* topk_ids, const float* topk_w,
             int32_t top_k, float* y, void* workspace, size_t workspace_bytes, void* stream) {
  if (n_tokens < 0 || top_k < 1) return QM_ERR_INVALID;
  int st = check_experts(ex);
  if (st == QM_ERR_INVALID) return st;
  if (n_tokens == 0) return QM_OK;
  if (!h || !topk_ids || !topk_w || !y) return QM_ERR_INVALID;
  if (st != QM_OK) return st;
  if (top_k > QM_TOPK_MAX) return QM_ERR_UNSUPPORTED;
  if (!aligned(h, 16) || !aligned(y, 4) || !aligned(topk_ids, 4) || !aligned(topk_w, 4)) return QM_ERR_UNSUPPORTED;
  bool grouped = false;
  st = moe_grouping(ex, &grouped);
  if (st != QM_OK) return st;
  const int tpp = dec_tokens(ex, top_k);
  if (tpp == 0) return QM_ERR_UNSUPPORTED;
  if (!workspace || !aligned(workspace, 256) || workspace_bytes < moe_expert_ffn_workspace(ex, n_tokens, top_k))
    return QM_ERR_WORKSPACE;
  hipError_t err = hipSuccess;
  for (int t0 = 0; t0 < n_tokens && err == hipSuccess; t0 += tpp) {
    const int nt = n_tokens - t0 < tpp ? n_tokens - t0 : tpp;
    const MoeDecArgs a = dec_args(expert_args(ex), nullptr, QM_F32, t0, nt, topk_ids, topk_w, top_k,
                                  const_cast<float*>(h), y, workspace);
    err = launch_moe_down2(ex->fmt, grouped, a, true, static_cast<hipStream_t>(stream));
  }
  if (err == hipErrorNotSupported) return QM_ERR_UNSUPPORTED;
  return err == hipSuccess ? QM_OK : QM_ERR_LAUNCH;
}

int moe_expert_ffn(const qm_experts* ex, const void* x, int32_t x_dtype, int32_t n_tokens,
                   const int32_t* topk_ids, const float* topk_w, int32_t top_k, float* y, void* workspace,
                   size_t workspace_bytes, void* stream) {
  return moe_expert_ffn_path(ex, x, x_dtype, n_tokens, topk_ids, topk_w, top_k, y, workspace, workspace_bytes,
                             stream, QM_PATH_AUTO);
}

}  // extern "C"

extern "C" int moe_expert_ffn_noalloc(const qm_experts* ex, const void* x, int32_t x_dtype, int32_t n_tokens,
                                      const int32_t* topk_ids, const float* topk_w, int32_t top_k, float* y,
                                      void* stream) {
  // argument checks first (host only), so a malformed call reports what is
  // wrong with it rather than its size
  if (x_dtype != QM_F32 && x_dtype != QM_BF16) return QM_ERR_INVALID;
  if (n_tokens < 0 || top_k < 1) return QM_ERR_INVALID;
  const int st = check_experts(ex);
  if (st == QM_ERR_INVALID) return st;
  if (n_tokens == 0) return QM_OK;
  if (!x || !topk_ids || !topk_w || !y) return QM_ERR_INVALID;
  if (st != QM_OK) return st;
  if (top_k > QM_TOPK_MAX) return QM_ERR_UNSUPPORTED;
  const size_t need = moe_expert_ffn_workspace(ex, n_tokens, top_k);
  if (need == 0) return QM_ERR_INVALID;
  if (need > (size_t)QM_NOALLOC_SCRATCH_BYTES) return QM_ERR_TOO_LARGE;
  void* ws = scratch_ptr();
  if (!ws) return QM_ERR_LAUNCH;
  return moe_expert_ffn_path(ex, x, x_dtype, n_tokens, topk_ids, topk_w, top_k, y, ws,
                             (size_t)QM_NOALLOC_SCRATCH_BYTES, stream, QM_PATH_AUTO);
}
