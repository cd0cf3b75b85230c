// launch.hpp -- kernel argument blocks and host-side launchers shared by the
// C ABI (qmoe.hip) and the kernel files.  Internal to libqmoe.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qm {

struct GemvArgs {
  const uint8_t* q;   // packed weights, row-major
  const float* s;     // scales: [n][G] (grouped) or [n]
  const void* x;      // activations [nb][ldx]
  float* y;           // outputs [nb][ldy]
  int n, k;
  int G, gshift;      // groups per row; chunk index >> gshift = group (grouped int4)
  int64_t row_bytes, ldx, ldy;
  int nb;             // batch actually used
  int segc;           // chunks per LDS segment (set by the launcher)
  int rounds;         // tiles per wave
  int max_blocks;     // pipelined kernels: grid size cap (0 = default)
};

// One set of stacked experts as seen by the kernels.
struct ExpertArgs {
  const uint8_t *gq, *uq, *dq;
  const float *gs, *us, *ds;
  int E, H, I;
  int G_h, G_i;       // scale groups per gate/up row (K = H) and per down row (K = I)
  int gshift;         // log2(group size / 32) for grouped int4
  int64_t rb_h, rb_i; // bytes per gate/up row and per down row
};

// Arguments of the decode kernels (moe_decode.hip) for one pass of up to
// kDecMaxTokens tokens.
struct MoeDecArgs {
  ExpertArgs ex;
  const void* x;       // [T][H] activations of the pass
  const int32_t* ids;  // [T][k] expert ids
  const float* w;      // [T][k] routing weights
  float* h;            // optional fp32 h [T*k][I] (stage output / caller input)
  float* y;            // [T][H]
  int T, topk;
  uint8_t* hrec;       // workspace: h records [T*k][kRecPairs][8 * ceil(I / 128)][96 B] (moe_decode.hip)
  float* ab;           // workspace: gate/up partial sums between passes [T*k][I][2]
};

constexpr int kDecMaxTokens = 8;            // tokens per decode pass at most
constexpr size_t kDecLdsMax = 128 * 1024;   // dynamic LDS of the decode kernels

// gemv.hip: y = W x for int4 (grouped or per row) and int8 per-row weights,
// a.nb (<= 8) activation rows per weight read; with b, a second matrix of the
// same k and x in the same launch (one activation row).  hipErrorNotSupported
// for formats it does not take.
hipError_t launch_gemv_planes(int fmt, int xdt, bool grouped, const GemvArgs& a, const GemvArgs* b, hipStream_t st);
// compute units of the current device (cached per device, thread-safe)
hipError_t device_cus(int* cus);
// int3-g64 rows (fmt 5) the library takes: k <= kI3KMax (the int4 kernels
// run them; this is the range the int3 parity tests cover).
constexpr int kI3KMax = 16384;
// u[i] <- u[i] / sqrt(mean u^2 + eps) * g[i] in place, one workgroup.
hipError_t launch_rmsnorm(float* u, const float* g, int n, float eps, hipStream_t st);

// moe_decode.hip: the decode kernels.  Workspace bytes for T tokens of a
// pass, and its split into the MoeDecArgs buffers.
size_t moe_decode_ws_bytes(int T, int topk, int H, int I);
void moe_decode_ws_split(MoeDecArgs& a, void* ws);
// shapes the decode kernels take; tokens per pass for these experts
bool moe_decode_supported(int fmt, int T, int topk, const ExpertArgs& e);
int moe_decode_tokens_per_pass(int fmt, int topk, const ExpertArgs& e);
// gate+up: h digits (and a.h when set); down: y from the h digits (made
// from a.h first when h_from_caller)
hipError_t launch_moe_gate_up2(int fmt, int xdt, bool grouped, const MoeDecArgs& a, hipStream_t st);
hipError_t launch_moe_down2(int fmt, bool grouped, const MoeDecArgs& a, bool h_from_caller, hipStream_t st);

// moe_prefill.hip: the grouped MFMA path takes int4 experts whose group size
// (or row length, per-row scales) is a multiple of 64 (grouped: a multiple of
// 4 groups per row, 16-byte aligned scale arrays), hidden % 512 == 0,
// inter % 256 == 0 and at most 8192 experts.
bool moe_prefill_supported(int fmt, int topk, const ExpertArgs& e);
size_t moe_prefill_workspace(int T, int topk, const ExpertArgs& e);
hipError_t launch_moe_prefill(int fmt, int xdt, const ExpertArgs& e, const void* x, const int32_t* ids,
                              const float* w, int T, int topk, float* y, void* ws, hipStream_t st);

}  // namespace qm
