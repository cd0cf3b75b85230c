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

struct MoeDecodeArgs {
  ExpertArgs ex;
  const void* x;       // [T][H]
  const int32_t* ids;  // [T][k]
  const float* w;      // [T][k]
  float* h;            // workspace [T*k][I] fp32
  float* pout;         // workspace [T*k][H] fp32, per-pair down outputs
  float* y;            // [T][H]
  int T, topk;
  int segc;            // chunks per LDS segment
  int parts;           // blocks per unique expert
  int rounds;          // tiles per wave
  int max_blocks;      // pipelined kernels: grid size cap (0 = default)
  uint32_t* hq;        // workspace: h as digit words [T*k][I/16][8] (single-token int4 kernels)
  float* hqs;          // workspace: their factors [T*k][I/16]
  int hq_ready;        // hq already holds the digits of h (written by the gate+up kernel)
  uint64_t* flags;     // workspace: one 64-bit flag per tile of h (one-launch layer)
  uint64_t nonce;      // value the flags take in this call (fresh per call)
};

// qgemv_q.hip: single-token int4 GEMV on integer dot products (k = 2048 *
// {1,2,3,4,6,8}); hipErrorNotSupported for other calls
hipError_t launch_qgemv_q(int xdt, bool grouped, const GemvArgs& a, hipStream_t st);
hipError_t launch_qgemv_q_pair(int xdt, bool grouped, const GemvArgs& a, const GemvArgs& b, hipStream_t st);
hipError_t launch_qgemv_qb(int xdt, bool grouped, const GemvArgs& a, hipStream_t st);  // 2..8 activation rows
// the same for int8 per-row weights (k = 1024 * {2,4,6,8,12,16}, v_dot4_i32_i8)
hipError_t launch_qgemv_q8(int xdt, const GemvArgs& a, hipStream_t st);
hipError_t launch_qgemv_q8_pair(int xdt, const GemvArgs& a, const GemvArgs& b, hipStream_t st);
// qgemv.hip
int lanes_per_row(int kchunks);
int rows_per_unit(int L, int NB);
int seg_chunks(int fmt, int xdt, int NB, int kchunks);
size_t stage_bytes(int fmt, int xdt, int NB, int segc);
hipError_t launch_qgemv(int fmt, int xdt, bool grouped, const GemvArgs& a, int NB, hipStream_t st);
// Two GEMVs of one x (same fmt, group structure and k) in one launch of the
// pipelined kernel; hipErrorNotSupported when that kernel does not take them
// (the caller then launches them one by one).
hipError_t launch_qgemv_pair(int fmt, int xdt, bool grouped, const GemvArgs& a, const GemvArgs& b, hipStream_t st);
// int3-g64 GEMV (fmt 5): y = W x for k <= kI3KMax; LDS bytes it stages.
constexpr int kI3KMax = 16384;
size_t qgemv_i3_lds(int k, int xdt);
hipError_t launch_qgemv_i3(const uint8_t* q, const float* sc, const void* x, int xdt, float* y, int n, int k,
                           hipStream_t st);
// u[i] <- u[i] / sqrt(mean u^2 + eps) * g[i] in place, one workgroup.
hipError_t launch_rmsnorm(float* u, const float* g, int n, float eps, hipStream_t st);
hipError_t launch_fill_zero(float* y, int64_t n, int64_t ld, int rows, hipStream_t st);

// per-instantiation launchers (qgemv_*.hip): grouped (_g) or row-scaled (_r)
#define QM_DECL_QGEMV(name) \
  hipError_t name(const GemvArgs& a, int L, int NB, int blocks, size_t lds, hipStream_t st);
QM_DECL_QGEMV(qgemv_launch_i4_bf16_g)
QM_DECL_QGEMV(qgemv_launch_i4_bf16_r)
QM_DECL_QGEMV(qgemv_launch_i4_f32_g)
QM_DECL_QGEMV(qgemv_launch_i4_f32_r)
QM_DECL_QGEMV(qgemv_launch_i8_bf16_r)
QM_DECL_QGEMV(qgemv_launch_i8_f32_r)
#define QM_DECL_QGEMV2(name) \
  hipError_t name(const GemvArgs& a, const GemvArgs& b, int na, int L, int CB, int blocks, size_t lds, hipStream_t st);
QM_DECL_QGEMV2(qgemv_v2_i4_bf16_g)
QM_DECL_QGEMV2(qgemv_v2_i4_bf16_r)
QM_DECL_QGEMV2(qgemv_v2_i8_bf16_r)
#undef QM_DECL_QGEMV2
#undef QM_DECL_QGEMV

// v2 (pipelined, single token, whole x in LDS) shape choices
int v2_cb(int kchunks, int L);
int v2_blocks(int ntiles, int max_blocks);

// moe_decode_*.hip: stage launchers per (format, activation type, grouping)
#define QM_DECL_MOE(name) hipError_t name(const MoeDecodeArgs& a, hipStream_t st);
QM_DECL_MOE(moe_gate_up_i4_bf16_g)
QM_DECL_MOE(moe_gate_up_i4_bf16_r)
QM_DECL_MOE(moe_gate_up_i4_f32_g)
QM_DECL_MOE(moe_gate_up_i4_f32_r)
QM_DECL_MOE(moe_gate_up_i8_bf16_r)
QM_DECL_MOE(moe_gate_up_i8_f32_r)
QM_DECL_MOE(moe_down_i4_g)
QM_DECL_MOE(moe_down_i4_r)
QM_DECL_MOE(moe_down_i8_r)
QM_DECL_MOE(moe_ffn_i4_bf16_g)  // the one-launch layer (hipErrorNotSupported: not taken)
QM_DECL_MOE(moe_ffn_i4_bf16_r)
QM_DECL_MOE(moe_ffn_i4_f32_g)
QM_DECL_MOE(moe_ffn_i4_f32_r)
#undef QM_DECL_MOE

// moe_decode.hip
hipError_t launch_moe_gate_up(int fmt, int xdt, bool grouped, const MoeDecodeArgs& a, hipStream_t st);
hipError_t launch_moe_down(int fmt, bool grouped, const MoeDecodeArgs& a, hipStream_t st);
// true when launch_moe_gate_up with these arguments also writes the digits of h to a.hq
bool moe_gate_up_writes_digits(int fmt, const MoeDecodeArgs& a);
// the whole decode layer in one launch when the one-launch kernel takes the
// call; hipErrorNotSupported otherwise (the caller then runs the two stages)
hipError_t launch_moe_ffn_layer(int fmt, int xdt, bool grouped, const MoeDecodeArgs& a, hipStream_t st);

// moe_prefill.hip: the grouped MFMA path takes int4 experts whose group size
// (or row length, per-row scales) is a multiple of 64 with at most 96 groups
// per row (grouped: a multiple of 4 groups, 16-byte aligned scale arrays),
// hidden % 512 == 0, inter % 256 == 0 and at most 8192 experts.
bool moe_prefill_supported(int fmt, int topk, const ExpertArgs& e);
size_t moe_prefill_workspace(int T, int topk, const ExpertArgs& e);
hipError_t launch_moe_prefill(int fmt, int xdt, const ExpertArgs& e, const void* x, const int32_t* ids,
                              const float* w, int T, int topk, float* y, void* ws, hipStream_t st);

}  // namespace qm
