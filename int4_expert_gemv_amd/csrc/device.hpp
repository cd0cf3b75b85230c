// device.hpp -- small building blocks shared by the kernels (gfx950, wave64):
// format and activation-type constants, vector types, streaming loads, bf16
// conversion, SiLU and lane-group sums.
//
// Weight formats (colibri page "Vulkan backend: expert tier + dense + MLA
// attention on any Vulkan 1.2 GPU", commit notes "backend_vulkan.c/.h +
// shaders/qmatmul.comp", "fmt=4 grouped scales" and the int3 notes): int4
// value = nibble - 8, two nibbles per byte with element 2j in the low nibble
// of byte j, one fp32 scale per gs consecutive inputs of a row (or one per
// row); int8 is two's complement with one fp32 scale per row; int3-g64 is
// described in planes.hpp, where its values become int4 nibbles.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qm {

constexpr int kThreads = 256;  // workgroup size of the prefill kernels
constexpr int kTopkMax = 32;   // largest top_k accepted by the C ABI

constexpr int kFmtInt8 = 1;
constexpr int kFmtInt4 = 4;
constexpr int kFmtInt3 = 5;
constexpr int kF32 = 0;
constexpr int kBF16 = 1;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ---- scalar helpers -----------------------------------------------------------

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

// Weights and scales are read exactly once per call: stream them with
// non-temporal loads so they do not displace the activations, the hidden
// vectors and the other waves' data from the caches.
__device__ __forceinline__ u32x4 ld_stream(const uint8_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ float ld_stream(const float* p) { return __builtin_nontemporal_load(p); }

// fp32 -> bf16 bits, round to nearest even (v_cvt_pk_bf16_f32 on gfx950)
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

// Sum over aligned groups of L lanes; every lane of a group ends with the sum.
template <int L>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (L >= 2)  // lane ^ 1
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
  if constexpr (L >= 4)  // lane ^ 2
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
  if constexpr (L >= 8)  // row_half_mirror: the other quad of the 8-lane half-row
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));
  if constexpr (L >= 16)  // row_mirror: the other half of the 16-lane row
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));
  if constexpr (L >= 32) v += __shfl_xor(v, 16, 64);
  if constexpr (L >= 64) v += __shfl_xor(v, 32, 64);
  return v;
}

}  // namespace qm
