// lds_ring.hpp -- building blocks of the kernels that stream weights into an
// LDS ring with gfx950's global_load_lds DMA (one 16- or 4-byte piece per
// lane, written lane-contiguously to a wave-uniform LDS address) and wait for
// them with explicit vmcnt counts (the compiler does not track LDS DMA).
//
// vmcnt bookkeeping: loads complete in issue order, so after issuing units in
// order, "unit u has landed" is "at most U * (units issued after u) VMEM
// operations are outstanding", U being the operations one unit issues.  Other
// VMEM operations issued later only make such a wait stricter.
#pragma once
#include <hip/hip_runtime.h>

namespace qm {

#define QM_LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

// One lane's 16 bytes (or 4 bytes) into a wave-uniform LDS block of 1 KiB
// (or 256 B) at lane-contiguous positions; non-temporal.
__device__ __forceinline__ void dma16(const void* g, char* lds_block) {
  __builtin_amdgcn_global_load_lds(g, QM_LDS_PTR(lds_block), 16, 0, 2);
}
__device__ __forceinline__ void dma4(const void* g, char* lds_block) {
  __builtin_amdgcn_global_load_lds(g, QM_LDS_PTR(lds_block), 4, 0, 2);
}

// s_waitcnt vmcnt(N) with the other counters untouched (gfx9 encoding:
// vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8], vmcnt[5:4] in bits [15:14]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | 0x0F70 | (((N >> 4) & 3) << 14));
}

// wait until at most n_after * U VMEM operations are outstanding (n_after < D)
template <int U, int D>
__device__ __forceinline__ void wait_units(int n_after) {
  static_assert(D >= 1 && D <= 4, "ring depth");
  if (n_after <= 0) {
    wait_vmcnt<0>();
  } else if (n_after == 1 || D <= 2) {
    wait_vmcnt<U>();
  } else if (n_after == 2 || D <= 3) {
    wait_vmcnt<(2 * U < 64 ? 2 * U : 63)>();
  } else {
    wait_vmcnt<(3 * U < 64 ? 3 * U : 63)>();
  }
}

// LDS reads of a slot must have returned before DMA refills it.
__device__ __forceinline__ void slot_release() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), vmcnt/expcnt untouched
  asm volatile("" ::: "memory");
}

// wait until at most n * U VMEM operations are outstanding (0 <= n <= N)
template <int U, int N>
__device__ __forceinline__ void wait_units_upto(int n) {
  if constexpr (N <= 0) {
    wait_vmcnt<0>();
  } else {
    if (n >= N)
      wait_vmcnt<(N * U < 64 ? N * U : 63)>();
    else
      wait_units_upto<U, N - 1>(n);
  }
}


}  // namespace qm
