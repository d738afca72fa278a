// Asynchronous global -> LDS copies on gfx950 and counted waits for them.
//
// __builtin_amdgcn_global_load_lds moves 16 bytes per lane straight into LDS
// (destination: the instruction's LDS base + 16 * lane) without passing
// through registers; each such load counts in the wave's vmcnt until its data
// is in LDS. A ring of stages is then synchronised with an s_waitcnt that
// leaves the younger stages in flight and a bare s_barrier (the fence of
// __syncthreads() would wait for every outstanding load and drain the ring).
#pragma once

#include <hip/hip_runtime.h>

namespace dg {

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) const void global_cvoid_t;

__device__ inline void dma16(const void* src, void* lds_base) {
  __builtin_amdgcn_global_load_lds((global_cvoid_t*)src, (lds_void_t*)lds_base, 16, 0, 0);
}

// s_waitcnt vmcnt(N) with the export and LDS counters left alone (gfx9 encoding:
// vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
template <int N>
__device__ inline void wait_vm_n() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

template <int LPS, int K>
__device__ inline void wait_stages_impl(int younger) {
  if constexpr (K == 0) {
    wait_vm_n<0>();
  } else {
    if (younger >= K) wait_vm_n<K * LPS>();
    else wait_stages_impl<LPS, K - 1>(younger);
  }
}

// Wait until at most `younger` (0 .. NS-2) stages of LPS loads each are still in flight.
template <int LPS, int NS>
__device__ inline void wait_stages(int younger) {
  wait_stages_impl<LPS, NS - 2>(younger);
}

}  // namespace dg
