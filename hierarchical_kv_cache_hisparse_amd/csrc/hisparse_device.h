// Device helpers shared by the gfx950 kernels of libhisparse.
#pragma once

#include <hip/hip_runtime.h>

namespace hsp {

// Workgroup barrier for LDS only, for kernels in which no wave reads global
// memory that another wave of the same workgroup wrote: the barrier then
// never has to wait for outstanding global stores (HIP's __syncthreads
// would: it fences global memory too, which costs a store round trip per
// barrier).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// A pointer to device-visible memory (HBM, or pinned host memory mapped into
// the device address space) in the global address space.  Host-row pointers
// are read from the handle's pointer table, so the compiler cannot infer
// their address space and would emit flat instructions; flat loads count in
// lgkmcnt as well as vmcnt, which makes every later LDS wait also wait for
// the host round trip.  Accesses through this cast are global_load /
// global_store, counted in vmcnt only.
template <typename T>
__device__ __forceinline__ __attribute__((address_space(1))) T* global_ptr(T* p) {
  return (__attribute__((address_space(1))) T*)p;
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP moves: shifts by
// 1, 2, 4, 8 inside each 16-lane row, then the row totals are carried with
// the row broadcasts of lane 15 (into rows 1 and 3) and lane 31 (into rows 2
// and 3).  Six VALU operations, no LDS traffic.
__device__ __forceinline__ int wave_inclusive_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return x;
}

}  // namespace hsp
