// Direct global-to-LDS loads (gfx950) and explicit vector-memory waits.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

// 16 bytes per lane from global memory straight into LDS: lane l's bytes land
// at lds_base + 16 l. Counted by vmcnt only; waits are explicit (wait_vmem,
// then a barrier before any wave reads the data).
__device__ __forceinline__ void lds_dma16(const void* gptr, uint32_t lds_base) {
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(gptr), "{m0}"(lds_base));
}

// 4 bytes per lane into LDS: lane l's word lands at lds_base + 4 l.
__device__ __forceinline__ void lds_dma4(const void* gptr, uint32_t lds_base) {
  asm volatile("global_load_lds_dword %0, off" ::"v"(gptr), "{m0}"(lds_base));
}

// wait until at most N of this wave's vector-memory operations are in flight
template <int N>
__device__ __forceinline__ void wait_vmem() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

}  // namespace pkv
