// lds_barrier.h -- work-group barrier for hand-offs through LDS (gfx950).
#pragma once

#include <hip/hip_runtime.h>

namespace gi {

// Waits for this wave's own LDS instructions, then for every wave of the
// work-group.  __syncthreads() also fences global memory, and the compiler
// implements that fence by waiting for every outstanding direct (buffer ->
// LDS) load, which drains the prefetches a pipeline keeps in flight across
// the barrier.  A kernel that hands off data landed by direct loads waits
// for them itself (s_waitcnt vmcnt) before this.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

}  // namespace gi
