// Hand-offs between workgroups of one launch on gfx950: completion counters
// on 128-byte lines and bounded waits with a sticky error word.
//
// Data that one workgroup leaves for another is written with agent-scope
// atomic stores (st_*<true>), which write through to the device coherence
// point; a producer waits for its stores to complete before it bumps its
// counter, and a consumer reads the data only once the count covers it.
#pragma once

#include "device_common.h"
#include "launch.h"

namespace moe {

struct Sync {
  uint32_t* base;
  __device__ uint32_t* line(int i) const { return base + static_cast<size_t>(i) * kSyncStride; }
};

// Bumps the counter on line `line` once this workgroup's coherent stores
// have completed.  The atomic's result is not used, so it is issued without
// a return and no thread waits for it.  Called by every thread.
__device__ __forceinline__ void bump(const Sync& sy, int line) {
  wait_memory();
  __syncthreads();
  if (threadIdx.x == 0)
    (void)__hip_atomic_fetch_add(sy.line(line), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Waits until the sum of the counters on lines [first, first + n) (n <= 64)
// reaches `target`: wave 0 polls them, one lane per line, then the
// workgroup meets at a barrier.  Bounded by `limit` polls (then the error
// word -- `err`, or line kSyncError of sy -- is set and the wait gives up).
// Called by every thread.
__device__ __forceinline__ void wait_count(const Sync& sy, int first, int n, uint32_t target,
                                           uint32_t limit, uint32_t* err = nullptr) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const uint32_t* p = sy.line(first + (lane < n ? lane : 0));
    uint32_t polls = 0;
    for (;;) {
      const uint32_t v = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      uint32_t sum = lane < n ? v : 0u;
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off, 64);
      if (sum >= target) break;  // uniform over the wave
      __builtin_amdgcn_s_sleep(2);
      if (++polls == limit) {
        if (lane == 0)
          __hip_atomic_fetch_or(err ? err : sy.line(kSyncError), 1u, __ATOMIC_RELAXED,
                                __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
    }
  }
  __syncthreads();
}

}  // namespace moe
