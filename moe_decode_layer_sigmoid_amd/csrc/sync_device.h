// Hand-offs between workgroups of one launch on gfx950: counters, flags
// replicated over 128-byte lines, bounded waits with a sticky error word, and
// the two-level exit count after which the last workgroup out resets every
// counter for the next launch (HIP-graph replays included).
//
// Data that one workgroup leaves for another is written with agent-scope
// atomic stores (st_*<true>), which write through to the device coherence
// point, and read with agent-scope atomic loads (ld_*<true>), so no L2
// write-back or invalidate is needed across the XCDs.  A producer waits for
// its stores to complete before it bumps its counter.
#pragma once

#include "device_common.h"
#include "launch.h"

namespace moe {

// Polls before a wait gives up (each poll is a memory round trip plus a
// short sleep, so this is far beyond any legitimate wait).
constexpr uint32_t kSpinLimit = 1u << 22;

struct Sync {
  uint32_t* base;
  __device__ uint32_t* line(int i) const { return base + static_cast<size_t>(i) * kSyncStride; }
};

// Sets flag f (all kFlagRep replicas).  Called by one thread.
__device__ __forceinline__ void raise_flag(const Sync& sy, int f) {
#pragma unroll
  for (int r = 0; r < kFlagRep; ++r)
    __hip_atomic_store(sy.line(f + r), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Publishes this workgroup's coherent stores, then bumps counter `cnt`; the
// bump that reaches `target` raises flag `f` (f < 0: no flag).  Returns, to
// every thread, whether this bump completed the counter.
__device__ __forceinline__ bool signal(const Sync& sy, int cnt, uint32_t target, int f, int* s_flag) {
  wait_memory();
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(sy.line(cnt), 1u, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    const bool last = prev + 1 == target;
    if (last && f >= 0) raise_flag(sy, f);
    *s_flag = last;
  }
  __syncthreads();
  return *s_flag != 0;
}

// Waits until flag f is up, polling this workgroup's replica (bounded: sets
// the error word and gives up after kSpinLimit polls).
__device__ __forceinline__ void wait_flag(const Sync& sy, int f) {
  if (threadIdx.x == 0) {
    const uint32_t* p = sy.line(f + static_cast<int>(blockIdx.x % kFlagRep));
    uint32_t n = 0;
    while (__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0u) {
      __builtin_amdgcn_s_sleep(2);
      if (++n == kSpinLimit) {
        __hip_atomic_fetch_or(sy.line(kSyncError), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
    }
  }
  __syncthreads();
}

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

// Two-level exit count over `grid` workgroups (kSyncExitLines first-level
// lines, then one top line).  Returns, to every thread, whether this
// workgroup is the last one out: then every other workgroup has finished
// and published its coherent stores.  Called once per workgroup, at its end.
__device__ __forceinline__ bool last_out(const Sync& sy, uint32_t grid, int* s_flag) {
  wait_memory();
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t lines = kSyncExitLines;
    const uint32_t line = blockIdx.x % lines;
    const uint32_t share = grid / lines + (line < grid % lines ? 1u : 0u);
    const uint32_t prev = __hip_atomic_fetch_add(sy.line(kSyncExit0 + static_cast<int>(line)), 1u,
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    int last = 0;
    if (prev == share - 1) {
      const uint32_t top = __hip_atomic_fetch_add(sy.line(kSyncExitTop), 1u, __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT);
      last = top == (grid < lines ? grid : lines) - 1;
    }
    *s_flag = last;
  }
  __syncthreads();
  return *s_flag != 0;
}

// Zeroes sync lines [0, n) except the error word (by the last workgroup out).
__device__ __forceinline__ void reset_sync(const Sync& sy, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x)
    if (i != kSyncError)
      __hip_atomic_store(sy.line(i), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace moe
