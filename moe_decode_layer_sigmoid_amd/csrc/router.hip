// Router of the MoE decode layer on gfx950: logits GEMV, sigmoid scores,
// top-k selection with renormalised weights and the token -> expert route
// tables, in one launch.
//
// Follows the vLLM API page "vllm.models.glm5next.nvidia.specialized_decode.
// runtime.decode": LayerStages._router (bf16 router weight, fp32 logits),
// LayerStages._build_mega (sigmoid scoring, one group, normalised top-k,
// routed_scaling_factor) and LayerStages._mega_moe (the route order table
// handed to the boundary with the unfinalized rows).
//
// Grid: x = blocks of 4 experts (one expert row per wave), y = blocks of
// kTokB tokens.  Phase 1: every wave loads its whole bf16 router row at once
// (one memory round trip), then dots it with the block's token rows.
// Phase 2: the last workgroup of each token block (an arrival counter per
// block) ranks that block's tokens, one wave per token.  Phase 3: the last
// token block to finish (a second counter) builds the route tables from
// per-expert token bitmasks in LDS.  Data handed between workgroups goes
// through coherent stores and loads; the counters reset themselves, so the
// launch replays from a HIP graph.
#include "device_common.h"
#include "gemv_tiles.h"
#include "launch.h"
#include "routing_device.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

template <int NJ2>
__global__ __launch_bounds__(kThreads) void router_kernel(
    const uint16_t* __restrict__ hidden, const uint16_t* __restrict__ router_w,
    const float* __restrict__ bias, int T, int H, int E, int k, float rsf, Workspace ws,
    int32_t* __restrict__ ids_out, float* __restrict__ w_out) {
  // 16-byte aligned: the 64-bit token masks need 8-byte aligned LDS
  // addresses, and dynamic LDS starts right after the static variables.
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __shared__ int s_last;
  const int wave = threadIdx.x >> 6;
  const int t0 = blockIdx.y * kRouterTokBlk;
  const int nt = min(kRouterTokBlk, T - t0);

  // ---- phase 1: logits of this wave's expert for the block's tokens
  const int e = blockIdx.x * 4 + wave;
  if (e < E)
    router_wave<NJ2, true>(hidden + static_cast<size_t>(t0) * H,
                           router_w + static_cast<size_t>(e) * H, H, nt, E, e,
                           ws.logits + static_cast<size_t>(t0) * E);
  wait_memory();
  __syncthreads();
  uint32_t* cnt = ws.counter + router_cnt_line(blockIdx.y);
  if (threadIdx.x == 0)
    s_last = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
             gridDim.x - 1;
  __syncthreads();
  if (!s_last) return;

  // ---- phase 2: top-k of the block's tokens
  const RouteSmem sm(smem, T, E, k);
  select_tokens<true>(t0, t0 + nt, E, k, rsf, ws.logits, bias, ws, ids_out, w_out, sm.ids);
  if (threadIdx.x == 0) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (gridDim.y > 1) {
    wait_memory();
    __syncthreads();
    uint32_t* top = ws.counter + router_cnt_line(kRouterMaxBlk);
    if (threadIdx.x == 0)
      s_last = __hip_atomic_fetch_add(top, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
               gridDim.y - 1;
    __syncthreads();
    if (!s_last) return;
    if (threadIdx.x == 0) __hip_atomic_store(top, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (int r = threadIdx.x; r < T * k; r += kThreads) sm.ids[r] = ld_i32<true>(ws.ids + r);
  }

  // ---- phase 3: route tables (read by later kernels)
  build_routes<false>(T, E, k, ws, sm);
}

}  // namespace

hipError_t launch_router(const LayerDims& d, const void* hidden, const void* router_w,
                         const float* bias, const Workspace& ws, int32_t* ids_out,
                         float* weights_out, hipStream_t s) {
  if (d.T > kRouterMaxBlk * kRouterTokBlk) return hipErrorInvalidValue;
  dim3 grid((d.E + 3) / 4, (d.T + kRouterTokBlk - 1) / kRouterTokBlk);
  const size_t smem = route_smem_bytes(d.T, d.E, d.k);
  const auto* x = static_cast<const uint16_t*>(hidden);
  const auto* w = static_cast<const uint16_t*>(router_w);
  switch ((d.H + 511) / 512) {
#define X(N)                                                                                  \
  case N:                                                                                     \
    hipLaunchKernelGGL((router_kernel<N>), grid, dim3(kThreads), smem, s, x, w, bias, d.T,    \
                       d.H, d.E, d.k, d.rsf, ws, ids_out, weights_out);                       \
    break;
    X(1) X(2) X(3) X(4) X(5) X(6) X(7) X(8) X(9) X(10) X(11) X(12) X(13) X(14) X(15) X(16)
#undef X
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace moe
