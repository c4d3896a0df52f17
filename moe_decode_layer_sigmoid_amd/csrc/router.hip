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
// Grid: x = blocks of 4 experts (one expert row per wave), then, when asked,
// the shared expert's gate_up tiles (8 SwiGLU rows each, grid row 0 only: it
// depends on no routing, so its weights stream while the router waits on
// its memory round trips); y = blocks of TB tokens (router_block_tokens).  Phase 1: every wave loads its whole bf16 router row at once
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

// NJ2 = 16-byte chunks per lane of a bf16 router row (ceil(H / 512)); E8 =
// e8m0 scales of the shared expert's weights.
template <int NJ2, bool E8>
__global__ __launch_bounds__(kThreads) void router_kernel(
    const uint16_t* __restrict__ hidden, const uint16_t* __restrict__ router_w,
    const float* __restrict__ bias, int T, int TB, int H, int E, int k, float rsf, Workspace ws,
    int32_t* __restrict__ ids_out, float* __restrict__ w_out, int n_router,
    const uint8_t* __restrict__ sw13, const void* __restrict__ sscale, int Is, float limit) {
  // 16-byte aligned: the 64-bit token masks need 8-byte aligned LDS
  // addresses, and dynamic LDS starts right after the static variables.
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __shared__ int s_last;
  const int wave = threadIdx.x >> 6;
  const int t0 = blockIdx.y * TB;
  const int nt = min(TB, T - t0);

  // ---- columns past the router's: the shared expert's gate_up + SwiGLU,
  // which needs no routing and so streams in the router's shadow
  if (static_cast<int>(blockIdx.x) >= n_router) {
    if (blockIdx.y != 0) return;
    constexpr int NJ = (NJ2 + 1) / 2;  // 16-byte fp8 chunks per lane = ceil(H / 1024)
    const int i0 = ((static_cast<int>(blockIdx.x) - n_router) * 4 + wave) * 2;
    if (i0 < Is)
      gate_up_wave<NJ, 1, false, E8>(hidden, sw13, sscale, 0, H, Is, i0, T, nullptr, 0, k,
                                      ws.act_s, limit);
    return;
  }

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
             static_cast<uint32_t>(n_router) - 1;
  __syncthreads();
  if (!s_last) return;

  // ---- phase 2: top-k of the block's tokens
  const RouteSmem sm(smem, T, E, k);
  select_tokens<true>(t0, t0 + nt, E, k, rsf, ws.logits, bias, ws, ids_out, w_out, sm);
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
  // The counters of the launch that follows (the split path's expert chain)
  // start from zero and its boundary slots empty (zero): it never resets
  // them itself.  The error word stays.
  const int lines = sync_lines(T * k < E ? T * k : E);
  for (int i = threadIdx.x; i < lines; i += kThreads)
    if (i != kSyncError)
      __hip_atomic_store(ws.sync + static_cast<size_t>(i) * kSyncStride, 0u, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  for (int i = threadIdx.x; i < T * kMaxBndSlices; i += kThreads)
    __hip_atomic_store(reinterpret_cast<uint32_t*>(ws.epi_part) + i, 0u, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

// Tokens per block: every wave of a block's workgroups loads all of the
// block's token rows, so small blocks shorten the logits phase; larger ones
// read the router weight fewer times (once per block).  One token per block
// up to 16 tokens (2 us shorter at 16 tokens than blocks of 4), then
// kRouterTokBlk (blocks of 2 measured slower at 64 and 128 tokens).
int router_block_tokens(int T) { return T <= 16 ? 1 : kRouterTokBlk; }

}  // namespace

hipError_t launch_router(const LayerDims& d, const void* hidden, const void* router_w,
                         const float* bias, const Workspace& ws, int32_t* ids_out,
                         float* weights_out, const void* sw13, const void* sw13_scale,
                         hipStream_t s, hipEvent_t evb, hipEvent_t eve) {
  if (d.T > kRouterMaxBlk * kRouterTokBlk) return hipErrorInvalidValue;
  const int n_router = (d.E + 3) / 4;
  const int n_shared = sw13 && d.Is > 0 ? d.Is / 8 : 0;  // 8 SwiGLU rows per workgroup
  const int TB = router_block_tokens(d.T);
  // no routed experts (a dense layer): only the gate_up tiles, one grid row
  dim3 grid(n_router + n_shared, d.E > 0 ? (d.T + TB - 1) / TB : 1);
  const size_t smem = route_smem_bytes(d.T, d.E, d.k);
  const auto* x = static_cast<const uint16_t*>(hidden);
  const auto* w = static_cast<const uint16_t*>(router_w);
  const auto* sw = static_cast<const uint8_t*>(sw13);
  const int Is = n_shared ? d.Is : 0;
  switch (((d.H + 511) / 512) * 2 + (d.e8m0 ? 1 : 0)) {
#define X(N)                                                                                   \
  case 2 * N:                                                                                  \
    MOE_LAUNCH((router_kernel<N, false>), grid, dim3(kThreads), smem, s, evb, eve, x, w, bias, \
               d.T, TB, d.H, d.E, d.k, d.rsf, ws, ids_out, weights_out, n_router, sw,          \
               sw13_scale, Is, d.limit);                                                       \
    break;                                                                                     \
  case 2 * N + 1:                                                                              \
    MOE_LAUNCH((router_kernel<N, true>), grid, dim3(kThreads), smem, s, evb, eve, x, w, bias,  \
               d.T, TB, d.H, d.E, d.k, d.rsf, ws, ids_out, weights_out, n_router, sw,          \
               sw13_scale, Is, d.limit);                                                       \
    break;
    X(1) X(2) X(3) X(4) X(5) X(6) X(7) X(8) X(9) X(10) X(11) X(12) X(13) X(14) X(15) X(16)
#undef X
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace moe
