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
// Phase 1 (every workgroup): each wave computes the logits of kEpw experts
// for a block of kTokB tokens, streaming 16-byte chunks of the bf16 router
// rows; lanes split the hidden dimension and a wave reduction finishes each
// dot product.  Phase 2 (the last workgroup to finish, found with an atomic
// counter): per token a wave ranks the experts with a packed (key, id)
// wave-max, k rounds; then the route tables are built from per-expert token
// bitmasks in LDS (popcounts give stable ranks, one block scan gives the
// offsets and the touched-expert list).  The counter is reset at the end so
// the launch can be replayed from a HIP graph.
#include "device_common.h"
#include "launch.h"
#include "routing_device.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kEpw = 2;   // experts per wave
constexpr int kTokB = 8;  // tokens per workgroup row of the grid

__global__ __launch_bounds__(kThreads) void router_kernel(
    const uint16_t* __restrict__ hidden, const uint16_t* __restrict__ router_w,
    const float* __restrict__ bias, int T, int H, int E, int k, float rsf, Workspace ws,
    int32_t* __restrict__ ids_out, float* __restrict__ w_out, uint32_t total_blocks) {
  // 16-byte aligned: the 64-bit token masks below need 8-byte aligned LDS
  // addresses, and dynamic LDS starts right after the static variables.
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __shared__ int s_last;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;

  // ---- phase 1: logits[t, e] for this block's experts and tokens
  {
    const int e0 = (blockIdx.x * 4 + wave) * kEpw;
    const int t0 = blockIdx.y * kTokB;
    const int nt = min(kTokB, T - t0);
    const int nchunk = H / 8;  // 16-byte chunks of a bf16 row
    float acc[kEpw][kTokB];
#pragma unroll
    for (int x = 0; x < kEpw; ++x)
#pragma unroll
      for (int q = 0; q < kTokB; ++q) acc[x][q] = 0.f;
    for (int c = lane; c < nchunk; c += 64) {
      float wf[kEpw][8];
#pragma unroll
      for (int x = 0; x < kEpw; ++x) {
        uint4 v = make_uint4(0, 0, 0, 0);
        if (e0 + x < E)
          v = *reinterpret_cast<const uint4*>(router_w + static_cast<size_t>(e0 + x) * H + 8 * c);
        uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          wf[x][2 * m] = bf16_lo(u[m]);
          wf[x][2 * m + 1] = bf16_hi(u[m]);
        }
      }
#pragma unroll
      for (int q = 0; q < kTokB; ++q) {
        if (q < nt) {
          uint4 v = *reinterpret_cast<const uint4*>(hidden + static_cast<size_t>(t0 + q) * H + 8 * c);
          uint32_t u[4] = {v.x, v.y, v.z, v.w};
          float xf[8];
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            xf[2 * m] = bf16_lo(u[m]);
            xf[2 * m + 1] = bf16_hi(u[m]);
          }
#pragma unroll
          for (int x = 0; x < kEpw; ++x)
#pragma unroll
            for (int m = 0; m < 8; ++m) acc[x][q] = fmaf(wf[x][m], xf[m], acc[x][q]);
        }
      }
    }
#pragma unroll
    for (int x = 0; x < kEpw; ++x)
#pragma unroll
      for (int q = 0; q < kTokB; ++q) {
        if (q < nt) {
          float v = wave_sum(acc[x][q]);
          if (lane == 0 && e0 + x < E) ws.logits[static_cast<size_t>(t0 + q) * E + e0 + x] = v;
        }
      }
  }

  // ---- hand-off: the last workgroup to arrive runs phase 2
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t prev = __hip_atomic_fetch_add(ws.counter, 1u, __ATOMIC_ACQ_REL,
                                           __HIP_MEMORY_SCOPE_AGENT);
    s_last = (prev == total_blocks - 1);
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();

  // ---- phase 2: top-k of every token and the route tables
  select_and_route<false>(T, E, k, rsf, ws.logits, bias, ws, ids_out, w_out, smem);
  if (threadIdx.x == 0)
    __hip_atomic_store(ws.counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace

hipError_t launch_router(const LayerDims& d, const void* hidden, const void* router_w,
                         const float* bias, const Workspace& ws, int32_t* ids_out,
                         float* weights_out, hipStream_t s) {
  dim3 grid((d.E + 4 * kEpw - 1) / (4 * kEpw), (d.T + kTokB - 1) / kTokB);
  const size_t smem = route_smem_bytes(d.T, d.E, d.k);
  hipLaunchKernelGGL(router_kernel, grid, dim3(kThreads), smem, s,
                     static_cast<const uint16_t*>(hidden), static_cast<const uint16_t*>(router_w),
                     bias, d.T, d.H, d.E, d.k, d.rsf, ws, ids_out, weights_out,
                     static_cast<uint32_t>(grid.x * grid.y));
  return hipGetLastError();
}

}  // namespace moe
