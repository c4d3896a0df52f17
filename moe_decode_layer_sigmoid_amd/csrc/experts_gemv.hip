// fp8 expert projections as GEMVs on gfx950 (the 1..16-token regime).
//
// Follows the vLLM API page "vllm.models.glm5next.nvidia.specialized_decode.
// runtime.decode": LayerStages._build_mega builds the routed experts from
// w13 / w2 fp8 weights with their block scales (w13_weight_scale_inv,
// w2_weight_scale_inv; power-of-two e8m0 scales when that flag is set) and
// swiglu_limit; the shared expert (SharedExpert) takes the same weight pair
// and limit.
//
// Each touched expert's weights are streamed from HBM once for all of its
// tokens: a wave owns a few weight rows, every lane loads 16-byte fp8 chunks
// of each row (coalesced 1 KiB per row per instruction), converts them
// exactly to fp32 with the gfx950 fp8 conversion, multiplies each 16-element
// partial dot product by its 128x128 block scale and accumulates in fp32; a
// wave reduction finishes every row.  gate_up fuses the clamped SwiGLU into
// its epilogue; down writes one fp32 row per route.
//
// Grid: x = row tiles of one expert, y = touched-expert slot (routed; slots
// past the step's touched count exit at once, so the grid size depends only
// on T and the launch can be captured) or a single row for the shared expert.
#include "device_common.h"
#include "gemv_tiles.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;

// Per-slot expert, token count and permuted base position.
struct SlotInfo {
  int e, n, base;
};

template <bool SHARED>
__device__ __forceinline__ bool slot_info(int T, const Workspace& ws, SlotInfo* si) {
  if (SHARED) {
    *si = {0, T, 0};
    return true;
  }
  const int d = blockIdx.y;
  if (d >= *ws.n_touched) return false;
  const int e = ws.touched[d];
  *si = {e, ws.counts[e], ws.offsets[e]};
  return true;
}

// SHARED: the shared expert (a separate instantiation, so that profiles tell
// the routed and shared launches apart).
template <int NJ, bool E8, bool SHARED>
__global__ __launch_bounds__(kThreads) void gate_up_kernel(
    const uint16_t* __restrict__ hidden, const uint8_t* __restrict__ w13,
    const void* __restrict__ scale, int H, int I, int k, int T, Workspace ws, float limit) {
  const int wave = threadIdx.x >> 6;
  const int i0 = (blockIdx.x * kWaves + wave) * 2;
  const bool shared = SHARED;
  SlotInfo si;
  if (!slot_info<SHARED>(T, ws, &si) || i0 >= I) return;
  const size_t rows_per_e = static_cast<size_t>(2) * I;
  const uint8_t* W = w13 + static_cast<size_t>(si.e) * rows_per_e * H;
  const size_t sbase = static_cast<size_t>(si.e) * (rows_per_e / kBlock) * (H / kBlock);
  gate_up_wave<NJ, 1, false, E8>(hidden, W, scale, sbase, H, I, i0, si.n,
                                  shared ? nullptr : ws.perm, si.base, k,
                                  shared ? ws.act_s : ws.act, limit);
}

template <int NJ, bool E8, bool SHARED>
__global__ __launch_bounds__(kThreads) void down_kernel(
    const uint8_t* __restrict__ w2, const void* __restrict__ scale, int H, int I, int T,
    Workspace ws) {
  const int wave = threadIdx.x >> 6;
  const int h0 = (blockIdx.x * kWaves + wave) * 4;
  const bool shared = SHARED;
  SlotInfo si;
  if (!slot_info<SHARED>(T, ws, &si) || h0 >= H) return;
  const uint8_t* W = w2 + static_cast<size_t>(si.e) * H * I;
  const size_t sbase = static_cast<size_t>(si.e) * (H / kBlock) * (I / kBlock);
  down_wave<NJ, 1, false, E8>(W, scale, sbase, H, I, h0, si.n, si.base,
                              shared ? nullptr : ws.perm, shared ? ws.act_s : ws.act,
                              shared ? ws.y_s : ws.rows);
}

template <int NJ, bool E8>
void launch_gu(dim3 grid, hipStream_t s, bool shared, const uint16_t* x, const uint8_t* w,
               const void* scale, const LayerDims& d, int I, const Workspace& ws) {
  if (shared)
    hipLaunchKernelGGL((gate_up_kernel<NJ, E8, true>), grid, dim3(kThreads), 0, s, x, w, scale,
                       d.H, I, d.k, d.T, ws, d.limit);
  else
    hipLaunchKernelGGL((gate_up_kernel<NJ, E8, false>), grid, dim3(kThreads), 0, s, x, w, scale,
                       d.H, I, d.k, d.T, ws, d.limit);
}

template <int NJ, bool E8>
void launch_dn(dim3 grid, hipStream_t s, bool shared, const uint8_t* w, const void* scale,
               const LayerDims& d, int I, const Workspace& ws) {
  if (shared)
    hipLaunchKernelGGL((down_kernel<NJ, E8, true>), grid, dim3(kThreads), 0, s, w, scale, d.H, I,
                       d.T, ws);
  else
    hipLaunchKernelGGL((down_kernel<NJ, E8, false>), grid, dim3(kThreads), 0, s, w, scale, d.H,
                       I, d.T, ws);
}

}  // namespace

#define MOE_NJ_CASES(X) X(1) X(2) X(3) X(4) X(5) X(6) X(7) X(8)

hipError_t launch_gate_up_gemv(const LayerDims& d, bool shared, const void* hidden,
                               const void* w13, const void* w13_scale, const Workspace& ws,
                               hipStream_t s) {
  const int I = shared ? d.Is : d.I;
  const int nj = (d.H + 1023) / 1024;
  const int slots = shared ? 1 : (d.T * d.k < d.E ? d.T * d.k : d.E);
  dim3 grid(I / (2 * kWaves), slots);
  const auto* x = static_cast<const uint16_t*>(hidden);
  const auto* w = static_cast<const uint8_t*>(w13);
  switch (nj * 2 + (d.e8m0 ? 1 : 0)) {
#define X(N)                                                              \
  case 2 * N:                                                             \
    launch_gu<N, false>(grid, s, shared, x, w, w13_scale, d, I, ws);      \
    break;                                                                \
  case 2 * N + 1:                                                         \
    launch_gu<N, true>(grid, s, shared, x, w, w13_scale, d, I, ws);       \
    break;
    MOE_NJ_CASES(X)
#undef X
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_down_gemv(const LayerDims& d, bool shared, const void* w2,
                            const void* w2_scale, const Workspace& ws, hipStream_t s) {
  const int I = shared ? d.Is : d.I;
  const int nj = (I + 1023) / 1024;
  const int slots = shared ? 1 : (d.T * d.k < d.E ? d.T * d.k : d.E);
  dim3 grid(d.H / (4 * kWaves), slots);
  const auto* w = static_cast<const uint8_t*>(w2);
  switch (nj * 2 + (d.e8m0 ? 1 : 0)) {
#define X(N)                                                     \
  case 2 * N:                                                    \
    launch_dn<N, false>(grid, s, shared, w, w2_scale, d, I, ws); \
    break;                                                       \
  case 2 * N + 1:                                                \
    launch_dn<N, true>(grid, s, shared, w, w2_scale, d, I, ws);  \
    break;
    MOE_NJ_CASES(X)
#undef X
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace moe
