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
// Grid: x = row tiles of one expert, y = slot.  gate_up: the touched
// experts (the shared expert's gate_up runs in the router launch).  down:
// the shared expert first (one more expert with all T tokens and weight 1),
// then the touched experts.  No second stream is needed on this path.
#include "device_common.h"
#include "gemv_tiles.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;

// One slot of the grid's y dimension: row 0 is the shared expert (when
// there is one), the next rows the touched experts in ascending id (rows
// past the step's touched count exit at once, so the grid size depends only
// on T and the launch can be captured).
struct Slot {
  bool shared;
  int e, n, base;
};

__device__ __forceinline__ bool slot_of(int T, int Is, const Workspace& ws, Slot* s) {
  const int y = static_cast<int>(blockIdx.y);
  if (Is > 0 && y == 0) {
    *s = {true, 0, T, 0};
    return true;
  }
  const int d = Is > 0 ? y - 1 : y;
  if (d >= *ws.n_touched) return false;
  const int e = ws.touched[d];
  *s = {false, e, ws.counts[e], ws.offsets[e]};
  return true;
}

// gate_up + clamped SwiGLU of the touched experts: a wave owns SwiGLU
// outputs i0, i0 + 1 of its slot's expert (grid row = touched slot).
template <int NJ, bool E8>
__global__ __launch_bounds__(kThreads) void gate_up_kernel(
    const uint16_t* __restrict__ hidden, const uint8_t* __restrict__ w13,
    const void* __restrict__ scale, int H, int I, int k, int T, Workspace ws, float limit) {
  const int wave = threadIdx.x >> 6;
  const int i0 = (blockIdx.x * kWaves + wave) * 2;
  Slot sl;
  if (!slot_of(T, 0, ws, &sl) || i0 >= I) return;
  const size_t rows_per_e = static_cast<size_t>(2) * I;
  const uint8_t* W = w13 + static_cast<size_t>(sl.e) * rows_per_e * H;
  const size_t sbase = static_cast<size_t>(sl.e) * (rows_per_e / kBlock) * (H / kBlock);
  gate_up_wave<NJ, 1, false, E8>(hidden, W, scale, sbase, H, I, i0, sl.n, ws.perm, sl.base, k,
                                  ws.act, limit);
}

// down projection of the routed experts and the shared expert in one
// launch: a wave owns output rows h0 .. h0 + 3 of its slot's expert.
// Routed rows land at their route index (t*k + j), shared rows at t.
template <int NJ, bool E8>
__global__ __launch_bounds__(kThreads) void down_kernel(
    const uint8_t* __restrict__ w2, const void* __restrict__ scale,
    const uint8_t* __restrict__ sw2, const void* __restrict__ sscale, int H, int I, int Is,
    int T, Workspace ws) {
  const int wave = threadIdx.x >> 6;
  const int h0 = (blockIdx.x * kWaves + wave) * 4;
  Slot sl;
  if (!slot_of(T, Is, ws, &sl) || h0 >= H) return;
  const int II = sl.shared ? Is : I;
  const uint8_t* W = sl.shared ? sw2 : w2 + static_cast<size_t>(sl.e) * H * II;
  const size_t sbase = static_cast<size_t>(sl.e) * (H / kBlock) * (II / kBlock);
  down_wave<NJ, 1, false, E8>(W, sl.shared ? sscale : scale, sbase, H, II, h0, sl.n, sl.base,
                              RouteTable<false>{sl.shared ? nullptr : ws.perm},
                              sl.shared ? ws.act_s : ws.act, sl.shared ? ws.y_s : ws.rows);
}

}  // namespace

#define MOE_NJ_CASES(X) X(1) X(2) X(3) X(4) X(5) X(6) X(7) X(8)

static int slot_rows(const LayerDims& d) {
  return (d.T * d.k < d.E ? d.T * d.k : d.E) + (d.Is > 0 ? 1 : 0);
}

hipError_t launch_gate_up_gemv(const LayerDims& d, const void* hidden, const void* w13,
                               const void* w13_scale, const Workspace& ws, hipStream_t s,
                               hipEvent_t evb, hipEvent_t eve) {
  const int nj = (d.H + 1023) / 1024;
  dim3 grid(d.I / (2 * kWaves), d.T * d.k < d.E ? d.T * d.k : d.E);
  const auto* x = static_cast<const uint16_t*>(hidden);
  const auto* w = static_cast<const uint8_t*>(w13);
  switch (nj * 2 + (d.e8m0 ? 1 : 0)) {
#define X(N)                                                                                  \
  case 2 * N:                                                                                 \
    MOE_LAUNCH((gate_up_kernel<N, false>), grid, dim3(kThreads), 0, s, evb, eve, x, w,        \
               w13_scale, d.H, d.I, d.k, d.T, ws, d.limit);                                   \
    break;                                                                                    \
  case 2 * N + 1:                                                                             \
    MOE_LAUNCH((gate_up_kernel<N, true>), grid, dim3(kThreads), 0, s, evb, eve, x, w,         \
               w13_scale, d.H, d.I, d.k, d.T, ws, d.limit);                                   \
    break;
    MOE_NJ_CASES(X)
#undef X
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_down_gemv(const LayerDims& d, const void* w2, const void* w2_scale,
                            const void* sw2, const void* sw2_scale, const Workspace& ws,
                            hipStream_t s) {
  const int Imax = d.I > d.Is ? d.I : d.Is;
  const int nj = (Imax + 1023) / 1024;  // chunks past a row's end are masked
  dim3 grid(d.H / (4 * kWaves), slot_rows(d));
  const auto* w = static_cast<const uint8_t*>(w2);
  const auto* sw = static_cast<const uint8_t*>(sw2);
  switch (nj * 2 + (d.e8m0 ? 1 : 0)) {
#define X(N)                                                                                   \
  case 2 * N:                                                                                  \
    hipLaunchKernelGGL((down_kernel<N, false>), grid, dim3(kThreads), 0, s, w, w2_scale, sw,    \
                       sw2_scale, d.H, d.I, d.Is, d.T, ws);                                    \
    break;                                                                                     \
  case 2 * N + 1:                                                                              \
    hipLaunchKernelGGL((down_kernel<N, true>), grid, dim3(kThreads), 0, s, w, w2_scale, sw,     \
                       sw2_scale, d.H, d.I, d.Is, d.T, ws);                                    \
    break;
    MOE_NJ_CASES(X)
#undef X
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace moe
