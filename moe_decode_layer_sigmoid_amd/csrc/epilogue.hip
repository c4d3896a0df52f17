// The MoE layer's boundary on gfx950: weighted combine of the routed rows,
// plus the shared expert and the residual, then RMSNorm * gamma.
//
// Follows the vLLM API page "vllm.models.glm5next.nvidia.specialized_decode.
// runtime.draft", SpecializedDraft.reduced_norm and _build_ar_norm: the
// boundary takes the unfinalized routed rows with their top-k weights
// (it is built with top_k), adds the residual and returns norm(x + residual)
// together with the new residual.  Page "...runtime.decode",
// LayerStages._mega_moe: the shared expert output arrives beside the routed
// rows and is added with weight 1.  With one GPU there is no all-reduce in it.
//
// One workgroup per token; each thread owns 8 consecutive hidden elements
// per pass and keeps its sums in registers between the two halves (sum of
// squares, then scaling), so h is read once.  Sums run in a fixed order
// (routes j = 0..k-1, shared, residual; waves 0..3), so results are
// bitwise reproducible.
#include "device_common.h"
#include "gemv_tiles.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void epilogue_kernel(
    const uint16_t* residual, const uint16_t* __restrict__ gamma, int H, int k, int has_shared,
    float eps, Workspace ws, uint16_t* out, uint16_t* residual_out) {
  __shared__ float s_part[kThreads / kWave];
  epilogue_token(blockIdx.x, residual, gamma, H, k, has_shared != 0, eps, ws, out, residual_out,
                 s_part);
}

}  // namespace

hipError_t launch_epilogue(const LayerDims& d, const void* residual, const void* gamma,
                           const Workspace& ws, void* out, void* residual_out, hipStream_t s) {
  hipLaunchKernelGGL(epilogue_kernel, dim3(d.T), dim3(kThreads), 0, s,
                     static_cast<const uint16_t*>(residual), static_cast<const uint16_t*>(gamma),
                     d.H, d.k, static_cast<int>(d.Is > 0), d.eps, ws, static_cast<uint16_t*>(out),
                     static_cast<uint16_t*>(residual_out));
  return hipGetLastError();
}

}  // namespace moe
