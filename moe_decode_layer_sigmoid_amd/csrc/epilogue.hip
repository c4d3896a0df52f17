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
#include "launch.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxPass = 4;  // H <= 8192 = 4 passes x 256 threads x 8

__global__ __launch_bounds__(kThreads) void epilogue_kernel(
    const uint16_t* residual, const uint16_t* __restrict__ gamma, int H, int k, int has_shared,
    float eps, Workspace ws, uint16_t* out, uint16_t* residual_out) {
  __shared__ float s_part[kThreads / kWave];
  const int t = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float hv[kMaxPass][8];
  float ss = 0.f;
#pragma unroll
  for (int p = 0; p < kMaxPass; ++p) {
    const int c0 = 8 * (threadIdx.x + kThreads * p);
    if (c0 >= H) continue;
    float acc[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) acc[m] = 0.f;
    for (int j = 0; j < k; ++j) {
      const int r = t * k + j;
      const float w = ws.weights[r];
      const float4* row = reinterpret_cast<const float4*>(
          ws.rows + static_cast<size_t>(ws.inv[r]) * H + c0);
      const float4 a = row[0], b = row[1];
      acc[0] = fmaf(w, a.x, acc[0]);
      acc[1] = fmaf(w, a.y, acc[1]);
      acc[2] = fmaf(w, a.z, acc[2]);
      acc[3] = fmaf(w, a.w, acc[3]);
      acc[4] = fmaf(w, b.x, acc[4]);
      acc[5] = fmaf(w, b.y, acc[5]);
      acc[6] = fmaf(w, b.z, acc[6]);
      acc[7] = fmaf(w, b.w, acc[7]);
    }
    if (has_shared) {
      const float4* ys = reinterpret_cast<const float4*>(ws.y_s + static_cast<size_t>(t) * H + c0);
      const float4 a = ys[0], b = ys[1];
      acc[0] += a.x; acc[1] += a.y; acc[2] += a.z; acc[3] += a.w;
      acc[4] += b.x; acc[5] += b.y; acc[6] += b.z; acc[7] += b.w;
    }
    const uint4 rv = *reinterpret_cast<const uint4*>(residual + static_cast<size_t>(t) * H + c0);
    const uint32_t u[4] = {rv.x, rv.y, rv.z, rv.w};
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      acc[2 * m] += bf16_lo(u[m]);
      acc[2 * m + 1] += bf16_hi(u[m]);
    }
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      hv[p][m] = acc[m];
      ss = fmaf(acc[m], acc[m], ss);
    }
  }
  ss = wave_sum(ss);
  if (lane == 0) s_part[wave] = ss;
  __syncthreads();
  const float tot = (s_part[0] + s_part[1]) + (s_part[2] + s_part[3]);
  const float inv_rms = 1.0f / sqrtf(tot / static_cast<float>(H) + eps);
#pragma unroll
  for (int p = 0; p < kMaxPass; ++p) {
    const int c0 = 8 * (threadIdx.x + kThreads * p);
    if (c0 >= H) continue;
    const uint4 gv = *reinterpret_cast<const uint4*>(gamma + c0);
    const uint32_t g[4] = {gv.x, gv.y, gv.z, gv.w};
    uint32_t o[4], r[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const float h0 = hv[p][2 * m], h1 = hv[p][2 * m + 1];
      o[m] = f32_to_bf16(h0 * inv_rms * bf16_lo(g[m])) |
             (f32_to_bf16(h1 * inv_rms * bf16_hi(g[m])) << 16);
      r[m] = f32_to_bf16(h0) | (f32_to_bf16(h1) << 16);
    }
    *reinterpret_cast<uint4*>(out + static_cast<size_t>(t) * H + c0) = make_uint4(o[0], o[1], o[2], o[3]);
    *reinterpret_cast<uint4*>(residual_out + static_cast<size_t>(t) * H + c0) =
        make_uint4(r[0], r[1], r[2], r[3]);
  }
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
