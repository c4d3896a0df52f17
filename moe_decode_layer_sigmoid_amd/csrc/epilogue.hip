// The MoE layer's boundary on gfx950: weighted combine of the routed rows,
// plus the shared expert and the residual, then RMSNorm * gamma; optionally
// also the finalized MoE output (the combine plus the shared expert, before
// the residual: what the decode page's LayerStages._grouped_moe takes from
// the grouped kernel with finalize=True).
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
// and keeps its sums in registers between the two halves (sum of squares,
// then scaling), so h is read once.  Sums run in a fixed order, so results
// are bitwise reproducible.  Column slices of 1024 or 2048 per workgroup
// exchanging their sums of squares (as the chain launch's boundary does)
// measured no faster at 48 to 256 tokens (H = 4096 and 6144).
#include "device_common.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kMaxThreads = 1024;  // 8 columns per thread: H <= 8192 in one pass
constexpr int kCols = 8;
constexpr int kGroup = 8;        // routes whose rows one round of loads fetches

// One workgroup per token, of ceil(H / 8) threads rounded up to whole waves
// (a thread past H would only repeat loads of the row's last columns).
// Every load (top-k weights, the first kGroup
// routed rows, the shared row, the residual and gamma) is issued before the
// first is used, and addresses are clamped instead of branched around, so
// the common case (k <= 8) costs one memory round trip before the sum of
// squares.  Sums run in a fixed order: routes j = 0..k-1, shared, residual;
// waves in order for the sum of squares.
__global__ __launch_bounds__(kMaxThreads) void epilogue_kernel(
    const uint16_t* residual, const uint16_t* __restrict__ gamma, int H, int k, int has_shared,
    float eps, Workspace ws, uint16_t* out, uint16_t* residual_out,
    uint16_t* moe_out) {
  __shared__ float s_part[kMaxThreads / kWave];
  const int t = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = kCols * threadIdx.x;
  const bool live = c < H;
  const int c0 = live ? c : H - kCols;  // clamped: loads stay in the row
  const float* rows_t = ws.rows + static_cast<size_t>(t) * k * H + c0;
  const float* ys = ws.y_s + static_cast<size_t>(t) * H + c0;
  const uint4 rv = *reinterpret_cast<const uint4*>(residual + static_cast<size_t>(t) * H + c0);
  const uint4 gv = *reinterpret_cast<const uint4*>(gamma + c0);
  // set when a bounded wait of an earlier launch of this run gave up: the
  // rows may then be incomplete, and out is written as NaN
  const uint32_t gave_up = ld_i32<true>(reinterpret_cast<const int*>(ws.sync) +
                                        kSyncError * kSyncStride);
  const float4 ya = *reinterpret_cast<const float4*>(ys);
  const float4 yb = *reinterpret_cast<const float4*>(ys + 4);
  float acc[kCols];
#pragma unroll
  for (int m = 0; m < kCols; ++m) acc[m] = 0.f;
  for (int j0 = 0; j0 < k; j0 += kGroup) {
    float wj[kGroup];
    float4 ra[kGroup], rb[kGroup];
#pragma unroll
    for (int q = 0; q < kGroup; ++q) {
      const int j = j0 + q < k ? j0 + q : k - 1;
      const float w = ws.weights[t * k + j];
      wj[q] = j0 + q < k ? w : 0.f;
      ra[q] = *reinterpret_cast<const float4*>(rows_t + static_cast<size_t>(j) * H);
      rb[q] = *reinterpret_cast<const float4*>(rows_t + static_cast<size_t>(j) * H + 4);
    }
#pragma unroll
    for (int q = 0; q < kGroup; ++q) {
      acc[0] = fmaf(wj[q], ra[q].x, acc[0]);
      acc[1] = fmaf(wj[q], ra[q].y, acc[1]);
      acc[2] = fmaf(wj[q], ra[q].z, acc[2]);
      acc[3] = fmaf(wj[q], ra[q].w, acc[3]);
      acc[4] = fmaf(wj[q], rb[q].x, acc[4]);
      acc[5] = fmaf(wj[q], rb[q].y, acc[5]);
      acc[6] = fmaf(wj[q], rb[q].z, acc[6]);
      acc[7] = fmaf(wj[q], rb[q].w, acc[7]);
    }
  }
  if (has_shared) {
    acc[0] += ya.x; acc[1] += ya.y; acc[2] += ya.z; acc[3] += ya.w;
    acc[4] += yb.x; acc[5] += yb.y; acc[6] += yb.z; acc[7] += yb.w;
  }
  if (moe_out && live) store_bf16x8(moe_out + static_cast<size_t>(t) * H + c, acc);
  const uint32_t u[4] = {rv.x, rv.y, rv.z, rv.w};
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    acc[2 * m] += bf16_lo(u[m]);
    acc[2 * m + 1] += bf16_hi(u[m]);
  }
  float ss = 0.f;
#pragma unroll
  for (int m = 0; m < kCols; ++m) ss = fmaf(acc[m], acc[m], ss);
  ss = wave_sum(live ? ss : 0.f);
  if (lane == 0) s_part[wave] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int w = 0; w < kMaxThreads / kWave; ++w)
    if (w < static_cast<int>(blockDim.x) / kWave) tot += s_part[w];
  const float inv_rms = 1.0f / sqrtf(tot / static_cast<float>(H) + eps);
  if (!live) return;
  const uint32_t g[4] = {gv.x, gv.y, gv.z, gv.w};
  uint32_t o[4], r[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const float h0 = acc[2 * m], h1 = acc[2 * m + 1];
    o[m] = f32_to_bf16(h0 * inv_rms * bf16_lo(g[m])) |
           (f32_to_bf16(h1 * inv_rms * bf16_hi(g[m])) << 16);
    r[m] = f32_to_bf16(h0) | (f32_to_bf16(h1) << 16);
    if (gave_up) o[m] = kBf16NanPair;
  }
  *reinterpret_cast<uint4*>(out + static_cast<size_t>(t) * H + c) =
      make_uint4(o[0], o[1], o[2], o[3]);
  *reinterpret_cast<uint4*>(residual_out + static_cast<size_t>(t) * H + c) =
      make_uint4(r[0], r[1], r[2], r[3]);
}

}  // namespace

hipError_t launch_epilogue(const LayerDims& d, const void* residual, const void* gamma,
                           const Workspace& ws, void* out, void* residual_out, void* moe_out,
                           hipStream_t s) {
  const int threads = ((d.H / kCols + kWave - 1) / kWave) * kWave;
  hipLaunchKernelGGL(epilogue_kernel, dim3(d.T), dim3(threads), 0, s,
                     static_cast<const uint16_t*>(residual), static_cast<const uint16_t*>(gamma),
                     d.H, d.k, static_cast<int>(d.Is > 0), d.eps, ws,
                     static_cast<uint16_t*>(out),
                     static_cast<uint16_t*>(residual_out), static_cast<uint16_t*>(moe_out));
  return hipGetLastError();
}

}  // namespace moe
