// Streaming-read ceiling of the GPU's memory path (a measurement kernel, not
// part of the layer): the benchmark states every layer time as a fraction of
// both the published HBM peak and of what a plain read of the same weight
// streams achieves on this GPU.
//
// Every lane reads 16-byte chunks with non-temporal loads, the load form the
// expert kernels stream their fp8 weights with; one load instruction of a
// wave covers 1 KiB contiguously (eight lanes per 128-byte line), and each
// lane keeps kUnroll loads in flight before it uses the first.  The XOR of
// the loaded words goes to `sink` only when it equals a value no buffer of
// the probe's sizes produces in practice, so the loads stay live without a
// store per lane.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "moe_decode.h"

namespace moe {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kUnroll = 8;
constexpr uint32_t kProbeGrid = 2048;  // 8 workgroups per CU on 256 CUs
constexpr size_t kProbeStep = static_cast<size_t>(kProbeGrid) * kProbeThreads * kUnroll * 16;

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const u32x4_t* __restrict__ p,
                                                                   size_t steps,
                                                                   uint32_t* __restrict__ sink) {
  const size_t per_step = kProbeStep / 16;
  const u32x4_t* q = p + static_cast<size_t>(blockIdx.x) * kProbeThreads * kUnroll + threadIdx.x;
  uint32_t acc = 0;
  for (size_t s = 0; s < steps; ++s) {
    u32x4_t v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(q + u * kProbeThreads);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    q += per_step;
  }
  if (acc == 0x9e3779b9u) sink[threadIdx.x] = acc;
}

}  // namespace
}  // namespace moe

extern "C" int moe_decode_read_probe(const void* buf, size_t bytes, uint32_t* sink,
                                     void* stream) {
  if (!buf || !sink || bytes == 0 || bytes % moe::kProbeStep != 0 ||
      (reinterpret_cast<uintptr_t>(buf) & 15u) != 0)
    return MOE_DECODE_ERR_INVALID_ARG;
  hipLaunchKernelGGL(moe::read_probe_kernel, dim3(moe::kProbeGrid), dim3(moe::kProbeThreads), 0,
                     static_cast<hipStream_t>(stream),
                     static_cast<const moe::u32x4_t*>(buf), bytes / moe::kProbeStep, sink);
  return hipGetLastError() == hipSuccess ? MOE_DECODE_OK : MOE_DECODE_ERR_HIP;
}
