// Device helpers shared by the gfx950 kernels of the MoE decode layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kBlock = 128;   // weight scale block edge
constexpr int kWave = 64;     // CDNA wavefront width
constexpr int kMaxTopK = 16;
constexpr int kMaxExperts = 1024;
constexpr int kMaxTokens = 256;

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Low and high bf16 halves of a dword as floats.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float -> bf16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// Four e4m3fn codes (one dword, byte 0 first) -> four floats (exact).
__device__ __forceinline__ void fp8x4_to_f32(uint32_t w, float* o) {
  auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), false);
  auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), true);
  o[0] = lo[0];
  o[1] = lo[1];
  o[2] = hi[0];
  o[3] = hi[1];
}

// e8m0 byte b -> 2^(b-127) as a float (b = 0 is the subnormal 2^-127).
__device__ __forceinline__ float e8m0_to_f32(uint32_t b) {
  return b == 0 ? __uint_as_float(0x00400000u) : __uint_as_float(b << 23);
}

// Block scale number `idx` of a scale tensor (fp32 or e8m0 bytes).
__device__ __forceinline__ float load_scale(const void* s, bool e8m0, size_t idx) {
  if (e8m0) return e8m0_to_f32(static_cast<const uint8_t*>(s)[idx]);
  return static_cast<const float*>(s)[idx];
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

__device__ __forceinline__ float sigmoidf_(float z) { return 1.0f / (1.0f + __expf(-z)); }

// silu(min(g, L)) * clamp(u, -L, L)
__device__ __forceinline__ float clamped_swiglu(float g, float u, float limit) {
  float gc = fminf(g, limit);
  float uc = fminf(fmaxf(u, -limit), limit);
  return gc / (1.0f + __expf(-gc)) * uc;
}

}  // namespace moe
