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

// Two bf16 quiet NaNs in one dword: what a boundary writes to `out` when a
// bounded wait of the run gave up.
constexpr uint32_t kBf16NanPair = 0x7fc07fc0u;

// Eight floats -> eight bf16 (RNE) in one 16-byte store (p 16-byte aligned).
__device__ __forceinline__ void store_bf16x8(uint16_t* p, const float* v) {
  uint32_t w[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) w[m] = f32_to_bf16(v[2 * m]) | (f32_to_bf16(v[2 * m + 1]) << 16);
  *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
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

// Block scale number `idx` of a scale tensor: fp32, or e8m0 bytes (E8).  A
// compile-time format keeps the load free of branches (a branch around a
// load makes the compiler wait for it at the join, serialising the loads).
template <bool E8>
__device__ __forceinline__ float load_scale(const void* s, size_t idx) {
  if (E8) return e8m0_to_f32(static_cast<const uint8_t*>(s)[idx]);
  return static_cast<const float*>(s)[idx];
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// Loads and stores of data that workgroups of one launch hand to each other.
// With C = true they are agent-scope relaxed atomics: the stores write
// through to the device coherence point and the loads read from it, so no
// cache flush or invalidate is needed around the hand-off (see
// wait_memory()).  With C = false they are plain accesses (a kernel
// boundary orders them).
template <bool C>
__device__ __forceinline__ float ld_f32(const float* p) {
  if (C) return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return *p;
}
template <bool C>
__device__ __forceinline__ int ld_i32(const int* p) {
  if (C) return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return *p;
}
template <bool C>
__device__ __forceinline__ void st_f32(float* p, float v) {
  if (C) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else *p = v;
}
template <bool C>
__device__ __forceinline__ void st_u32(uint32_t* p, uint32_t v) {
  if (C) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else *p = v;
}
template <bool C>
__device__ __forceinline__ void st_i32(int* p, int v) {
  if (C) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else *p = v;
}
// 16-byte versions (two 8-byte atomics when C; p must be 16-byte aligned).
template <bool C>
__device__ __forceinline__ float4 ld_f32x4(const float* p) {
  if (C) {
    const auto* q = reinterpret_cast<const unsigned long long*>(p);
    const unsigned long long a = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const unsigned long long b = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return make_float4(__uint_as_float(static_cast<uint32_t>(a)),
                       __uint_as_float(static_cast<uint32_t>(a >> 32)),
                       __uint_as_float(static_cast<uint32_t>(b)),
                       __uint_as_float(static_cast<uint32_t>(b >> 32)));
  }
  return *reinterpret_cast<const float4*>(p);
}
template <bool C>
__device__ __forceinline__ void st_f32x4(float* p, float4 v) {
  if (C) {
    auto* q = reinterpret_cast<unsigned long long*>(p);
    const unsigned long long a = (static_cast<unsigned long long>(__float_as_uint(v.y)) << 32) |
                                 __float_as_uint(v.x);
    const unsigned long long b = (static_cast<unsigned long long>(__float_as_uint(v.w)) << 32) |
                                 __float_as_uint(v.z);
    __hip_atomic_store(q, a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(q + 1, b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else {
    *reinterpret_cast<float4*>(p) = v;
  }
}

// Every lane waits until its earlier memory operations have completed (for
// the coherent stores above: reached the device coherence point).  Also a
// compiler barrier.
__device__ __forceinline__ void wait_memory() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// 1 / (1 + e^-z) with the hardware exponential and reciprocal (about 1 ulp
// each) instead of an IEEE division sequence.
__device__ __forceinline__ float sigmoidf_(float z) {
  return __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

// silu(min(g, L)) * clamp(u, -L, L)
__device__ __forceinline__ float clamped_swiglu(float g, float u, float limit) {
  float gc = fminf(g, limit);
  float uc = fminf(fmaxf(u, -limit), limit);
  return gc * sigmoidf_(gc) * uc;
}

}  // namespace moe
