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
#include "launch.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kTokB = 4;  // tokens per register pass over the loaded weights

// Per-slot expert, token count and permuted base position.
struct SlotInfo {
  int e, n, base;
};

__device__ __forceinline__ bool slot_info(bool shared, int T, const Workspace& ws, SlotInfo* si) {
  if (shared) {
    *si = {0, T, 0};
    return true;
  }
  const int d = blockIdx.y;
  if (d >= *ws.n_touched) return false;
  const int e = ws.touched[d];
  *si = {e, ws.counts[e], ws.offsets[e]};
  return true;
}

__device__ __forceinline__ float dot16_fp8(const uint4& w, const float* x) {
  float wf[16];
  fp8x4_to_f32(w.x, wf);
  fp8x4_to_f32(w.y, wf + 4);
  fp8x4_to_f32(w.z, wf + 8);
  fp8x4_to_f32(w.w, wf + 12);
  float p = 0.f;
#pragma unroll
  for (int m = 0; m < 16; ++m) p = fmaf(wf[m], x[m], p);
  return p;
}

// NJ: 16-byte chunks per lane per weight row = ceil(H / 1024).
// Each wave computes two SwiGLU outputs i0, i0+1 from the gate rows i0, i0+1
// and the up rows I+i0, I+i0+1 (one scale row-block each).
template <int NJ>
__global__ __launch_bounds__(kThreads) void gate_up_kernel(
    const uint16_t* __restrict__ hidden, const uint8_t* __restrict__ w13,
    const void* __restrict__ scale, int e8m0, int H, int I, int k, int T, int shared,
    Workspace ws, float limit) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i0 = (blockIdx.x * kWaves + wave) * 2;
  SlotInfo si;
  if (!slot_info(shared, T, ws, &si) || i0 >= I) return;
  const size_t rows_per_e = static_cast<size_t>(2) * I;
  const uint8_t* W = w13 + static_cast<size_t>(si.e) * rows_per_e * H;
  const int kb_n = H / kBlock;
  const size_t sbase = static_cast<size_t>(si.e) * (rows_per_e / kBlock) * kb_n;
  const int nchunk = H / 16;
  const int rows[4] = {i0, i0 + 1, I + i0, I + i0 + 1};

  uint4 wv[4][NJ];
  float sc[2][NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int c = lane + 64 * j;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      wv[r][j] = c < nchunk
                     ? *reinterpret_cast<const uint4*>(W + static_cast<size_t>(rows[r]) * H + 16 * c)
                     : make_uint4(0, 0, 0, 0);
    const int kb = min(c, nchunk - 1) / 8;
    sc[0][j] = load_scale(scale, e8m0, sbase + static_cast<size_t>(i0 / kBlock) * kb_n + kb);
    sc[1][j] = load_scale(scale, e8m0, sbase + static_cast<size_t>((I + i0) / kBlock) * kb_n + kb);
  }

  float* act = shared ? ws.act_s : ws.act;
  for (int q0 = 0; q0 < si.n; q0 += kTokB) {
    int tok[kTokB];
#pragma unroll
    for (int qq = 0; qq < kTokB; ++qq) {
      const int q = q0 + qq;
      tok[qq] = q < si.n ? (shared ? q : ws.perm[si.base + q] / k) : -1;
    }
    float acc[4][kTokB];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int qq = 0; qq < kTokB; ++qq) acc[r][qq] = 0.f;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int c = lane + 64 * j;
      if (c >= nchunk) continue;
#pragma unroll
      for (int qq = 0; qq < kTokB; ++qq) {
        if (tok[qq] < 0) continue;
        const uint4* xp =
            reinterpret_cast<const uint4*>(hidden + static_cast<size_t>(tok[qq]) * H + 16 * c);
        const uint4 xa = xp[0], xb = xp[1];
        const uint32_t u[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
        float xf[16];
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          xf[2 * m] = bf16_lo(u[m]);
          xf[2 * m + 1] = bf16_hi(u[m]);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r][qq] = fmaf(sc[r >> 1][j], dot16_fp8(wv[r][j], xf), acc[r][qq]);
      }
    }
#pragma unroll
    for (int qq = 0; qq < kTokB; ++qq) {
      if (tok[qq] < 0) continue;
      const float g0 = wave_sum(acc[0][qq]), g1 = wave_sum(acc[1][qq]);
      const float u0 = wave_sum(acc[2][qq]), u1 = wave_sum(acc[3][qq]);
      if (lane == 0) {
        float* o = act + static_cast<size_t>(si.base + q0 + qq) * I + i0;
        o[0] = clamped_swiglu(g0, u0, limit);
        o[1] = clamped_swiglu(g1, u1, limit);
      }
    }
  }
}

// NJ: 16-byte chunks per lane per w2 row = ceil(I / 1024).
// Each wave computes four output rows h0 .. h0+3 (one scale row-block).
template <int NJ>
__global__ __launch_bounds__(kThreads) void down_kernel(
    const uint8_t* __restrict__ w2, const void* __restrict__ scale, int e8m0, int H, int I,
    int T, int shared, Workspace ws) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h0 = (blockIdx.x * kWaves + wave) * 4;
  SlotInfo si;
  if (!slot_info(shared, T, ws, &si) || h0 >= H) return;
  const uint8_t* W = w2 + static_cast<size_t>(si.e) * H * I;
  const int ib_n = I / kBlock;
  const size_t sbase = static_cast<size_t>(si.e) * (H / kBlock) * ib_n;
  const int nchunk = I / 16;

  uint4 wv[4][NJ];
  float sc[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int c = lane + 64 * j;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      wv[r][j] = c < nchunk
                     ? *reinterpret_cast<const uint4*>(W + static_cast<size_t>(h0 + r) * I + 16 * c)
                     : make_uint4(0, 0, 0, 0);
    sc[j] = load_scale(scale, e8m0, sbase + static_cast<size_t>(h0 / kBlock) * ib_n +
                                        min(c, nchunk - 1) / 8);
  }

  const float* act = shared ? ws.act_s : ws.act;
  float* out = shared ? ws.y_s : ws.rows;
  for (int q0 = 0; q0 < si.n; q0 += kTokB) {
    const int nq = min(kTokB, si.n - q0);
    float acc[4][kTokB];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int qq = 0; qq < kTokB; ++qq) acc[r][qq] = 0.f;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int c = lane + 64 * j;
      if (c >= nchunk) continue;
#pragma unroll
      for (int qq = 0; qq < kTokB; ++qq) {
        if (qq >= nq) continue;
        const float4* ap =
            reinterpret_cast<const float4*>(act + static_cast<size_t>(si.base + q0 + qq) * I + 16 * c);
        float af[16];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const float4 v = ap[m];
          af[4 * m] = v.x;
          af[4 * m + 1] = v.y;
          af[4 * m + 2] = v.z;
          af[4 * m + 3] = v.w;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r][qq] = fmaf(sc[j], dot16_fp8(wv[r][j], af), acc[r][qq]);
      }
    }
#pragma unroll
    for (int qq = 0; qq < kTokB; ++qq) {
      if (qq >= nq) continue;
      float v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = wave_sum(acc[r][qq]);
      if (lane == 0) {
        float4* o = reinterpret_cast<float4*>(out + static_cast<size_t>(si.base + q0 + qq) * H + h0);
        *o = make_float4(v[0], v[1], v[2], v[3]);
      }
    }
  }
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
  switch (nj) {
#define X(N)                                                                                  \
  case N:                                                                                     \
    hipLaunchKernelGGL(gate_up_kernel<N>, grid, dim3(kThreads), 0, s, x, w, w13_scale,        \
                       static_cast<int>(d.e8m0), d.H, I, d.k, d.T, static_cast<int>(shared), ws, \
                       d.limit);                                                              \
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
  switch (nj) {
#define X(N)                                                                                  \
  case N:                                                                                     \
    hipLaunchKernelGGL(down_kernel<N>, grid, dim3(kThreads), 0, s, w, w2_scale,               \
                       static_cast<int>(d.e8m0), d.H, I, d.T, static_cast<int>(shared), ws); \
    break;
    MOE_NJ_CASES(X)
#undef X
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace moe
