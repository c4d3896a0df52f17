// The boundary of the decode layer as workgroups of a launch that also runs
// the projections (the expert chain, the single-launch step, the grouped
// merged launch): the weighted combine of a token's routed rows, the shared
// expert and the residual, then RMSNorm * gamma, over column slices of the
// token whose sums of squares the slices exchange.
//
// Follows the vLLM API page "vllm.models.glm5next.nvidia.specialized_decode.
// runtime.draft", SpecializedDraft.reduced_norm (norm(x + residual) with the
// new residual) and page "...runtime.decode", LayerStages._mega_moe (the
// shared expert's output added beside the weighted routed rows).
#pragma once

#include "device_common.h"
#include "launch.h"

namespace moe {

constexpr int kBndThreads = 256;  // threads of a boundary workgroup (4 or 8 columns each)
constexpr int kBndWaves = kBndThreads / kWave;
// Polls before the slices' exchange gives up (a poll is a memory round trip
// plus a short sleep; a legitimate wait lasts microseconds).
constexpr uint32_t kBndSpin = 1u << 17;

// N bf16 (N = 4 or 8, 8- or 16-byte aligned) as N / 2 packed pairs, and back.
template <int N>
__device__ __forceinline__ void load_bf16_pairs(const uint16_t* p, uint32_t* u) {
  if constexpr (N == 8) {
    const uint4 v = *reinterpret_cast<const uint4*>(p);
    u[0] = v.x; u[1] = v.y; u[2] = v.z; u[3] = v.w;
  } else {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    u[0] = v.x; u[1] = v.y;
  }
}
template <int N>
__device__ __forceinline__ void store_bf16_pairs(uint16_t* p, const uint32_t* u) {
  if constexpr (N == 8)
    *reinterpret_cast<uint4*>(p) = make_uint4(u[0], u[1], u[2], u[3]);
  else
    *reinterpret_cast<uint2*>(p) = make_uint2(u[0], u[1]);
}

// What a boundary slice reads and writes besides the workspace rows.
struct BndArgs {
  const uint16_t* residual;
  const uint16_t* gamma;
  uint16_t* out;
  uint16_t* residual_out;
  uint16_t* moe_out;  // nullable
  int H, k, Is, ns;   // ns = slices per token
  float eps;
  float* part;        // [T][kMaxBndSlices] slice sums of squares, inverted bits (0 = empty)
  uint32_t* err;      // the error word
};

// What the step launch's last boundary slice clears for the next launch.
struct StepTail {
  uint32_t* bnd;      // the boundary slices' count (msync line kStepBnd)
  uint32_t total;     // boundary slices of the launch
  uint32_t* sync;     // msync
  int sync_lines;
  float* logits;      // mlogits, n_logits words
  int n_logits;
  int n_part;         // words of the boundary slots
};

// The boundary of token t, columns [CPT kBndThreads s, + CPT kBndThreads)
// (CPT = 4 or 8 per thread), by one of the token's ns workgroups: h = sum_j w[t, j] * rows[t*k + j]
// + y_s[t] + residual[t] (fixed order; with moe_out, the sum before the
// residual goes there too); the slice's sum of squares (waves in order) goes
// to part[t][s] as inverted bits; once every slice of the token is in, their
// sums in slice order give the RMS, and the slice of residual_out = bf16(h),
// out = bf16(h / sqrt(mean(h^2) + eps) * gamma) is written (NaN if a bounded
// wait of the launch gave up).  The loads that do not depend on the down rows
// are issued before `wait`: the residual, gamma and, in the chain launch,
// the top-k weights (the step launch writes those itself, so it loads them
// after the wait, coherently); the rest of the slice's loads all before
// their first use.  STEP: the step launch's slice, which afterwards counts
// itself done, and the last one clears the launch's state (`tail`).
template <bool STEP, int CPT, typename Wait>
__device__ __forceinline__ void boundary_slice(const BndArgs& b, const Workspace& ws, int t,
                                               int s, Wait wait, const StepTail& tail) {
  __shared__ float s_part[kBndWaves];
  __shared__ float s_tot[kMaxBndSlices];
  __shared__ uint32_t s_bad;
  __shared__ int s_last;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int H = b.H, k = b.k, ns = b.ns;
  static_assert(CPT == 4 || CPT == 8, "4 or 8 columns per thread");
  constexpr int NQ = CPT / 4;  // float4 per routed row piece
  const int c = CPT * (kBndThreads * s + static_cast<int>(threadIdx.x));
  const bool live = c < H;
  const int c0 = live ? c : H - CPT;  // clamped: loads stay in the row
  // residual and gamma, CPT / 2 pairs of bf16
  uint32_t rv[CPT / 2], gv[CPT / 2];
  load_bf16_pairs<CPT>(b.residual + static_cast<size_t>(t) * H + c0, rv);
  load_bf16_pairs<CPT>(b.gamma + c0, gv);
  float wts[kMaxTopK];
  if (!STEP) {
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) wts[j] = ws.weights[t * k + (j < k ? j : k - 1)];
  }
  wait();
  if (STEP) {
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) wts[j] = ld_f32<true>(ws.weights + t * k + (j < k ? j : k - 1));
  }
  const float* rows_t = ws.rows + static_cast<size_t>(t) * k * H + c0;
  const float* ys = ws.y_s + static_cast<size_t>(t) * H + c0;
  float4 yv[NQ];
#pragma unroll
  for (int h = 0; h < NQ; ++h) yv[h] = *reinterpret_cast<const float4*>(ys + 4 * h);
  float acc[CPT];
#pragma unroll
  for (int m = 0; m < CPT; ++m) acc[m] = 0.f;
#pragma unroll
  for (int j0 = 0; j0 < kMaxTopK; j0 += 8) {
    if (j0 >= k) break;  // uniform
    float4 r[8][NQ];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int j = j0 + q < k ? j0 + q : k - 1;  // clamped: no branch around the loads
#pragma unroll
      for (int h = 0; h < NQ; ++h)
        r[q][h] = *reinterpret_cast<const float4*>(rows_t + static_cast<size_t>(j) * H + 4 * h);
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const float w = j0 + q < k ? wts[j0 + q] : 0.f;
#pragma unroll
      for (int h = 0; h < NQ; ++h) {
        acc[4 * h + 0] = fmaf(w, r[q][h].x, acc[4 * h + 0]);
        acc[4 * h + 1] = fmaf(w, r[q][h].y, acc[4 * h + 1]);
        acc[4 * h + 2] = fmaf(w, r[q][h].z, acc[4 * h + 2]);
        acc[4 * h + 3] = fmaf(w, r[q][h].w, acc[4 * h + 3]);
      }
    }
  }
  if (b.Is > 0) {
#pragma unroll
    for (int h = 0; h < NQ; ++h) {
      acc[4 * h + 0] += yv[h].x;
      acc[4 * h + 1] += yv[h].y;
      acc[4 * h + 2] += yv[h].z;
      acc[4 * h + 3] += yv[h].w;
    }
  }
  if (b.moe_out && live) {
    uint32_t w[CPT / 2];
#pragma unroll
    for (int m = 0; m < CPT / 2; ++m)
      w[m] = f32_to_bf16(acc[2 * m]) | (f32_to_bf16(acc[2 * m + 1]) << 16);
    store_bf16_pairs<CPT>(b.moe_out + static_cast<size_t>(t) * H + c, w);
  }
#pragma unroll
  for (int m = 0; m < CPT / 2; ++m) {
    acc[2 * m] += bf16_lo(rv[m]);
    acc[2 * m + 1] += bf16_hi(rv[m]);
  }
  float ss = 0.f;
#pragma unroll
  for (int m = 0; m < CPT; ++m) ss = fmaf(acc[m], acc[m], ss);
  ss = wave_sum(live ? ss : 0.f);
  if (lane == 0) s_part[wave] = ss;
  __syncthreads();
  float* part = b.part + t * kMaxBndSlices;
  if (wave == 0) {
    // publish this slice's sum (no wait for the store), then poll the token's
    // slices, one lane each, until none is empty; lane 63 reads the error
    // word in the same round trips
    if (lane == 0) {
      const float mine = (s_part[0] + s_part[1]) + (s_part[2] + s_part[3]);
      st_u32<true>(reinterpret_cast<uint32_t*>(part + s), ~__float_as_uint(mine));
    }
    const float* src = lane < ns ? part + lane
                                 : (lane == 63 ? reinterpret_cast<const float*>(b.err) : part);
    uint32_t polls = 0;
    uint32_t v = 0;
    for (;;) {
      v = __float_as_uint(ld_f32<true>(src));
      const bool in = lane >= ns || v != 0u;
      if (__builtin_amdgcn_ballot_w64(!in) == 0) break;  // uniform over the wave
      __builtin_amdgcn_s_sleep(1);
      if (++polls == kBndSpin) {
        if (lane == 0) __hip_atomic_fetch_or(b.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
    }
    if (lane < ns) s_tot[lane] = __uint_as_float(~v);
    if (lane == 63) s_bad = (v != 0u || polls == kBndSpin) ? 1u : 0u;
  }
  __syncthreads();
  // step launch: this slice is done with the shared state; the count comes
  // back while the outputs are computed and stored
  uint32_t prev = 0;
  if (STEP && threadIdx.x == 0)
    prev = __hip_atomic_fetch_add(tail.bnd, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const bool gave_up = s_bad != 0u;
  float tot = 0.f;
  for (int i = 0; i < ns; ++i) tot += s_tot[i];
  const float inv_rms = 1.0f / sqrtf(tot / static_cast<float>(H) + b.eps);
  if (live) {
    uint32_t o[CPT / 2], r[CPT / 2];
#pragma unroll
    for (int m = 0; m < CPT / 2; ++m) {
      const float h0 = acc[2 * m], h1 = acc[2 * m + 1];
      o[m] = f32_to_bf16(h0 * inv_rms * bf16_lo(gv[m])) |
             (f32_to_bf16(h1 * inv_rms * bf16_hi(gv[m])) << 16);
      r[m] = f32_to_bf16(h0) | (f32_to_bf16(h1) << 16);
      if (gave_up) o[m] = kBf16NanPair;
    }
    store_bf16_pairs<CPT>(b.out + static_cast<size_t>(t) * H + c, o);
    store_bf16_pairs<CPT>(b.residual_out + static_cast<size_t>(t) * H + c, r);
  }
  if (STEP) {
    if (threadIdx.x == 0) s_last = prev + 1 == tail.total;
    __syncthreads();
    if (s_last) {
      // every other workgroup of the launch is past its last use of these
      for (int i = threadIdx.x; i < tail.sync_lines; i += kBndThreads)
        st_u32<true>(tail.sync + static_cast<size_t>(i) * kSyncStride, 0u);
      for (int i = threadIdx.x; i < tail.n_logits; i += kBndThreads)
        st_u32<true>(reinterpret_cast<uint32_t*>(tail.logits) + i, 0u);
      for (int i = threadIdx.x; i < tail.n_part; i += kBndThreads)
        st_u32<true>(reinterpret_cast<uint32_t*>(b.part) + i, 0u);
    }
  }
}

}  // namespace moe
