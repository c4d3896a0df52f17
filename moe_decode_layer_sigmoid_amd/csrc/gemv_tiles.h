// One-wave GEMV tiles of the fp8 expert projections, the router logits and
// the per-token boundary, shared by the separate kernels and the fused
// persistent decode kernel.
//
// Follows the vLLM API page "vllm.models.glm5next.nvidia.specialized_decode.
// runtime.decode" (LayerStages._build_mega: fp8 w13/w2 with block scales,
// swiglu_limit; LayerStages._router: bf16 router weight, fp32 logits) and
// the page "...runtime.draft" (SpecializedDraft.reduced_norm: the boundary
// returns norm(x + residual) and the new residual).
//
// Layout of a wave's work: lanes split a weight row into 16-byte chunks
// (chunk c = lane + 64 j), so every load instruction of the wave reads 1 KiB
// of one row contiguously; all of a wave's weight loads are issued before the
// first one is used.  Weights are read with non-temporal loads: they are
// streamed once per step and should not displace the activations in L2.
#pragma once

#include "device_common.h"
#include "launch.h"

namespace moe {

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// Streamed (read-once) 16-byte load.
__device__ __forceinline__ uint4 ld_stream16(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// 16 fp8 weights (one 16-byte chunk) dotted with 16 floats.
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

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Four e4m3fn codes -> two dwords of bf16 pairs (exact: an e4m3 value has at
// most 4 significant bits, so the top half of its float is the value).
__device__ __forceinline__ void fp8x4_to_bf16x4(uint32_t w, uint32_t* lo, uint32_t* hi) {
  const auto a = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), false);
  const auto b = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), true);
  *lo = __builtin_amdgcn_perm(__float_as_uint(a[1]), __float_as_uint(a[0]), 0x07060302u);
  *hi = __builtin_amdgcn_perm(__float_as_uint(b[1]), __float_as_uint(b[0]), 0x07060302u);
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// Keeps the compiler from hoisting work on `v` out of a loop (the weights
// stay raw fp8 in registers; each token pass converts them again instead of
// holding 4x as many converted registers).
__device__ __forceinline__ void opaque(uint4& v) {
  asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w));
}


// All loads below are branch-free: out-of-range chunks and tokens read a
// clamped, valid address and are masked afterwards.  A load under a branch
// makes the compiler wait for it where the branches join, which serialises
// the loads of a wave; these tiles issue every weight load of the wave
// before the first one is used.

// gate_up + clamped SwiGLU of one wave: SwiGLU outputs i0, i0+1 (i0 even)
// from gate rows i0, i0+1 and up rows I+i0, I+i0+1 of one expert, for its n
// tokens (n >= 1).  Token q is row perm[base+q] / k of hidden (perm ==
// nullptr: row q).  Writes act[(base + q) * I + i0 + {0, 1}].  Products are
// exact (bf16 x e4m3 in the bf16 dot2 unit), sums in fp32.
// NJ = 16-byte chunks per lane per row = ceil(H / 1024); TB = tokens per
// register pass over the loaded weights; C = coherent hand-off of perm/act;
// E8 = e8m0 scales.
template <int NJ, int TB, bool C, bool E8>
__device__ __forceinline__ void gate_up_wave(const uint16_t* __restrict__ hidden,
                                             const uint8_t* __restrict__ W,
                                             const void* __restrict__ scale, size_t sbase, int H,
                                             int I, int i0, int n, const int32_t* perm, int base,
                                             int k, float* __restrict__ act, float limit) {
  const int lane = threadIdx.x & 63;
  const int kb_n = H / kBlock;
  const int nchunk = H / 16;
  const int rows[4] = {i0, i0 + 1, I + i0, I + i0 + 1};
  uint4 wv[4][NJ];
  float sc[2][NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int c = lane + 64 * j;
    const int cc = c < nchunk ? c : nchunk - 1;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      wv[r][j] = ld_stream16(W + static_cast<size_t>(rows[r]) * H + 16 * cc);
    const int kb = cc / 8;
    const float s0 = load_scale<E8>(scale, sbase + static_cast<size_t>(i0 / kBlock) * kb_n + kb);
    const float s1 =
        load_scale<E8>(scale, sbase + static_cast<size_t>((I + i0) / kBlock) * kb_n + kb);
    // a chunk past the row end contributes nothing
    sc[0][j] = c < nchunk ? s0 : 0.f;
    sc[1][j] = c < nchunk ? s1 : 0.f;
  }
  for (int q0 = 0; q0 < n; q0 += TB) {
    int tok[TB];
#pragma unroll
    for (int qq = 0; qq < TB; ++qq) {
      const int q = q0 + qq < n ? q0 + qq : n - 1;
      tok[qq] = perm ? ld_i32<C>(perm + base + q) / k : q;
    }
    float acc[4][TB];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int qq = 0; qq < TB; ++qq) acc[r][qq] = 0.f;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int c = lane + 64 * j;
      const int cc = c < nchunk ? c : nchunk - 1;
      uint32_t xs[TB][8];
#pragma unroll
      for (int qq = 0; qq < TB; ++qq) {
        const uint4* xp =
            reinterpret_cast<const uint4*>(hidden + static_cast<size_t>(tok[qq]) * H + 16 * cc);
        const uint4 a = xp[0], b = xp[1];
        xs[qq][0] = a.x; xs[qq][1] = a.y; xs[qq][2] = a.z; xs[qq][3] = a.w;
        xs[qq][4] = b.x; xs[qq][5] = b.y; xs[qq][6] = b.z; xs[qq][7] = b.w;
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        uint32_t wb[8];
        fp8x4_to_bf16x4(wv[r][j].x, &wb[0], &wb[1]);
        fp8x4_to_bf16x4(wv[r][j].y, &wb[2], &wb[3]);
        fp8x4_to_bf16x4(wv[r][j].z, &wb[4], &wb[5]);
        fp8x4_to_bf16x4(wv[r][j].w, &wb[6], &wb[7]);
#pragma unroll
        for (int qq = 0; qq < TB; ++qq) {
          float p = 0.f;
#pragma unroll
          for (int m = 0; m < 8; ++m) p = dot2_bf16(wb[m], xs[qq][m], p);
          acc[r][qq] = fmaf(sc[r >> 1][j], p, acc[r][qq]);
        }
      }
    }
#pragma unroll
    for (int qq = 0; qq < TB; ++qq) {
      if (q0 + qq >= n) continue;  // uniform: no loads below
      const float g0 = wave_sum(acc[0][qq]), g1 = wave_sum(acc[1][qq]);
      const float u0 = wave_sum(acc[2][qq]), u1 = wave_sum(acc[3][qq]);
      if (lane == 0) {
        float* o = act + static_cast<size_t>(base + q0 + qq) * I + i0;
        st_f32<C>(o, clamped_swiglu(g0, u0, limit));
        st_f32<C>(o + 1, clamped_swiglu(g1, u1, limit));
      }
    }
    if (q0 + TB < n) {
      // another pass follows: keep the raw weights, convert them again
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int j = 0; j < NJ; ++j) opaque(wv[r][j]);
    }
  }
}

// No wait between a tile's weight loads and its first use of activations.
struct NoWait {
  __device__ void operator()() const {}
};

// Where the down output of SwiGLU row `pos` goes: out row route_of(pos).
struct RouteIdentity {  // row pos itself (the shared expert: token pos)
  __device__ int operator()(int pos) const { return pos; }
};
template <bool C>
struct RouteTable {  // perm[pos]: the route index t*k+j (C: coherent load); pos when
                     // perm is null (the shared expert)
  const int32_t* perm;
  __device__ int operator()(int pos) const { return perm ? ld_i32<C>(perm + pos) : pos; }
};
struct RouteFixed {  // one known route (a slot with one route)
  int route;
  __device__ int operator()(int) const { return route; }
};

// down projection of one wave: output rows h0 .. h0+R-1 (h0 % R == 0, R = 4
// or 8) of one expert for its n >= 1 SwiGLU rows act[(base + q) * I],
// written to out[o * H + h0 .. +R-1] with o = route_of(base + q) (the route
// index t*k+j, or base + q).  fp32 products and sums (the SwiGLU activations
// stay fp32).  NJ = ceil(I / 1024); TB, C, E8 as above, C for the stores;
// CL = coherent loads of act.  wait() runs after the weight loads are issued
// and before act is read (a workgroup whose activations come from other
// workgroups of the same launch waits there for them while its weights
// stream in; it must be called by every wave of the workgroup).
template <int NJ, int TB, bool C, bool E8, bool CL = C, typename Wait = NoWait, int R = 4,
          typename RouteOf = RouteIdentity>
__device__ __forceinline__ void down_wave(const uint8_t* __restrict__ W,
                                          const void* __restrict__ scale, size_t sbase, int H,
                                          int I, int h0, int n, int base, RouteOf route_of,
                                          const float* act, float* out, Wait wait = Wait()) {
  static_assert(R == 4 || R == 8, "4 or 8 rows per wave");
  const int lane = threadIdx.x & 63;
  const int ib_n = I / kBlock;
  const int nchunk = I / 16;
  uint4 wv[R][NJ];
  float sc[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int c = lane + 64 * j;
    const int cc = c < nchunk ? c : nchunk - 1;
#pragma unroll
    for (int r = 0; r < R; ++r)
      wv[r][j] = ld_stream16(W + static_cast<size_t>(h0 + r) * I + 16 * cc);
    const float s0 = load_scale<E8>(scale, sbase + static_cast<size_t>(h0 / kBlock) * ib_n + cc / 8);
    sc[j] = c < nchunk ? s0 : 0.f;
  }
  wait();
  for (int q0 = 0; q0 < n; q0 += TB) {
    float acc[R][TB];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int qq = 0; qq < TB; ++qq) acc[r][qq] = 0.f;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int c = lane + 64 * j;
      const int cc = c < nchunk ? c : nchunk - 1;
#pragma unroll
      for (int qq = 0; qq < TB; ++qq) {
        const int q = q0 + qq < n ? q0 + qq : n - 1;
        const float* ap = act + static_cast<size_t>(base + q) * I + 16 * cc;
        float af[16];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const float4 v = ld_f32x4<CL>(ap + 4 * m);
          af[4 * m] = v.x;
          af[4 * m + 1] = v.y;
          af[4 * m + 2] = v.z;
          af[4 * m + 3] = v.w;
        }
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r][qq] = fmaf(sc[j], dot16_fp8(wv[r][j], af), acc[r][qq]);
      }
    }
#pragma unroll
    for (int qq = 0; qq < TB; ++qq) {
      if (q0 + qq >= n) continue;
      float v[R];
#pragma unroll
      for (int r = 0; r < R; ++r) v[r] = wave_sum(acc[r][qq]);
      if (lane == 0) {
        const int o = route_of(base + q0 + qq);
#pragma unroll
        for (int r = 0; r < R; r += 4)
          st_f32x4<C>(out + static_cast<size_t>(o) * H + h0 + r,
                      make_float4(v[r], v[r + 1], v[r + 2], v[r + 3]));
      }
    }
    if (q0 + TB < n) {
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int j = 0; j < NJ; ++j) opaque(wv[r][j]);
    }
  }
}

constexpr int kRouterTokB = 2;  // tokens per register pass of a router wave

// Router logits of one expert row for tokens [0, T) (T >= 1):
// logits[t * E + e] = sum_h hidden[t, h] * router_w[e, h] in fp32.
// The row stays in registers; tokens go in passes of kRouterTokB.
// NJ2 = 16-byte chunks per lane = ceil(H / 512).
// ENC: stored with inverted bits (load_logit); reps copies, rep_stride
// floats apart (pollers spread over the copies).
template <int NJ2, bool C = false, bool ENC = false>
__device__ __forceinline__ void router_wave(const uint16_t* __restrict__ hidden,
                                            const uint16_t* __restrict__ row, int H, int T,
                                            int E, int e, float* logits, int reps = 1,
                                            size_t rep_stride = 0) {
  const int lane = threadIdx.x & 63;
  const int nchunk = H / 8;
  uint4 wv[NJ2];
#pragma unroll
  for (int j = 0; j < NJ2; ++j) {
    const int c = lane + 64 * j;
    const uint4 v = ld_stream16(row + 8 * (c < nchunk ? c : nchunk - 1));
    wv[j] = c < nchunk ? v : make_uint4(0, 0, 0, 0);
  }
#pragma unroll 1
  for (int t0 = 0; t0 < T; t0 += kRouterTokB) {
    float acc[kRouterTokB];
#pragma unroll
    for (int q = 0; q < kRouterTokB; ++q) acc[q] = 0.f;
#pragma unroll
    for (int j = 0; j < NJ2; ++j) {
      const int c = lane + 64 * j;
      const int cc = c < nchunk ? c : nchunk - 1;
      const uint32_t w[4] = {wv[j].x, wv[j].y, wv[j].z, wv[j].w};
#pragma unroll
      for (int q = 0; q < kRouterTokB; ++q) {
        const int t = t0 + q < T ? t0 + q : T - 1;
        const uint4 xv = *reinterpret_cast<const uint4*>(hidden + static_cast<size_t>(t) * H + 8 * cc);
        const uint32_t x[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
        for (int m = 0; m < 4; ++m) acc[q] = dot2_bf16(w[m], x[m], acc[q]);
      }
    }
#pragma unroll
    for (int q = 0; q < kRouterTokB; ++q) {
      if (t0 + q >= T) continue;
      const float v = wave_sum(acc[q]);
      const float stored = ENC ? __uint_as_float(~__float_as_uint(v)) : v;
      if (lane < reps)
        st_f32<C>(logits + lane * rep_stride + static_cast<size_t>(t0 + q) * E + e, stored);
    }
  }
}

constexpr int kEpiPass = 4;  // H <= 8192 = 4 passes x 256 threads x 8

// The boundary for token t, by one 256-thread workgroup:
// h = sum_j w[t, j] * rows[inv[t, j]] + y_s[t] + residual[t] (fixed order),
// residual_out = bf16(h), out = bf16(h / sqrt(mean(h^2) + eps) * gamma).
// s_part: 4 floats of LDS.
constexpr int kEpiGroup = 8;  // routes whose rows one round of loads fetches

// The boundary for token t, by one 256-thread workgroup:
// h = sum_j w[t, j] * rows[t*k + j] + y_s[t] + residual[t] (fixed order),
// residual_out = bf16(h), out = bf16(h / sqrt(mean(h^2) + eps) * gamma),
// and, when moe_out is not null, moe_out = bf16(h - residual) (the sum before
// the residual is added).  Every load of a group of routes is issued before
// any is used.
// s_part: 4 floats of LDS.
// GRP = routes whose rows one round of loads fetches (fewer registers with a
// smaller group).
template <bool C = false, int GRP = kEpiGroup>
__device__ __forceinline__ void epilogue_token(int t, const uint16_t* residual,
                                               const uint16_t* __restrict__ gamma, int H, int k,
                                               bool has_shared, float eps, const Workspace& ws,
                                               uint16_t* out, uint16_t* residual_out,
                                               uint16_t* moe_out, float* s_part) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float* rows_t = ws.rows + static_cast<size_t>(t) * k * H;
  float hv[kEpiPass][8];
  float ss = 0.f;
#pragma unroll
  for (int p = 0; p < kEpiPass; ++p) {
    const int c0 = 8 * (threadIdx.x + 256 * p);
    if (c0 >= H) continue;  // uniform up to the last partial pass
    float acc[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) acc[m] = 0.f;
    for (int j0 = 0; j0 < k; j0 += GRP) {
      float wj[GRP];
      float4 ra[GRP], rb[GRP];
#pragma unroll
      for (int q = 0; q < GRP; ++q) {
        const int j = j0 + q < k ? j0 + q : k - 1;  // clamped: no branch around the loads
        const float w = ld_f32<C>(ws.weights + t * k + j);
        wj[q] = j0 + q < k ? w : 0.f;
        const float* row = rows_t + static_cast<size_t>(j) * H + c0;
        ra[q] = ld_f32x4<C>(row);
        rb[q] = ld_f32x4<C>(row + 4);
      }
#pragma unroll
      for (int q = 0; q < GRP; ++q) {
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
    const float* ys = ws.y_s + static_cast<size_t>(t) * H + c0;
    const float4 ya = ld_f32x4<C>(ys), yb = ld_f32x4<C>(ys + 4);
    const uint4 rv = *reinterpret_cast<const uint4*>(residual + static_cast<size_t>(t) * H + c0);
    if (has_shared) {
      acc[0] += ya.x; acc[1] += ya.y; acc[2] += ya.z; acc[3] += ya.w;
      acc[4] += yb.x; acc[5] += yb.y; acc[6] += yb.z; acc[7] += yb.w;
    }
    if (moe_out) store_bf16x8(moe_out + static_cast<size_t>(t) * H + c0, acc);
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
  __syncthreads();
  const float inv_rms = 1.0f / sqrtf(tot / static_cast<float>(H) + eps);
#pragma unroll
  for (int p = 0; p < kEpiPass; ++p) {
    const int c0 = 8 * (threadIdx.x + 256 * p);
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
    *reinterpret_cast<uint4*>(out + static_cast<size_t>(t) * H + c0) =
        make_uint4(o[0], o[1], o[2], o[3]);
    *reinterpret_cast<uint4*>(residual_out + static_cast<size_t>(t) * H + c0) =
        make_uint4(r[0], r[1], r[2], r[3]);
  }
}

}  // namespace moe
