// Router of the MoE decode layer on gfx950: logits GEMV, sigmoid scores,
// top-k selection with renormalised weights and the token -> expert route
// tables, in one launch.
//
// Follows the vLLM API page "vllm.models.glm5next.nvidia.specialized_decode.
// runtime.decode": LayerStages._router (bf16 router weight, fp32 logits),
// LayerStages._build_mega (sigmoid scoring, one group, normalised top-k,
// routed_scaling_factor) and LayerStages._mega_moe (the route order table
// handed to the boundary with the unfinalized rows).
//
// Grid: x = blocks of 4 experts (one expert row per wave), then, when asked,
// the shared expert's gate_up tiles (8 SwiGLU rows each, grid row 0 only: it
// depends on no routing, so its weights stream while the router waits on
// its memory round trips); y = blocks of TB tokens (router_block_tokens).
// Phase 1: every wave loads its whole bf16 router row at once (one memory
// round trip), dots it with the block's token rows and stores the logits
// with inverted bits.  Phase 2: the last router workgroup of each token
// block polls the block's logits until all are written, ranks its tokens
// (one wave per token) and zeroes the logits again.  Phase 3: the last token
// block to finish (a counter) builds the route tables from per-expert token
// bitmasks in LDS.  Data handed between workgroups goes through coherent
// stores and loads; the counter and the logits reset themselves, so the
// launch replays from a HIP graph.
#include <algorithm>

#include "device_common.h"
#include "gemv_tiles.h"
#include "launch.h"
#include "routing_device.h"
#include "sync_device.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

// NJ2 = 16-byte chunks per lane of a bf16 router row (ceil(H / 512)); E8 =
// e8m0 scales of the shared expert's weights.
template <int NJ2, bool E8>
__global__ __launch_bounds__(kThreads) void router_kernel(
    const uint16_t* __restrict__ hidden, const uint16_t* __restrict__ router_w,
    const float* __restrict__ bias, int T, int TB, int H, int E, int k, float rsf, Workspace ws,
    int32_t* __restrict__ ids_out, float* __restrict__ w_out, int n_router,
    const uint8_t* __restrict__ sw13, const void* __restrict__ sscale, int Is, float limit) {
  // 16-byte aligned: the 64-bit token masks need 8-byte aligned LDS
  // addresses, and dynamic LDS starts right after the static variables.
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __shared__ int s_last;
  const int wave = threadIdx.x >> 6;
  const int t0 = blockIdx.y * TB;
  const int nt = min(TB, T - t0);

  // ---- columns past the router's: the shared expert's gate_up + SwiGLU,
  // which needs no routing and so streams in the router's shadow
  if (static_cast<int>(blockIdx.x) >= n_router) {
    if (blockIdx.y != 0) return;
    constexpr int NJ = (NJ2 + 1) / 2;  // 16-byte fp8 chunks per lane = ceil(H / 1024)
    const int i0 = ((static_cast<int>(blockIdx.x) - n_router) * 4 + wave) * 2;
    if (i0 < Is)
      gate_up_wave<NJ, 1, false, E8>(hidden, sw13, sscale, 0, H, Is, i0, T, nullptr, 0, k,
                                      ws.act_s, limit);
    return;
  }

  // ---- phase 1: logits of this wave's expert for the block's tokens, stored
  // with inverted bits (ws.rlogits reads 0 until a logit is written)
  const int e = blockIdx.x * 4 + wave;
  if (e < E)
    router_wave<NJ2, true, true>(hidden + static_cast<size_t>(t0) * H,
                                 router_w + static_cast<size_t>(e) * H, H, nt, E, e,
                                 ws.rlogits + static_cast<size_t>(t0) * E);
  // The block's last router workgroup ranks its tokens: it polls their
  // logits until every one is written (workgroups of lower index, which the
  // dispatcher starts first; a bounded wait sets the error word), where a
  // counter would cost each producer a store acknowledgement and an atomic
  // before the reader's first load.
  if (static_cast<int>(blockIdx.x) != n_router - 1) return;
  uint32_t* err = ws.sync + static_cast<size_t>(kSyncError) * kSyncStride;

  // ---- phase 2: top-k of the block's tokens (one wave per token), then,
  // once every wave's selection has read them, their logits back to zero
  // for the next launch
  const RouteSmem sm(smem, T, E, k);
  select_tokens<true, true, true>(t0, t0 + nt, E, k, rsf, ws.rlogits, bias, ws, ids_out, w_out,
                                  sm, err);
  __syncthreads();
  for (int i = threadIdx.x; i < nt * E; i += kThreads)
    st_f32<true>(ws.rlogits + static_cast<size_t>(t0) * E + i, 0.f);
  if (gridDim.y > 1) {
    wait_memory();
    __syncthreads();
    uint32_t* top = ws.counter + router_cnt_line(kRouterMaxBlk);
    if (threadIdx.x == 0)
      s_last = __hip_atomic_fetch_add(top, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
               gridDim.y - 1;
    __syncthreads();
    if (!s_last) return;
    if (threadIdx.x == 0) __hip_atomic_store(top, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (int r = threadIdx.x; r < T * k; r += kThreads) sm.ids[r] = ld_i32<true>(ws.ids + r);
  }

  // ---- phase 3: route tables (read by later kernels)
  build_routes<false>(T, E, k, ws, sm);
  // The counters of the launch that follows (the split path's expert chain)
  // start from zero and its boundary slots empty (zero): it never resets
  // them itself.  The error word stays.
  const int lines = sync_lines(T * k < E ? T * k : E);
  for (int i = threadIdx.x; i < lines; i += kThreads)
    if (i != kSyncError)
      __hip_atomic_store(ws.sync + static_cast<size_t>(i) * kSyncStride, 0u, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  for (int i = threadIdx.x; i < T * kMaxBndSlices; i += kThreads)
    __hip_atomic_store(reinterpret_cast<uint32_t*>(ws.epi_part) + i, 0u, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

// Tokens per block: every wave of a block's workgroups loads all of the
// block's token rows, so small blocks shorten the logits phase; larger ones
// read the router weight fewer times (once per block).  With the logits
// polled by each block's selecting workgroup (one wave per token), measured
// on MI355X at E = 128, H = 4096 (us per launch, blocks of 1 / 2 / 4): 16
// tokens 18.3 / 12.3 / 13.8, 8 tokens 10.8 / 11.1 / 12.5, 4 tokens 10.7 /
// 11.6 / 11.8.  So one token per block up to 8 tokens, two up to 16, then
// kRouterTokBlk (blocks of 2 measured slower at 64 and 128 tokens).
int router_block_tokens(int T) { return T <= 8 ? 1 : (T <= 16 ? 2 : kRouterTokBlk); }

// ---------------------------------------------------------------------------
// The router for many tokens on the matrix cores.  The logits are a small
// GEMM, x [T, H] . W_r^T [H, E]; read one row at a time per wave (above),
// every wave re-reads its block's token rows, which at 128 tokens and
// H = 6144 moves hundreds of MB through L2.  Here each workgroup computes a
// tile of 16 tokens x 64 experts (one v_mfma_f32_16x16x32_bf16 per wave per
// 32 columns: bf16 products are exact, sums fp32) over one slice of the
// contraction, so each operand row is read once per tile.  Phases:
//   1 partials   workgroup (expert tile, token tile, slice): the tile's
//                partial logits to ws.rpart[slice][expert][token]; each
//                round's token rows are staged into LDS once for the four
//                waves, which load their own expert rows
//   2 logits     the last slice of a (token tile, expert tile) to finish
//                sums the slices in slice order (deterministic) into
//                ws.logits
//   3 top-k      that workgroup then waits for the token tile's other
//                expert tiles (every workgroup of the launch is resident:
//                the grid is capped at kRtMaxGrid) and ranks its share of
//                the tile's tokens, one token per wave while the share
//                allows
//   4 routes     the last of those to finish builds the route tables and
//                empties the counters of the launch that follows
// Measured on MI355X (rocprofv3, 128 tokens, E = 256, H = 6144): 24.8 us
// with 384 workgroups whose waves each loaded the token rows, 22.9 us with
// the rows staged once per workgroup and one workgroup per CU.  Ranking
// workgroups that sum their token's slices themselves (no logits round
// trip, no wait per expert tile) measured no faster (25.0 us): the launch
// is a chain of dependent memory round trips (partials, counts, logits,
// ids, route tables), not bound by its loads.
// The MFMA takes any one-to-one assignment of contraction columns to lanes
// as long as both operands use it: lane (g, c) holds, for steps 2j and
// 2j + 1, columns 64 j + 16 g + [0, 8) and [8, 16) of its row, so that it
// loads 32 contiguous bytes per two steps (the four lanes of a row cover a
// whole 128-byte line).
// Counts are arrival counters (one 128-byte line each) in ws.rcnt that are
// reset once nothing reads them; partials and logits are handed over with
// write-through stores, read after the count that covers them.
constexpr int kRtTok = 16;     // tokens per tile (MFMA rows)
constexpr int kRtExp = 64;     // experts per workgroup (16 per wave)
constexpr int kRtSteps = 16;   // MFMA steps (32 columns each) per round of loads
constexpr int kRtMaxGrid = 256;  // workgroups: one per CU, all resident at once
constexpr int kRtStageBytes = kRtTok * kRtSteps * 32 * 2;  // a round's token rows (16 KB)
constexpr uint32_t kRtSpin = 1u << 17;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;

__global__ __launch_bounds__(kThreads) void router_mfma_kernel(
    const uint16_t* __restrict__ hidden, const uint16_t* __restrict__ router_w,
    const float* __restrict__ bias, int T, int H, int E, int k, float rsf, int S, int Ks,
    int Tp, int zero_lines, Workspace ws, int32_t* __restrict__ ids_out,
    float* __restrict__ w_out) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __shared__ int s_last;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int et = blockIdx.x, tt = blockIdx.y, sl = blockIdx.z;
  const int n_et = gridDim.x, n_tt = gridDim.y;
  const int t0 = tt * kRtTok;
  const int e0 = et * kRtExp + wave * 16;
  uint32_t* err = ws.sync + kSyncError * kSyncStride;

  // ---- phase 1: partial logits of tokens t0.., experts e0.. over the slice.
  // The token rows of a round (16 x 512 columns) are staged into LDS once for
  // the four waves (double-buffered: one barrier per round); each wave loads
  // its own expert rows into registers.
  {
    const bool live = e0 < E;  // uniform per wave; the others only stage
    const int kb = sl * Ks;
    const int kend = min(H, kb + Ks);
    const int nst = (kend - kb) / 32;  // even: H and Ks are multiples of 64
    // rows past T or E repeat the last one (loads stay in bounds; never stored)
    const uint16_t* wb = router_w + static_cast<size_t>(min(e0 + c, E - 1)) * H + kb + 16 * g;
    // staging: piece L = 256 q + tid of the round's tile is token L / 64, LDS
    // slot L % 64, and fetches 16-byte piece (L % 64) ^ token of that token's
    // 512 columns, so that piece p of token c sits at slot p ^ c
    const uint16_t* xs[4];
    int xcol[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int L = 256 * q + static_cast<int>(threadIdx.x);
      const int tok = L >> 6;
      xs[q] = hidden + static_cast<size_t>(min(t0 + tok, T - 1)) * H;
      xcol[q] = kb + 8 * ((L & 63) ^ tok);
    }
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    for (int r0 = 0, rd = 0; r0 < nst; r0 += kRtSteps, ++rd) {
      unsigned char* stage = smem + (rd & 1) * kRtStageBytes;
#pragma unroll
      for (int q = 0; q < 4; ++q)  // columns past the slice are staged but not used
        __builtin_amdgcn_global_load_lds(xs[q] + min(xcol[q] + 32 * r0, H - 8),
                                         (lds_void_t*)(stage + 4096 * q + 1024 * wave), 16, 0,
                                         0);
      uint4 bv[kRtSteps];
      if (live) {
#pragma unroll
        for (int i = 0; i < kRtSteps; ++i) {
          // step i of the round: columns 64 (i / 2) + 16 g + 8 (i % 2), clamped
          const int st = min(r0 + i, nst - 1);
          bv[i] = *reinterpret_cast<const uint4*>(wb + 64 * (st >> 1) + 8 * (st & 1));
        }
      }
      wait_memory();    // this thread's staged pieces are in LDS
      __syncthreads();  // and every other thread's
      if (live) {
#pragma unroll
        for (int i = 0; i < kRtSteps; ++i)
          if (r0 + i < nst) {  // uniform
            // token c's piece 8 (i / 2) + 2 g + i % 2: the same columns as bv[i]
            const int pc = (8 * (i >> 1) + 2 * g + (i & 1)) ^ c;
            const uint4 av = *reinterpret_cast<const uint4*>(stage + 1024 * c + 16 * pc);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av),
                                                          __builtin_bit_cast(bf16x8_t, bv[i]),
                                                          acc, 0, 0, 0);
          }
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS reads are done
    }
    // lane holds tokens t0 + 4g .. +3 of expert e0 + c
    if (live && e0 + c < E)
      st_f32x4<true>(ws.rpart + (static_cast<size_t>(sl) * E + e0 + c) * Tp + t0 + 4 * g,
                     make_float4(acc[0], acc[1], acc[2], acc[3]));
  }
  wait_memory();
  __syncthreads();
  uint32_t* cnt1 = ws.rcnt + static_cast<size_t>(tt * n_et + et) * kSyncStride;
  if (threadIdx.x == 0)
    s_last = __hip_atomic_fetch_add(cnt1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
             static_cast<uint32_t>(S) - 1;
  __syncthreads();
  if (!s_last) return;

  // ---- phase 2: the tile's logits, slices summed in slice order; thread:
  // expert et * 64 + tid / 4, tokens t0 + 4 (tid % 4) .. +3
  if (threadIdx.x == 0) __hip_atomic_store(cnt1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  {
    const int e = et * kRtExp + static_cast<int>(threadIdx.x >> 2);
    const int tq = t0 + 4 * static_cast<int>(threadIdx.x & 3);
    if (e < E) {
      float4 v[16];
#pragma unroll
      for (int i = 0; i < 16; ++i)  // S <= 16; clamped, masked below
        v[i] = *reinterpret_cast<const float4*>(
            ws.rpart + (static_cast<size_t>(i < S ? i : S - 1) * E + e) * Tp + tq);
      float4 sum = v[0];
#pragma unroll
      for (int i = 1; i < 16; ++i)
        if (i < S) {
          sum.x += v[i].x; sum.y += v[i].y; sum.z += v[i].z; sum.w += v[i].w;
        }
      const float r[4] = {sum.x, sum.y, sum.z, sum.w};
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (tq + i < T) st_f32<true>(ws.logits + static_cast<size_t>(tq + i) * E + e, r[i]);
    }
  }

  // ---- phase 3: once every expert tile of the token tile has its logits,
  // this workgroup ranks tokens t0 + et, t0 + et + n_et, ... (one per wave)
  uint32_t* cnt2 = ws.rcnt + static_cast<size_t>(n_tt * n_et + tt) * kSyncStride;
  bump(Sync{cnt2}, 0);
  wait_count(Sync{cnt2}, 0, 1, static_cast<uint32_t>(n_et), kRtSpin, err);
  const RouteSmem sm(smem, T, E, k);
  {
    unsigned long long* sel = sm.sel + static_cast<size_t>(wave) * kSelWaveWords;
    for (int j = wave; et + j * n_et < kRtTok; j += kThreads / 64) {
      const int t = t0 + et + j * n_et;
      if (t >= T) break;  // uniform
      int id = 0;
      float w = 0.f;
      select_token<true>(ws.logits + static_cast<size_t>(t) * E, bias, E, k, rsf, sel, &id, &w);
      if (lane < k) {
        const int r = t * k + lane;
        st_i32<true>(ws.ids + r, id);
        st_f32<true>(ws.weights + r, w);
        if (ids_out) ids_out[r] = id;
        if (w_out) w_out[r] = w;
      }
    }
  }
  wait_memory();
  __syncthreads();
  uint32_t* top = ws.rcnt + static_cast<size_t>(n_tt * n_et + n_tt) * kSyncStride;
  if (threadIdx.x == 0)
    s_last = __hip_atomic_fetch_add(top, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
             static_cast<uint32_t>(n_tt * n_et) - 1;
  __syncthreads();
  if (!s_last) return;

  // ---- phase 4: route tables (read by later kernels); every other
  // workgroup is past its waits, so the tile counts reset here
  for (int i = threadIdx.x; i <= n_tt; i += kThreads)
    __hip_atomic_store(ws.rcnt + static_cast<size_t>(n_tt * n_et + i) * kSyncStride, 0u,
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  for (int r = threadIdx.x; r < T * k; r += kThreads) sm.ids[r] = ld_i32<true>(ws.ids + r);
  build_routes<false>(T, E, k, ws, sm);
  // the counters and boundary slots of the grouped merged launch that
  // follows (zero_lines of them; none when separate launches follow)
  for (int i = threadIdx.x; i < zero_lines; i += kThreads)
    if (i != kSyncError)
      __hip_atomic_store(ws.sync + static_cast<size_t>(i) * kSyncStride, 0u, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  if (zero_lines > 0)
    for (int i = threadIdx.x; i < T * kMaxBndSlices; i += kThreads)
      __hip_atomic_store(reinterpret_cast<uint32_t*>(ws.epi_part) + i, 0u, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace

int router_mfma_tokens_padded(int T) { return (T + kRtTok - 1) / kRtTok * kRtTok; }
int router_mfma_count_lines(int T, int E) {
  const int n_tt = (T + kRtTok - 1) / kRtTok, n_et = (E + kRtExp - 1) / kRtExp;
  return n_tt * n_et + n_tt + 1;
}
// Contraction slices: one per 512 columns, fewer where the grid would pass
// kRtMaxGrid (at most 16: H <= 8192).
int router_mfma_slices(int T, int E, int H) {
  const int tiles = ((T + kRtTok - 1) / kRtTok) * ((E + kRtExp - 1) / kRtExp);
  int S = (H + 511) / 512;
  const int cap = kRtMaxGrid / tiles;
  if (S > cap) S = cap > 1 ? cap : 1;
  return S;
}

hipError_t launch_router_mfma(const LayerDims& d, const void* hidden, const void* router_w,
                              const float* bias, const Workspace& ws, int Tp_alloc,
                              int zero_lines, int32_t* ids_out, float* weights_out,
                              hipStream_t s) {
  const int S = router_mfma_slices(d.T, d.E, d.H);
  // slice width: a multiple of 64 columns
  const int Ks = ((d.H + S - 1) / S + 63) / 64 * 64;
  const int n_tt = (d.T + kRtTok - 1) / kRtTok, n_et = (d.E + kRtExp - 1) / kRtExp;
  if (d.T < 1 || d.E < 1 || d.k < 1 || d.H % 64 || S > 16 || n_tt * n_et * S > kRtMaxGrid ||
      router_mfma_tokens_padded(d.T) > Tp_alloc)
    return hipErrorInvalidValue;
  dim3 grid(n_et, n_tt, (d.H + Ks - 1) / Ks);
  // the staged token rows (two rounds), or the routing step's scratch after them
  const size_t smem =
      std::max(route_smem_bytes(d.T, d.E, d.k), 2 * static_cast<size_t>(kRtStageBytes));
  hipLaunchKernelGGL(router_mfma_kernel, grid, dim3(kThreads), smem, s,
                     static_cast<const uint16_t*>(hidden), static_cast<const uint16_t*>(router_w),
                     bias, d.T, d.H, d.E, d.k, d.rsf, static_cast<int>(grid.z), Ks, Tp_alloc,
                     zero_lines, ws, ids_out, weights_out);
  return hipGetLastError();
}

hipError_t launch_router(const LayerDims& d, const void* hidden, const void* router_w,
                         const float* bias, const Workspace& ws, int32_t* ids_out,
                         float* weights_out, const void* sw13, const void* sw13_scale,
                         hipStream_t s, hipEvent_t evb, hipEvent_t eve) {
  if (d.T > kRouterMaxBlk * kRouterTokBlk) return hipErrorInvalidValue;
  const int n_router = (d.E + 3) / 4;
  const int n_shared = sw13 && d.Is > 0 ? d.Is / 8 : 0;  // 8 SwiGLU rows per workgroup
  const int TB = router_block_tokens(d.T);
  // no routed experts (a dense layer): only the gate_up tiles, one grid row
  dim3 grid(n_router + n_shared, d.E > 0 ? (d.T + TB - 1) / TB : 1);
  const size_t smem = route_smem_bytes(d.T, d.E, d.k);
  const auto* x = static_cast<const uint16_t*>(hidden);
  const auto* w = static_cast<const uint16_t*>(router_w);
  const auto* sw = static_cast<const uint8_t*>(sw13);
  const int Is = n_shared ? d.Is : 0;
  switch (((d.H + 511) / 512) * 2 + (d.e8m0 ? 1 : 0)) {
#define X(N)                                                                                   \
  case 2 * N:                                                                                  \
    MOE_LAUNCH((router_kernel<N, false>), grid, dim3(kThreads), smem, s, evb, eve, x, w, bias, \
               d.T, TB, d.H, d.E, d.k, d.rsf, ws, ids_out, weights_out, n_router, sw,          \
               sw13_scale, Is, d.limit);                                                       \
    break;                                                                                     \
  case 2 * N + 1:                                                                              \
    MOE_LAUNCH((router_kernel<N, true>), grid, dim3(kThreads), smem, s, evb, eve, x, w, bias,  \
               d.T, TB, d.H, d.E, d.k, d.rsf, ws, ids_out, weights_out, n_router, sw,          \
               sw13_scale, Is, d.limit);                                                       \
    break;
    X(1) X(2) X(3) X(4) X(5) X(6) X(7) X(8) X(9) X(10) X(11) X(12) X(13) X(14) X(15) X(16)
#undef X
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace moe
