// The expert projections and the boundary of a few-token decode step in one
// launch on gfx950 (after the router launch).
//
// Follows the vLLM API page "vllm.models.glm5next.nvidia.specialized_decode.
// runtime.decode": LayerStages._build_mega (fp8 w13 / w2 with 128x128 block
// scales, swiglu_limit), LayerStages._mega_moe (the shared expert beside the
// routed experts; the boundary receives the unfinalized rows with the route
// order) and the page "...runtime.draft", SpecializedDraft.reduced_norm
// (norm(x + residual) with the new residual).
//
// At one token the step is a chain of short weight streams (gate_up 100 MB,
// down 57 MB at the 4096 x 1536 decode shape).  As separate launches each
// pays its own ramp and tail; here one launch streams them back to back, one
// workgroup per item, in this order of workgroup index:
//   shared down      32 output rows of the shared expert (16 when I_s >
//                    2048; its SwiGLU rows come from the router launch)
//   routed gate_up   8 SwiGLU rows of one touched slot
//   routed down      32 (or 16) output rows of one touched slot; it issues its weight
//                    loads first and then waits for the slot's gate_up
//                    count, so the down weights stream while gate_up ends
//   boundary         the last T * ceil(H / 2048) workgroups: after every
//                    down item, combine + shared + residual of a 2048-column
//                    slice of one token, the slices' sums of squares
//                    exchanged, then RMSNorm * gamma of the slice
// The down items read the SwiGLU rows, and the boundary the down rows, with
// plain (L2-cached) loads: they are written with write-through stores that
// complete before the writer's count is bumped, the L2s hold no line of them
// when the launch starts (every launch begins with an L2 invalidate), and no
// workgroup touches them (whole 128-byte lines per slot and per route) before
// the count that covers them is complete.  Coherent loads instead would
// fetch a slot's SwiGLU rows from memory once per down workgroup (50 MB at
// one token, as much as the down weights).
// A workgroup waits only for workgroups of lower index, which the dispatcher
// has started before it (workgroups are dispatched in index order), so
// every wait ends; waits are bounded anyway (a sticky error word,
// moe_decode_check_waits).  Completion counts are bumped with atomics whose
// result is not used (no workgroup waits for them); the router launch that
// precedes every chain launch zeroes them (and arms the boundary's slots).  SwiGLU rows and down rows are
// written with agent-scope atomic stores (sync_device.h).
#include "device_common.h"
#include "gemv_tiles.h"
#include "launch.h"
#include "sync_device.h"

namespace moe {
namespace chain {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
// Output rows per wave of a down item: 8 while a w2 row takes at most two
// 16-byte chunks per lane (the weights then hold as many registers as a
// gate_up wave's), else 4.
__host__ __device__ constexpr int rows_dn_wave(int njd) { return njd <= 2 ? 8 : 4; }
constexpr int kRowsGu = 2 * kWaves;  // SwiGLU rows per gate_up item
constexpr int kMaxNjd = 4;           // I, I_s <= 4096
constexpr int kMaxSlots = kChainMaxTokens * kMaxTopK;
// Polls before a wait gives up: a legitimate wait here lasts microseconds
// (a poll is a memory round trip plus a short sleep).
constexpr uint32_t kChainSpin = 1u << 17;

template <int NJG, int NJD, bool E8>
hipError_t launch_t(const ChainArgs& a, const Workspace& ws, hipStream_t s, hipEvent_t evb,
                    hipEvent_t eve);

#ifdef MOE_CHAIN_NJG
// The boundary of token t, columns [kBndCols * s, +kBndCols) (8 per thread),
// by one of the token's bnd_ns workgroups: h = sum_j w[t, j] * rows[t*k + j]
// + y_s[t] + residual[t] (fixed order; with moe_out, the sum before the
// residual goes there too); the slice's sum of squares (waves in
// order) goes to ws.epi_part[t][s], which the router launch armed with
// kEpiEmpty; once every slice of the token is in, their sums in slice order
// give the RMS, and the slice of residual_out = bf16(h), out = bf16(h /
// sqrt(mean(h^2) + eps) * gamma) is written.  The loads that do not depend on
// the down rows (top-k weights, residual, gamma) are issued before `wait`;
// the rest of the slice's loads all before their first use.
template <typename Wait>
__device__ __forceinline__ void boundary_slice(const ChainArgs& a, const Workspace& ws, int t,
                                               int s, float* s_part, float* s_tot, Wait wait) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int H = a.H, k = a.k, ns = a.bnd_ns;
  const int c = kBndCols * s + 8 * static_cast<int>(threadIdx.x);
  const bool live = c < H;
  const int c0 = live ? c : H - 8;  // clamped: loads stay in the row
  const uint4 rv = *reinterpret_cast<const uint4*>(a.residual + static_cast<size_t>(t) * H + c0);
  const uint4 gv = *reinterpret_cast<const uint4*>(a.gamma + c0);
  float wts[kMaxTopK];
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) wts[j] = ws.weights[t * k + (j < k ? j : k - 1)];
  wait();
  const float* rows_t = ws.rows + static_cast<size_t>(t) * k * H + c0;
  const float* ys = ws.y_s + static_cast<size_t>(t) * H + c0;
  const float4 ya = *reinterpret_cast<const float4*>(ys);
  const float4 yb = *reinterpret_cast<const float4*>(ys + 4);
  float acc[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) acc[m] = 0.f;
#pragma unroll
  for (int j0 = 0; j0 < kMaxTopK; j0 += 8) {
    if (j0 >= k) break;  // uniform
    float4 ra[8], rb[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int j = j0 + q < k ? j0 + q : k - 1;  // clamped: no branch around the loads
      ra[q] = *reinterpret_cast<const float4*>(rows_t + static_cast<size_t>(j) * H);
      rb[q] = *reinterpret_cast<const float4*>(rows_t + static_cast<size_t>(j) * H + 4);
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const float w = j0 + q < k ? wts[j0 + q] : 0.f;
      acc[0] = fmaf(w, ra[q].x, acc[0]);
      acc[1] = fmaf(w, ra[q].y, acc[1]);
      acc[2] = fmaf(w, ra[q].z, acc[2]);
      acc[3] = fmaf(w, ra[q].w, acc[3]);
      acc[4] = fmaf(w, rb[q].x, acc[4]);
      acc[5] = fmaf(w, rb[q].y, acc[5]);
      acc[6] = fmaf(w, rb[q].z, acc[6]);
      acc[7] = fmaf(w, rb[q].w, acc[7]);
    }
  }
  if (a.Is > 0) {
    acc[0] += ya.x; acc[1] += ya.y; acc[2] += ya.z; acc[3] += ya.w;
    acc[4] += yb.x; acc[5] += yb.y; acc[6] += yb.z; acc[7] += yb.w;
  }
  if (a.moe_out && live) store_bf16x8(a.moe_out + static_cast<size_t>(t) * H + c, acc);
  const uint32_t u[4] = {rv.x, rv.y, rv.z, rv.w};
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    acc[2 * m] += bf16_lo(u[m]);
    acc[2 * m + 1] += bf16_hi(u[m]);
  }
  float ss = 0.f;
#pragma unroll
  for (int m = 0; m < 8; ++m) ss = fmaf(acc[m], acc[m], ss);
  ss = wave_sum(live ? ss : 0.f);
  if (lane == 0) s_part[wave] = ss;
  __syncthreads();
  float* part = ws.epi_part + t * kMaxBndSlices;
  __shared__ uint32_t s_bad;
  if (wave == 0) {
    // publish this slice's sum (no wait for the store), then poll the token's
    // slices, one lane each, until none is empty; lane 63 reads the error
    // word in the same round trips (a wait of the launch that gave up)
    if (lane == 0) st_f32<true>(part + s, (s_part[0] + s_part[1]) + (s_part[2] + s_part[3]));
    const float* src = lane < ns ? part + lane
                                 : (lane == 63 ? reinterpret_cast<const float*>(
                                                     ws.sync + kSyncError * kSyncStride)
                                               : part);
    uint32_t polls = 0;
    float v = 0.f;
    for (;;) {
      v = ld_f32<true>(src);
      const bool in = lane >= ns || __float_as_uint(v) != kEpiEmpty;
      if (__builtin_amdgcn_ballot_w64(!in) == 0) break;  // uniform over the wave
      __builtin_amdgcn_s_sleep(1);
      if (++polls == kChainSpin) {
        if (lane == 0)
          __hip_atomic_fetch_or(ws.sync + kSyncError * kSyncStride, 1u, __ATOMIC_RELAXED,
                                __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
    }
    if (lane < ns) s_tot[lane] = v;
    if (lane == 63) s_bad = (__float_as_uint(v) != 0u || polls == kChainSpin) ? 1u : 0u;
  }
  __syncthreads();
  const bool gave_up = s_bad != 0u;
  float tot = 0.f;
  for (int i = 0; i < ns; ++i) tot += s_tot[i];
  const float inv_rms = 1.0f / sqrtf(tot / static_cast<float>(H) + a.eps);
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
  *reinterpret_cast<uint4*>(a.out + static_cast<size_t>(t) * H + c) =
      make_uint4(o[0], o[1], o[2], o[3]);
  *reinterpret_cast<uint4*>(a.residual_out + static_cast<size_t>(t) * H + c) =
      make_uint4(r[0], r[1], r[2], r[3]);
}

// NJG = 16-byte chunks per lane of a w13 row (ceil(H / 1024)); NJD = the same
// for w2 rows (ceil(max(I, I_s) / 1024)); E8 = e8m0 scales.
template <int NJG, int NJD, bool E8>
__global__ __launch_bounds__(kThreads) void expert_chain_kernel(ChainArgs a, Workspace ws) {
  __shared__ float s_part[kWaves];
  const Sync sy{ws.sync};
  const int wave = threadIdx.x >> 6;
  const int H = a.H, I = a.I, k = a.k;
  const int it = blockIdx.x;

  constexpr int RD = rows_dn_wave(NJD);
  if (it < a.o_rgu) {
    // ---- shared down: rows RD * (4 * it + wave) .. +RD-1 of y_s
    down_wave<NJD, 1, true, E8, false, NoWait, RD>(a.sw2, a.sw2_scale, 0, H, a.Is,
                                                   (it * kWaves + wave) * RD, a.T, 0,
                                                   RouteIdentity{}, ws.act_s, ws.y_s);
    bump(sy, kSyncExit0 + it % kSyncExitLines);
    return;
  }
  if (it < a.o_rdn) {
    // ---- routed gate_up + SwiGLU: slot d, SwiGLU rows 8 * tile + 2 * wave, +1
    const int u = it - a.o_rgu;
    const int d = u / a.gu_per;
    // the slot's record (expert, route count, first position) from the router
    const int4 rec = *reinterpret_cast<const int4*>(ws.slot_tab +
                                                    static_cast<size_t>(d) * kSlotInts);
    if (rec.x < 0) return;  // a slot past the touched count (uniform)
    const int e = rec.x;
    gate_up_wave<NJG, 1, true, E8>(a.hidden, a.w13 + static_cast<size_t>(e) * 2 * I * H,
                                   a.w13_scale,
                                   static_cast<size_t>(e) * (2 * I / kBlock) * (H / kBlock), H, I,
                                   (u - d * a.gu_per) * kRowsGu + 2 * wave, rec.y, ws.perm,
                                   rec.z, k, ws.act, a.limit);
    bump(sy, sync_gu_cnt(d));
    return;
  }
  if (it < a.n_items) {
    // ---- routed down: slot d, rows RD * (4 * tile + wave) .. +RD-1, at route
    // index t * k + j; the weights are in flight while the slot's gate_up ends
    const int v = it - a.o_rdn;
    const int d = v / a.dn_per;
    const int4 rec = *reinterpret_cast<const int4*>(ws.slot_tab +
                                                    static_cast<size_t>(d) * kSlotInts);
    if (rec.x >= 0) {
      const int e = rec.x;
      auto wait = [&]() {
        wait_count(sy, sync_gu_cnt(d), 1, static_cast<uint32_t>(a.gu_per), kChainSpin);
      };
      down_wave<NJD, 1, true, E8, false, decltype(wait), RD>(
          a.w2 + static_cast<size_t>(e) * H * I, a.w2_scale,
          static_cast<size_t>(e) * (H / kBlock) * (I / kBlock), H, I,
          ((v - d * a.dn_per) * kWaves + wave) * RD, rec.y, rec.z, RouteTable<false>{ws.perm},
          ws.act, ws.rows, wait);
    }
    bump(sy, kSyncExit0 + it % kSyncExitLines);
    return;
  }

  // ---- the boundary (the last T * bnd_ns workgroups), after every down item
  // (shared and routed, empty slots included)
  __shared__ float s_tot[kMaxBndSlices];
  const int b = it - a.n_items;
  boundary_slice(a, ws, b / a.bnd_ns, b % a.bnd_ns, s_part, s_tot, [&]() {
    wait_count(sy, kSyncExit0, kSyncExitLines, static_cast<uint32_t>(a.n_items - a.gu_items),
               kChainSpin);
  });
}

template <int NJG, int NJD, bool E8>
hipError_t launch_t(const ChainArgs& a, const Workspace& ws, hipStream_t s, hipEvent_t evb,
                    hipEvent_t eve) {
  MOE_LAUNCH((expert_chain_kernel<NJG, NJD, E8>), dim3(a.grid), dim3(kThreads), 0, s, evb, eve, a,
             ws);
  return hipGetLastError();
}

#define MOE_CHAIN_INST(NJD, E8)                                                              \
  template hipError_t launch_t<MOE_CHAIN_NJG, NJD, E8>(const ChainArgs&, const Workspace&,   \
                                                        hipStream_t, hipEvent_t, hipEvent_t);
MOE_CHAIN_INST(1, false) MOE_CHAIN_INST(1, true)
MOE_CHAIN_INST(2, false) MOE_CHAIN_INST(2, true)
MOE_CHAIN_INST(3, false) MOE_CHAIN_INST(3, true)
MOE_CHAIN_INST(4, false) MOE_CHAIN_INST(4, true)
#undef MOE_CHAIN_INST
#endif  // MOE_CHAIN_NJG

}  // namespace chain

#ifndef MOE_CHAIN_NJG
namespace {

int chain_njg(int H) { return (H + 1023) / 1024; }
int chain_njd(int I, int Is) {
  const int m = I > Is ? I : Is;
  return (m + 1023) / 1024;
}

// Dispatch over the instantiated (NJG, NJD, E8).
#define MOE_CHAIN_CASES(NJG)                                            \
  X(NJG, 1, false) X(NJG, 1, true) X(NJG, 2, false) X(NJG, 2, true)     \
  X(NJG, 3, false) X(NJG, 3, true) X(NJG, 4, false) X(NJG, 4, true)
#define MOE_CHAIN_ALL                                                     \
  MOE_CHAIN_CASES(1) MOE_CHAIN_CASES(2) MOE_CHAIN_CASES(3) MOE_CHAIN_CASES(4) \
  MOE_CHAIN_CASES(5) MOE_CHAIN_CASES(6) MOE_CHAIN_CASES(7) MOE_CHAIN_CASES(8)

int key(int njg, int njd, bool e8) { return (njg * 8 + njd) * 2 + (e8 ? 1 : 0); }

}  // namespace

bool chain_supported(int H, int I, int Is) {
  return chain_njg(H) <= 8 && chain_njd(I, Is) <= chain::kMaxNjd;
}

void chain_items(const LayerDims& d, ChainArgs* a) {
  a->T = d.T;
  a->H = d.H;
  a->k = d.k;
  a->I = d.I;
  a->Is = d.Is;
  a->e8m0 = d.e8m0 ? 1 : 0;
  a->limit = d.limit;
  a->eps = d.eps;
  a->gu_per = d.I / chain::kRowsGu;
  const int rd = chain::kWaves * chain::rows_dn_wave(chain_njd(d.I, d.Is));
  a->dn_per = d.H / rd;
  a->dmax = d.T * d.k < d.E ? d.T * d.k : d.E;
  a->o_rgu = d.Is ? d.H / rd : 0;
  a->o_rdn = a->o_rgu + a->dmax * a->gu_per;
  a->n_items = a->o_rdn + a->dmax * a->dn_per;
  a->gu_items = a->dmax * a->gu_per;
  a->bnd_ns = (d.H + kBndCols - 1) / kBndCols;
  a->grid = static_cast<uint32_t>(a->n_items + d.T * a->bnd_ns);
}

hipError_t launch_expert_chain(const ChainArgs& a, const Workspace& ws, hipStream_t s,
                               hipEvent_t evb, hipEvent_t eve) {
  if (a.T < 1 || a.T > kChainMaxTokens || a.bnd_ns > kMaxBndSlices ||
      a.grid != static_cast<uint32_t>(a.n_items + a.T * a.bnd_ns) ||
      a.dmax > chain::kMaxSlots ||
      !chain_supported(a.H, a.I, a.Is))
    return hipErrorInvalidValue;
  switch (key(chain_njg(a.H), chain_njd(a.I, a.Is), a.e8m0 != 0)) {
#define X(G, D, E)          \
  case (G * 8 + D) * 2 + E: \
    return chain::launch_t<G, D, E>(a, ws, s, evb, eve);
    MOE_CHAIN_ALL
#undef X
    default:
      return hipErrorInvalidValue;
  }
}
#endif  // !MOE_CHAIN_NJG

}  // namespace moe
