// The whole layer step for 1..16 tokens as one persistent kernel on gfx950.
//
// The pages run the decode-step MoE as one fused "mega MoE" kernel per layer
// (vLLM API page "vllm.models.glm5next.nvidia.specialized_decode.runtime.
// decode", LayerStages._build_mega logs the MoE layers it runs as one
// kernel), with the shared expert overlapping the router and the routed
// experts (LayerStages._mega_moe) and the boundary finalizing the routed rows
// (page "...runtime.draft", SpecializedDraft.reduced_norm).  Here one launch
// does all of it: the shared expert's work is queued ahead of the routed
// experts, so its weight stream overlaps the router and the top-k instead of
// running on a second stream.
//
// Work items, in order:
//   router items     logits of 4 experts (one per wave) for all tokens; the
//                    last router item to finish selects the top-k of every
//                    token, builds the route tables and raises the route flag
//   shared gate_up   8 SwiGLU rows of the shared expert
//   shared down      16 output rows of the shared expert   (after all shared gate_up)
//   routed gate_up   8 SwiGLU rows of one touched expert    (after the route flag)
//   routed down      16 output rows of one touched expert   (after its gate_up)
//   boundary         one token: combine + shared + residual + RMSNorm (after all down)
// The routed items are counted from the touched experts only, so their
// number is known once the route flag is up.  Workgroup w runs items w,
// w + G, w + 2G, ... (G = grid size) in increasing order, one loop per kind
// of item so that each kind's registers are allocated on their own.  An item
// waits only for items with smaller numbers, so when all G workgroups are
// resident at once (the grid is sized to the device's occupancy for this
// kernel) every wait ends.  Waits are bounded anyway: a wait that runs out of
// its spin budget raises a sticky error word (moe_decode_check_waits) and
// gives up instead of hanging.  The last workgroup out (two-level exit
// count) zeroes the counters and flags for the next launch.
//
// Hand-off across workgroups (and XCDs): everything one item leaves for
// another (logits, route tables, SwiGLU rows, down rows) is written with
// agent-scope atomic stores, which write through to the device coherence
// point; the producer waits for its stores to complete before it bumps its
// counter, and consumers read that data with agent-scope atomic loads once
// the flag is up.  No L2 write-back or invalidate is needed.  Counters are
// only bumped by producers; the producer that completes a counter sets a
// flag replicated over several 128-byte lines, and each waiting workgroup
// polls its own replica, so a flip reaches hundreds of waiters without all
// of them hammering one line.
#include "device_common.h"
#include "gemv_tiles.h"
#include "launch.h"
#include "routing_device.h"
#include "sync_device.h"

namespace moe {
namespace fused {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr size_t kRouteSmem =
    kSelBytes + 16 * 16 * 4 + kMaxExperts * 8 + kMaxExperts * 8 + 16;
constexpr int kMaxRoutes = kFusedMaxTokens * kMaxTopK;  // most touched-expert slots
static_assert(3 * kMaxRoutes * 4 <= kRouteSmem, "slot table must fit the routing scratch");

template <int NJ, bool E8>
hipError_t launch_nj(const FusedArgs& a, const Workspace& ws, hipStream_t s, hipEvent_t evb,
                     hipEvent_t eve);
template <int NJ, bool E8>
int occupancy_nj();

#ifdef MOE_FUSED_NJ
// This object holds the kernel for one chunk count and scale format (the
// build compiles this file once per pair, in parallel).
template <int NJ, bool E8>
__global__ __launch_bounds__(kThreads) void decode_fused_kernel(FusedArgs a, Workspace ws) {
  // Routing scratch of the routing workgroup; afterwards every workgroup
  // keeps the touched-expert table (expert, token count, first position) here.
  __shared__ __attribute__((aligned(16))) unsigned char s_route[kRouteSmem];
  __shared__ int s_flag;
  __shared__ float s_part[kWaves];
  const Sync sy{ws.sync};
  const int wave = threadIdx.x >> 6;
  const int H = a.H, I = a.I, Is = a.Is, k = a.k, T = a.T, E = a.E;
  const int G = static_cast<int>(gridDim.x);
  int it = blockIdx.x;

  // Each kind of item has a loop of its own (a workgroup's items still run in
  // increasing order); one loop per kind keeps the register allocation of
  // each kind separate.

  // ---- router items: logits of experts 4*it + wave; the last one to finish
  // selects the top-k of every token and builds the route tables
  for (; it < a.o_sgu; it += G) {
    const int e = it * kWaves + wave;
    if (e < E)
      router_wave<2 * NJ, true>(a.hidden, a.router_w + static_cast<size_t>(e) * H, H, T, E, e,
                                ws.logits);
    if (signal(sy, kSyncRouterCnt, static_cast<uint32_t>(a.n_router), -1, &s_flag)) {
      select_and_route<true>(T, E, k, a.rsf, ws.logits, a.bias, ws, a.ids_out, a.w_out, s_route);
      wait_memory();
      __syncthreads();
      if (threadIdx.x == 0) raise_flag(sy, sync_flag(kFlagRoute));
    }
    __syncthreads();
  }

  // ---- shared gate_up: SwiGLU rows 8*s + 2*wave, +1
  for (; it < a.o_sdn; it += G) {
    const int i0 = (it - a.o_sgu) * 2 * kWaves + 2 * wave;
    gate_up_wave<NJ, 1, true, E8>(a.hidden, a.sw13, a.sw13_scale, 0, H, Is, i0, T, nullptr, 0, k,
                                  ws.act_s, a.limit);
    signal(sy, kSyncSguCnt, static_cast<uint32_t>(a.n_sgu), sync_flag(kFlagSgu), &s_flag);
  }

  // ---- shared down: rows 16*j + 4*wave .. +3, after all shared gate_up
  for (; it < a.o_rgu; it += G) {
    wait_flag(sy, sync_flag(kFlagSgu));
    const int h0 = (it - a.o_sdn) * 4 * kWaves + 4 * wave;
    down_wave<NJ, 1, true, E8>(a.sw2, a.sw2_scale, 0, H, Is, h0, T, 0, RouteIdentity{},
                               ws.act_s, ws.y_s);
    signal(sy, kSyncSdnCnt, static_cast<uint32_t>(a.n_sdn), sync_flag(kFlagSdn), &s_flag);
  }

  // ---- the routed items exist once the router has counted the touched experts
  wait_flag(sy, sync_flag(kFlagRoute));
  const int n_touched = ld_i32<true>(ws.n_touched);
  int* s_e = reinterpret_cast<int*>(s_route);
  int* s_n = s_e + kMaxRoutes;
  int* s_b = s_n + kMaxRoutes;
  for (int d = threadIdx.x; d < n_touched; d += kThreads) {
    const int e = ld_i32<true>(ws.touched + d);
    s_e[d] = e;
    s_n[d] = ld_i32<true>(ws.counts + e);
    s_b[d] = ld_i32<true>(ws.offsets + e);
  }
  __syncthreads();
  const int o_rdn = a.o_rgu + n_touched * a.gu_per;
  const int o_epi = o_rdn + n_touched * a.dn_per;

  // ---- routed gate_up
  for (; it < o_rdn; it += G) {
    const int u = it - a.o_rgu;
    const int d = u / a.gu_per, tile = u % a.gu_per;
    const int e = s_e[d];
    const int i0 = tile * 2 * kWaves + 2 * wave;
    gate_up_wave<NJ, 1, true, E8>(a.hidden, a.w13 + static_cast<size_t>(e) * 2 * I * H,
                                  a.w13_scale,
                                  static_cast<size_t>(e) * (2 * I / kBlock) * (H / kBlock), H, I,
                                  i0, s_n[d], ws.perm, s_b[d], k, ws.act, a.limit);
    signal(sy, sync_gu_cnt(d), static_cast<uint32_t>(a.gu_per), sync_gu_flag(d), &s_flag);
  }

  // ---- routed down, after its expert's gate_up; rows land at their route
  // index t*k + j, where the boundary reads them
  for (; it < o_epi; it += G) {
    const int v = it - o_rdn;
    const int d = v / a.dn_per, tile = v % a.dn_per;
    wait_flag(sy, sync_gu_flag(d));
    const int e = s_e[d];
    const int h0 = tile * 4 * kWaves + 4 * wave;
    down_wave<NJ, 1, true, E8>(a.w2 + static_cast<size_t>(e) * H * I, a.w2_scale,
                               static_cast<size_t>(e) * (H / kBlock) * (I / kBlock), H, I, h0,
                               s_n[d], s_b[d], RouteTable<true>{ws.perm}, ws.act, ws.rows);
    if (signal(sy, sync_dn_cnt(d), static_cast<uint32_t>(a.dn_per), -1, &s_flag) &&
        threadIdx.x == 0) {
      // this expert is complete; the last expert to complete raises the flag
      const uint32_t prev = __hip_atomic_fetch_add(sy.line(kSyncDnSlots), 1u, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
      if (prev + 1 == static_cast<uint32_t>(n_touched)) raise_flag(sy, sync_flag(kFlagDnAll));
    }
    __syncthreads();
  }

  // ---- the boundary, one token per item, after every down row
  const int total = o_epi + T;
  if (it < total) {
    wait_flag(sy, sync_flag(kFlagDnAll));
    if (Is) wait_flag(sy, sync_flag(kFlagSdn));
  }
  for (; it < total; it += G) {
    epilogue_token<true>(it - o_epi, a.residual, a.gamma, H, k, Is > 0, a.eps, ws, a.out,
                         a.residual_out, a.moe_out, s_part);
    __syncthreads();
  }

  // The last workgroup out zeroes every counter and flag for the next launch
  // (HIP-graph replays included).  The error word stays.
  if (last_out(sy, a.grid, &s_flag)) reset_sync(sy, sync_lines(a.dmax));
}

template <int NJ, bool E8>
hipError_t launch_nj(const FusedArgs& a, const Workspace& ws, hipStream_t s, hipEvent_t evb,
                     hipEvent_t eve) {
  MOE_LAUNCH((decode_fused_kernel<NJ, E8>), dim3(a.grid), dim3(kThreads), 0, s, evb, eve, a, ws);
  return hipGetLastError();
}

template <int NJ, bool E8>
int occupancy_nj() {
  int blocks = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, decode_fused_kernel<NJ, E8>, kThreads,
                                                   0) != hipSuccess)
    return 0;
  return blocks;
}

template hipError_t launch_nj<MOE_FUSED_NJ, (MOE_FUSED_E8 != 0)>(const FusedArgs&,
                                                                  const Workspace&, hipStream_t,
                                                                  hipEvent_t, hipEvent_t);
template int occupancy_nj<MOE_FUSED_NJ, (MOE_FUSED_E8 != 0)>();
#endif  // MOE_FUSED_NJ

}  // namespace fused

#ifndef MOE_FUSED_NJ
using fused::kWaves;
using fused::launch_nj;
using fused::occupancy_nj;

int fused_nj(int H, int I, int Is) {
  int nj = (H + 1023) / 1024;
  nj = nj > (I + 1023) / 1024 ? nj : (I + 1023) / 1024;
  nj = nj > (Is + 1023) / 1024 ? nj : (Is + 1023) / 1024;
  return nj;
}

int fused_blocks_per_cu(int nj, bool e8m0) {
  switch (nj * 2 + (e8m0 ? 1 : 0)) {
#define X(N)                           \
  case 2 * N:                          \
    return occupancy_nj<N, false>();   \
  case 2 * N + 1:                      \
    return occupancy_nj<N, true>();
    X(1) X(2) X(3) X(4) X(5) X(6) X(7) X(8)
#undef X
    default:
      return 0;
  }
}

void fused_items(const LayerDims& d, FusedArgs* a) {
  a->T = d.T;
  a->H = d.H;
  a->E = d.E;
  a->k = d.k;
  a->I = d.I;
  a->Is = d.Is;
  a->e8m0 = d.e8m0 ? 1 : 0;
  a->limit = d.limit;
  a->rsf = d.rsf;
  a->eps = d.eps;
  a->n_router = (d.E + kWaves - 1) / kWaves;
  a->n_sgu = d.Is ? d.Is / (2 * kWaves) : 0;
  a->n_sdn = d.Is ? d.H / (4 * kWaves) : 0;
  a->gu_per = d.I / (2 * kWaves);
  a->dn_per = d.H / (4 * kWaves);
  a->dmax = d.T * d.k < d.E ? d.T * d.k : d.E;
  a->o_sgu = a->n_router;
  a->o_sdn = a->o_sgu + a->n_sgu;
  a->o_rgu = a->o_sdn + a->n_sdn;
}

hipError_t launch_decode_fused(const FusedArgs& a, const Workspace& ws, hipStream_t s,
                               hipEvent_t evb, hipEvent_t eve) {
  switch (fused_nj(a.H, a.I, a.Is) * 2 + (a.e8m0 ? 1 : 0)) {
#define X(N)                          \
  case 2 * N:                         \
    return launch_nj<N, false>(a, ws, s, evb, eve); \
  case 2 * N + 1:                     \
    return launch_nj<N, true>(a, ws, s, evb, eve);
    X(1) X(2) X(3) X(4) X(5) X(6) X(7) X(8)
#undef X
    default:
      return hipErrorInvalidValue;
  }
}
#endif  // !MOE_FUSED_NJ

}  // namespace moe
