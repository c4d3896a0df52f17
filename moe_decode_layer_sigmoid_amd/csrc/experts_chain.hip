// The few-token decode step on gfx950 as one or two launches of ordered work
// items: the expert chain (after the router launch), and the whole step in
// one launch with the router's items in front.
//
// Follows the vLLM API page "vllm.models.glm5next.nvidia.specialized_decode.
// runtime.decode": LayerStages._build_mega (fp8 w13 / w2 with 128x128 block
// scales, swiglu_limit; the MoE layer logged as one kernel),
// LayerStages._mega_moe (router logits, the shared expert beside the routed
// experts; the boundary receives the unfinalized rows with the route order),
// LayerStages._router (fp32 logits from the bf16 router weight) and the page
// "...runtime.draft", SpecializedDraft.reduced_norm (norm(x + residual) with
// the new residual).
//
// At one token the step is a chain of short weight streams (gate_up 100 MB,
// down 57 MB at the 4096 x 1536 decode shape).  As separate launches each
// pays its own ramp and tail; here one launch streams them back to back, one
// workgroup per item, in this order of workgroup index.
//
// expert_chain_kernel (after the router launch, which also ran the shared
// expert's gate_up):
//   shared down      32 output rows of the shared expert (16 when I_s > 2048)
//   routed gate_up   8 SwiGLU rows of one touched slot
//   routed down      32 (or 16) output rows of one touched slot; it issues its
//                    weight loads first and then waits for the slot's gate_up
//                    count, so the down weights stream while gate_up ends
//   boundary         the last T * ceil(H / 1024) workgroups: after every
//                    down item, combine + shared + residual of a 1024-column
//                    slice of one token, the slices' sums of squares
//                    exchanged, then RMSNorm * gamma of the slice
// decode_step_kernel (the whole step):
//   router           logits of 4 experts (one per wave) for one token, stored
//                    with inverted bits so that zeroed memory means "not
//                    written yet"; the last router item then selects every
//                    token's top-k, builds the route tables and raises the
//                    route flag
//   shared gate_up   8 SwiGLU rows of the shared expert (no routing needed:
//                    its weights stream while the router runs)
//   shared down      as above, after every shared gate_up item
//   routed gate_up, routed down, boundary: as above (2048-column boundary
//                    slices).  At one token each
//                    routed item finds its slot's expert itself, from the
//                    logits (it polls them until every router item has
//                    stored its logits, then runs the same selection as the
//                    last router item on the same bits), so no routed item
//                    waits for the route tables; above one token they wait
//                    for the route flag and read the slot's record.
// The step launch leaves its counters, flags, logits and boundary slots
// zeroed for the next step launch: the last boundary slice to finish clears
// them, once every other workgroup is past its last use of them.
//
// Hand-offs.  The down items read the SwiGLU rows, and the boundary the down
// rows, with plain (L2-cached) loads: they are written with write-through
// stores that complete before the writer's count is bumped, the L2s hold no
// line of them when the launch starts (every launch begins with an L2
// invalidate), and no workgroup touches them (whole 128-byte lines per slot
// and per route) before the count that covers them is complete.  Coherent
// loads instead would fetch a slot's SwiGLU rows from memory once per down
// workgroup (50 MB at one token, as much as the down weights).  Everything
// else handed over inside a launch (logits, route tables, top-k weights,
// counters, the boundary slots) is written and read coherently.
// A workgroup waits only for workgroups of lower index, which the dispatcher
// has started before it (workgroups are dispatched in index order), except
// that a token's boundary slices wait for each other: all of a launch's
// boundary workgroups (T * ceil(H / 1024) in the chain, T * ceil(H / 2048)
// in the step launch, at most 128) must be resident together, which they
// are once every other item has ended.  Every wait is bounded anyway: an
// exhausted wait sets the sticky error word (moe_decode_check_waits) and
// goes on, and the boundary then writes NaN to out.  Completion counts are
// bumped with atomics whose result is not used.
#include "device_common.h"
#include "gemv_tiles.h"
#include "launch.h"
#include "routing_device.h"
#include "boundary_device.h"
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
[[maybe_unused]] constexpr int kMaxNjd = 4;  // I, I_s <= 4096
[[maybe_unused]] constexpr int kMaxSlots = kChainMaxTokens * kMaxTopK;
// Polls before a wait gives up: a legitimate wait here lasts microseconds
// (a poll is a memory round trip plus a short sleep).
constexpr uint32_t kChainSpin = 1u << 17;

template <int NJG, int NJD, bool E8>
hipError_t launch_t(const ChainArgs& a, const Workspace& ws, hipStream_t s, hipEvent_t evb,
                    hipEvent_t eve);
template <int NJG, int NJD, bool E8>
hipError_t step_launch_t(const StepArgs& a, const Workspace& ws, size_t smem, hipStream_t s,
                         hipEvent_t evb, hipEvent_t eve);

#ifdef MOE_CHAIN_NJG
// NJG = 16-byte chunks per lane of a w13 row (ceil(H / 1024)); NJD = the same
// for w2 rows (ceil(max(I, I_s) / 1024)); E8 = e8m0 scales.
template <int NJG, int NJD, bool E8>
__global__ __launch_bounds__(kThreads) void expert_chain_kernel(ChainArgs a, Workspace ws) {
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
  const int b = it - a.n_items;
  const BndArgs bn{a.residual, a.gamma, a.out, a.residual_out, a.moe_out, H, k, a.Is, a.bnd_ns,
                   a.eps, ws.epi_part, sy.line(kSyncError)};
  constexpr int kCpt = kBndColsChain / kBndThreads;
  boundary_slice<false, kCpt>(bn, ws, b / a.bnd_ns, b % a.bnd_ns, [&]() {
    wait_count(sy, kSyncExit0, kSyncExitLines, static_cast<uint32_t>(a.n_items - a.gu_items),
               kChainSpin);
  }, StepTail{});
}

// ---------------------------------------------------------------- step launch

// Where a routed down item of the step launch writes its rows: the slot's
// route table (several tokens) or its one route (one token).
struct RouteStep {
  const int32_t* perm;  // null: `fixed`
  int fixed;
  __device__ int operator()(int pos) const { return perm ? ld_i32<true>(perm + pos) : fixed; }
};

// Counts this item done once its coherent stores have completed: `cnt`
// (a counter line of msync, or -1) and its exit line.  Every thread calls it.
__device__ __forceinline__ void item_done(const Sync& sy, int it, int cnt) {
  wait_memory();
  __syncthreads();
  if (threadIdx.x == 0) {
    if (cnt >= 0)
      (void)__hip_atomic_fetch_add(sy.line(cnt), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    (void)__hip_atomic_fetch_add(sy.line(kStepExit0 + it % kSyncExitLines), 1u, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Waits (wave 0, bounded) for the route flag's replica of this workgroup.
__device__ __forceinline__ void wait_route(const Sync& sy, uint32_t* err) {
  if (threadIdx.x < 64) {
    const uint32_t* p = sy.line(kStepRoute + static_cast<int>(blockIdx.x % kFlagRep));
    uint32_t polls = 0;
    while (__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0u) {
      __builtin_amdgcn_s_sleep(1);
      if (++polls == kChainSpin) {
        if (threadIdx.x == 0)
          __hip_atomic_fetch_or(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
    }
  }
  __syncthreads();
}

// One token: the expert and route of every slot, from the logits, in wave 0
// (polling replica blockIdx % kFlagRep of the logits until every router item
// has stored them).  It is the selection the last router item runs, on the
// same bits, so all workgroups agree with the route tables.  Slots are the
// picks in ascending expert order (the route tables' order): s_slot[d] =
// expert of slot d, s_slot[kMaxTopK + d] = its route j (rank in the top-k).
__device__ __forceinline__ void route_one_token(const StepArgs& a, const Workspace& ws,
                                                unsigned long long* sel, int* s_slot,
                                                uint32_t* err) {
  const int lane = threadIdx.x & 63;
  if (threadIdx.x < 64) {
    const float* logits = ws.mlogits + static_cast<size_t>(blockIdx.x % kFlagRep) * a.T * a.E;
    int id = 0;
    float w = 0.f;
    select_token<true, true, true, false>(logits, a.bias, a.E, a.k, a.rsf, sel, &id, &w, err);
    int* ids = reinterpret_cast<int*>(sel);  // the selection is done with its scratch
    if (lane < a.k) ids[lane] = id;
    wave_lds_order();
    if (lane < a.k) {
      int below = 0;
      for (int i = 0; i < a.k; ++i) below += ids[i] < id ? 1 : 0;
      s_slot[below] = id;
      s_slot[kMaxTopK + below] = lane;
    }
  }
  __syncthreads();
}

template <int NJG, int NJD, bool E8>
__global__ __launch_bounds__(kThreads) void decode_step_kernel(StepArgs a, Workspace ws) {
  // routing scratch (route_smem_bytes(T, E, k)): the last router item's, or
  // wave 0's selection scratch at one token
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __shared__ int s_slot[2 * kMaxTopK];
  const Sync sy{ws.msync};
  uint32_t* err = ws.sync + kSyncError * kSyncStride;
  const int wave = threadIdx.x >> 6;
  const int H = a.H, I = a.I, k = a.k, T = a.T, E = a.E;
  const int it = blockIdx.x;
  constexpr int RD = rows_dn_wave(NJD);

  if (it < a.o_sgu) {
    // ---- router: experts 4 * eb + wave for token t; logits go to every
    // replica (inverted bits)
    const int t = it / a.n_eb;
    const int e = (it - t * a.n_eb) * kWaves + wave;
    if (e < E)
      router_wave<2 * NJG, true, true>(a.hidden + static_cast<size_t>(t) * H,
                                       a.router_w + static_cast<size_t>(e) * H, H, 1, E, e,
                                       ws.mlogits + static_cast<size_t>(t) * E, kFlagRep,
                                       static_cast<size_t>(T) * E);
    if (it == a.o_sgu - 1) {
      // the last router item: top-k of every token (polling replica 0 of its
      // logits), the route tables and the caller's ids / weights, then the
      // route flag
      const RouteSmem sm(smem, T, E, k);
      select_tokens<true, true, true, false>(0, T, E, k, a.rsf, ws.mlogits, a.bias, ws,
                                             a.ids_out, a.w_out, sm, err);
      build_routes<true>(T, E, k, ws, sm);
      wait_memory();
      __syncthreads();
      if (threadIdx.x < kFlagRep)
        st_u32<true>(sy.line(kStepRoute + static_cast<int>(threadIdx.x)), 1u);
    }
    item_done(sy, it, -1);
    return;
  }
  if (it < a.o_sdn) {
    // ---- shared gate_up + SwiGLU: SwiGLU rows 8 * item + 2 * wave, +1
    const int i0 = ((it - a.o_sgu) * kWaves + wave) * 2;
    gate_up_wave<NJG, 1, true, E8>(a.hidden, a.sw13, a.sw13_scale, 0, H, a.Is, i0, T, nullptr, 0,
                                   k, ws.act_s, a.limit);
    item_done(sy, it, kStepSgu);
    return;
  }
  if (it < a.o_rgu) {
    // ---- shared down: rows RD * (4 * item + wave) .. +RD-1 of y_s, after
    // every shared gate_up item (its weights stream meanwhile)
    auto wait = [&]() {
      wait_count(sy, kStepSgu, 1, static_cast<uint32_t>(a.sgu_n), kChainSpin, err);
    };
    down_wave<NJD, 1, true, E8, false, decltype(wait), RD>(
        a.sw2, a.sw2_scale, 0, H, a.Is, ((it - a.o_sdn) * kWaves + wave) * RD, T, 0,
        RouteIdentity{}, ws.act_s, ws.y_s, wait);
    item_done(sy, it, -1);
    return;
  }
  if (it < a.n_items) {
    // ---- routed items: slot d's expert e, its route count n, first
    // position base (and, at one token, its route j)
    const bool gu = it < a.o_rdn;
    const int u = gu ? it - a.o_rgu : it - a.o_rdn;
    const int per = gu ? a.gu_per : a.dn_per;
    const int d = u / per;
    int e, n, base, j = 0;
    if (T == 1) {
      route_one_token(a, ws, reinterpret_cast<unsigned long long*>(smem), s_slot, err);
      // clamped: only a selection on logits that never arrived (a wait that
      // gave up, out then NaN) could leave a slot unset
      e = min(max(s_slot[d], 0), E - 1);
      j = min(max(s_slot[kMaxTopK + d], 0), k - 1);
      n = 1;
      base = d;
    } else {
      wait_route(sy, err);
      const int32_t* rec = ws.slot_tab + static_cast<size_t>(d) * kSlotInts;
      e = ld_i32<true>(rec);
      n = ld_i32<true>(rec + 1);
      base = ld_i32<true>(rec + 2);
    }
    if (gu) {
      // gate_up + SwiGLU: SwiGLU rows 8 * tile + 2 * wave, +1
      if (e >= 0)
        gate_up_wave<NJG, 1, true, E8>(
            a.hidden, a.w13 + static_cast<size_t>(e) * 2 * I * H, a.w13_scale,
            static_cast<size_t>(e) * (2 * I / kBlock) * (H / kBlock), H, I,
            (u - d * per) * kRowsGu + 2 * wave, n, T == 1 ? nullptr : ws.perm, base, k, ws.act,
            a.limit);
      item_done(sy, it, e >= 0 ? kStepSlot0 + d : -1);
      return;
    }
    // down: rows RD * (4 * tile + wave) .. +RD-1 at route index t * k + j,
    // the weights in flight while the slot's gate_up ends
    if (e >= 0) {
      auto wait = [&]() {
        wait_count(sy, kStepSlot0 + d, 1, static_cast<uint32_t>(a.gu_per), kChainSpin, err);
      };
      down_wave<NJD, 1, true, E8, false, decltype(wait), RD>(
          a.w2 + static_cast<size_t>(e) * H * I, a.w2_scale,
          static_cast<size_t>(e) * (H / kBlock) * (I / kBlock), H, I,
          ((u - d * per) * kWaves + wave) * RD, n, base,
          RouteStep{T == 1 ? nullptr : ws.perm, j}, ws.act, ws.rows, wait);
    }
    item_done(sy, it, -1);
    return;
  }

  // ---- the boundary (the last T * bnd_ns workgroups), after every other item
  const int b = it - a.n_items;
  const BndArgs bn{a.residual, a.gamma, a.out, a.residual_out, a.moe_out, H, k, a.Is, a.bnd_ns,
                   a.eps, ws.mepi, err};
  const StepTail tail{sy.line(kStepBnd), static_cast<uint32_t>(T * a.bnd_ns), ws.msync,
                      step_sync_lines(a.dmax), ws.mlogits, kFlagRep * T * E,
                      T * kMaxBndSlices};
  constexpr int kCpt = kBndCols / kBndThreads;
  boundary_slice<true, kCpt>(bn, ws, b / a.bnd_ns, b % a.bnd_ns, [&]() {
    wait_count(sy, kStepExit0, kSyncExitLines, static_cast<uint32_t>(a.n_items), kChainSpin, err);
  }, tail);
}

template <int NJG, int NJD, bool E8>
hipError_t launch_t(const ChainArgs& a, const Workspace& ws, hipStream_t s, hipEvent_t evb,
                    hipEvent_t eve) {
  MOE_LAUNCH((expert_chain_kernel<NJG, NJD, E8>), dim3(a.grid), dim3(kThreads), 0, s, evb, eve, a,
             ws);
  return hipGetLastError();
}

template <int NJG, int NJD, bool E8>
hipError_t step_launch_t(const StepArgs& a, const Workspace& ws, size_t smem, hipStream_t s,
                         hipEvent_t evb, hipEvent_t eve) {
  MOE_LAUNCH((decode_step_kernel<NJG, NJD, E8>), dim3(a.grid), dim3(kThreads), smem, s, evb, eve,
             a, ws);
  return hipGetLastError();
}

#define MOE_CHAIN_INST(NJD, E8)                                                              \
  template hipError_t launch_t<MOE_CHAIN_NJG, NJD, E8>(const ChainArgs&, const Workspace&,   \
                                                        hipStream_t, hipEvent_t, hipEvent_t); \
  template hipError_t step_launch_t<MOE_CHAIN_NJG, NJD, E8>(                                 \
      const StepArgs&, const Workspace&, size_t, hipStream_t, hipEvent_t, hipEvent_t);
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
  a->bnd_ns = (d.H + kBndColsChain - 1) / kBndColsChain;
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

void step_items(const LayerDims& d, StepArgs* a) {
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
  a->n_eb = (d.E + chain::kWaves - 1) / chain::kWaves;
  const int rd = chain::kWaves * chain::rows_dn_wave(chain_njd(d.I, d.Is));
  a->sgu_n = d.Is ? d.Is / chain::kRowsGu : 0;
  a->sdn_n = d.Is ? d.H / rd : 0;
  a->gu_per = d.I / chain::kRowsGu;
  a->dn_per = d.H / rd;
  a->dmax = d.T * d.k < d.E ? d.T * d.k : d.E;
  a->o_sgu = a->n_eb * d.T;
  a->o_sdn = a->o_sgu + a->sgu_n;
  a->o_rgu = a->o_sdn + a->sdn_n;
  a->o_rdn = a->o_rgu + a->dmax * a->gu_per;
  a->n_items = a->o_rdn + a->dmax * a->dn_per;
  a->bnd_ns = (d.H + kBndCols - 1) / kBndCols;
  a->grid = static_cast<uint32_t>(a->n_items + d.T * a->bnd_ns);
}

size_t step_smem_bytes(const LayerDims& d) { return route_smem_bytes(d.T, d.E, d.k); }

hipError_t launch_decode_step(const StepArgs& a, const Workspace& ws, hipStream_t s,
                              hipEvent_t evb, hipEvent_t eve) {
  if (a.T < 1 || a.T > kChainMaxTokens || a.E < 1 || a.E > kStepMaxExperts || a.k < 1 ||
      a.k > kMaxTopK || a.k > a.E || a.bnd_ns > kMaxBndSlices || a.dmax > chain::kMaxSlots ||
      a.grid != static_cast<uint32_t>(a.n_items + a.T * a.bnd_ns) ||
      !chain_supported(a.H, a.I, a.Is))
    return hipErrorInvalidValue;
  const size_t smem = route_smem_bytes(a.T, a.E, a.k);
  switch (key(chain_njg(a.H), chain_njd(a.I, a.Is), a.e8m0 != 0)) {
#define X(G, D, E)          \
  case (G * 8 + D) * 2 + E: \
    return chain::step_launch_t<G, D, E>(a, ws, smem, s, evb, eve);
    MOE_CHAIN_ALL
#undef X
    default:
      return hipErrorInvalidValue;
  }
}
#endif  // !MOE_CHAIN_NJG

}  // namespace moe
