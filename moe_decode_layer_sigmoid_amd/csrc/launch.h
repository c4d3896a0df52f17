// Host-side launchers of the MoE decode kernels (internal to the library).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Launches `kernel`; with a non-null `evb` through hipExtLaunchKernelGGL,
// which records evb / eve at the kernel's own start and end (the measurement
// hook: an event recorded on the stream around the launch would also count
// the dispatch and completion of the launch).
#define MOE_LAUNCH(kernel, grid, block, lds, s, evb, eve, ...)                             \
  do {                                                                                   \
    if (evb)                                                                             \
      hipExtLaunchKernelGGL(kernel, grid, block, lds, s, evb, eve, 0, __VA_ARGS__);      \
    else                                                                                 \
      hipLaunchKernelGGL(kernel, grid, block, lds, s, __VA_ARGS__);                      \
  } while (0)

// Device workspace of one plan, sized for max_tokens.
struct Workspace {
  float* logits;       // [maxT, E]
  int32_t* ids;        // [maxT, k]
  float* weights;      // [maxT, k]
  int32_t* counts;     // [E]
  int32_t* offsets;    // [E + 1]
  int32_t* touched;    // [E]
  int32_t* n_touched;  // [1]
  int32_t* perm;       // [maxT * k]  permuted position -> route t*k+j
  int32_t* inv;        // [maxT * k]  route -> permuted position
  float* act;          // [maxT * k, I]   routed SwiGLU output, permuted order; a dense
                       // layer's partial sums (dense_part_floats)
  float* act_s;        // [maxT, Is]      shared SwiGLU output
  float* rows;         // [maxT * k, H]   routed down output, at route index t*k+j
  float* y_s;          // [maxT, H] shared expert (or dense MLP) output
  uint32_t* counter;   // router arrival counters, router_cnt_words() (self-resetting)
  uint32_t* sync;      // [sync_words(E)] counters of the expert chain and grouped merged
                       // launches (zeroed by the router launch before them); the error word
  float* zero_bias;    // [E] zeros: the router bias when the caller passes none
  int32_t* slot_tab;   // [E][kSlotInts] touched slot d: expert (-1: no expert), route
                       // count, first permuted position, -, first kSlotRoutes routes
  float* epi_part;     // [maxT][kMaxBndSlices] boundary slices' sums of squares (inverted
                       // bits; 0 = not published yet)
  // State of the single-launch step (decode_step_kernel), left zeroed by
  // every such launch for the next one:
  uint32_t* msync;     // [step_sync_lines(dmax)] lines: route flag, counts, exit lines
  float* mlogits;      // [min(maxT, kChainMaxTokens), E] logits, inverted bits (0 = not yet)
  float* mepi;         // [min(maxT, kChainMaxTokens)][kMaxBndSlices] like epi_part
  // The router launch's logits [maxT, E] with inverted bits (0 = not yet
  // written), zeroed again by the workgroup that reads them.
  float* rlogits;
  // The matrix-core router (many tokens): partial logits [slices][E][Tp]
  // and its arrival counters (one line each, self-resetting); a dense
  // layer's arrival counters (dense_count_lines).
  float* rpart;
  uint32_t* rcnt;
};

// Per-slot record the router leaves for the expert kernels, so that a
// workgroup finds its expert and its first routes with one load instead of a
// chain of dependent ones.
constexpr int kSlotInts = 16;
constexpr int kSlotRoutes = 12;

// Counters and flags in Workspace::sync, one 128-byte line each: atomics and
// polls on one line serialise, separate lines proceed in parallel.  Lines:
// the sticky error word; the exit lines of the expert chain launch; lines
// kSyncFlags + y for the grouped merged launch's shared-expert rows; one
// line per touched slot (its gate_up items done).  Waiting workgroups poll
// replicas of a flag (kFlagRep lines) so that no line is polled by many.
constexpr int kSyncStride = 32;  // uint32 words per line
constexpr int kFlagRep = 8;      // replicas of a polled flag
enum : int {
  kSyncError = 4,       // sticky: set when a bounded wait gave up
  kSyncExit0 = 5,       // kSyncExitLines exit counters
  kSyncExitLines = 8,
  kSyncFlags = 16,      // lines of the grouped merged launch's shared rows
  kSyncSlot0 = 48,      // per touched slot: gate_up items done
};
__host__ __device__ constexpr int sync_gu_cnt(int d) { return kSyncSlot0 + d; }
__host__ __device__ constexpr int sync_lines(int slots) { return kSyncSlot0 + slots; }
__host__ __device__ constexpr size_t sync_words(int E) {
  return static_cast<size_t>(sync_lines(E)) * kSyncStride;
}

// Arrival counters of the router kernel in Workspace::counter: one 128-byte
// line per token block, then one for the token blocks.  A block holds at most
// kRouterTokBlk tokens (one per wave when ranking); launches of few tokens
// use smaller blocks (router_block_tokens).
constexpr int kRouterTokBlk = 4;
constexpr int kRouterMaxBlk = 64;  // 256 tokens
__host__ __device__ constexpr int router_cnt_line(int b) { return b * kSyncStride; }
__host__ __device__ constexpr size_t router_cnt_words() {
  return static_cast<size_t>(kRouterMaxBlk + 1) * kSyncStride;
}

// Up to this many tokens the MFMA path runs the shared expert's passes in the
// routed experts' launches; above it (several 16-token passes, each streaming
// the shared weights again) on a second stream, beside the routed launches.
constexpr int kMergeSharedMaxTokens = 64;
// AUTO takes the MFMA projections from this many tokens on.  Measured on
// MI355X at the 4096 x 1536, 128-expert decode shape (µs per step, split /
// grouped): 1 token 46.5 / 74.2, 2: 75.3 / 87.0, 3: 103.1 / 109.9,
// 4: 127.9 / 118.9, 8: 215.8 / 183.5, 16: 378.8 / 295.6.
constexpr int kGroupedMinTokens = 4;
// AUTO takes the single-launch step up to this many tokens (where it fits).
// Measured on MI355X at the decode shape (H = 4096, E = 128, k = 8,
// I = 1536), µs per step, single launch / router launch + expert chain:
// 1 token 53.8 / 47.0, 2: 80.7 / 73.1, 3: 117.2 / 103.1.  A per-workgroup
// timeline of the single launch showed why: every routed item there learns
// its expert from coherent reads of the logits plus its own selection
// (2.4-3 us), where an expert chain item reads the finished route tables
// from L2 (1.1 us), and the routing delay (about 5 us) is more than the
// shared expert's weights can fill.  So AUTO keeps the two launches.
constexpr int kStepAutoMaxTokens = 0;
// The same for a dense layer (no routed experts).  Its MFMA kernels split
// the contraction over waves and workgroups and win from one token on
// (MI355X, H = 4096, I_s = 8192, us per step GEMV / MFMA: 1 token 35.7 /
// 30.4, 4: 71.4 / 32.0, 8: 119.5 / 33.4, 16: 213.9 / 38.7).
constexpr int kDenseGroupedMinTokens = 1;

// Arguments of the expert chain launch of the few-token GEMV path (see
// experts_chain.hip): item offsets and counts, the grid (items + 1).
constexpr int kChainMaxTokens = 16;
// Columns of one boundary workgroup: 2048 (8 per thread) in the grouped
// merged launch and the single-launch step, 1024 (4 per thread) in the
// expert chain.  Measured on MI355X (us per layer, H = 4096): 1024-column
// slices took one token 48.0 -> 47.4 and two 76.9 -> 76.5 in the chain
// (512-column slices: no further gain), and 16 tokens 276.1 -> 279.5 in the
// grouped launch (twice the workgroups exchanging their sums).
constexpr int kBndCols = 2048;
constexpr int kBndColsChain = 1024;
constexpr int kMaxBndSlices = 8;   // H <= 8192 at 1024 columns
struct ChainArgs {
  const uint16_t* hidden;
  const uint16_t* residual;
  const uint8_t* w13;
  const void* w13_scale;
  const uint8_t* w2;
  const void* w2_scale;
  const uint8_t* sw2;
  const void* sw2_scale;
  const uint16_t* gamma;
  uint16_t* out;
  uint16_t* residual_out;
  uint16_t* moe_out;  // nullable
  int T, H, k, I, Is, e8m0;
  float limit, eps;
  int gu_per, dn_per, dmax;  // items per slot; touched-slot rows of the grid
  int o_rgu, o_rdn, n_items, gu_items;
  int bnd_ns;  // boundary workgroups per token (kBndCols columns each)
  uint32_t grid;
};

// Arguments of the single-launch step (experts_chain.hip, decode_step_kernel):
// router items, the shared expert's gate_up and down items, the touched
// slots' gate_up and down items, the boundary slices, in this index order.
struct StepArgs {
  const uint16_t* hidden;
  const uint16_t* residual;
  const uint16_t* router_w;
  const float* bias;  // never null (the zero bias stands in)
  const uint8_t* w13;
  const void* w13_scale;
  const uint8_t* w2;
  const void* w2_scale;
  const uint8_t* sw13;
  const void* sw13_scale;
  const uint8_t* sw2;
  const void* sw2_scale;
  const uint16_t* gamma;
  uint16_t* out;
  uint16_t* residual_out;
  uint16_t* moe_out;  // nullable
  int32_t* ids_out;   // nullable
  float* w_out;       // nullable
  int T, H, E, k, I, Is, e8m0;
  float limit, rsf, eps;
  int n_eb;                  // router expert blocks (4 experts each); n_eb * T router items
  int sgu_n, sdn_n;          // shared gate_up and down items
  int gu_per, dn_per, dmax;  // items per slot; slots
  int o_sgu, o_sdn, o_rgu, o_rdn, n_items;
  int bnd_ns;
  uint32_t grid;
};

// Most experts the single-launch step routes (its top-k holds at most four
// keys per lane; wider routers take the router launch and the chain).
constexpr int kStepMaxExperts = 256;

// Lines of Workspace::msync (one 128-byte line each).
enum : int {
  kStepRoute = 0,                     // route flag, kFlagRep replicas (T > 1)
  kStepSgu = kStepRoute + kFlagRep,   // shared gate_up items done
  kStepExit0 = kStepSgu + 1,          // kSyncExitLines lines: items done
  kStepBnd = kStepExit0 + kSyncExitLines,  // boundary slices done
  kStepSlot0 = kStepBnd + 1           // gate_up items done, one line per slot
};
__host__ __device__ constexpr int step_sync_lines(int dmax) { return kStepSlot0 + dmax; }

// Arguments of the grouped path's merged gate_up + down launch (see
// experts_mfma.hip, grouped_chain_kernel).
struct GChainArgs {
  const uint16_t* hidden;
  const uint8_t* w13;
  const void* w13_scale;
  const uint8_t* sw13;
  const void* sw13_scale;
  const uint8_t* w2;
  const void* w2_scale;
  const uint8_t* sw2;
  const void* sw2_scale;
  const uint16_t* residual;
  const uint16_t* gamma;
  uint16_t* out;
  uint16_t* residual_out;
  uint16_t* moe_out;  // nullable
  int H, I, Is, k, T, SP;
  float limit, eps;
  int gx, dx, n_gu;  // tiles per grid row (gate_up, down); gate_up workgroups
  int n_dn, bnd_ns;  // down workgroups; boundary workgroups per token
};

struct LayerDims {
  int T, H, E, k, I, Is;
  bool e8m0;
  float limit, rsf, eps;
};

// Router logits, sigmoid, top-k, weights and the route tables; with sw13
// non-null also the shared expert's gate_up + SwiGLU (into ws.act_s).
// With d.E == 0 (a dense layer) only the gate_up tiles run.  evb / eve: the
// measurement hook (MOE_LAUNCH).
hipError_t launch_router(const LayerDims& d, const void* hidden, const void* router_w,
                         const float* bias, const Workspace& ws, int32_t* ids_out,
                         float* weights_out, const void* sw13, const void* sw13_scale,
                         hipStream_t s, hipEvent_t evb = nullptr, hipEvent_t eve = nullptr);

// The router for many tokens on the matrix cores (logits as 16 x 64 MFMA
// tiles over 512-column slices of the contraction), then the same top-k and
// route tables; no shared-expert tiles.  Tp_alloc: the token stride of
// ws.rpart (router_mfma_tokens_padded of the plan's max tokens).
// zero_lines: lines of ws.sync the launch that follows expects at zero.
int router_mfma_slices(int T, int E, int H);
int router_mfma_tokens_padded(int T);
int router_mfma_count_lines(int T, int E);
hipError_t launch_router_mfma(const LayerDims& d, const void* hidden, const void* router_w,
                              const float* bias, const Workspace& ws, int Tp_alloc,
                              int zero_lines, int32_t* ids_out, float* weights_out,
                              hipStream_t s);
// The matrix-core router takes over from this many tokens.
constexpr int kRouterMfmaMinTokens = 17;

// gate_up + clamped SwiGLU (GEMV) of the touched experts (one grid row
// each; the shared expert's runs in the router launch).
hipError_t launch_gate_up_gemv(const LayerDims& d, const void* hidden, const void* w13,
                               const void* w13_scale, const Workspace& ws, hipStream_t s,
                               hipEvent_t evb = nullptr, hipEvent_t eve = nullptr);

// down projection (GEMV) of the same slots.
hipError_t launch_down_gemv(const LayerDims& d, const void* w2, const void* w2_scale,
                            const void* sw2, const void* sw2_scale, const Workspace& ws,
                            hipStream_t s);

// The same two projections on the matrix cores (bf16 MFMA on exactly
// converted fp8 weights; SwiGLU activations as hi + lo bf16 planes).  Grid
// rows: the shared expert's 16-token passes, then the touched experts;
// `rows` launches both or one of the two kinds.
enum : int { kAllRows = 0, kSharedRows = 1, kRoutedRows = 2 };
hipError_t launch_gate_up_mfma(const LayerDims& d, int rows, const void* hidden, const void* w13,
                               const void* w13_scale, const void* sw13, const void* sw13_scale,
                               const Workspace& ws, hipStream_t s, hipEvent_t evb = nullptr,
                               hipEvent_t eve = nullptr);
hipError_t launch_down_mfma(const LayerDims& d, int rows, const void* w2, const void* w2_scale,
                            const void* sw2, const void* sw2_scale, const Workspace& ws,
                            hipStream_t s);

// The same gate_up and down projections (shared passes and touched slots,
// T <= kMergeSharedMaxTokens) as one launch whose down tiles wait for their
// row's gate_up tiles; up to kFusedBoundaryMaxTokens tokens the boundary
// joins it (grouped_boundary_fused), its slices waiting for every down tile,
// which then writes its rows through to the coherence point.  Measured on
// MI355X (us per step, boundary launched apart / in the launch): 16 tokens
// 279.3 / 278.0, 8 tokens 180.9 / 180.0, 32 tokens 372.5 / 372.1, 64 tokens
// at H = 6144 1296 / 1310 (the coherent stores of the down rows cost more
// than the boundary launch they save).  grouped_chain_supported tells
// whether the shape fits.  The router launch before it leaves the counters
// and boundary slots at zero.
constexpr int kFusedBoundaryMaxTokens = 16;
bool grouped_chain_supported(const LayerDims& d);
bool grouped_boundary_fused(const LayerDims& d);
hipError_t launch_grouped_chain(const LayerDims& d, const void* hidden, const void* w13,
                                const void* w13_scale, const void* sw13, const void* sw13_scale,
                                const void* w2, const void* w2_scale, const void* sw2,
                                const void* sw2_scale, const void* residual, const void* gamma,
                                void* out, void* residual_out, void* moe_out,
                                const Workspace& ws, hipStream_t s, hipEvent_t evb = nullptr,
                                hipEvent_t eve = nullptr);

// Shared down, routed gate_up, routed down and the boundary in one launch
// (T <= kChainMaxTokens; H <= 8192; I and I_s <= 4096).
bool chain_supported(int H, int I, int Is);
void chain_items(const LayerDims& d, ChainArgs* a);
hipError_t launch_expert_chain(const ChainArgs& a, const Workspace& ws, hipStream_t s,
                               hipEvent_t evb = nullptr, hipEvent_t eve = nullptr);

// The whole step in one launch: the router items and the chain's items
// (T <= kChainMaxTokens, E <= kStepMaxExperts, chain_supported).
void step_items(const LayerDims& d, StepArgs* a);
size_t step_smem_bytes(const LayerDims& d);
hipError_t launch_decode_step(const StepArgs& a, const Workspace& ws, hipStream_t s,
                              hipEvent_t evb = nullptr, hipEvent_t eve = nullptr);

// A dense layer's MLP (d.E == 0) on the matrix cores: gate_up + SwiGLU, then
// down, each with the contraction split over workgroups whose fp32 partial
// sums the last of a tile's workgroups adds up; the down output goes to
// ws.y_s.  The partial sums use ws.act (a dense layer has no routed rows),
// dense_part_floats(maxT, H, Is) floats; the arrival counters use ws.rcnt,
// dense_count_lines(maxT, H, Is) lines (zero before the first run, reset by
// the workgroups that use them).
size_t dense_part_floats(int maxT, int H, int Is);
int dense_count_lines(int maxT, int H, int Is);
hipError_t launch_dense_mfma(const LayerDims& d, const void* hidden, const void* sw13,
                             const void* sw13_scale, const void* sw2, const void* sw2_scale,
                             const Workspace& ws, hipStream_t s, hipEvent_t evb = nullptr,
                             hipEvent_t eve = nullptr);

// Weighted combine + shared + residual, RMSNorm * gamma, bf16 outputs.
// moe_out (nullable): also the finalized MoE output (before the residual).
hipError_t launch_epilogue(const LayerDims& d, const void* residual, const void* gamma,
                           const Workspace& ws, void* out, void* residual_out, void* moe_out,
                           hipStream_t s);

}  // namespace moe
