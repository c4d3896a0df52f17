// C ABI of the MoE decode layer: validation, plan (workspace, events), run
// (kernel sequence), destroy.
//
// Follows the vLLM API page "vllm.models.glm5next.nvidia.specialized_decode.
// runtime.decode": LayerStages._build_mega allocates the route-order buffer
// and its other buffers once, before any capture, and LayerStages._mega_moe
// runs the shared expert beside the routed experts.  There the shared expert
// gets a second stream; on MI355X a fork and join inside a HIP graph cost
// about 5 and 10 us per step (measured), more than running the shared
// expert's tiles as extra workgroups of the same launches, which is what
// this library does up to 64 tokens: its gate_up rides in the router launch
// (GEMV path) or in the routed gate_up launch (MFMA path), its down
// projection in the routed down launch.  Above 64 tokens the shared expert
// needs several passes over its weights and runs on the plan's side stream
// (default priority), forked after the router and joined before the
// boundary; an error after the fork still joins it, as the page "vllm.
// models.deepseek_v41.nvidia.specialized_decode.runtime.draft",
// DraftDecode.run, rejoins its side stream before reporting.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <new>

#include "moe_decode.h"
#include "device_common.h"
#include "launch.h"

struct moe_decode_plan_s {
  moe_decode_desc desc;
  int device;
  void* ws_base;
  size_t ws_bytes;
  size_t state_bytes;  // the leading workspace regions that carry state between runs
  moe::Workspace ws;
  hipStream_t side;      // the shared expert's stream on the MFMA path above
                         // kMergeSharedMaxTokens tokens
  hipEvent_t fork, join;
  hipEvent_t user_begin, user_end;
  bool chain;  // the expert chain and the single-launch step support this layer shape
};

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Whether the single-launch step runs T tokens of this layer.
bool step_fits(const moe_decode_plan_s& p, int32_t T) {
  return p.chain && T <= moe::kChainMaxTokens && p.desc.num_experts <= moe::kStepMaxExperts;
}

// AUTO: the single-launch step below kGroupedMinTokens tokens (where it fits;
// else the router launch and the chain), the MFMA kernels from there.
int path_for(const moe_decode_plan_s& p, int32_t T) {
  const int want = p.desc.path;
  if (p.desc.num_experts == 0)  // a dense layer: the GEMV or the MFMA kernels
    return want == MOE_DECODE_PATH_GROUPED ||
                   (want == MOE_DECODE_PATH_AUTO && T >= moe::kDenseGroupedMinTokens)
               ? MOE_DECODE_PATH_GROUPED
               : MOE_DECODE_PATH_GEMV_SPLIT;
  if (want == MOE_DECODE_PATH_GEMV_SPLIT || want == MOE_DECODE_PATH_GROUPED) return want;
  if (want == MOE_DECODE_PATH_AUTO && T >= moe::kGroupedMinTokens) return MOE_DECODE_PATH_GROUPED;
  if ((want == MOE_DECODE_PATH_GEMV || T <= moe::kStepAutoMaxTokens) && step_fits(p, T))
    return MOE_DECODE_PATH_GEMV;
  return MOE_DECODE_PATH_GEMV_SPLIT;
}

size_t align256(size_t n) { return (n + 255) & ~static_cast<size_t>(255); }

// Lays the workspace out from `base` (nullptr: only sizes it).  The regions
// that carry state from one run to the next (counters, flags, the boundary
// slots, the zero bias) come first, `state_bytes` of them: they must be zero
// before the first run.
size_t layout(const moe_decode_desc& d, char* base, moe::Workspace* ws,
              size_t* state_bytes = nullptr) {
  const size_t T = d.max_tokens, E = d.num_experts, k = d.top_k, H = d.hidden;
  const size_t I = d.intermediate, Is = d.shared_intermediate;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* p = base ? base + off : nullptr;
    off += align256(bytes);
    return p;
  };
  moe::Workspace w{};
  w.counter = reinterpret_cast<uint32_t*>(take(moe::router_cnt_words() * 4));
  w.sync = reinterpret_cast<uint32_t*>(take(moe::sync_words(static_cast<int>(E)) * 4));
  w.zero_bias = reinterpret_cast<float*>(take(E * 4));
  w.epi_part = reinterpret_cast<float*>(take(T * moe::kMaxBndSlices * 4));
  // the single-launch step's state (at most kChainMaxTokens tokens)
  const size_t Ts = T < moe::kChainMaxTokens ? T : moe::kChainMaxTokens;
  const int dmax_s = static_cast<int>(Ts * k < E ? Ts * k : E);
  w.msync = reinterpret_cast<uint32_t*>(take(moe::step_sync_lines(dmax_s) * moe::kSyncStride * 4));
  w.mlogits = reinterpret_cast<float*>(take(moe::kFlagRep * Ts * E * 4));
  w.mepi = reinterpret_cast<float*>(take(Ts * moe::kMaxBndSlices * 4));
  // the router launch's encoded logits
  w.rlogits = reinterpret_cast<float*>(take(T * E * 4));
  // the matrix-core router's counters (many tokens only)
  const bool rmfma = T >= moe::kRouterMfmaMinTokens && E > 0;
  // (a dense layer: the arrival counters of its matrix-core launches)
  const size_t rcnt_lines =
      rmfma ? moe::router_mfma_count_lines(static_cast<int>(T), static_cast<int>(E))
            : (E == 0 ? moe::dense_count_lines(static_cast<int>(T), static_cast<int>(H),
                                               static_cast<int>(Is))
                      : 0);
  w.rcnt = reinterpret_cast<uint32_t*>(take(rcnt_lines * moe::kSyncStride * 4));
  if (state_bytes) *state_bytes = off;
  w.logits = reinterpret_cast<float*>(take(T * E * 4));
  w.ids = reinterpret_cast<int32_t*>(take(T * k * 4));
  w.weights = reinterpret_cast<float*>(take(T * k * 4));
  w.counts = reinterpret_cast<int32_t*>(take(E * 4));
  w.offsets = reinterpret_cast<int32_t*>(take((E + 1) * 4));
  w.touched = reinterpret_cast<int32_t*>(take(E * 4));
  w.n_touched = reinterpret_cast<int32_t*>(take(4));
  w.perm = reinterpret_cast<int32_t*>(take(T * k * 4));
  w.inv = reinterpret_cast<int32_t*>(take(T * k * 4));
  // (a dense layer: the partial sums of its matrix-core launches)
  w.act = reinterpret_cast<float*>(
      take(E == 0 ? moe::dense_part_floats(static_cast<int>(T), static_cast<int>(H),
                                           static_cast<int>(Is)) * 4
                  : T * k * I * 4));
  w.act_s = reinterpret_cast<float*>(take(T * (Is ? Is : 1) * 4));
  w.rows = reinterpret_cast<float*>(take(T * k * H * 4));
  w.y_s = reinterpret_cast<float*>(take(T * H * 4));
  w.slot_tab = reinterpret_cast<int32_t*>(take(E * moe::kSlotInts * 4));
  w.rpart = reinterpret_cast<float*>(
      take(rmfma ? static_cast<size_t>(moe::router_mfma_slices(static_cast<int>(T),
                                                               static_cast<int>(E),
                                                               static_cast<int>(H))) *
                       E * moe::router_mfma_tokens_padded(static_cast<int>(T)) * 4
                 : 0));
  if (ws) *ws = w;
  return off;
}

moe::LayerDims dims(const moe_decode_desc& d, int32_t T) {
  moe::LayerDims x;
  x.T = T;
  x.H = d.hidden;
  x.E = d.num_experts;
  x.k = d.top_k;
  x.I = d.intermediate;
  x.Is = d.shared_intermediate;
  x.e8m0 = d.scale_fmt == MOE_DECODE_SCALE_E8M0;
  x.limit = d.swiglu_limit;
  x.rsf = d.routed_scaling_factor;
  x.eps = d.rms_eps;
  return x;
}

}  // namespace

static int run_on_device(moe_decode_plan_t p, const moe_decode_args* a, int32_t T,
                         hipStream_t s);

extern "C" {

const char* moe_decode_strerror(int code) {
  switch (code) {
    case MOE_DECODE_OK: return "ok";
    case MOE_DECODE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_DECODE_ERR_UNSUPPORTED: return "unsupported size or device";
    case MOE_DECODE_ERR_HIP: return "HIP runtime error";
    case MOE_DECODE_ERR_NO_MEMORY: return "device allocation failed";
    case MOE_DECODE_ERR_SCRATCH:
      return "workspace for this size exceeds the static scratch (moe_decode_run_static)";
    default: return "unknown status";
  }
}

int moe_decode_desc_check(const moe_decode_desc* d) {
  if (!d) return MOE_DECODE_ERR_INVALID_ARG;
  if (d->hidden <= 0 || d->num_experts < 0 || d->top_k < 0 || d->intermediate < 0 ||
      d->shared_intermediate < 0 || d->max_tokens <= 0)
    return MOE_DECODE_ERR_INVALID_ARG;
  // a dense layer (no routed experts) has its MLP in the shared-expert slot
  if (d->num_experts == 0 ? (d->top_k != 0 || d->shared_intermediate == 0)
                          : (d->top_k == 0 || d->intermediate == 0))
    return MOE_DECODE_ERR_INVALID_ARG;
  if (d->scale_fmt != MOE_DECODE_SCALE_FP32 && d->scale_fmt != MOE_DECODE_SCALE_E8M0)
    return MOE_DECODE_ERR_INVALID_ARG;
  if (d->path < MOE_DECODE_PATH_AUTO || d->path > MOE_DECODE_PATH_GEMV_SPLIT)
    return MOE_DECODE_ERR_INVALID_ARG;
  if (!(d->swiglu_limit > 0.f) || !(d->rms_eps >= 0.f) ||
      !(d->routed_scaling_factor == d->routed_scaling_factor))
    return MOE_DECODE_ERR_INVALID_ARG;
  if (d->hidden % moe::kBlock || d->intermediate % moe::kBlock ||
      d->shared_intermediate % moe::kBlock)
    return MOE_DECODE_ERR_UNSUPPORTED;
  if (d->hidden > 8192 || d->intermediate > 8192 || d->shared_intermediate > 8192)
    return MOE_DECODE_ERR_UNSUPPORTED;
  if (d->top_k > moe::kMaxTopK || d->top_k > d->num_experts ||
      d->num_experts > moe::kMaxExperts || d->max_tokens > moe::kMaxTokens)
    return MOE_DECODE_ERR_UNSUPPORTED;
  return MOE_DECODE_OK;
}

int moe_decode_args_check(const moe_decode_desc* d, const moe_decode_args* a, int32_t T) {
  if (!d || !a) return MOE_DECODE_ERR_INVALID_ARG;
  if (T < 0 || T > d->max_tokens) return MOE_DECODE_ERR_INVALID_ARG;
  const void* req[] = {a->hidden, a->residual, a->gamma, a->out, a->residual_out};
  for (const void* p : req)
    if (!p) return MOE_DECODE_ERR_INVALID_ARG;
  const void* routed[] = {a->router_w, a->w13, a->w13_scale, a->w2, a->w2_scale};
  if (d->num_experts > 0)
    for (const void* p : routed)
      if (!p) return MOE_DECODE_ERR_INVALID_ARG;
  if (d->shared_intermediate > 0 && (!a->sw13 || !a->sw13_scale || !a->sw2 || !a->sw2_scale))
    return MOE_DECODE_ERR_INVALID_ARG;
  // 16-byte vector loads and stores need 16-byte aligned tensors.
  const void* vec[] = {a->hidden, a->residual, a->router_w, a->w13, a->w2, a->gamma,
                       a->out, a->residual_out, a->sw13, a->sw2, a->moe_out};
  for (const void* p : vec)
    if (p && !aligned16(p)) return MOE_DECODE_ERR_INVALID_ARG;
  // out is written while hidden/residual/gamma are still being read.
  if (a->out == a->hidden || a->out == a->residual || a->out == a->residual_out ||
      a->residual_out == a->hidden)
    return MOE_DECODE_ERR_INVALID_ARG;
  if (a->moe_out && (a->moe_out == a->hidden || a->moe_out == a->residual ||
                     a->moe_out == a->out || a->moe_out == a->residual_out))
    return MOE_DECODE_ERR_INVALID_ARG;
  return MOE_DECODE_OK;
}

int moe_decode_plan(const moe_decode_desc* d, int device, moe_decode_plan_t* out) {
  if (!out) return MOE_DECODE_ERR_INVALID_ARG;
  *out = nullptr;
  int rc = moe_decode_desc_check(d);
  if (rc) return rc;
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || device < 0 || device >= ndev)
    return MOE_DECODE_ERR_INVALID_ARG;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, device) != hipSuccess) return MOE_DECODE_ERR_HIP;
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) return MOE_DECODE_ERR_UNSUPPORTED;
  int prev = 0;
  if (hipGetDevice(&prev) != hipSuccess) return MOE_DECODE_ERR_HIP;
  if (hipSetDevice(device) != hipSuccess) return MOE_DECODE_ERR_HIP;

  auto* p = new (std::nothrow) moe_decode_plan_s();
  if (!p) {
    (void)hipSetDevice(prev);
    return MOE_DECODE_ERR_NO_MEMORY;
  }
  p->desc = *d;
  p->device = device;
  p->ws_bytes = layout(*d, nullptr, nullptr, &p->state_bytes);
  rc = MOE_DECODE_OK;
  if (hipMalloc(&p->ws_base, p->ws_bytes) != hipSuccess) {
    p->ws_base = nullptr;
    rc = MOE_DECODE_ERR_NO_MEMORY;
  }
  if (!rc) {
    layout(*d, static_cast<char*>(p->ws_base), &p->ws);
    if (hipMemset(p->ws_base, 0, p->ws_bytes) != hipSuccess ||
        hipStreamCreateWithFlags(&p->side, hipStreamNonBlocking) != hipSuccess)
      rc = MOE_DECODE_ERR_HIP;
  }
  if (!rc && (hipEventCreateWithFlags(&p->fork, hipEventDisableTiming) != hipSuccess ||
              hipEventCreateWithFlags(&p->join, hipEventDisableTiming) != hipSuccess))
    rc = MOE_DECODE_ERR_HIP;
  if (!rc) p->chain = moe::chain_supported(d->hidden, d->intermediate, d->shared_intermediate);
  if (!rc && hipDeviceSynchronize() != hipSuccess) rc = MOE_DECODE_ERR_HIP;
  (void)hipSetDevice(prev);
  if (rc) {
    moe_decode_destroy(p);
    return rc;
  }
  *out = p;
  return MOE_DECODE_OK;
}

int moe_decode_destroy(moe_decode_plan_t p) {
  if (!p) return MOE_DECODE_OK;
  int prev = 0;
  (void)hipGetDevice(&prev);
  (void)hipSetDevice(p->device);
  if (p->side) (void)hipStreamSynchronize(p->side);
  if (p->fork) (void)hipEventDestroy(p->fork);
  if (p->join) (void)hipEventDestroy(p->join);
  if (p->side) (void)hipStreamDestroy(p->side);
  if (p->ws_base) {
    (void)hipDeviceSynchronize();  // no launch of this plan may still use the workspace
    (void)hipFree(p->ws_base);
  }
  (void)hipSetDevice(prev);
  delete p;
  return MOE_DECODE_OK;
}

int moe_decode_run(moe_decode_plan_t p, const moe_decode_args* a, int32_t T, void* stream) {
  if (!p) return MOE_DECODE_ERR_INVALID_ARG;
  int rc = moe_decode_args_check(&p->desc, a, T);
  if (rc) return rc;
  if (T == 0) return MOE_DECODE_OK;
  int prev = -1;
  if (hipGetDevice(&prev) != hipSuccess) return MOE_DECODE_ERR_HIP;
  if (prev != p->device && hipSetDevice(p->device) != hipSuccess) return MOE_DECODE_ERR_HIP;
  rc = run_on_device(p, a, T, static_cast<hipStream_t>(stream));
  if (prev != p->device) (void)hipSetDevice(prev);
  return rc;
}

// The whole step in one launch (router, shared expert, routed experts,
// boundary: decode_step_kernel).
static int run_step(moe_decode_plan_t p, const moe_decode_args* a, int32_t T, hipStream_t s) {
  moe::StepArgs st{};
  moe::step_items(dims(p->desc, T), &st);
  st.hidden = static_cast<const uint16_t*>(a->hidden);
  st.residual = static_cast<const uint16_t*>(a->residual);
  st.router_w = static_cast<const uint16_t*>(a->router_w);
  st.bias = a->router_bias ? a->router_bias : p->ws.zero_bias;
  st.w13 = static_cast<const uint8_t*>(a->w13);
  st.w13_scale = a->w13_scale;
  st.w2 = static_cast<const uint8_t*>(a->w2);
  st.w2_scale = a->w2_scale;
  st.sw13 = static_cast<const uint8_t*>(a->sw13);
  st.sw13_scale = a->sw13_scale;
  st.sw2 = static_cast<const uint8_t*>(a->sw2);
  st.sw2_scale = a->sw2_scale;
  st.gamma = static_cast<const uint16_t*>(a->gamma);
  st.out = static_cast<uint16_t*>(a->out);
  st.residual_out = static_cast<uint16_t*>(a->residual_out);
  st.moe_out = static_cast<uint16_t*>(a->moe_out);
  st.ids_out = a->topk_ids;
  st.w_out = a->topk_weights;
  const hipError_t err = moe::launch_decode_step(st, p->ws, s, p->user_begin, p->user_end);
  return err == hipSuccess ? MOE_DECODE_OK : MOE_DECODE_ERR_HIP;
}

// A dense layer (no routed experts): the shared-expert slot's MLP and the
// boundary with no routed rows.  The decode page's LayerStages._build_dense
// builds such layers' DenseMlp from the same fp8 weight pair with block
// scales and swiglu_limit, and LayerStages.mlp sends dense(x) to the same
// boundary as the MoE output.  GEMV path: the router kernel with no router
// rows (only the gate_up tiles), the down kernel's shared row, the boundary;
// MFMA path: the dense gate_up and down launches (launch_dense_mfma), the
// boundary.
static int run_dense(moe_decode_plan_t p, const moe_decode_args* a, int32_t T, hipStream_t s) {
  const moe::LayerDims d = dims(p->desc, T);
  hipError_t err = hipSuccess;
  auto step = [&](hipError_t e) {
    if (err == hipSuccess && e != hipSuccess) err = e;
  };
  if (path_for(*p, T) == MOE_DECODE_PATH_GROUPED) {
    step(moe::launch_dense_mfma(d, a->hidden, a->sw13, a->sw13_scale, a->sw2, a->sw2_scale,
                                p->ws, s, p->user_begin, p->user_end));
  } else {
    step(moe::launch_router(d, a->hidden, nullptr, p->ws.zero_bias, p->ws, nullptr, nullptr,
                            a->sw13, a->sw13_scale, s, p->user_begin, p->user_end));
    if (err == hipSuccess)
      step(moe::launch_down_gemv(d, nullptr, nullptr, a->sw2, a->sw2_scale, p->ws, s));
  }
  if (err == hipSuccess)
    step(moe::launch_epilogue(d, a->residual, a->gamma, p->ws, a->out, a->residual_out,
                              a->moe_out, s));
  return err == hipSuccess ? MOE_DECODE_OK : MOE_DECODE_ERR_HIP;
}

static int run_on_device(moe_decode_plan_t p, const moe_decode_args* a, int32_t T,
                         hipStream_t s) {
  if (p->desc.num_experts == 0) return run_dense(p, a, T, s);
  const int path = path_for(*p, T);
  if (path == MOE_DECODE_PATH_GEMV) return run_step(p, a, T, s);
  const moe::LayerDims d = dims(p->desc, T);
  const bool has_shared = d.Is > 0;
  const void* bias = a->router_bias ? a->router_bias : p->ws.zero_bias;
  hipError_t err = hipSuccess;
  auto step = [&](hipError_t e) {
    if (err == hipSuccess && e != hipSuccess) err = e;
  };

  if (path == MOE_DECODE_PATH_GEMV_SPLIT) {
    // router (with the shared expert's gate_up beside it), then either the
    // expert chain launch (shared down, routed gate_up and down, boundary) or,
    // above its token limit, the routed gate_up, the shared and routed down
    // projections in one launch, and the boundary
    step(moe::launch_router(d, a->hidden, a->router_w, static_cast<const float*>(bias), p->ws,
                            a->topk_ids, a->topk_weights, has_shared ? a->sw13 : nullptr,
                            a->sw13_scale, s));
    if (T <= moe::kChainMaxTokens && p->chain) {
      moe::ChainArgs c{};
      moe::chain_items(d, &c);
      c.hidden = static_cast<const uint16_t*>(a->hidden);
      c.residual = static_cast<const uint16_t*>(a->residual);
      c.w13 = static_cast<const uint8_t*>(a->w13);
      c.w13_scale = a->w13_scale;
      c.w2 = static_cast<const uint8_t*>(a->w2);
      c.w2_scale = a->w2_scale;
      c.sw2 = static_cast<const uint8_t*>(a->sw2);
      c.sw2_scale = a->sw2_scale;
      c.gamma = static_cast<const uint16_t*>(a->gamma);
      c.out = static_cast<uint16_t*>(a->out);
      c.moe_out = static_cast<uint16_t*>(a->moe_out);
      c.residual_out = static_cast<uint16_t*>(a->residual_out);
      if (err == hipSuccess)
        step(moe::launch_expert_chain(c, p->ws, s, p->user_begin, p->user_end));
      return err == hipSuccess ? MOE_DECODE_OK : MOE_DECODE_ERR_HIP;
    }
    if (err == hipSuccess)
      step(moe::launch_gate_up_gemv(d, a->hidden, a->w13, a->w13_scale, p->ws, s,
                                    p->user_begin, p->user_end));
    if (err == hipSuccess)
      step(moe::launch_down_gemv(d, a->w2, a->w2_scale, a->sw2, a->sw2_scale, p->ws, s));
    if (err == hipSuccess)
      step(moe::launch_epilogue(d, a->residual, a->gamma, p->ws, a->out, a->residual_out,
                                a->moe_out, s));
    return err == hipSuccess ? MOE_DECODE_OK : MOE_DECODE_ERR_HIP;
  }

  // GROUPED: router, the projections, the boundary.  Up to
  // kMergeSharedMaxTokens tokens the shared expert's passes are extra rows of
  // the routed launches; above that they run on the side stream, forked once
  // the router is queued and joined before the boundary.  Many tokens take
  // the matrix-core router.
  if (T >= moe::kRouterMfmaMinTokens)
    step(moe::launch_router_mfma(
        d, a->hidden, a->router_w, static_cast<const float*>(bias), p->ws,
        moe::router_mfma_tokens_padded(p->desc.max_tokens),
        T <= moe::kMergeSharedMaxTokens ? moe::sync_lines(T * d.k < d.E ? T * d.k : d.E) : 0,
        a->topk_ids, a->topk_weights, s));
  else
    step(moe::launch_router(d, a->hidden, a->router_w, static_cast<const float*>(bias), p->ws,
                            a->topk_ids, a->topk_weights, nullptr, nullptr, s));
  if (err != hipSuccess) return MOE_DECODE_ERR_HIP;
  const bool side = has_shared && T > moe::kMergeSharedMaxTokens;
  const int rows = side ? moe::kRoutedRows : moe::kAllRows;
  const void* sw13 = has_shared ? a->sw13 : nullptr;
  const void* sw2 = has_shared ? a->sw2 : nullptr;
  // a run without a side stream (moe_decode_run_static) queues the shared
  // passes on `s`, ahead of the routed launches
  const bool fork = side && p->side != nullptr;
  const hipStream_t ss = fork ? p->side : s;
  if (side) {
    if (fork) {
      if (hipEventRecord(p->fork, s) != hipSuccess) return MOE_DECODE_ERR_HIP;
      if (hipStreamWaitEvent(p->side, p->fork, 0) != hipSuccess) return MOE_DECODE_ERR_HIP;
    }
    step(moe::launch_gate_up_mfma(d, moe::kSharedRows, a->hidden, a->w13, a->w13_scale, sw13,
                                  a->sw13_scale, p->ws, ss));
    if (err == hipSuccess)
      step(moe::launch_down_mfma(d, moe::kSharedRows, a->w2, a->w2_scale, sw2, a->sw2_scale,
                                 p->ws, ss));
  }
  if (!side && moe::grouped_chain_supported(d)) {
    // gate_up and down in one launch (the down tiles start in the gate_up
    // drain), with few tokens the boundary too (right after the last down tile)
    if (err == hipSuccess)
      step(moe::launch_grouped_chain(d, a->hidden, a->w13, a->w13_scale, sw13, a->sw13_scale,
                                     a->w2, a->w2_scale, sw2, a->sw2_scale, a->residual,
                                     a->gamma, a->out, a->residual_out, a->moe_out, p->ws, s,
                                     p->user_begin, p->user_end));
    if (moe::grouped_boundary_fused(d))
      return err == hipSuccess ? MOE_DECODE_OK : MOE_DECODE_ERR_HIP;
  } else {
    if (err == hipSuccess)
      step(moe::launch_gate_up_mfma(d, rows, a->hidden, a->w13, a->w13_scale, sw13,
                                    a->sw13_scale, p->ws, s, p->user_begin, p->user_end));
    if (err == hipSuccess)
      step(moe::launch_down_mfma(d, rows, a->w2, a->w2_scale, sw2, a->sw2_scale, p->ws, s));
  }
  if (fork) {
    // joined on every path, errors included, so a capture sees no loose work
    hipError_t jerr = hipEventRecord(p->join, p->side);
    if (jerr == hipSuccess) jerr = hipStreamWaitEvent(s, p->join, 0);
    if (err == hipSuccess) err = jerr;
  }
  if (err == hipSuccess)
    step(moe::launch_epilogue(d, a->residual, a->gamma, p->ws, a->out, a->residual_out,
                                a->moe_out, s));
  return err == hipSuccess ? MOE_DECODE_OK : MOE_DECODE_ERR_HIP;
}

int moe_decode_last_routes(moe_decode_plan_t p, int32_t T, int32_t* counts, int32_t* offsets,
                           int32_t* perm, int32_t* touched, int32_t* n_touched, void* stream) {
  if (!p || T < 0 || T > p->desc.max_tokens) return MOE_DECODE_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t E = p->desc.num_experts, R = static_cast<size_t>(T) * p->desc.top_k;
  struct {
    void* dst;
    const void* src;
    size_t n;
  } cp[] = {{counts, p->ws.counts, E * 4},
            {offsets, p->ws.offsets, (E + 1) * 4},
            {perm, p->ws.perm, R * 4},
            {touched, p->ws.touched, E * 4},
            {n_touched, p->ws.n_touched, 4}};
  for (auto& c : cp)
    if (c.dst && c.n &&
        hipMemcpyAsync(c.dst, c.src, c.n, hipMemcpyDeviceToDevice, s) != hipSuccess)
      return MOE_DECODE_ERR_HIP;
  return MOE_DECODE_OK;
}

int moe_decode_set_expert_events(moe_decode_plan_t p, void* begin, void* end) {
  if (!p || (!begin) != (!end)) return MOE_DECODE_ERR_INVALID_ARG;
  p->user_begin = static_cast<hipEvent_t>(begin);
  p->user_end = static_cast<hipEvent_t>(end);
  return MOE_DECODE_OK;
}

int moe_decode_path_for(moe_decode_plan_t p, int32_t T) {
  if (!p || T < 0 || T > p->desc.max_tokens) return -MOE_DECODE_ERR_INVALID_ARG;
  return path_for(*p, T);
}

int moe_decode_check_waits(moe_decode_plan_t p, int32_t* gave_up) {
  if (!p || !gave_up) return MOE_DECODE_ERR_INVALID_ARG;
  int prev = 0;
  if (hipGetDevice(&prev) != hipSuccess || hipSetDevice(p->device) != hipSuccess)
    return MOE_DECODE_ERR_HIP;
  uint32_t flag = 0;
  int rc = MOE_DECODE_OK;
  if (hipDeviceSynchronize() != hipSuccess ||
      hipMemcpy(&flag, p->ws.sync + moe::kSyncError * moe::kSyncStride, 4,
                hipMemcpyDeviceToHost) != hipSuccess ||
      hipMemset(p->ws.sync + moe::kSyncError * moe::kSyncStride, 0, 4) != hipSuccess)
    rc = MOE_DECODE_ERR_HIP;
  // a wait that gave up may have left counters part-way: start the next run
  // from the zeroed state a new plan has
  if (!rc && flag && hipMemset(p->ws_base, 0, p->state_bytes) != hipSuccess)
    rc = MOE_DECODE_ERR_HIP;
  if (!rc && hipDeviceSynchronize() != hipSuccess) rc = MOE_DECODE_ERR_HIP;
  (void)hipSetDevice(prev);
  *gave_up = flag != 0;
  return rc;
}

size_t moe_decode_workspace_bytes(moe_decode_plan_t p) { return p ? p->ws_bytes : 0; }

}  // extern "C"

// ---- the entry point that allocates nothing ---------------------------------
// For callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid it).  Its workspace is
// `scratch`, a file-scope device array: every GPU the library runs on holds
// its own copy, at its own address, until the process ends.
namespace {
constexpr size_t kStaticScratchBytes = MOE_DECODE_STATIC_SCRATCH_BYTES;
constexpr int kStaticMaxDevices = 64;
}  // namespace

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {

std::mutex g_scratch_mu;
// The device address of `scratch` on each device (nullptr: not set up yet).
// Host code uses these, never the array's name, which on the host is only a
// stand-in for the symbol.
void* g_scratch_ptr[kStaticMaxDevices];

// Sets up device `dev` (current) once: checks it is gfx950 and takes the
// address of its copy of `scratch`.
int scratch_for_device(int dev, void** out) {
  if (dev < 0 || dev >= kStaticMaxDevices) return MOE_DECODE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MOE_DECODE_ERR_HIP;
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) return MOE_DECODE_ERR_UNSUPPORTED;
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr)
      return MOE_DECODE_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return MOE_DECODE_OK;
}

// Zeroes n 32-bit words (a kernel, not hipMemsetAsync, so that a captured
// graph replays it correctly).
__global__ __launch_bounds__(256) void zero_words_kernel(uint32_t* p, size_t n) {
  const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride)
    p[i] = 0u;
}

}  // namespace

extern "C" int moe_decode_run_static(const moe_decode_desc* d, const moe_decode_args* a,
                                     int32_t T, void* stream) {
  int rc = moe_decode_desc_check(d);
  if (rc) return rc;
  rc = moe_decode_args_check(d, a, T);
  if (rc) return rc;
  if (T == 0) return MOE_DECODE_OK;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_DECODE_ERR_HIP;
  void* base = nullptr;
  rc = scratch_for_device(dev, &base);
  if (rc) return rc;

  // a plan on the host stack: workspace in the scratch array, sized for T
  moe_decode_plan_s p{};
  p.desc = *d;
  p.desc.max_tokens = T;
  p.device = dev;
  size_t state = 0;
  p.ws_bytes = layout(p.desc, nullptr, nullptr, &state);
  p.state_bytes = state;
  if (p.ws_bytes > kStaticScratchBytes) return MOE_DECODE_ERR_SCRATCH;
  layout(p.desc, static_cast<char*>(base), &p.ws);
  p.ws_base = base;
  p.side = nullptr;  // the shared expert's passes go on `stream` too
  p.chain = moe::chain_supported(d->hidden, d->intermediate, d->shared_intermediate);

  // The array keeps the last call's contents: clear the counters, flags,
  // boundary slots, zero bias and error word that a run expects at zero.
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t words = state / 4;
  const unsigned blocks = static_cast<unsigned>(std::min<size_t>((words + 255) / 256, 1024));
  hipLaunchKernelGGL(zero_words_kernel, dim3(blocks), dim3(256), 0, s,
                     static_cast<uint32_t*>(base), words);
  if (hipGetLastError() != hipSuccess) return MOE_DECODE_ERR_HIP;
  return run_on_device(&p, a, T, s);
}
