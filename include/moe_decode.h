/*
 * moe_decode.h -- C ABI of the MI355X (gfx950) decode-step MoE layer.
 *
 * One call runs one MoE layer of a decode (or speculative-verify) step for T
 * tokens, from the router to the residual-add + RMSNorm boundary:
 *
 *   logits   = x . W_r^T                       (fp32 accumulation)
 *   s        = sigmoid(logits)
 *   ids      = top-k experts by s (+ bias), ties to the lower id
 *   w        = R * s[ids] / sum s[ids]          (unbiased scores)
 *   for each route (t, j), e = ids[t, j]:
 *     g, u   = W13[e][0:I] . x_t, W13[e][I:2I] . x_t   (fp8 block-scaled)
 *     a      = silu(min(g, L)) * clamp(u, -L, L)
 *     y      = W2[e] . a
 *   y_s      = the same expert MLP with the shared weights (weight 1)
 *   h        = sum_j w[t, j] * y[t, j] + y_s[t] + residual[t]
 *   residual_out = bf16(h);  out = bf16(h / sqrt(mean(h^2) + eps) * gamma)
 *
 * Where this comes from (vLLM API pages on the GLM-5.3-Flash specialized
 * decode):
 *   - page "vllm.models.glm5next.nvidia.specialized_decode.runtime.decode",
 *     LayerStages._build_mega: the fused MoE stage is built only for sigmoid
 *     scoring, one expert group and normalised top-k; its constructor takes
 *     w13/w2 fp8 weights with their block scales, top_k, swiglu_limit,
 *     routed_scaling_factor and the power-of-two (e8m0) scale flag; its
 *     buffers are made once at build time.
 *   - same page, LayerStages._mega_moe: the shared expert runs beside the
 *     routed experts; the routed rows come back unfinalized with their
 *     expert weights and the shared output beside them; the router bias is
 *     handed to the expert kernel.  (There the shared expert has a second
 *     stream; here its tiles are extra workgroups of the same launches,
 *     which costs less on MI355X than a fork and join per step.)
 *   - same page, LayerStages._router: router logits in fp32 from a bf16
 *     router weight.
 *   - page "vllm.models.glm5next.nvidia.specialized_decode.runtime.draft",
 *     SpecializedDraft.reduced_norm / _build_ar_norm: the boundary after the
 *     MoE finalizes the routed rows (it is built with top_k) and returns
 *     norm(x + residual) together with the new residual.  On one GPU there is
 *     no all-reduce to fuse into it.
 *
 * Conventions
 *   - All tensors are row-major and contiguous, in device memory of the
 *     plan's device, owned by the caller.  The library never frees them and
 *     never writes an input.
 *   - bf16 = 16-bit brain float bit patterns; fp8 = OCP e4m3fn codes;
 *     e8m0 = one unsigned byte b per block meaning 2^(b-127) (255 invalid).
 *   - Block scales cover 128x128 weight blocks and are multiplied in:
 *     weight = code value * scale.
 *   - Every entry point returns 0 on success or a moe_decode_status code; none
 *     aborts.  moe_decode_strerror names a code.
 */
#ifndef MOE_DECODE_H
#define MOE_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_DECODE_OK = 0,
  MOE_DECODE_ERR_INVALID_ARG = 1, /* null required pointer, T out of range, bad enum */
  MOE_DECODE_ERR_UNSUPPORTED = 2, /* a size or device this library does not handle */
  MOE_DECODE_ERR_HIP = 3,         /* a HIP runtime call failed */
  MOE_DECODE_ERR_NO_MEMORY = 4,   /* workspace allocation failed at plan time */
  MOE_DECODE_ERR_SCRATCH = 5      /* moe_decode_run_static: the workspace for this size
                                     exceeds the static scratch array */
} moe_decode_status;

typedef enum { MOE_DECODE_SCALE_FP32 = 0, MOE_DECODE_SCALE_E8M0 = 1 } moe_decode_scale_fmt;

/* Expert kernel family.  AUTO picks by token count; the others force one. */
typedef enum {
  /* The faster path for the token count as measured on MI355X: GEMV_SPLIT
   * below 4 tokens, GROUPED from 4 tokens on. */
  MOE_DECODE_PATH_AUTO = 0,
  /* fp8 dequant-FMA GEMV, one weight pass per touched expert.  Up to 16
   * tokens and 256 experts the whole step is one launch of ordered work
   * items: router, shared expert, routed experts, boundary; at one token
   * each routed item selects its own expert from the logits.  Otherwise the
   * GEMV_SPLIT kernels run. */
  MOE_DECODE_PATH_GEMV = 1,
  /* Tokens grouped by expert on the matrix cores: exactly converted fp8
   * weights (staged through LDS) times bf16 activations in
   * v_mfma_f32_16x16x32_bf16, fp32 accumulation per 128-wide scale block;
   * the SwiGLU output goes to the down projection as hi + lo bf16 parts.
   * Kernels: router; up to 64 tokens one launch of the gate_up and down tiles
   * (shared expert's 16-token passes and the touched experts; a down tile
   * waits for its row's gate_up tiles through a bounded wait); boundary.
   * Above 64 tokens: separate gate_up and down launches of the touched
   * experts, and the shared expert's passes on the plan's side stream. */
  MOE_DECODE_PATH_GROUPED = 2,
  /* The GEMV kernels launched one after another: the router (with the
   * shared expert's gate_up beside it), then, up to 16 tokens, one expert
   * chain launch (the shared expert's down, the touched experts' gate_up and
   * down, the boundary; its workgroups hand rows to each other through
   * counters with bounded waits), above 16 tokens the routed gate_up, down
   * (shared and routed) and boundary kernels. */
  MOE_DECODE_PATH_GEMV_SPLIT = 3
} moe_decode_path;

/*
 * Layer constants, fixed at plan time (the pages fix them in the stage
 * constructors).  Limits: H, I and Is multiples of 128 with H <= 8192,
 * I <= 8192 and Is <= 8192; 1 <= top_k <= 16; top_k <= E <= 1024;
 * 1 <= max_tokens <= 256.  shared_intermediate = 0 means no shared expert.
 * num_experts = 0 (with top_k = 0, shared_intermediate > 0, and intermediate
 * unused: 0, or any size within the limits) is a dense layer: its fp8 clamped-SwiGLU MLP (the decode page's
 * DenseMlp, LayerStages._build_dense) goes in the shared-expert slot
 * (sw13, sw2 and their scales), the router and routed-expert pointers may be
 * NULL, and a run computes out, residual_out and moe_out (= the MLP output)
 * through the same boundary.  AUTO takes the MFMA kernels at every token
 * count: gate_up (up to 16 tokens with each workgroup's contraction split
 * over its four waves; above, with the contraction split over up to four
 * workgroups), then down with the contraction split over up to eight
 * workgroups; the last workgroup of a tile adds the partial sums in a fixed
 * order.  Such a plan's workspace also holds those partial sums and their
 * arrival counters.
 */
typedef struct {
  int32_t hidden;              /* H */
  int32_t num_experts;         /* E */
  int32_t top_k;               /* k */
  int32_t intermediate;        /* I, routed expert */
  int32_t shared_intermediate; /* Is, shared expert (0 = none) */
  int32_t max_tokens;          /* largest T a run may pass */
  int32_t scale_fmt;           /* moe_decode_scale_fmt, for routed and shared weights */
  int32_t path;                /* moe_decode_path */
  float swiglu_limit;          /* L > 0 */
  float routed_scaling_factor; /* R */
  float rms_eps;               /* eps >= 0 */
} moe_decode_desc;

/*
 * Per-call device pointers.  Shapes use T (the run's token count) and the
 * plan's constants.  Scale tensors are float32 for MOE_DECODE_SCALE_FP32 and
 * uint8 for MOE_DECODE_SCALE_E8M0.
 */
typedef struct {
  const void* hidden;       /* [T, H] bf16: the MoE input x */
  const void* residual;     /* [T, H] bf16 */
  const void* router_w;     /* [E, H] bf16 */
  const float* router_bias; /* [E] fp32 score-correction bias, or NULL */
  const void* w13;          /* [E, 2I, H] fp8: rows [0, I) gate, [I, 2I) up */
  const void* w13_scale;    /* [E, 2I/128, H/128] */
  const void* w2;           /* [E, H, I] fp8 */
  const void* w2_scale;     /* [E, H/128, I/128] */
  const void* sw13;         /* [2Is, H] fp8 (ignored when Is = 0) */
  const void* sw13_scale;   /* [2Is/128, H/128] */
  const void* sw2;          /* [H, Is] fp8 */
  const void* sw2_scale;    /* [H/128, Is/128] */
  const void* gamma;        /* [H] bf16 RMSNorm weight */
  void* out;                /* [T, H] bf16: RMSNorm(h) * gamma */
  void* residual_out;       /* [T, H] bf16: h; may alias residual, nothing else */
  int32_t* topk_ids;        /* [T, k] selected experts in rank order, or NULL */
  float* topk_weights;      /* [T, k] their weights (R-scaled), or NULL */
  /* [T, H] bf16: the finalized MoE output sum_j w_j y_j + y_shared, before
   * the residual add and the norm (the decode page's LayerStages._grouped_moe
   * takes this from the grouped kernel with finalize=True, for token counts
   * whose boundary is not fused), or NULL.  Written by the boundary beside
   * out and residual_out; it may alias no other tensor. */
  void* moe_out;
} moe_decode_args;

typedef struct moe_decode_plan_s* moe_decode_plan_t;

/*
 * Checks a descriptor on the host without touching any device.
 * Returns OK, INVALID_ARG (null, bad enum, non-positive size) or
 * UNSUPPORTED (outside the limits above).
 */
int moe_decode_desc_check(const moe_decode_desc* d);

/*
 * Checks a run's arguments against a descriptor on the host (pointers are
 * not dereferenced).  Returns OK or INVALID_ARG (T < 0, T > max_tokens, a
 * required pointer NULL, out aliasing an input).
 */
int moe_decode_args_check(const moe_decode_desc* d, const moe_decode_args* a, int32_t T);

/*
 * Builds a plan on HIP device `device`: validates the descriptor, checks the
 * device is gfx950, allocates the workspace for max_tokens and creates a side
 * stream (default priority) with two events.  On success *out owns them
 * until moe_decode_destroy; on failure *out is set to NULL and nothing is
 * leaked.
 *
 * Defined by the decode page's LayerStages._build_mega: the MoE stage is
 * built once per layer from the layer constants (top_k, swiglu_limit,
 * routed_scaling_factor, the e8m0 flag), and its route-order buffer and the
 * shared expert's stream are made once at build time, sized for the largest
 * token count, before any graph capture.  Errors: INVALID_ARG (null out, bad
 * descriptor or device index), UNSUPPORTED (a size outside the limits, or a
 * device that is not gfx950), NO_MEMORY, HIP.
 */
int moe_decode_plan(const moe_decode_desc* d, int device, moe_decode_plan_t* out);

/*
 * Runs the layer for T tokens, asynchronously on `stream` (a hipStream_t of
 * the plan's device; NULL = the null stream).  No allocation and no host
 * synchronisation, so the call may be captured into a HIP graph.  Every
 * kernel goes to `stream`, except the shared expert's on the MFMA path above
 * 64 tokens: those run on the plan's side stream, forked from `stream` after
 * the router and joined back before the boundary (also when an error occurs
 * after the fork).  T = 0 returns OK and launches nothing.  Runs on one plan
 * must not overlap (they share its workspace).
 *
 * Defined by the decode page's LayerStages._mega_moe (router logits, the
 * routed experts as one stage, the shared expert beside them, the routed
 * rows handed on with their weights and route order) and LayerStages._router
 * (fp32 logits from the bf16 router weight), followed by the draft page's
 * SpecializedDraft.reduced_norm (norm(x + residual) and the new residual).
 * An error after the fork still joins the side stream before it returns, as
 * the v41 draft page's DraftDecode.run rejoins its side stream before it
 * reports an error, so a capture sees no unjoined work.
 *
 * Errors: INVALID_ARG (moe_decode_args_check), HIP (a launch failed).  The
 * launches hand work between workgroups through bounded waits; if one ever
 * gave up, the run still returns OK but out, residual_out and moe_out are
 * not trustworthy: the boundary then writes NaN to out, and
 * moe_decode_check_waits reports it.
 */
int moe_decode_run(moe_decode_plan_t p, const moe_decode_args* a, int32_t T, void* stream);

/* Waits for the plan's device, then frees the plan's workspace, side stream
 * and events (what LayerStages._build_mega made for the stage).  NULL is a
 * no-op; always returns OK. */
int moe_decode_destroy(moe_decode_plan_t p);

/* Static text naming a status code.  Where the decode page's
 * LayerStages._build_mega meets a routing it does not support it warns and
 * runs the stock layers; this library has no second compute path, so it
 * returns the reason to the caller, and this names it. */
const char* moe_decode_strerror(int code);

/*
 * Token -> expert permutation of the plan's last run, copied on `stream`
 * into caller device buffers (any may be NULL):
 *   counts [E]      routes per expert
 *   offsets [E+1]   exclusive prefix sum of counts
 *   perm [T*k]      routes r = t*k + j sorted by expert, in r order within one
 *   touched [E]     experts with count > 0 in ascending id; n_touched [1] of them
 * T must be the last run's T.  This is the pages' expanded-index-to-permuted-
 * index table (LayerStages._mega_moe) in inverse form.
 */
int moe_decode_last_routes(moe_decode_plan_t p, int32_t T, int32_t* counts, int32_t* offsets,
                           int32_t* perm, int32_t* touched, int32_t* n_touched, void* stream);

/*
 * Measurement hook: when both are non-NULL, each later run launches its
 * dominant kernel with hipExtLaunchKernel, which records hipEvent_t `begin`
 * and `end` (created by the caller, timing enabled) at that kernel's own start
 * and end.  The dominant kernel is the single-launch step on
 * MOE_DECODE_PATH_GEMV; on MOE_DECODE_PATH_GEMV_SPLIT the expert chain launch
 * (up to 16 tokens) or the routed-expert gate/up projection kernel; on
 * MOE_DECODE_PATH_GROUPED the gate_up + down launch (up to 64 tokens) or the
 * routed gate/up projection kernel.  NULL, NULL switches
 * it off.  Eager runs only: not for use under graph capture.
 */
int moe_decode_set_expert_events(moe_decode_plan_t p, void* begin, void* end);

/* Which kernels a run with T tokens takes: MOE_DECODE_PATH_GEMV (the
 * single-launch step), MOE_DECODE_PATH_GEMV_SPLIT or MOE_DECODE_PATH_GROUPED;
 * negative status on a bad argument. */
int moe_decode_path_for(moe_decode_plan_t p, int32_t T);

/*
 * Health check of the bounded waits (the single-launch path's, the expert
 * chain launch's and the grouped gate_up + down launch's): synchronises the
 * plan's device, returns in *gave_up whether any wait since the last check
 * ran out of its spin budget (outputs of the runs since the last check are
 * then not trustworthy) and clears the flag.  After a give-up it also
 * re-zeroes the plan's counters, so later runs start from a clean state.
 * Not capturable; for tests and monitoring.
 */
int moe_decode_check_waits(moe_decode_plan_t p, int32_t* gave_up);

/* Device bytes the plan holds for its workspace. */
size_t moe_decode_workspace_bytes(moe_decode_plan_t p);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * layer as moe_decode_run, on the current HIP device, without a plan.  It
 * calls no allocating routine.  Its workspace is a static device array of
 * 64 MiB (MOE_DECODE_STATIC_SCRATCH_BYTES) that every GPU the library runs on
 * holds, one copy each, until the process ends; the first call on a device
 * looks up that device's copy (and checks the device is gfx950).
 *
 * Arguments as moe_decode_run, with the descriptor in place of a plan
 * (d->max_tokens bounds T as before; the workspace is laid out for T).
 * Differences: the shared expert's passes above 64 tokens run on `stream`
 * ahead of the routed launches (there is no side stream); no measurement
 * hook and no moe_decode_check_waits (a bounded wait that gives up shows as
 * NaN in out).  Every call clears the array's counters and flags first, so a call
 * never depends on the one before it.  Calls on one GPU share its array:
 * calls that overlap on one GPU (other streams, other threads) race and give
 * undefined results; serialise them.
 *
 * Errors: INVALID_ARG, UNSUPPORTED (as moe_decode_plan; also a device index
 * of 64 or more), SCRATCH (the workspace for this descriptor and T exceeds
 * the array: for example 128 tokens at H = 6144, k = 8, I = 2048 need about
 * 38 MiB and fit, 256 tokens do not), HIP.
 */
#define MOE_DECODE_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
int moe_decode_run_static(const moe_decode_desc* d, const moe_decode_args* a, int32_t T,
                          void* stream);

/*
 * Measurement only (not part of the layer): one streaming read of `bytes`
 * bytes at device pointer `buf` (16-byte aligned; bytes a non-zero multiple
 * of 64 MiB) with the non-temporal 16-byte loads the expert kernels stream
 * their weights with, queued on `stream`.  `sink` (device, 256 uint32) is
 * written only to keep the loads live.  A benchmark times it with events to
 * state layer times as a fraction of a measured read ceiling besides the
 * published peak.  Errors: INVALID_ARG, HIP.
 */
int moe_decode_read_probe(const void* buf, size_t bytes, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_DECODE_H */
