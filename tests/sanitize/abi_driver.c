/*
 * Calls the host-side part of the C-ABI (include/moe_decode.h) for a build
 * with AddressSanitizer and UndefinedBehaviorSanitizer on the host code: the
 * descriptor and argument checks on every branch, the status strings, and
 * each entry point's rejection of a null plan or a bad argument, all before
 * any device is touched.  Exit status 0 when every return code is the
 * documented one.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "moe_decode.h"

static int bad = 0;
#define EXPECT(expr, want)                                                        \
  do {                                                                            \
    int got_ = (expr);                                                            \
    if (got_ != (want)) {                                                         \
      printf("FAIL %s:%d: %s = %d, want %d\n", __FILE__, __LINE__, #expr, got_,   \
             (int)(want));                                                        \
      bad = 1;                                                                    \
    }                                                                             \
  } while (0)

static moe_decode_desc good(void) {
  moe_decode_desc d;
  memset(&d, 0, sizeof d);
  d.hidden = 4096;
  d.num_experts = 128;
  d.top_k = 8;
  d.intermediate = 1536;
  d.shared_intermediate = 1536;
  d.max_tokens = 16;
  d.scale_fmt = MOE_DECODE_SCALE_FP32;
  d.path = MOE_DECODE_PATH_AUTO;
  d.swiglu_limit = 7.0f;
  d.routed_scaling_factor = 2.5f;
  d.rms_eps = 1e-5f;
  return d;
}

/* distinct, 16-byte aligned fake addresses; never dereferenced */
static moe_decode_args args(void) {
  moe_decode_args a;
  memset(&a, 0, sizeof a);
  const void** f[] = {&a.hidden, &a.residual, &a.router_w, &a.w13, &a.w13_scale, &a.w2,
                      &a.w2_scale, &a.sw13, &a.sw13_scale, &a.sw2, &a.sw2_scale, &a.gamma};
  for (size_t i = 0; i < sizeof f / sizeof f[0]; ++i) *f[i] = (const void*)(0x100000u * (i + 1));
  a.out = (void*)0x2000000u;
  a.residual_out = (void*)0x2100000u;
  return a;
}

int main(void) {
  moe_decode_desc d = good();
  EXPECT(moe_decode_desc_check(&d), MOE_DECODE_OK);
  EXPECT(moe_decode_desc_check(NULL), MOE_DECODE_ERR_INVALID_ARG);
  const struct {
    int field, value, want;
  } cases[] = {
      {0, 4000, MOE_DECODE_ERR_UNSUPPORTED}, {0, 8320, MOE_DECODE_ERR_UNSUPPORTED},
      {0, 0, MOE_DECODE_ERR_INVALID_ARG},    {0, -128, MOE_DECODE_ERR_INVALID_ARG},
      {1, 1025, MOE_DECODE_ERR_UNSUPPORTED}, {1, 4, MOE_DECODE_ERR_UNSUPPORTED},
      {1, -1, MOE_DECODE_ERR_INVALID_ARG},   {2, 17, MOE_DECODE_ERR_UNSUPPORTED},
      {2, 0, MOE_DECODE_ERR_INVALID_ARG},    {3, 100, MOE_DECODE_ERR_UNSUPPORTED},
      {3, 0, MOE_DECODE_ERR_INVALID_ARG},    {4, 64, MOE_DECODE_ERR_UNSUPPORTED},
      {4, -128, MOE_DECODE_ERR_INVALID_ARG}, {5, 257, MOE_DECODE_ERR_UNSUPPORTED},
      {5, 0, MOE_DECODE_ERR_INVALID_ARG},    {6, 7, MOE_DECODE_ERR_INVALID_ARG},
      {7, 9, MOE_DECODE_ERR_INVALID_ARG},    {7, -1, MOE_DECODE_ERR_INVALID_ARG},
  };
  for (size_t i = 0; i < sizeof cases / sizeof cases[0]; ++i) {
    moe_decode_desc x = good();
    int32_t* f[] = {&x.hidden, &x.num_experts, &x.top_k, &x.intermediate,
                    &x.shared_intermediate, &x.max_tokens, &x.scale_fmt, &x.path};
    *f[cases[i].field] = cases[i].value;
    EXPECT(moe_decode_desc_check(&x), cases[i].want);
  }
  {
    moe_decode_desc x = good();
    x.swiglu_limit = 0.0f;
    EXPECT(moe_decode_desc_check(&x), MOE_DECODE_ERR_INVALID_ARG);
    x = good();
    x.rms_eps = -1.0f;
    EXPECT(moe_decode_desc_check(&x), MOE_DECODE_ERR_INVALID_ARG);
    x = good();
    x.routed_scaling_factor = 0.0f / 0.0f;
    EXPECT(moe_decode_desc_check(&x), MOE_DECODE_ERR_INVALID_ARG);
    /* a dense layer: no routed experts, the MLP in the shared slot */
    x = good();
    x.num_experts = 0;
    x.top_k = 0;
    x.intermediate = 0;
    EXPECT(moe_decode_desc_check(&x), MOE_DECODE_OK);
    x.shared_intermediate = 0;
    EXPECT(moe_decode_desc_check(&x), MOE_DECODE_ERR_INVALID_ARG);
  }

  moe_decode_args a = args();
  EXPECT(moe_decode_args_check(&d, &a, 1), MOE_DECODE_OK);
  EXPECT(moe_decode_args_check(&d, &a, 0), MOE_DECODE_OK);
  EXPECT(moe_decode_args_check(&d, &a, 16), MOE_DECODE_OK);
  EXPECT(moe_decode_args_check(&d, &a, 17), MOE_DECODE_ERR_INVALID_ARG);
  EXPECT(moe_decode_args_check(&d, &a, -1), MOE_DECODE_ERR_INVALID_ARG);
  EXPECT(moe_decode_args_check(NULL, &a, 1), MOE_DECODE_ERR_INVALID_ARG);
  EXPECT(moe_decode_args_check(&d, NULL, 1), MOE_DECODE_ERR_INVALID_ARG);
  {
    moe_decode_args x = args();
    x.w13 = (const void*)0x100008u; /* misaligned */
    EXPECT(moe_decode_args_check(&d, &x, 1), MOE_DECODE_ERR_INVALID_ARG);
    x = args();
    x.out = (void*)x.hidden;
    EXPECT(moe_decode_args_check(&d, &x, 1), MOE_DECODE_ERR_INVALID_ARG);
    x = args();
    x.residual_out = (void*)x.residual;
    EXPECT(moe_decode_args_check(&d, &x, 1), MOE_DECODE_OK);
    x.moe_out = x.out;
    EXPECT(moe_decode_args_check(&d, &x, 1), MOE_DECODE_ERR_INVALID_ARG);
    x = args();
    x.sw2 = NULL;
    EXPECT(moe_decode_args_check(&d, &x, 1), MOE_DECODE_ERR_INVALID_ARG);
    moe_decode_desc n = good();
    n.shared_intermediate = 0;
    EXPECT(moe_decode_args_check(&n, &x, 1), MOE_DECODE_OK);
  }

  for (int code = -1; code <= 6; ++code)
    if (!moe_decode_strerror(code) || !moe_decode_strerror(code)[0]) bad = 1;

  /* entry points: null plan, null descriptor, bad arguments */
  moe_decode_plan_t p = (moe_decode_plan_t)0x1;
  EXPECT(moe_decode_plan(&d, 0, NULL), MOE_DECODE_ERR_INVALID_ARG);
  moe_decode_desc x = good();
  x.hidden = 100;
  EXPECT(moe_decode_plan(&x, 0, &p), MOE_DECODE_ERR_UNSUPPORTED);
  EXPECT(p == NULL, 1);
  EXPECT(moe_decode_run(NULL, &a, 1, NULL), MOE_DECODE_ERR_INVALID_ARG);
  EXPECT(moe_decode_destroy(NULL), MOE_DECODE_OK);
  EXPECT(moe_decode_path_for(NULL, 1), -MOE_DECODE_ERR_INVALID_ARG);
  EXPECT(moe_decode_last_routes(NULL, 1, NULL, NULL, NULL, NULL, NULL, NULL),
         MOE_DECODE_ERR_INVALID_ARG);
  EXPECT(moe_decode_set_expert_events(NULL, NULL, NULL), MOE_DECODE_ERR_INVALID_ARG);
  EXPECT(moe_decode_run_static(NULL, &a, 1, NULL), MOE_DECODE_ERR_INVALID_ARG);
  EXPECT(moe_decode_run_static(&d, &a, 17, NULL), MOE_DECODE_ERR_INVALID_ARG);
  EXPECT(moe_decode_run_static(&x, &a, 1, NULL), MOE_DECODE_ERR_UNSUPPORTED);
  uint32_t sink;
  EXPECT(moe_decode_read_probe(NULL, (size_t)64 << 20, &sink, NULL), MOE_DECODE_ERR_INVALID_ARG);
  EXPECT(moe_decode_read_probe((const void*)0x100000u, 12345, &sink, NULL),
         MOE_DECODE_ERR_INVALID_ARG);
  printf("%s\n", bad ? "abi checks: FAIL" : "abi checks: ok");
  return bad;
}
