/*
 * Runs the C oracle (oracle/moe_oracle.c) on small synthetic layers, for a
 * build with AddressSanitizer and UndefinedBehaviorSanitizer: every branch
 * of the oracle is taken at least once (fp32 and e8m0 scales, bias or none,
 * a shared expert or none, a row subset, forced ids, k = E, a rejected
 * argument), and the invariants that do not need a reference are checked:
 * the weights sum to the routed scaling factor and the outputs are finite.
 * Exit status 0 when every check holds.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int moe_oracle_layer(int T, int H, int E, int k, int I, int Is, int e8m0, double limit,
                     double rsf, double eps, const uint16_t* hidden, const uint16_t* residual,
                     const uint16_t* router_w, const float* bias, const uint8_t* w13,
                     const void* w13_scale, const uint8_t* w2, const void* w2_scale,
                     const uint8_t* sw13, const void* sw13_scale, const uint8_t* sw2,
                     const void* sw2_scale, const uint16_t* gamma, const int32_t* rows,
                     int n_rows, const int32_t* forced_ids, double* out, double* h_out,
                     int32_t* ids_out, double* w_out, double* gaps_out, double* logits_out,
                     int nthreads);

static uint32_t rng = 12345u;
static uint32_t next(void) { rng = rng * 1664525u + 1013904223u; return rng >> 8; }
/* bf16 bits of a small value in [-2, 2) */
static uint16_t bf16_small(void) {
  float f = ((float)(next() % 4096) / 1024.0f) - 2.0f;
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}
/* an e4m3fn code that is not NaN */
static uint8_t fp8_code(void) {
  uint8_t c = (uint8_t)(next() & 0xff);
  return (c & 0x7f) == 0x7f ? 0x38 : c;
}

static int run_case(int T, int H, int E, int k, int I, int Is, int e8m0, int with_bias,
                    int subset, int forced) {
  const size_t sblk13 = (size_t)(2 * I / 128) * (H / 128), sblk2 = (size_t)(H / 128) * (I / 128);
  const size_t ssb13 = (size_t)(2 * (Is ? Is : 128) / 128) * (H / 128);
  const size_t ssb2 = (size_t)(H / 128) * ((Is ? Is : 128) / 128);
  const size_t selem = e8m0 ? 1 : 4;
  uint16_t* hidden = malloc(sizeof(uint16_t) * T * H);
  uint16_t* residual = malloc(sizeof(uint16_t) * T * H);
  uint16_t* router = malloc(sizeof(uint16_t) * E * H);
  uint16_t* gamma = malloc(sizeof(uint16_t) * H);
  float* bias = malloc(sizeof(float) * E);
  uint8_t* w13 = malloc((size_t)E * 2 * I * H);
  uint8_t* w2 = malloc((size_t)E * H * I);
  unsigned char* s13 = malloc(E * sblk13 * selem);
  unsigned char* s2 = malloc(E * sblk2 * selem);
  uint8_t* sw13 = malloc((size_t)2 * (Is ? Is : 128) * H);
  uint8_t* sw2 = malloc((size_t)H * (Is ? Is : 128));
  unsigned char* ss13 = malloc(ssb13 * selem);
  unsigned char* ss2 = malloc(ssb2 * selem);
  for (int i = 0; i < T * H; ++i) { hidden[i] = bf16_small(); residual[i] = bf16_small(); }
  for (int i = 0; i < E * H; ++i) router[i] = bf16_small();
  for (int i = 0; i < H; ++i) gamma[i] = 0x3f80;  /* 1.0 */
  for (int i = 0; i < E; ++i) bias[i] = (float)((int)(next() % 200) - 100) * 1e-3f;
  for (size_t i = 0; i < (size_t)E * 2 * I * H; ++i) w13[i] = fp8_code();
  for (size_t i = 0; i < (size_t)E * H * I; ++i) w2[i] = fp8_code();
  for (size_t i = 0; i < (size_t)2 * (Is ? Is : 128) * H; ++i) sw13[i] = fp8_code();
  for (size_t i = 0; i < (size_t)H * (Is ? Is : 128); ++i) sw2[i] = fp8_code();
  /* scales: 1/448 as fp32, or e8m0 byte 118 (2^-9) */
  const float fs = 1.0f / 448.0f;
  for (size_t i = 0; i < E * sblk13; ++i)
    e8m0 ? (void)(s13[i] = 118) : (void)memcpy(s13 + 4 * i, &fs, 4);
  for (size_t i = 0; i < E * sblk2; ++i)
    e8m0 ? (void)(s2[i] = 118) : (void)memcpy(s2 + 4 * i, &fs, 4);
  for (size_t i = 0; i < ssb13; ++i) e8m0 ? (void)(ss13[i] = 118) : (void)memcpy(ss13 + 4 * i, &fs, 4);
  for (size_t i = 0; i < ssb2; ++i) e8m0 ? (void)(ss2[i] = 118) : (void)memcpy(ss2 + 4 * i, &fs, 4);

  int32_t rows[2] = {T - 1, 0};
  const int n = subset ? 2 : T;
  int32_t* fids = malloc(sizeof(int32_t) * T * k);
  /* forced ids, distinct per token: a rotation */
  for (int t = 0; t < T; ++t)
    for (int j = 0; j < k; ++j) fids[t * k + j] = (t + j) % E;
  double* out = malloc(sizeof(double) * n * H);
  double* h = malloc(sizeof(double) * n * H);
  int32_t* ids = malloc(sizeof(int32_t) * n * k);
  double* w = malloc(sizeof(double) * n * k);
  double* gaps = malloc(sizeof(double) * n);
  double* logits = malloc(sizeof(double) * n * E);
  const double rsf = 2.5;
  int rc = moe_oracle_layer(T, H, E, k, I, Is, e8m0, 7.0, rsf, 1e-5, hidden, residual, router,
                            with_bias ? bias : NULL, w13, s13, w2, s2, Is ? sw13 : NULL,
                            Is ? ss13 : NULL, Is ? sw2 : NULL, Is ? ss2 : NULL, gamma,
                            subset ? rows : NULL, n, forced ? fids : NULL, out, h, ids, w, gaps,
                            logits, 2);
  int bad = rc != 0;
  for (int p = 0; p < n && !bad; ++p) {
    double sw = 0.0;
    for (int j = 0; j < k; ++j) sw += w[p * k + j];
    if (fabs(sw - rsf) > 1e-12) bad = 1;
    for (int c = 0; c < H; ++c)
      if (!isfinite(out[p * H + c]) || !isfinite(h[p * H + c])) bad = 1;
  }
  printf("case T=%d H=%d E=%d k=%d I=%d Is=%d e8m0=%d bias=%d subset=%d forced=%d: %s\n", T,
         H, E, k, I, Is, e8m0, with_bias, subset, forced, bad ? "FAIL" : "ok");
  free(hidden); free(residual); free(router); free(gamma); free(bias); free(w13); free(w2);
  free(s13); free(s2); free(sw13); free(sw2); free(ss13); free(ss2); free(fids); free(out);
  free(h); free(ids); free(w); free(gaps); free(logits);
  return bad;
}

int main(void) {
  int bad = 0;
  bad |= run_case(3, 256, 8, 2, 128, 128, 0, 0, 0, 0);
  bad |= run_case(3, 256, 8, 2, 128, 128, 1, 1, 1, 0);
  bad |= run_case(2, 384, 6, 6, 256, 0, 0, 1, 0, 1);  /* k = E, no shared expert, forced ids */
  bad |= run_case(1, 128, 16, 4, 128, 256, 1, 0, 0, 0);
  /* a rejected argument: H not a multiple of 128 */
  {
    double o[1];
    int32_t i[1];
    int rc = moe_oracle_layer(1, 100, 4, 1, 128, 0, 0, 7.0, 2.5, 1e-5, NULL, NULL, NULL, NULL,
                              NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0,
                              NULL, o, o, i, o, o, NULL, 1);
    printf("rejected argument: %s\n", rc == -1 ? "ok" : "FAIL");
    bad |= rc != -1;
  }
  return bad;
}
