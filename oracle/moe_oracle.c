/*
 * Float64 C oracle of one decode-step MoE layer with a sigmoid router.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the test suite, the smoke check and the
 * benchmark's CPU-baseline leg; the product path never links or calls it.
 *
 * A second, independent writing of the layer defined on the vLLM API pages
 * "vllm.models.glm5next.nvidia.specialized_decode.runtime.decode"
 * (LayerStages._build_mega: sigmoid scoring, one group, renormalised top-k
 * times routed_scaling_factor, fp8 w13/w2 with block scales, swiglu_limit;
 * LayerStages._mega_moe: shared expert added unweighted beside the routed
 * rows) and "vllm.models.glm5next.nvidia.specialized_decode.runtime.draft"
 * (SpecializedDraft.reduced_norm: the boundary returns norm(x + residual) and
 * the new residual).  Same readings as the NumPy version: ties to the lower
 * expert id, weights from unbiased scores, gate rows [0, I) and up rows
 * [I, 2I) of w13, silu(min(g, L)) * clamp(u, -L, L), RMSNorm with gamma
 * multiplied in.
 *
 * Plain loops in float64; OpenMP only splits independent output rows over
 * threads, so no sum changes its order with the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define BLK 128

/* OCP FP8 E4M3 (e4m3fn): sign, 4-bit exponent with bias 7, 3-bit mantissa,
 * no infinities, S.1111.111 = NaN, exponent 0 = subnormal. */
static double e4m3_value(unsigned code) {
  double sign = (code & 0x80u) ? -1.0 : 1.0;
  unsigned ex = (code >> 3) & 0xFu, man = code & 0x7u;
  if (ex == 0xFu && man == 0x7u) return NAN;
  if (ex == 0) return sign * ldexp((double)man, -9);
  return sign * ldexp(1.0 + man / 8.0, (int)ex - 7);
}

static double bf16_value(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* Block scale: float32 as stored, or e8m0 byte b meaning 2^(b-127). */
static double block_scale(const void* scales, int e8m0, size_t idx) {
  if (e8m0) {
    uint8_t b = ((const uint8_t*)scales)[idx];
    return b == 255 ? NAN : ldexp(1.0, (int)b - 127);
  }
  return (double)((const float*)scales)[idx];
}

static double sigmoid(double z) { return 1.0 / (1.0 + exp(-z)); }

/* y[r] = sum_c W[r, c] * v[c] for a block-quantised W [R, C]. */
static void deq_matvec(const uint8_t* W, const void* S, int e8m0, const double* lut,
                       int R, int C, const double* v, double* y) {
  int cb = C / BLK;
#pragma omp parallel for schedule(static)
  for (int r = 0; r < R; ++r) {
    const uint8_t* row = W + (size_t)r * C;
    double acc = 0.0;
    for (int c = 0; c < C; ++c)
      acc += lut[row[c]] * block_scale(S, e8m0, (size_t)(r / BLK) * cb + c / BLK) * v[c];
    y[r] = acc;
  }
}

/* One expert on one token: gate/up projections, clamped SwiGLU, down. */
static void expert(const uint8_t* w13, const void* s13, const uint8_t* w2, const void* s2,
                   int e8m0, const double* lut, int H, int I, double limit,
                   const double* x, double* gu, double* a, double* y) {
  deq_matvec(w13, s13, e8m0, lut, 2 * I, H, x, gu);
  for (int i = 0; i < I; ++i) {
    double g = gu[i] < limit ? gu[i] : limit;
    double u = gu[I + i];
    u = u < -limit ? -limit : (u > limit ? limit : u);
    a[i] = g * sigmoid(g) * u;
  }
  deq_matvec(w2, s2, e8m0, lut, H, I, a, y);
}

/*
 * The layer on the token rows listed in `rows` (all T when rows == NULL).
 * Outputs are indexed by position in `rows`:
 *   out, h_out [n, H]; ids_out [n, k]; w_out [n, k]; gaps_out [n];
 *   logits_out [n, E] (nullable).
 * forced_ids [T, k] (nullable) replaces the selection.
 * Returns 0, or -1 on a bad argument.
 */
int moe_oracle_layer(int T, int H, int E, int k, int I, int Is, int e8m0, double limit,
                     double rsf, double eps, const uint16_t* hidden, const uint16_t* residual,
                     const uint16_t* router_w, const float* bias, const uint8_t* w13,
                     const void* w13_scale, const uint8_t* w2, const void* w2_scale,
                     const uint8_t* sw13, const void* sw13_scale, const uint8_t* sw2,
                     const void* sw2_scale, const uint16_t* gamma, const int32_t* rows,
                     int n_rows, const int32_t* forced_ids, double* out, double* h_out,
                     int32_t* ids_out, double* w_out, double* gaps_out, double* logits_out,
                     int nthreads) {
  if (T < 0 || H % BLK || I % BLK || Is % BLK || k < 1 || k > E) return -1;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#endif
  int n = rows ? n_rows : T;
  double lut[256];
  for (unsigned c = 0; c < 256; ++c) lut[c] = e4m3_value(c);
  int maxI = I > Is ? I : Is;
  double* x = malloc(sizeof(double) * H);
  double* logit = malloc(sizeof(double) * E);
  double* score = malloc(sizeof(double) * E);
  double* key = malloc(sizeof(double) * E);
  char* taken = malloc(E);
  double* gu = malloc(sizeof(double) * 2 * maxI);
  double* a = malloc(sizeof(double) * maxI);
  double* y = malloc(sizeof(double) * H);
  double* h = malloc(sizeof(double) * H);
  size_t w13_per = (size_t)2 * I * H, w2_per = (size_t)H * I;
  size_t s13_per = (size_t)(2 * I / BLK) * (H / BLK), s2_per = (size_t)(H / BLK) * (I / BLK);
  size_t selem = e8m0 ? 1 : 4;

  for (int p = 0; p < n; ++p) {
    int t = rows ? rows[p] : p;
    for (int c = 0; c < H; ++c) x[c] = bf16_value(hidden[(size_t)t * H + c]);

    /* Router: logits, sigmoid scores, ranking keys. */
    for (int e = 0; e < E; ++e) {
      double acc = 0.0;
      for (int c = 0; c < H; ++c) acc += x[c] * bf16_value(router_w[(size_t)e * H + c]);
      logit[e] = acc;
      score[e] = sigmoid(acc);
      key[e] = score[e] + (bias ? (double)bias[e] : 0.0);
      taken[e] = 0;
      if (logits_out) logits_out[(size_t)p * E + e] = acc;
    }
    /* Top-k by repeated selection of the largest key; the scan keeps the
     * first (lowest id) of equal keys. */
    double ssum = 0.0;
    for (int j = 0; j < k; ++j) {
      int best = -1;
      if (forced_ids) {
        best = forced_ids[(size_t)t * k + j];
      } else {
        for (int e = 0; e < E; ++e)
          if (!taken[e] && (best < 0 || key[e] > key[best])) best = e;
      }
      taken[best] = 1;
      ids_out[(size_t)p * k + j] = best;
      ssum += score[best];
    }
    /* Gap between the k-th and the (k+1)-th largest key. */
    {
      double kk, next;
      double* srt = malloc(sizeof(double) * E);
      memcpy(srt, key, sizeof(double) * E);
      for (int j = 0; j <= k && j < E; ++j) { /* partial selection sort */
        int b = j;
        for (int e = j + 1; e < E; ++e)
          if (srt[e] > srt[b]) b = e;
        double tmp = srt[j];
        srt[j] = srt[b];
        srt[b] = tmp;
      }
      kk = srt[k - 1];
      next = k < E ? srt[k] : -INFINITY;
      gaps_out[p] = k < E ? kk - next : INFINITY;
      free(srt);
    }

    for (int c = 0; c < H; ++c) h[c] = bf16_value(residual[(size_t)t * H + c]);
    for (int j = 0; j < k; ++j) {
      int e = ids_out[(size_t)p * k + j];
      double w = rsf * score[e] / ssum;
      w_out[(size_t)p * k + j] = w;
      expert(w13 + e * w13_per, (const char*)w13_scale + e * s13_per * selem,
             w2 + e * w2_per, (const char*)w2_scale + e * s2_per * selem, e8m0, lut, H, I,
             limit, x, gu, a, y);
      for (int c = 0; c < H; ++c) h[c] += w * y[c];
    }
    if (Is) {
      expert(sw13, sw13_scale, sw2, sw2_scale, e8m0, lut, H, Is, limit, x, gu, a, y);
      for (int c = 0; c < H; ++c) h[c] += y[c];
    }
    double ms = 0.0;
    for (int c = 0; c < H; ++c) ms += h[c] * h[c];
    ms /= H;
    double inv = 1.0 / sqrt(ms + eps);
    for (int c = 0; c < H; ++c) {
      h_out[(size_t)p * H + c] = h[c];
      out[(size_t)p * H + c] = h[c] * inv * bf16_value(gamma[c]);
    }
  }
  free(x); free(logit); free(score); free(key); free(taken);
  free(gu); free(a); free(y); free(h);
  return 0;
}
