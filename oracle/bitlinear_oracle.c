/*
 * bitlinear_oracle.c -- plain CPU oracle of the BitNet b1.58 BitLinear forward.
 *
 * TEST INFRASTRUCTURE. Only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark may load this library. It shares no code, header, table or helper
 * with the HIP kernels of ternary_quantized_linear_amd/, and the product path never
 * calls it.
 *
 * Built with:  gcc -O2 -std=c11 -fPIC -shared -ffp-contract=off -fno-fast-math -fopenmp
 * (no contraction of a*b+c into an FMA, no reassociation: every rounding below is
 * the one written).
 *
 * Sources (abbreviations used in the comments):
 *   [HF-1.58]   "Fine-tuning LLMs to 1.58 bits: extreme quantization with BitNet"
 *               (summary of the Hugging Face post, agentlenshq.com)
 *   [bitnet.cpp] "Microsoft's inference framework brings 1-bit large language models
 *               to local devices" (unite.ai)
 *   [b1.58]     "[Paper review] The Era of 1-bit LLMs: All Large Language Models are
 *               in 1.58 Bits" (nubint.ai)
 *   [BitDelta]  "BitDelta: Your Fine-Tune May Only Be Worth One Bit" (note.com summary)
 *
 * What each step computes, and the precision of each rounding:
 *   1. gamma = mean |W| over the whole matrix, one scale per tensor
 *      ([HF-1.58] "How quantization works", weights; [b1.58] "Proposed method",
 *      absmean bullet; the same mean over all n*m entries is [BitDelta] Eq. (4)).
 *      The sum is exact and rounded once to fp64; gamma64 = sum / (N*K) in fp64;
 *      beta = fp32(gamma64).
 *   2. codes: scale s = 1/beta (fp32), t = w*s (one fp32 product),
 *      q = clamp(round-half-even(t), -1, 1)  ([HF-1.58] "How quantization works":
 *      scale by the reciprocal of the absolute mean, round, clamp to [-1, 1]).
 *      beta below FLT_MIN (all-zero or denormal-only W) gives all codes 0.
 *   3. pack 4 codes per byte ([HF-1.58] "Key findings", model size): byte j of row o
 *      holds code k = 4j+i in bits [2i+1:2i] as u = q+1 in {0,1,2}; u = 3 is invalid.
 *   4. RMSNorm per token ([b1.58] "Proposed method", RMSNorm; [HF-1.58] "How
 *      quantization works", activations: a norm before the activation quantizer):
 *      ss = sum_k x_k^2 exact, rounded once to fp64; r = 1/sqrt(ss/K + eps) in fp64;
 *      y_k = fp32((x_k * r) * g_k) with both products in fp64 (g = 1 when absent).
 *   5. absmax int8 per token ([HF-1.58] "How quantization works", activations, range
 *      [-128, 127]; [bitnet.cpp] "2. Activation quantization": gamma = ||x||_inf and a
 *      small epsilon): m = max_k |y_k|; s_t = 127 / max(m, 1e-5) in fp32;
 *      q = clamp(round-half-even(y*s_t), -128, 127) with y*s_t one fp32 product.
 *   6. acc[t,o] = sum_k Xq[t,k] * q[o,k] in integers ([HF-1.58] "Computation paradigm":
 *      integer additions replace the multiply-adds).
 *   7. Y[t,o] = acc * beta / s_t, computed in fp64 and rounded once to fp32
 *      ([bitnet.cpp] "3. BitLinear operation": the product is multiplied by the
 *      weight scale and by the activation dequantization factor; no bias, [b1.58]
 *      "Proposed method").
 *
 * The 1-bit sign variant (the original BitNet that [bitnet.cpp] "1. Weight
 * binarization" describes), same activations and rescale:
 *   S1. alpha = mean(W): exact signed sum rounded once to fp64, alpha = sum / (N*K)
 *       in fp64 ([bitnet.cpp] "1. Weight binarization": the weights are centred on
 *       their mean).
 *   S2. c = Sign(w - alpha) with Sign(x) = +1 for x > 0 and -1 otherwise, so a weight
 *       equal to alpha gets -1 ([bitnet.cpp] the definition under "1. Weight
 *       binarization"; [BitDelta] Eq. (2) is the same rule). The sign of w - alpha is
 *       taken exactly: fp64(w) > alpha.
 *   S3. beta = fp32(mean |W|), the scale of step 1 ([BitDelta] Eq. (3)-(4): mean |W|
 *       is the scale that minimizes the L2 error of a sign code).
 *   S4. eight codes per byte: code k = 8j+i in bit i of byte j, 1 for +1, 0 for -1.
 *   S5. acc = sum_k Xq[t,k] * c[o,k] in integers; Y = fp32(acc * beta / s_t) in fp64.
 *
 * Group quantization ([bitnet.cpp] "Group quantization and normalization": weights and
 * activations split into G groups whose parameters are estimated separately, so that
 * no group needs another's): the weight matrix is cut into G blocks of N/G consecutive
 * output rows, and steps 1-2 run on each block alone (beta_g); activations are already
 * scaled per token (step 5), and RMSNorm is per token. The rescale of row o uses the
 * scale of its block: Y[t,o] = fp32(acc * beta_{o / (N/G)} / s_t) in fp64.
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_OK = 0, ORC_NONFINITE = -1, ORC_DIM = -2, ORC_NOMEM = -3, ORC_BADCODE = -4,
       ORC_OVERFLOW = -5 };

#define ORC_NO_NORM 0x1u

/* ------------------------------------------------------------------------------
 * Exact floating-point summation.
 *
 * Published method: J. R. Shewchuk, "Adaptive Precision Floating-Point Arithmetic and
 * Fast Robust Geometric Predicates" (1997). A running sum is kept as an expansion: a
 * list of doubles of increasing magnitude whose bits do not overlap and whose exact
 * real sum is the exact sum of everything added so far. Adding x walks the list with
 * the error-free two-sum (hi = fl(a+b), lo = exact a+b-hi), keeping the non-zero
 * low parts and carrying hi upward. Overflow cannot happen here: the inputs are fp32
 * values or their squares, whose sum stays far below DBL_MAX.
 * ------------------------------------------------------------------------------ */
typedef struct {
  double* v;
  int n, cap;
} expansion;

static int exp_init(expansion* e) {
  e->cap = 64;
  e->n = 0;
  e->v = (double*)malloc(sizeof(double) * (size_t)e->cap);
  return e->v ? ORC_OK : ORC_NOMEM;
}

static void exp_free(expansion* e) { free(e->v); e->v = NULL; e->n = e->cap = 0; }

static int exp_add(expansion* e, double x) {
  int kept = 0;
  for (int j = 0; j < e->n; ++j) {
    double a = x, b = e->v[j];
    if (fabs(a) < fabs(b)) { double t = a; a = b; b = t; }
    double hi = a + b;
    double lo = b - (hi - a);          /* exact because |a| >= |b| */
    if (lo != 0.0) e->v[kept++] = lo;  /* zero parts carry nothing */
    x = hi;
  }
  if (kept + 1 > e->cap) {
    int nc = e->cap * 2;
    double* nv = (double*)realloc(e->v, sizeof(double) * (size_t)nc);
    if (!nv) return ORC_NOMEM;
    e->v = nv;
    e->cap = nc;
  }
  e->v[kept] = x;
  e->n = kept + 1;
  return ORC_OK;
}

/* The exact value of the expansion, rounded once to the nearest double (ties to
 * even). Walking down from the largest part, sums stay exact until one addition
 * leaves a non-zero remainder `rem`; the rounded result is then `hi`, except when
 * `rem` is exactly half an ulp of hi and the parts still below push the true value
 * past that midpoint in rem's direction -- then the correctly rounded value is the
 * neighbour hi + 2*rem. */
static double exp_round(const expansion* e) {
  int j = e->n;
  if (j == 0) return 0.0;
  double hi = e->v[--j];
  double rem = 0.0;
  while (j > 0) {
    double part = e->v[--j];
    double s = hi + part;
    rem = part - (s - hi);
    hi = s;
    if (rem != 0.0) break;
  }
  if (rem != 0.0 && j > 0) {
    double below = e->v[j - 1];
    if ((rem > 0.0 && below > 0.0) || (rem < 0.0 && below < 0.0)) {
      double twice = rem * 2.0;
      double up = hi + twice;
      if (up - hi == twice) hi = up; /* rem was exactly half an ulp: a midpoint */
    }
  }
  return hi;
}

/* Exact sum of doubles d(i) for i in [0, n), produced by `get`, rounded once. The
 * range is cut into chunks summed exactly in parallel; the chunk expansions are then
 * merged exactly, so the result does not depend on the thread count or the order. */
typedef double (*term_fn)(const float* base, int64_t i);

static double term_abs(const float* b, int64_t i) { return fabs((double)b[i]); }
static double term_sq(const float* b, int64_t i) { double x = (double)b[i]; return x * x; }

static int exact_sum(const float* base, int64_t n, term_fn get, double* out) {
  const int64_t chunk = 1 << 20;
  int64_t nchunks = (n + chunk - 1) / chunk;
  if (nchunks <= 1) {
    expansion e;
    if (exp_init(&e)) return ORC_NOMEM;
    for (int64_t i = 0; i < n; ++i) {
      if (!isfinite(base[i])) { exp_free(&e); return ORC_NONFINITE; }
      if (exp_add(&e, get(base, i))) { exp_free(&e); return ORC_NOMEM; }
    }
    *out = exp_round(&e);
    exp_free(&e);
    return ORC_OK;
  }
  expansion* parts = (expansion*)calloc((size_t)nchunks, sizeof(expansion));
  if (!parts) return ORC_NOMEM;
  int status = ORC_OK;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t c = 0; c < nchunks; ++c) {
    int st = exp_init(&parts[c]);
    int64_t lo = c * chunk, hi = lo + chunk < n ? lo + chunk : n;
    for (int64_t i = lo; i < hi && st == ORC_OK; ++i) {
      if (!isfinite(base[i])) st = ORC_NONFINITE;
      else st = exp_add(&parts[c], get(base, i));
    }
    if (st != ORC_OK) {
#pragma omp critical
      status = st;
    }
  }
  expansion all;
  if (status == ORC_OK && exp_init(&all)) status = ORC_NOMEM;
  if (status == ORC_OK) {
    for (int64_t c = 0; c < nchunks && status == ORC_OK; ++c)
      for (int j = 0; j < parts[c].n && status == ORC_OK; ++j)
        status = exp_add(&all, parts[c].v[j]);
    if (status == ORC_OK) *out = exp_round(&all);
    exp_free(&all);
  }
  for (int64_t c = 0; c < nchunks; ++c) exp_free(&parts[c]);
  free(parts);
  return status;
}

/* ------------------------------------------------------------------------------ */

int orc_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
  return omp_get_max_threads();
#else
  (void)n;
  return 1;
#endif
}

/* Exact sum of |w| over n fp32 values, rounded once to fp64. */
int orc_abs_sum(const float* w, int64_t n, double* out) {
  if (n < 0) return ORC_DIM;
  return exact_sum(w, n, term_abs, out);
}

/* Exact sum of x^2 over n fp32 values (each square is exact in fp64), rounded once. */
int orc_sum_sq(const float* x, int64_t n, double* out) {
  if (n < 0) return ORC_DIM;
  return exact_sum(x, n, term_sq, out);
}

/* Step 1: gamma64 = (exact sum |W|) / (N*K) in fp64; beta = fp32(gamma64). */
int orc_weight_scale(const float* W, int64_t N, int64_t K, double* gamma, float* beta) {
  if (N <= 0 || K <= 0) return ORC_DIM;
  double s;
  int st = orc_abs_sum(W, N * K, &s);
  if (st) return st;
  double g = s / (double)(N * K);
  *gamma = g;
  *beta = (float)g;
  return ORC_OK;
}

/* Step 2: ternary codes of n weights under the per-tensor scale beta. */
int orc_ternarize(const float* W, int64_t n, float beta, int8_t* q) {
  if (n < 0) return ORC_DIM;
  if (!(beta >= FLT_MIN)) {           /* zero or denormal scale: every code is 0 */
    if (!isfinite(beta)) return ORC_NONFINITE;
    memset(q, 0, (size_t)n);
    return ORC_OK;
  }
  float s = 1.0f / beta;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    float t = W[i] * s;
    float r = rintf(t);                /* default rounding mode: half to even */
    if (r > 1.0f) r = 1.0f;
    if (r < -1.0f) r = -1.0f;
    q[i] = (int8_t)r;
  }
  return ORC_OK;
}

/* Step 3: pack codes [N, K] into bytes [N, K/4]. */
int orc_pack(const int8_t* q, int64_t N, int64_t K, uint8_t* P) {
  if (N <= 0 || K <= 0 || K % 4) return ORC_DIM;
  int64_t nb = K / 4;
  for (int64_t o = 0; o < N; ++o)
    for (int64_t j = 0; j < nb; ++j) {
      unsigned byte = 0;
      for (int i = 0; i < 4; ++i) {
        int c = q[o * K + 4 * j + i];
        if (c < -1 || c > 1) return ORC_BADCODE;
        byte |= (unsigned)(c + 1) << (2 * i);
      }
      P[o * nb + j] = (uint8_t)byte;
    }
  return ORC_OK;
}

/* Inverse of step 3; rejects the unused pattern 0b11. */
int orc_unpack(const uint8_t* P, int64_t N, int64_t K, int8_t* q) {
  if (N <= 0 || K <= 0 || K % 4) return ORC_DIM;
  int64_t nb = K / 4;
  for (int64_t o = 0; o < N; ++o)
    for (int64_t k = 0; k < K; ++k) {
      unsigned u = (P[o * nb + k / 4] >> (2 * (k % 4))) & 3u;
      if (u == 3u) return ORC_BADCODE;
      q[o * K + k] = (int8_t)((int)u - 1);
    }
  return ORC_OK;
}

/* Steps 1-3 together: W [N, K] fp32 -> packed bytes [N, K/4], beta, gamma64. */
int orc_quantize_weights(const float* W, int64_t N, int64_t K, uint8_t* P, float* beta,
                         double* gamma) {
  if (N <= 0 || K <= 0 || K % 4) return ORC_DIM;
  int st = orc_weight_scale(W, N, K, gamma, beta);
  if (st) return st;
  int8_t* q = (int8_t*)malloc((size_t)(N * K));
  if (!q) return ORC_NOMEM;
  st = orc_ternarize(W, N * K, *beta, q);
  if (!st) st = orc_pack(q, N, K, P);
  free(q);
  return st;
}

/* Step 4: RMSNorm of X [T, K] into Y [T, K] (fp32). gain may be NULL (unit gain). */
int orc_rmsnorm(const float* X, const float* gain, int64_t T, int64_t K, float eps,
                float* Y) {
  if (T <= 0 || K <= 0) return ORC_DIM;
  if (!isfinite(eps) || eps < 0.0f) return ORC_NONFINITE;
  int status = ORC_OK;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t t = 0; t < T; ++t) {
    const float* x = X + t * K;
    double ss;
    int st = orc_sum_sq(x, K, &ss);
    if (st) {
#pragma omp critical
      status = st;
      continue;
    }
    double r = 1.0 / sqrt(ss / (double)K + (double)eps);
    for (int64_t k = 0; k < K; ++k) {
      double v = (double)x[k] * r;
      if (gain) v = v * (double)gain[k];
      Y[t * K + k] = (float)v;
    }
  }
  return status;
}

/* Step 5: per-token absmax int8 quantization of Y [T, K]. */
int orc_absmax_quant(const float* Y, int64_t T, int64_t K, int8_t* Xq, float* s_out) {
  if (T <= 0 || K <= 0) return ORC_DIM;
  for (int64_t i = 0; i < T * K; ++i)
    if (!isfinite(Y[i])) return ORC_NONFINITE;
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    const float* y = Y + t * K;
    float m = 0.0f;
    for (int64_t k = 0; k < K; ++k) {
      float a = fabsf(y[k]);
      if (a > m) m = a;
    }
    float s = 127.0f / fmaxf(m, 1e-5f);
    s_out[t] = s;
    for (int64_t k = 0; k < K; ++k) {
      float v = y[k] * s;
      float r = rintf(v);
      if (r > 127.0f) r = 127.0f;
      if (r < -128.0f) r = -128.0f;
      Xq[t * K + k] = (int8_t)r;
    }
  }
  return ORC_OK;
}

/* Steps 4-5 together; ORC_NO_NORM in flags quantizes X itself (y = x). */
int orc_quantize_acts(const float* X, const float* gain, int64_t T, int64_t K, float eps,
                      uint32_t flags, int8_t* Xq, float* s_out) {
  if (T <= 0 || K <= 0) return ORC_DIM;
  if (flags & ORC_NO_NORM) return orc_absmax_quant(X, T, K, Xq, s_out);
  float* Y = (float*)malloc(sizeof(float) * (size_t)(T * K));
  if (!Y) return ORC_NOMEM;
  int st = orc_rmsnorm(X, gain, T, K, eps, Y);
  if (!st) st = orc_absmax_quant(Y, T, K, Xq, s_out);
  free(Y);
  return st;
}

/* Step 6: acc [T, N] = Xq [T, K] times the codes decoded from P [N, K/4]. */
int orc_product(const int8_t* Xq, const uint8_t* P, int64_t T, int64_t N, int64_t K,
                int32_t* acc) {
  if (T <= 0 || N <= 0 || K <= 0 || K % 4) return ORC_DIM;
  int64_t nb = K / 4;
  int status = ORC_OK;
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t o = 0; o < N; ++o) {
    const uint8_t* row = P + o * nb;
    for (int64_t t = 0; t < T; ++t) {
      const int8_t* x = Xq + t * K;
      int64_t sum = 0;
      for (int64_t k = 0; k < K; ++k) {
        int u = (row[k / 4] >> (2 * (k % 4))) & 3;
        if (u == 3) { sum = INT64_MIN; break; }
        sum += (int64_t)x[k] * (int64_t)(u - 1);
      }
      if (sum == INT64_MIN || sum > INT32_MAX || sum < INT32_MIN) {
#pragma omp critical
        status = (sum == INT64_MIN) ? ORC_BADCODE : ORC_OVERFLOW;
        continue;
      }
      acc[t * N + o] = (int32_t)sum;
    }
  }
  return status;
}

/* Step 7: Y [T, N] = acc * beta / s_t, in fp64, rounded once to fp32. */
int orc_rescale(const int32_t* acc, const float* s, float beta, int64_t T, int64_t N,
                float* Y) {
  if (T <= 0 || N <= 0) return ORC_DIM;
  for (int64_t t = 0; t < T; ++t) {
    double st = (double)s[t];
    for (int64_t o = 0; o < N; ++o)
      Y[t * N + o] = (float)((double)acc[t * N + o] * (double)beta / st);
  }
  return ORC_OK;
}

/* Steps 6-7 together: the forward from quantized activations and packed weights.
 * acc may be NULL. */
int orc_forward(const int8_t* Xq, const float* s, int64_t T, int64_t K, const uint8_t* P,
                float beta, int64_t N, float* Y, int32_t* acc) {
  if (T <= 0 || N <= 0 || K <= 0 || K % 4) return ORC_DIM;
  int32_t* a = acc ? acc : (int32_t*)malloc(sizeof(int32_t) * (size_t)(T * N));
  if (!a) return ORC_NOMEM;
  int st = orc_product(Xq, P, T, N, K, a);
  if (!st) st = orc_rescale(a, s, beta, T, N, Y);
  if (!acc) free(a);
  return st;
}

/* ---------------------------------------------------------------- sign variant */

static double term_id(const float* b, int64_t i) { return (double)b[i]; }

/* Exact sum of n fp32 values (signed), rounded once to fp64. */
int orc_sum(const float* w, int64_t n, double* out) {
  if (n < 0) return ORC_DIM;
  return exact_sum(w, n, term_id, out);
}

/* S2: c = +1 where fp64(w) > alpha, else -1. */
int orc_sign_codes(const float* W, int64_t n, double alpha, int8_t* c) {
  if (n < 0) return ORC_DIM;
  for (int64_t i = 0; i < n; ++i) {
    if (!isfinite(W[i])) return ORC_NONFINITE;
    c[i] = ((double)W[i] > alpha) ? (int8_t)1 : (int8_t)-1;
  }
  return ORC_OK;
}

/* S1-S3 for W [N, K]: codes c [N, K], alpha (fp64), gamma = mean|W| (fp64), beta. */
int orc_sign_weights(const float* W, int64_t N, int64_t K, int8_t* c, double* alpha,
                     double* gamma, float* beta) {
  if (N <= 0 || K <= 0) return ORC_DIM;
  double sum;
  int st = orc_sum(W, N * K, &sum);
  if (st) return st;
  const double a = sum / (double)(N * K);
  st = orc_weight_scale(W, N, K, gamma, beta);
  if (st) return st;
  *alpha = a;
  return orc_sign_codes(W, N * K, a, c);
}

/* S4: pack codes c [N, K] (K % 8 == 0) into P [N, K/8]. */
int orc_pack1(const int8_t* c, int64_t N, int64_t K, uint8_t* P) {
  if (N <= 0 || K <= 0 || K % 8) return ORC_DIM;
  const int64_t nb = K / 8;
  for (int64_t o = 0; o < N; ++o)
    for (int64_t j = 0; j < nb; ++j) {
      unsigned byte = 0u;
      for (int i = 0; i < 8; ++i) {
        const int8_t v = c[o * K + 8 * j + i];
        if (v != 1 && v != -1) return ORC_BADCODE;
        if (v == 1) byte |= 1u << i;
      }
      P[o * nb + j] = (uint8_t)byte;
    }
  return ORC_OK;
}

int orc_unpack1(const uint8_t* P, int64_t N, int64_t K, int8_t* c) {
  if (N <= 0 || K <= 0 || K % 8) return ORC_DIM;
  const int64_t nb = K / 8;
  for (int64_t o = 0; o < N; ++o)
    for (int64_t k = 0; k < K; ++k)
      c[o * K + k] = ((P[o * nb + k / 8] >> (k % 8)) & 1u) ? (int8_t)1 : (int8_t)-1;
  return ORC_OK;
}

/* S5, integer part: acc [T, N] = Xq [T, K] times the sign codes of P [N, K/8]. */
int orc_product_sign(const int8_t* Xq, const uint8_t* P, int64_t T, int64_t N, int64_t K,
                     int32_t* acc) {
  if (T <= 0 || N <= 0 || K <= 0 || K % 8) return ORC_DIM;
  const int64_t nb = K / 8;
  int status = ORC_OK;
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t o = 0; o < N; ++o) {
    const uint8_t* row = P + o * nb;
    for (int64_t t = 0; t < T; ++t) {
      const int8_t* x = Xq + t * K;
      int64_t sum = 0;
      for (int64_t k = 0; k < K; ++k) {
        const int c = ((row[k / 8] >> (k % 8)) & 1u) ? 1 : -1;
        sum += (int64_t)x[k] * (int64_t)c;
      }
      if (sum > INT32_MAX || sum < INT32_MIN) {
#pragma omp critical
        status = ORC_OVERFLOW;
        continue;
      }
      acc[t * N + o] = (int32_t)sum;
    }
  }
  return status;
}

/* S5: Y = fp32(acc * beta / s_t) (the rescale of step 7). acc may be NULL. */
int orc_forward_sign(const int8_t* Xq, const float* s, int64_t T, int64_t K, const uint8_t* P,
                     float beta, int64_t N, float* Y, int32_t* acc) {
  if (T <= 0 || N <= 0 || K <= 0 || K % 8) return ORC_DIM;
  int32_t* a = acc ? acc : (int32_t*)malloc(sizeof(int32_t) * (size_t)(T * N));
  if (!a) return ORC_NOMEM;
  int st = orc_product_sign(Xq, P, T, N, K, a);
  if (!st) st = orc_rescale(a, s, beta, T, N, Y);
  if (!acc) free(a);
  return st;
}

/* ---------------------------------------------------------------- group quantization */

/* Steps 1-3 on each of G blocks of N/G rows: P [N, K/4], beta [G], gamma [G]. */
int orc_quantize_weights_groups(const float* W, int64_t N, int64_t K, int64_t G, uint8_t* P,
                                float* beta, double* gamma) {
  if (N <= 0 || K <= 0 || K % 4 || G <= 0 || N % G) return ORC_DIM;
  const int64_t rows = N / G;
  for (int64_t g = 0; g < G; ++g) {
    int st = orc_quantize_weights(W + g * rows * K, rows, K, P + g * rows * (K / 4), &beta[g],
                                  &gamma[g]);
    if (st) return st;
  }
  return ORC_OK;
}

/* Y [T, N] = acc * beta_{o / (N/G)} / s_t in fp64, rounded once to fp32. */
int orc_rescale_groups(const int32_t* acc, const float* s, const float* beta, int64_t T,
                       int64_t N, int64_t G, float* Y) {
  if (T <= 0 || N <= 0 || G <= 0 || N % G) return ORC_DIM;
  const int64_t rows = N / G;
  for (int64_t t = 0; t < T; ++t) {
    const double st = (double)s[t];
    for (int64_t o = 0; o < N; ++o)
      Y[t * N + o] = (float)((double)acc[t * N + o] * (double)beta[o / rows] / st);
  }
  return ORC_OK;
}
