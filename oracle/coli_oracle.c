/*
 * coli_oracle.c -- plain CPU oracle of the routed-expert MoE layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark load this file's library.  The product path
 * never calls it, and it shares no code, header, table or constant with the
 * HIP library: the container layout and the quantiser below are written out
 * again here from their definitions.
 *
 * Everything is straight loops in the order the definitions read, with fp64
 * accumulation (built with -ffp-contract=off).  OpenMP splits only
 * independent output rows / tokens; every sum runs sequentially.  Tokens
 * are split across threads when there are at least as many tokens as
 * threads; otherwise each token's output rows are (OR_ROWS_PARALLEL), so a
 * single token also uses every core.
 *
 * Definitions followed (web pages about the colibri engine):
 *  - int4, one fp16 scale per 64 weights ("gs64"): tantan.ink post
 *    "colibri: 把 744B 模型当数据流...", section "我看到的几个坑".
 *  - int8-weight experts (the MTP layer's experts must be int8, same post
 *    and section; the OLMoE container is int8, ai-tools-nav review, model
 *    family table): read as the same container with one two's-complement
 *    byte per weight in place of a nibble, the same fp16 scale per 64.
 *  - fp4 experts (the Kimi K3 and DeepSeek V4 rows of the ai-tools-nav
 *    model family table): read as OCP MXFP4 -- FP4 E2M1 codes packed two
 *    per byte like the int4 nibbles, one E8M0 scale byte per 32 weights.
 *  - three matrices gate/up/down per expert, each distinct expert read once
 *    per batch: same post, section "几个关键工程动作".
 *  - Q8_0-style int8 activations on the integer path: alphamatch.ai blog
 *    "Colibri：革命性 AI 引擎...", section "優化整數核心".
 *  - fp4 experts with fp8 activations (the MX path): the DeepSeek V4 row of
 *    the ai-tools-nav model family table pairs fp4 experts with fp8-e4m3;
 *    read as OCP MXFP8 (E4M3 elements, one E8M0 scale per 32 values) for
 *    the activations of an MXFP4 layer's expert GEMMs.
 *  - router choice decides the experts: aixq.cc article, section
 *    "为什么值得关注".
 * Readings where the pages are silent (routing function, tie order, nibble
 * order, SwiGLU, the Q8_0 rounding rule) are the ones stated in the library
 * header and repeated at each function below.
 *
 * Pins: every function here is checked by tests against an independent
 * numpy brute force, closed forms, invariants and hand-derived fixtures.
 * Parity unpinned: for softmax-routed layers, whether the k selected
 * probabilities are renormalised.  No page decides it; both readings are
 * implemented (the RENORM flag) and each is pinned to its own definition.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_OK 0
#define OR_EINVAL -1

/* Split a loop over independent output rows across threads, unless the
 * caller's token loop already runs in parallel. */
#define OR_ROWS_PARALLEL _Pragma("omp parallel for schedule(static) if(!omp_in_parallel())")

/* Whether a token loop of T iterations should itself run in parallel. */
static int or_tokens_parallel(int64_t T) { return T >= omp_get_max_threads(); }

/* ---------------------------------------------------------------- numbers */

/* IEEE binary16 bits -> value (exact). */
static double or_f16(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 31;
  int m = h & 1023;
  double v;
  if (e == 0)
    v = ldexp((double)m, -24);
  else if (e == 31)
    v = m ? NAN : INFINITY;
  else
    v = ldexp((double)(m + 1024), e - 25);
  return sign ? -v : v;
}

/* bfloat16 bits -> value (exact: the upper half of an IEEE binary32). */
static double or_bf16(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* binary32 -> binary16 bits, round to nearest, ties to even. */
uint16_t oracle_f32_to_f16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
  double a = fabs((double)f);
  if (f != f) return (uint16_t)(sign | 0x7e00u);
  if (a >= 65520.0) return (uint16_t)(sign | 0x7c00u); /* 65520 ties to inf */
  if (a < ldexp(1.0, -14)) {
    /* subnormal range: value = m * 2^-24, m = 0..1024 (1024 = min normal) */
    double m = nearbyint(a * ldexp(1.0, 24)); /* default mode: ties-to-even */
    return (uint16_t)(sign | (uint16_t)m);
  }
  int e2;
  frexp(a, &e2);               /* a = f * 2^e2, f in [0.5, 1) */
  int E = e2 - 1;              /* a in [2^E, 2^(E+1)) */
  double m = nearbyint(ldexp(a, 10 - E)); /* 11-bit significand in [1024, 2048] */
  if (m == 2048.0) {
    m = 1024.0;
    E += 1;
  }
  if (E > 15) return (uint16_t)(sign | 0x7c00u);
  return (uint16_t)(sign | (uint16_t)((E + 15) << 10) | (uint16_t)((int)m - 1024));
}

/* nibble -> signed int4: two's complement in 4 bits. */
static int or_nib(uint8_t byte, int high) {
  int v = high ? (byte >> 4) : (byte & 15);
  return v >= 8 ? v - 16 : v;
}

/* weight formats of the container */
#define OR_INT4 0  /* nibble codes, fp16 scale per 64 */
#define OR_INT8 1  /* byte codes, fp16 scale per 64 */
#define OR_FP4 2   /* MXFP4: E2M1 nibbles, E8M0 scale byte per 32 */

/* FP4 E2M1 value of a nibble (OCP microscaling formats): bit 3 sign, bits
 * 2-1 exponent e with bias 1, bit 0 mantissa m; e = 0 is subnormal:
 * m / 2; otherwise 2^(e-1) * (1 + m/2).  Values 0, .5, 1, 1.5, 2, 3, 4, 6. */
static double or_e2m1(int nib) {
  const int e = (nib >> 1) & 3, m = nib & 1;
  const double v = e ? ldexp(1.0 + 0.5 * m, e - 1) : 0.5 * m;
  return (nib & 8) ? -v : v;
}

/* integer code of weight [n][k] of a row-major code matrix.
 *  int4: rows hold K/2 bytes, byte k/2, low nibble for even k, high nibble
 *        for odd k, two's complement.
 *  int8: rows hold K bytes, byte k, two's complement.
 *  fp4:  nibbles placed as for int4; the code is twice the E2M1 value, an
 *        integer in [-12, 12] (its scale below carries the 1/2). */
static int or_q(const uint8_t *mat, int64_t K, int64_t n, int64_t k, int fmt) {
  if (fmt == OR_INT8) return (int)(int8_t)mat[n * K + k];
  const uint8_t byte = mat[n * (K / 2) + k / 2];
  if (fmt == OR_FP4) return (int)(2.0 * or_e2m1((k & 1) ? byte >> 4 : byte & 15));
  return or_nib(byte, (int)(k & 1));
}

/* scale of weight [n][k] of a matrix: fp16 s[n][k/64] (int4, int8), or for
 * fp4 the E8M0 byte E[n][k/32] as 2^(E-127), halved. */
static double or_s(const uint8_t *sc, int64_t K, int64_t n, int64_t k, int fmt) {
  if (fmt == OR_FP4) return ldexp(1.0, (int)sc[n * (K / 32) + k / 32] - 128);
  return or_f16(((const uint16_t *)sc)[n * (K / 64) + k / 64]);
}

/* --------------------------------------------------------------- container */

typedef struct {
  int64_t H, I, E, S;
  const uint8_t *q4;     /* host copy of the container's codes */
  const uint8_t *scales; /* host copy of its scales (fp16 bits or E8M0) */
  int fmt;               /* OR_INT4, OR_INT8 or OR_FP4 */
} or_layer;

/* matrix m (0 gate, 1 up, 2 down) of expert e: code base and scale base.
 * A matrix holds I*H codes: I*H/2 bytes (int4, fp4) or I*H bytes (int8),
 * and I*H/64 fp16 scales (int4, int8) or I*H/32 E8M0 bytes (fp4).  Expert e
 * occupies three matrices of codes and three of scales, in order. */
static int64_t or_mat_bytes(const or_layer *L) {
  return L->fmt == OR_INT8 ? L->I * L->H : L->I * L->H / 2;
}
static int64_t or_sc_bytes(const or_layer *L) {  /* the same for every format */
  return L->fmt == OR_FP4 ? L->I * L->H / 32 : 2 * (L->I * L->H / 64);
}
static const uint8_t *or_mat(const or_layer *L, int64_t e, int m) {
  return L->q4 + e * 3 * or_mat_bytes(L) + (int64_t)m * or_mat_bytes(L);
}
static const uint8_t *or_sc(const or_layer *L, int64_t e, int m) {
  return L->scales + e * 3 * or_sc_bytes(L) + (int64_t)m * or_sc_bytes(L);
}

/* --------------------------------------------------------- router logits */

/* Router logits of T tokens: logit[t][e] = sum over k < H of x[t][k] *
 * w[e][k], with bf16 inputs (exact in fp64), the sum in fp64 in k order,
 * rounded once to fp32.  The router decides which experts a token loads and
 * runs ahead of the expert loads (aixq.cc article, sections "为什么值得关注"
 * and "我的真实看法"); the pages give no formula, so it is read as a dense
 * linear layer without bias over the layer input, with bf16 weights stored
 * row-major [E][H]. */
int oracle_router_logits(int64_t T, int64_t E, int64_t H, const uint16_t *w,
                         const uint16_t *x, float *logits) {
  if (T < 1 || E < 1 || H < 1 || !w || !x || !logits) return OR_EINVAL;
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t)
    for (int64_t e = 0; e < E; ++e) {
      double acc = 0.0;
      for (int64_t k = 0; k < H; ++k) acc += or_bf16(x[t * H + k]) * or_bf16(w[e * H + k]);
      logits[t * E + e] = (float)acc;
    }
  return OR_OK;
}

/* ------------------------------------------------------------------ route */

/* Top-k selection, weights and grouping for T tokens.
 * Selection: score = fp32(logit + sel_bias) (sel_bias may be NULL); the k
 * largest scores, taken largest first, a tie going to the lower expert index.
 * Weights (from the raw logits, computed in fp64, stored fp32):
 *   flags&1 == 0: softmax over all E logits, w_j = p[idx_j];
 *   flags&1 == 1: w_j = 1/(1+exp(-logit[idx_j]));
 *   flags&256   : w_j /= sum of the k weights;
 *   then w_j *= routed_scale.
 * Grouping (the batch union): counts per expert, exclusive offsets, and the
 * pair ids p = t*k + j listed expert by expert in ascending p.
 * Source: aixq.cc article, section "为什么值得关注"; tantan.ink post,
 * section "几个关键工程动作". */
int oracle_route(int32_t T, int32_t E, int32_t k, uint32_t flags,
                 float routed_scale, const float *logits, const float *sel_bias,
                 int32_t *topk_idx, float *topk_w, int32_t *counts,
                 int32_t *offsets, int32_t *pairs) {
  if (T < 0 || E < 1 || k < 1 || k > E) return OR_EINVAL;
  char *taken = (char *)malloc((size_t)E);
  double *w = (double *)malloc(sizeof(double) * (size_t)k);
  if (!taken || !w) {
    free(taken);
    free(w);
    return OR_EINVAL;
  }
  for (int32_t t = 0; t < T; ++t) {
    const float *l = logits + (int64_t)t * E;
    memset(taken, 0, (size_t)E);
    for (int32_t j = 0; j < k; ++j) {
      int32_t best = -1;
      float best_s = 0.0f;
      for (int32_t e = 0; e < E; ++e) {
        if (taken[e]) continue;
        float s = sel_bias ? (float)(l[e] + sel_bias[e]) : l[e];
        if (best < 0 || s > best_s) { /* strict: earlier (lower) index wins ties */
          best = e;
          best_s = s;
        }
      }
      taken[best] = 1;
      topk_idx[(int64_t)t * k + j] = best;
    }
    if ((flags & 1u) == 0) {
      double mx = l[0];
      for (int32_t e = 1; e < E; ++e)
        if (l[e] > mx) mx = l[e];
      double z = 0.0;
      for (int32_t e = 0; e < E; ++e) z += exp((double)l[e] - mx);
      for (int32_t j = 0; j < k; ++j)
        w[j] = exp((double)l[topk_idx[(int64_t)t * k + j]] - mx) / z;
    } else {
      for (int32_t j = 0; j < k; ++j)
        w[j] = 1.0 / (1.0 + exp(-(double)l[topk_idx[(int64_t)t * k + j]]));
    }
    if (flags & 256u) {
      double sum = 0.0;
      for (int32_t j = 0; j < k; ++j) sum += w[j];
      for (int32_t j = 0; j < k; ++j) w[j] /= sum;
    }
    for (int32_t j = 0; j < k; ++j)
      topk_w[(int64_t)t * k + j] = (float)(w[j] * (double)routed_scale);
  }
  free(taken);
  free(w);

  int64_t P = (int64_t)T * k;
  for (int32_t e = 0; e < E; ++e) counts[e] = 0;
  for (int64_t p = 0; p < P; ++p) counts[topk_idx[p]] += 1;
  offsets[0] = 0;
  for (int32_t e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  int32_t *fill = (int32_t *)malloc(sizeof(int32_t) * (size_t)E);
  if (!fill) return OR_EINVAL;
  for (int32_t e = 0; e < E; ++e) fill[e] = offsets[e];
  for (int64_t p = 0; p < P; ++p) pairs[fill[topk_idx[p]]++] = (int32_t)p;
  free(fill);
  return OR_OK;
}

/* ------------------------------------------------------------------- FFN */

static double or_silu(double g) { return g / (1.0 + exp(-g)); }

/* Decode-mode expert FFN on one fp64 activation vector x[H]:
 *   g[n] = sum_k q_g[n][k] s_g[n][k/64] x[k]   (likewise u)
 *   h[n] = silu(g[n]) * u[n]
 *   o[m] = sum_n q_d[m][n] s_d[m][n/64] h[n]
 * SwiGLU is the reading of "gate / up / down" (tantan.ink post, section
 * "几个关键工程动作"); the pages do not name the activation. */
static void or_ffn_f64(const or_layer *L, int64_t e, const double *x, double *h,
                       double *o) {
  const int64_t H = L->H, I = L->I;
  const uint8_t *qg = or_mat(L, e, 0), *qu = or_mat(L, e, 1), *qd = or_mat(L, e, 2);
  const uint8_t *sg = or_sc(L, e, 0), *su = or_sc(L, e, 1), *sd = or_sc(L, e, 2);
  const int f = L->fmt;
  OR_ROWS_PARALLEL
  for (int64_t n = 0; n < I; ++n) {
    double g = 0.0, u = 0.0;
    for (int64_t k = 0; k < H; ++k) {
      g += (double)or_q(qg, H, n, k, f) * or_s(sg, H, n, k, f) * x[k];
      u += (double)or_q(qu, H, n, k, f) * or_s(su, H, n, k, f) * x[k];
    }
    h[n] = or_silu(g) * u;
  }
  OR_ROWS_PARALLEL
  for (int64_t m = 0; m < H; ++m) {
    double acc = 0.0;
    for (int64_t n = 0; n < I; ++n)
      acc += (double)or_q(qd, I, m, n, f) * or_s(sd, I, m, n, f) * h[n];
    o[m] = acc;
  }
}

/* Decode-mode layer output for T tokens (x bf16, y fp64 [T][H]):
 *   y[t] = sum_j topk_w[t][j] * FFN_{topk_idx[t][j]}(x[t]) + [S] FFN_E(x[t])
 * Each token is computed on its own, so the batch union (which only changes
 * how often weights are read) does not appear here. */
int oracle_forward_decode(int64_t H, int64_t I, int64_t E, int64_t S, int64_t k,
                          const uint8_t *q4, const void *scales,
                          const int32_t *topk_idx, const float *topk_w,
                          const uint16_t *x_bf16, int64_t T, double *y, int32_t fmt) {
  if (H <= 0 || I <= 0 || H % 64 || I % 64 || E < 1 || S < 0 || S > 1 || k < 1 ||
      fmt < OR_INT4 || fmt > OR_FP4)
    return OR_EINVAL;
  or_layer L = {H, I, E, S, q4, (const uint8_t *)scales, fmt};
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad) if(or_tokens_parallel(T))
  for (int64_t t = 0; t < T; ++t) {
    double *x = (double *)malloc(sizeof(double) * (size_t)H);
    double *h = (double *)malloc(sizeof(double) * (size_t)I);
    double *o = (double *)malloc(sizeof(double) * (size_t)H);
    if (!x || !h || !o) {
      bad = 1;
    } else {
      for (int64_t i = 0; i < H; ++i) x[i] = or_bf16(x_bf16[t * H + i]);
      double *yt = y + t * H;
      for (int64_t i = 0; i < H; ++i) yt[i] = 0.0;
      for (int64_t j = 0; j < k; ++j) {
        int64_t e = topk_idx[t * k + j];
        double w = (double)topk_w[t * k + j];
        or_ffn_f64(&L, e, x, h, o);
        for (int64_t i = 0; i < H; ++i) yt[i] += w * o[i];
      }
      if (S) {
        or_ffn_f64(&L, E, x, h, o);
        for (int64_t i = 0; i < H; ++i) yt[i] += o[i];
      }
    }
    free(x);
    free(h);
    free(o);
  }
  return bad ? OR_EINVAL : OR_OK;
}

/* ------------------------------------------------------------------ Q8_0 */

/* Q8_0 of n fp32 values (n % 32 == 0), per block of 32:
 *   a = max |v|;  d = a / 127 in fp32;  q = round half away from zero of
 *   fp32(v / d), clamped to [-127, 127], or 0 when a == 0;  stored scale =
 *   d rounded to fp16 (nearest-even).
 * The pages give only "Q8_0-style int8 activations" (alphamatch.ai blog,
 * section "優化整數核心"); this rounding rule is the reading taken. */
int oracle_quantize_q8_0(const float *v, int64_t n, int8_t *q, uint16_t *d16) {
  if (n < 0 || n % 32) return OR_EINVAL;
  for (int64_t b = 0; b < n / 32; ++b) {
    const float *vb = v + 32 * b;
    float a = 0.0f;
    for (int i = 0; i < 32; ++i)
      if (fabsf(vb[i]) > a) a = fabsf(vb[i]);
    volatile float d = a / 127.0f;
    d16[b] = oracle_f32_to_f16(d);
    for (int i = 0; i < 32; ++i) {
      int r = 0;
      if (a != 0.0f) {
        volatile float ratio = vb[i] / d;
        r = (int)roundf(ratio); /* C roundf: halfway cases away from zero */
        if (r > 127) r = 127;
        if (r < -127) r = -127;
      }
      q[32 * b + i] = (int8_t)r;
    }
  }
  return OR_OK;
}

/* int4 gs64 container from float weights: rows x K values (K % 64 == 0),
 * row-major.  Per group of 64 consecutive weights of a row: a = max |w|;
 * s = a / 7 (IEEE fp32 division), stored as fp16 (nearest, ties to even);
 * each weight becomes q = round-half-away-from-zero(w / s16) with the
 * stored scale s16 (fp32 division), clamped to [-8, 7]; a group whose
 * stored scale is 0 gives q = 0.  Nibbles are packed two's complement, the
 * even k in the low nibble.  The pages fix the container -- int4, one fp16
 * scale per 64 weights, symmetric (tantan.ink post, section "我看到的几个坑")
 * -- but not the quantiser; this rule (the largest magnitude maps to 7,
 * quantised against the scale the decoder will use) is the reading taken.
 * Inputs must be finite with max |w| <= 7 * 65504. */
int oracle_quantize_int4_gs64(const float *w, int64_t rows, int64_t K, uint8_t *q4,
                              uint16_t *scales) {
  if (rows < 0 || K <= 0 || K % 64) return OR_EINVAL;
  for (int64_t n = 0; n < rows; ++n)
    for (int64_t g = 0; g < K / 64; ++g) {
      const float *wg = w + n * K + 64 * g;
      float a = 0.0f;
      for (int i = 0; i < 64; ++i)
        if (fabsf(wg[i]) > a) a = fabsf(wg[i]);
      volatile float s = a / 7.0f;
      const uint16_t s16 = oracle_f32_to_f16(s);
      scales[n * (K / 64) + g] = s16;
      const float sf = (float)or_f16(s16);
      for (int i = 0; i < 64; ++i) {
        int r = 0;
        if (sf != 0.0f) {
          volatile float u = wg[i] / sf;
          r = (int)roundf(u); /* halfway cases away from zero */
          if (r > 7) r = 7;
          if (r < -8) r = -8;
        }
        const int64_t k = 64 * g + i;
        uint8_t *byte = q4 + n * (K / 2) + k / 2;
        const uint8_t nib = (uint8_t)(r & 15);
        *byte = (k & 1) ? (uint8_t)((*byte & 0x0f) | (nib << 4)) : (uint8_t)((*byte & 0xf0) | nib);
      }
    }
  return OR_OK;
}

/* int8 gs64 container from float weights: the int4 rule above with 127 in
 * place of 7 and byte codes: per group of 64, s = max|w| / 127 (fp32
 * division), s16 = fp16_RNE(s), q = round-half-away(w / s16) clamped to
 * [-128, 127] (0 when s16 == 0); q[n][k] at byte n*K + k.  The pages give
 * int8 experts (tantan.ink post, section "我看到的几个坑") but no quantiser;
 * this rule, the int4 one widened, is the reading taken. */
int oracle_quantize_int8_gs64(const float *w, int64_t rows, int64_t K, int8_t *q,
                              uint16_t *scales) {
  if (rows < 0 || K <= 0 || K % 64) return OR_EINVAL;
  for (int64_t n = 0; n < rows; ++n)
    for (int64_t g = 0; g < K / 64; ++g) {
      const float *wg = w + n * K + 64 * g;
      float a = 0.0f;
      for (int i = 0; i < 64; ++i)
        if (fabsf(wg[i]) > a) a = fabsf(wg[i]);
      volatile float t = a / 127.0f;
      const uint16_t t16 = oracle_f32_to_f16(t);
      scales[n * (K / 64) + g] = t16;
      const float tf = (float)or_f16(t16);
      for (int i = 0; i < 64; ++i) {
        int r = 0;
        if (tf != 0.0f) {
          volatile float v = wg[i] / tf;
          r = (int)roundf(v); /* halfway cases away from zero */
          if (r > 127) r = 127;
          if (r < -128) r = -128;
        }
        q[n * K + 64 * g + i] = (int8_t)r;
      }
    }
  return OR_OK;
}

/* MXFP4 from float weights, following the OCP microscaling formats
 * conversion: per block of 32 consecutive weights of a row, the shared
 * exponent is X = floor(log2(max|w|)) - 2 (2 = the largest E2M1 exponent),
 * stored as E8M0 byte E = X + 127 clamped to [0, 254] (E = 0 for an all-zero
 * block); each weight becomes the E2M1 code nearest to w / 2^(E-127), ties
 * to the even code, saturating at +-6 (sign kept, also for zero).  Codes are
 * packed like the int4 nibbles (even k low).  The pages list fp4 experts
 * (ai-tools-nav review, model family table) without the converter; this is
 * the published MX conversion. */
int oracle_quantize_mxfp4(const float *w, int64_t rows, int64_t K, uint8_t *q4, uint8_t *e8) {
  static const double grid[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
  if (rows < 0 || K <= 0 || K % 32) return OR_EINVAL;
  for (int64_t n = 0; n < rows; ++n)
    for (int64_t b = 0; b < K / 32; ++b) {
      const float *wb = w + n * K + 32 * b;
      double a = 0.0;
      for (int i = 0; i < 32; ++i)
        if (fabs((double)wb[i]) > a) a = fabs((double)wb[i]);
      int E = 0;
      if (a > 0.0) {
        int ex;
        frexp(a, &ex); /* a = f * 2^ex, f in [0.5, 1): floor(log2 a) = ex - 1 */
        E = (ex - 1) - 2 + 127;
        if (E < 0) E = 0;
        if (E > 254) E = 254;
      }
      e8[n * (K / 32) + b] = (uint8_t)E;
      for (int i = 0; i < 32; ++i) {
        const double v = ldexp((double)wb[i], 127 - E);
        const double m = fabs(v);
        int c = 7; /* saturate above 6 */
        for (int j = 0; j < 7; ++j) {
          const double mid = 0.5 * (grid[j] + grid[j + 1]);
          if (m < mid || (m == mid && (j & 1) == 0)) { /* tie: the even code j */
            c = j;
            break;
          }
        }
        const uint8_t nib = (uint8_t)(c | ((wb[i] < 0.0f || (wb[i] == 0.0f && signbit(wb[i]))) ? 8 : 0));
        const int64_t k = 32 * b + i;
        uint8_t *dst = q4 + n * (K / 2) + k / 2;
        *dst = (k & 1) ? (uint8_t)((*dst & 0x0f) | (nib << 4)) : (uint8_t)((*dst & 0xf0) | nib);
      }
    }
  return OR_OK;
}

/* Exact int32 dot of one 32-block: weights of row n of a code matrix
 * against int8 activations a[K], over k in [32b, 32b+32). */
static int32_t or_block_dot(const uint8_t *mat, int64_t K, int64_t n, int fmt,
                            const int8_t *a, int64_t b) {
  int32_t acc = 0;
  for (int64_t k = 32 * b; k < 32 * b + 32; ++k)
    acc += or_q(mat, K, n, k, fmt) * (int32_t)a[k];
  return acc;
}

/* dots[t][n][b] for matrix m (0 gate, 1 up, 2 down) of expert e. */
int oracle_block_dots(int64_t H, int64_t I, int64_t E, int64_t S,
                      const uint8_t *q4, const void *scales, int64_t e,
                      int m, const int8_t *q_act, int64_t T, int32_t *dots, int32_t fmt) {
  if (H <= 0 || I <= 0 || H % 64 || I % 64 || m < 0 || m > 2 || e < 0 || e >= E + S ||
      fmt < OR_INT4 || fmt > OR_FP4)
    return OR_EINVAL;
  or_layer L = {H, I, E, S, q4, (const uint8_t *)scales, fmt};
  const int64_t K = (m == 2) ? I : H, rows = (m == 2) ? H : I, nb = K / 32;
  const uint8_t *mat = or_mat(&L, e, m);
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t)
    for (int64_t n = 0; n < rows; ++n)
      for (int64_t b = 0; b < nb; ++b)
        dots[(t * rows + n) * nb + b] = or_block_dot(mat, K, n, L.fmt, q_act + t * K, b);
  return OR_OK;
}

/* Integer-path expert FFN for one Q8_0 activation row (qx[H], dx[H/32]):
 *   g[n] = sum_b s_g[n][b/2] * d_x[b] * dot_b(q_g[n], q_x)   (likewise u)
 *   h = fp32(silu(g) * u);  (q_h, d_h) = Q8_0(h)
 *   o[m] = sum_b s_d[m][b/2] * d_h[b] * dot_b(q_d[m], q_h)
 * Source: alphamatch.ai blog, section "優化整數核心". */
static int or_ffn_q8(const or_layer *L, int64_t e, const int8_t *qx,
                     const uint16_t *dx, float *hf, int8_t *qh, uint16_t *dh,
                     double *o) {
  const int64_t H = L->H, I = L->I;
  const uint8_t *qg = or_mat(L, e, 0), *qu = or_mat(L, e, 1), *qd = or_mat(L, e, 2);
  const uint8_t *sg = or_sc(L, e, 0), *su = or_sc(L, e, 1), *sd = or_sc(L, e, 2);
  const int f = L->fmt;
  OR_ROWS_PARALLEL
  for (int64_t n = 0; n < I; ++n) {
    double g = 0.0, u = 0.0;
    for (int64_t b = 0; b < H / 32; ++b) {
      double d = or_f16(dx[b]);
      g += or_s(sg, H, n, 32 * b, f) * d * (double)or_block_dot(qg, H, n, f, qx, b);
      u += or_s(su, H, n, 32 * b, f) * d * (double)or_block_dot(qu, H, n, f, qx, b);
    }
    hf[n] = (float)(or_silu(g) * u);
  }
  if (oracle_quantize_q8_0(hf, I, qh, dh) != OR_OK) return OR_EINVAL;
  OR_ROWS_PARALLEL
  for (int64_t m = 0; m < H; ++m) {
    double acc = 0.0;
    for (int64_t b = 0; b < I / 32; ++b)
      acc += or_s(sd, I, m, 32 * b, f) * or_f16(dh[b]) *
             (double)or_block_dot(qd, I, m, f, qh, b);
    o[m] = acc;
  }
  return OR_OK;
}

/* Prefill-mode layer output for T tokens (x bf16, y fp64 [T][H]):
 * x[t] -> fp32 -> Q8_0, then as decode but with or_ffn_q8 per expert.
 * If h_out is not NULL it receives the fp32 h of every (token, slot) in
 * [T][k+S][I] order (slot k = shared expert), for diagnosis in tests. */
int oracle_forward_prefill(int64_t H, int64_t I, int64_t E, int64_t S, int64_t k,
                           const uint8_t *q4, const void *scales,
                           const int32_t *topk_idx, const float *topk_w,
                           const uint16_t *x_bf16, int64_t T, double *y,
                           float *h_out, int32_t fmt) {
  if (H <= 0 || I <= 0 || H % 64 || I % 64 || E < 1 || S < 0 || S > 1 || k < 1 ||
      fmt < OR_INT4 || fmt > OR_FP4)
    return OR_EINVAL;
  or_layer L = {H, I, E, S, q4, (const uint8_t *)scales, fmt};
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad) if(or_tokens_parallel(T))
  for (int64_t t = 0; t < T; ++t) {
    float *xf = (float *)malloc(sizeof(float) * (size_t)H);
    int8_t *qx = (int8_t *)malloc((size_t)H);
    uint16_t *dx = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)(H / 32));
    float *hf = (float *)malloc(sizeof(float) * (size_t)I);
    int8_t *qh = (int8_t *)malloc((size_t)I);
    uint16_t *dh = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)(I / 32));
    double *o = (double *)malloc(sizeof(double) * (size_t)H);
    if (!xf || !qx || !dx || !hf || !qh || !dh || !o) {
      bad = 1;
    } else {
      for (int64_t i = 0; i < H; ++i) xf[i] = (float)or_bf16(x_bf16[t * H + i]);
      if (oracle_quantize_q8_0(xf, H, qx, dx) != OR_OK) bad = 1;
      double *yt = y + t * H;
      for (int64_t i = 0; i < H; ++i) yt[i] = 0.0;
      for (int64_t j = 0; j < k + S && !bad; ++j) {
        int64_t e = (j < k) ? topk_idx[t * k + j] : E;
        double w = (j < k) ? (double)topk_w[t * k + j] : 1.0;
        if (or_ffn_q8(&L, e, qx, dx, hf, qh, dh, o) != OR_OK) bad = 1;
        if (h_out) memcpy(h_out + (t * (k + S) + j) * I, hf, sizeof(float) * (size_t)I);
        for (int64_t i = 0; i < H; ++i) yt[i] += w * o[i];
      }
    }
    free(xf);
    free(qx);
    free(dx);
    free(hf);
    free(qh);
    free(dh);
    free(o);
  }
  return bad ? OR_EINVAL : OR_OK;
}

/* ====================================================== MX activation path
 *
 * fp4 experts with fp8 activations.  The pages pair fp4 experts with
 * fp8-e4m3 elsewhere in the same model (ai-tools-nav review, model family
 * table, the DeepSeek V4 row) and give no activation format for the expert
 * GEMMs; read here as OCP MXFP8: FP8 E4M3 elements with one E8M0 scale per
 * 32 consecutive values, the block format of the MXFP4 weights. */

/* FP8 E4M3 value of a code (OCP 8-bit floating point, the E4M3 variant): bit
 * 7 sign, bits 6-3 exponent e with bias 7, bits 2-0 mantissa m; e = 0 is
 * subnormal: m/8 * 2^-6; otherwise 2^(e-7) * (1 + m/8).  Magnitude code
 * 0x7f is NaN; the largest finite magnitude is 0x7e = 448. */
static double or_e4m3(int code) {
  const int e = (code >> 3) & 15, m = code & 7;
  const double v = e ? ldexp(1.0 + m / 8.0, e - 7) : ldexp(m / 8.0, -6);
  return (code & 0x80) ? -v : v;
}

/* MXFP8 (E4M3) of n fp32 values (n % 32 == 0), per block of 32, following
 * the OCP microscaling conversion: shared exponent X = floor(log2(max|v|))
 * - 8 (8 = the largest E4M3 exponent), stored as E8M0 byte E = X + 127
 * clamped to [0, 254] (E = 0 for an all-zero block); each value becomes the
 * E4M3 code nearest to v / 2^(E-127), ties to the even code, saturating at
 * +-448 (sign kept, also for zero). */
int oracle_quantize_mxfp8(const float *v, int64_t n, uint8_t *q, uint8_t *e8) {
  if (n < 0 || n % 32) return OR_EINVAL;
  for (int64_t b = 0; b < n / 32; ++b) {
    const float *vb = v + 32 * b;
    double a = 0.0;
    for (int i = 0; i < 32; ++i)
      if (fabs((double)vb[i]) > a) a = fabs((double)vb[i]);
    int E = 0;
    if (a > 0.0) {
      int ex;
      frexp(a, &ex); /* a = f * 2^ex, f in [0.5, 1): floor(log2 a) = ex - 1 */
      E = (ex - 1) - 8 + 127;
      if (E < 0) E = 0;
      if (E > 254) E = 254;
    }
    e8[b] = (uint8_t)E;
    for (int i = 0; i < 32; ++i) {
      const double m = fabs(ldexp((double)vb[i], 127 - E));
      int c = 0x7e; /* saturate at 448 */
      for (int j = 0; j < 0x7e; ++j) {
        const double mid = 0.5 * (or_e4m3(j) + or_e4m3(j + 1));
        if (m < mid || (m == mid && !(j & 1))) { /* tie: the even code j */
          c = j;
          break;
        }
      }
      const int neg = vb[i] < 0.0f || (vb[i] == 0.0f && signbit(vb[i]));
      q[32 * b + i] = (uint8_t)(c | (neg ? 0x80 : 0));
    }
  }
  return OR_OK;
}

/* Scaled dot of one 32-block of MXFP4 weight row n (codes + E8M0) with
 * MXFP8 activations a (codes + E8M0 per block): 2^(Ew-127) * 2^(Ea-127) *
 * sum over the block of e2m1(w_k) * e4m3(a_k), every product and the sum
 * exact in fp64. */
static double or_mx_block(const uint8_t *mat, const uint8_t *sc, int64_t K, int64_t n,
                          const uint8_t *qa, const uint8_t *ea, int64_t b) {
  double acc = 0.0;
  for (int64_t k = 32 * b; k < 32 * (b + 1); ++k) {
    const uint8_t byte = mat[n * (K / 2) + k / 2];
    acc += or_e2m1((k & 1) ? (byte >> 4) : (byte & 15)) * or_e4m3(qa[k]);
  }
  return ldexp(acc, ((int)sc[n * (K / 32) + b] - 127) + ((int)ea[b] - 127));
}

/* out[t][n] = sum over blocks b of or_mx_block for matrix m (0 gate, 1 up,
 * 2 down) of expert e of an MXFP4 container, against T rows of MXFP8
 * activations (qa [T][K] codes, ea [T][K/32] E8M0), sum in block order. */
int oracle_mx_dots(int64_t H, int64_t I, int64_t E, int64_t S, const uint8_t *q4,
                   const uint8_t *scales, int64_t e, int m, const uint8_t *qa,
                   const uint8_t *ea, int64_t T, double *out) {
  if (H <= 0 || I <= 0 || H % 64 || I % 64 || m < 0 || m > 2 || e < 0 || e >= E + S || T < 0)
    return OR_EINVAL;
  or_layer L = {H, I, E, S, q4, scales, OR_FP4};
  const int64_t K = (m == 2) ? I : H, rows = (m == 2) ? H : I;
  const uint8_t *mat = or_mat(&L, e, m), *sc = or_sc(&L, e, m);
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t)
    for (int64_t n = 0; n < rows; ++n) {
      double acc = 0.0;
      for (int64_t b = 0; b < K / 32; ++b)
        acc += or_mx_block(mat, sc, K, n, qa + t * K, ea + t * (K / 32), b);
      out[t * rows + n] = acc;
    }
  return OR_OK;
}

/* MX-path expert FFN for one MXFP8 activation row (qx[H], ex[H/32]):
 *   g[n] = sum_b mx_block(w_g[n], x, b)   (likewise u)
 *   h = fp32(silu(g) * u);  (q_h, e_h) = MXFP8(h)
 *   o[m] = sum_b mx_block(w_d[m], h, b) */
static int or_ffn_mx(const or_layer *L, int64_t e, const uint8_t *qx, const uint8_t *ex,
                     float *hf, uint8_t *qh, uint8_t *eh, double *o) {
  const int64_t H = L->H, I = L->I;
  const uint8_t *qg = or_mat(L, e, 0), *qu = or_mat(L, e, 1), *qd = or_mat(L, e, 2);
  const uint8_t *sg = or_sc(L, e, 0), *su = or_sc(L, e, 1), *sd = or_sc(L, e, 2);
  OR_ROWS_PARALLEL
  for (int64_t n = 0; n < I; ++n) {
    double g = 0.0, u = 0.0;
    for (int64_t b = 0; b < H / 32; ++b) {
      g += or_mx_block(qg, sg, H, n, qx, ex, b);
      u += or_mx_block(qu, su, H, n, qx, ex, b);
    }
    hf[n] = (float)(or_silu(g) * u);
  }
  if (oracle_quantize_mxfp8(hf, I, qh, eh) != OR_OK) return OR_EINVAL;
  OR_ROWS_PARALLEL
  for (int64_t m = 0; m < H; ++m) {
    double acc = 0.0;
    for (int64_t b = 0; b < I / 32; ++b) acc += or_mx_block(qd, sd, I, m, qh, eh, b);
    o[m] = acc;
  }
  return OR_OK;
}

/* MX-path prefill layer output of an MXFP4 container for T tokens (x bf16,
 * y fp64 [T][H]): x[t] -> fp32 -> MXFP8, or_ffn_mx per routed expert and the
 * shared expert, y[t] = sum_j w[t][j] * o_j + o_shared.  h_out as in
 * oracle_forward_prefill. */
int oracle_forward_prefill_mx(int64_t H, int64_t I, int64_t E, int64_t S, int64_t k,
                              const uint8_t *q4, const uint8_t *scales,
                              const int32_t *topk_idx, const float *topk_w,
                              const uint16_t *x_bf16, int64_t T, double *y, float *h_out) {
  if (H <= 0 || I <= 0 || H % 64 || I % 64 || E < 1 || S < 0 || S > 1 || k < 1) return OR_EINVAL;
  or_layer L = {H, I, E, S, q4, scales, OR_FP4};
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad) if(or_tokens_parallel(T))
  for (int64_t t = 0; t < T; ++t) {
    float *xf = (float *)malloc(sizeof(float) * (size_t)H);
    uint8_t *qx = (uint8_t *)malloc((size_t)H);
    uint8_t *ex = (uint8_t *)malloc((size_t)(H / 32));
    float *hf = (float *)malloc(sizeof(float) * (size_t)I);
    uint8_t *qh = (uint8_t *)malloc((size_t)I);
    uint8_t *eh = (uint8_t *)malloc((size_t)(I / 32));
    double *o = (double *)malloc(sizeof(double) * (size_t)H);
    if (!xf || !qx || !ex || !hf || !qh || !eh || !o) {
      bad = 1;
    } else {
      for (int64_t i = 0; i < H; ++i) xf[i] = (float)or_bf16(x_bf16[t * H + i]);
      if (oracle_quantize_mxfp8(xf, H, qx, ex) != OR_OK) bad = 1;
      double *yt = y + t * H;
      for (int64_t i = 0; i < H; ++i) yt[i] = 0.0;
      for (int64_t j = 0; j < k + S && !bad; ++j) {
        int64_t e = (j < k) ? topk_idx[t * k + j] : E;
        double w = (j < k) ? (double)topk_w[t * k + j] : 1.0;
        if (or_ffn_mx(&L, e, qx, ex, hf, qh, eh, o) != OR_OK) bad = 1;
        if (h_out) memcpy(h_out + (t * (k + S) + j) * I, hf, sizeof(float) * (size_t)I);
        for (int64_t i = 0; i < H; ++i) yt[i] += w * o[i];
      }
    }
    free(xf);
    free(qx);
    free(ex);
    free(hf);
    free(qh);
    free(eh);
    free(o);
  }
  return bad ? OR_EINVAL : OR_OK;
}
