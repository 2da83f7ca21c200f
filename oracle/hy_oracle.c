/*
 * fp64 CPU oracle of one sparse-MoE FFN layer's forward pass.
 *
 * TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load or call this library. It shares no code with the
 * HIP path (no headers, helpers, tables or generators); the two meet only in
 * the seeded inputs they are both given.
 *
 * What the layer computes, and where it is stated:
 *  - The FFN of a Transformer block is split into many parallel FFN sub-networks
 *    ("experts"); attention is untouched. (m.xxqk.cn Hy4 preview explainer,
 *    section 2.1 "FFN 层拆分".)
 *  - A router scores every token against every expert, the K best-scoring
 *    experts are activated, they process the token in parallel, and their
 *    results are merged into the layer output. (Same page, section 2.2
 *    "路由机制".)
 *  - Hy4 preview: 256 routed experts, top-8, plus 1 shared expert that every
 *    token also goes through. (Tencent Hy4 preview model card, configuration
 *    summary; app.myzaker.com Hy4 Preview news, section "770B 不是简单堆参数".)
 * The pages leave these steps open; the readings taken here are:
 *  - score = logit x.W_r[e] (+ optional per-expert bias b[e]); selection ranks
 *    experts by logit descending, ties to the lower expert index;
 *  - merge weights = softmax of the logits renormalised over the selected set;
 *  - expert = SwiGLU without biases, y = W_down (silu(W_gate x) * (W_up x)),
 *    silu(z) = z / (1 + e^-z), weights stored [out][in];
 *  - the shared expert is added with weight 1;
 *  - output = shared + sum over the selected experts of weight * expert output.
 * Every value is computed in fp64 from the exact bf16 inputs, each sum taken
 * sequentially in index order, with no intermediate rounding.
 *
 * Sherry ternary weights (ai.chattools.top article on compressing Hy4 preview
 * to 214GB, section "极限压缩背后的技术支柱：Sherry 与 MIX-STQ1_0"): weights in
 * groups of 4 along a row take values in {-1,0,+1}; 5 bits per group give
 * 1.25 bits per weight, which fits exactly one zero per group (4 zero
 * positions x 2^3 signs = 32 codes). Code layout read here: within a block of
 * 128 weights (32 groups) held in 5 little-endian uint32 words read as one
 * 160-bit integer B, group g's code is bits [5g, 5g+5) of B; code bits 0-1 give
 * the zero's position in the group, bits 2, 3, 4 the signs (1 = negative) of
 * the first, second and third non-zero in ascending position. The weight is
 * the row's bf16 scale times the ternary value.
 *
 * FP8 weights (the Hy4 preview release ships BF16 and FP8 weights, FP8 halving
 * the weight storage: app.myzaker.com Hy4 Preview news, section "MTP、FP8 与
 * 低价 API"; the model card lists an official FP8 checkpoint). The pages fix
 * no format, scale layout or activation precision. Reading taken here: routed
 * experts' weights are OCP 8-bit floats in the E4M3 encoding (no infinities:
 * sign bit 7, exponent bits 6-3 with bias 7, mantissa bits 2-0; exponent 0 is
 * subnormal m/8 * 2^-6; exponent 15 with mantissa 7 is NaN), each output row
 * carries one fp32 scale, weight = scale * value; activations stay bf16 and the
 * shared expert stays bf16.
 *
 * FP8 weights with FP8 activations (W8A8; same pages and section, which name no
 * activation format). Reading taken here: the routed experts take the FP8 weights
 * above, and their activations (the token rows entering gate/up and the hidden
 * rows entering down) are quantized to MXFP8 as the OCP Microscaling Formats v1.0
 * specification defines it: along K, each block of 32 consecutive values shares
 * one power-of-two scale 2^e stored as an E8M0 byte e + 127, with
 * e = floor(log2(max |v|)) - 8 (8 being the exponent of E4M3's largest normal,
 * 448 = 1.75 * 2^8) clamped to [-127, 127] (a block of zeros takes -127), and
 * each value becomes the E4M3 value nearest to v * 2^-e, ties to the even
 * mantissa, saturated to +-448. The hidden values are rounded to fp32 before they
 * are quantized (the precision in which the GPU path quantizes them). The router
 * and the shared expert stay bf16.
 *
 * Sparse-attention indexer (Hy4 preview config summary, Tencent Hy4 preview model
 * card: every layer is DeepSeek-style sparse attention with an indexer of 32 heads,
 * head_dim 128 and top-k 2048, whose 128-dim key per token is shared by all heads;
 * IndexCache: 21 "full" layers run the indexer, the other 57 reuse the top-k of the
 * layer before them). The pages give no score function. Reading taken: score(t, s) =
 * sum over heads h of w[t][h] * max(0, q[t][h] . k[s]) (per-head query and weight of
 * the query token, shared key of token s); selection = the K highest scores among the
 * visible keys, ties to the lower key index, reported in ascending key order (all
 * visible keys when there are at most K).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define HYO_OK 0
#define HYO_ERR_ARG (-1)

/* ------------------------------------------------------------- helpers --- */

/* A bf16 value is the upper 16 bits of an IEEE fp32; widening is exact. */
static double bf16_value(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

typedef void (*range_fn)(void* ctx, int64_t lo, int64_t hi);
typedef struct { range_fn fn; void* ctx; int64_t lo, hi; } span_t;

static void* span_run(void* p) {
  span_t* s = (span_t*)p;
  s->fn(s->ctx, s->lo, s->hi);
  return NULL;
}

/* Runs fn over [0, n) split into contiguous spans, one per thread. Each index
 * is handled by exactly one call, so results do not depend on nthreads. */
static void parallel_for(int64_t n, range_fn fn, void* ctx, int nthreads) {
  if (n <= 0) return;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if (nthreads > n) nthreads = (int)n;
  if (nthreads == 1) { fn(ctx, 0, n); return; }
  pthread_t th[256];
  span_t sp[256];
  int made[256];
  int64_t per = (n + nthreads - 1) / nthreads;
  for (int t = 0; t < nthreads; ++t) {
    sp[t].fn = fn; sp[t].ctx = ctx;
    sp[t].lo = (int64_t)t * per;
    sp[t].hi = sp[t].lo + per < n ? sp[t].lo + per : n;
    made[t] = 0;
    if (t > 0 && sp[t].lo < sp[t].hi)
      made[t] = pthread_create(&th[t], NULL, span_run, &sp[t]) == 0;
  }
  if (sp[0].lo < sp[0].hi) span_run(&sp[0]);
  for (int t = 1; t < nthreads; ++t) {
    if (made[t]) pthread_join(th[t], NULL);
    else if (sp[t].lo < sp[t].hi) span_run(&sp[t]);
  }
}

/* ----------------------------------------------------- router logits ----- */

typedef struct {
  const uint16_t *x, *wr;
  const float* bias;
  int64_t d, E;
  double* logits;
} logits_ctx;

static void logits_rows(void* p, int64_t t0, int64_t t1) {
  logits_ctx* c = (logits_ctx*)p;
  for (int64_t t = t0; t < t1; ++t) {
    const uint16_t* xt = c->x + t * c->d;
    for (int64_t e = 0; e < c->E; ++e) {
      const uint16_t* we = c->wr + e * c->d;
      double s = 0.0;
      for (int64_t i = 0; i < c->d; ++i) s += bf16_value(xt[i]) * bf16_value(we[i]);
      if (c->bias) s += (double)c->bias[e];
      c->logits[t * c->E + e] = s;
    }
  }
}

/* Router scores: logits[t][e] = sum_i x[t][i] W_r[e][i] (+ bias[e]).
 * x: bf16 [T][d]; wr: bf16 [E][d]; bias: fp32 [E] or NULL; logits: fp64 [T][E]. */
int hyo_logits(const uint16_t* x, const uint16_t* wr, const float* bias, int64_t T, int64_t d,
               int64_t E, double* logits, int nthreads) {
  if (T < 0 || d <= 0 || E <= 0 || (T > 0 && (!x || !wr || !logits))) return HYO_ERR_ARG;
  logits_ctx c = {x, wr, bias, d, E, logits};
  parallel_for(T, logits_rows, &c, nthreads);
  return HYO_OK;
}

/* ---------------------------------------------------------- top-k -------- */

static const double* g_sort_logits; /* used only under the single-threaded qsort below */

static int by_logit_desc_then_index(const void* a, const void* b) {
  int32_t i = *(const int32_t*)a, j = *(const int32_t*)b;
  double li = g_sort_logits[i], lj = g_sort_logits[j];
  if (li > lj) return -1;
  if (li < lj) return 1;
  return (i > j) - (i < j);
}

static int by_index(const void* a, const void* b) {
  int32_t i = *(const int32_t*)a, j = *(const int32_t*)b;
  return (i > j) - (i < j);
}

/* Top-k selection: experts ranked by (logit descending, index ascending); the
 * first k are selected and written in ascending expert order to sets[t][0..k).
 * margin[t] = (k-th largest logit) - ((k+1)-th largest), +inf when k == E.
 * logits: fp64 [T][E]; sets: int32 [T][k]; margin: fp64 [T] or NULL. */
int hyo_select(const double* logits, int64_t T, int64_t E, int64_t k, int32_t* sets, double* margin) {
  if (T < 0 || E <= 0 || k < 1 || k > E || (T > 0 && (!logits || !sets))) return HYO_ERR_ARG;
  int32_t* order = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
  if (!order) return HYO_ERR_ARG;
  for (int64_t t = 0; t < T; ++t) {
    const double* l = logits + t * E;
    for (int64_t e = 0; e < E; ++e) order[e] = (int32_t)e;
    g_sort_logits = l;
    qsort(order, (size_t)E, sizeof(int32_t), by_logit_desc_then_index);
    if (margin) margin[t] = (k == E) ? INFINITY : l[order[k - 1]] - l[order[k]];
    qsort(order, (size_t)k, sizeof(int32_t), by_index);
    memcpy(sets + t * k, order, sizeof(int32_t) * (size_t)k);
  }
  free(order);
  return HYO_OK;
}

/* ------------------------------------------------------- merge weights --- */

/* w[t][j] = exp(l[e_j]) / sum_{e in S_t} exp(l[e]) for the set S_t = sets[t],
 * evaluated as exp(l - m) with m the largest logit in S_t. This is the softmax
 * over all experts renormalised over S_t. */
int hyo_weights(const double* logits, const int32_t* sets, int64_t T, int64_t E, int64_t k, double* w) {
  if (T < 0 || E <= 0 || k < 1 || k > E || (T > 0 && (!logits || !sets || !w))) return HYO_ERR_ARG;
  for (int64_t t = 0; t < T; ++t) {
    const double* l = logits + t * E;
    const int32_t* s = sets + t * k;
    double m = -INFINITY;
    for (int64_t j = 0; j < k; ++j) {
      if (s[j] < 0 || s[j] >= E) return HYO_ERR_ARG;
      if (l[s[j]] > m) m = l[s[j]];
    }
    double z = 0.0;
    for (int64_t j = 0; j < k; ++j) z += exp(l[s[j]] - m);
    for (int64_t j = 0; j < k; ++j) w[t * k + j] = exp(l[s[j]] - m) / z;
  }
  return HYO_OK;
}

/* ---------------------------------------------------------- dispatch ----- */

/* Expert-contiguous order of the routed (token, slot) pairs: expert-major,
 * tokens ascending within an expert.
 *  counts[e]    number of tokens whose set holds e              int32 [E]
 *  offsets[e]   sum of counts[0..e), offsets[E] = T*k           int32 [E+1]
 *  perm_src[p]  t*k + j of the pair stored at row p             int32 [T*k]
 *  pos[t*k+j]   row p holding pair (t, j), or NULL              int32 [T*k]
 * Sets must hold distinct experts in [0, E). */
int hyo_permute(const int32_t* sets, int64_t T, int64_t E, int64_t k, int32_t* counts,
                int32_t* offsets, int32_t* perm_src, int32_t* pos) {
  if (T < 0 || E <= 0 || k < 1 || k > E || !counts || !offsets || (T > 0 && (!sets || !perm_src)))
    return HYO_ERR_ARG;
  for (int64_t e = 0; e < E; ++e) counts[e] = 0;
  for (int64_t i = 0; i < T * k; ++i) {
    if (sets[i] < 0 || sets[i] >= E) return HYO_ERR_ARG;
    counts[sets[i]] += 1;
  }
  offsets[0] = 0;
  for (int64_t e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  int64_t p = 0;
  for (int64_t e = 0; e < E; ++e)
    for (int64_t t = 0; t < T; ++t)
      for (int64_t j = 0; j < k; ++j)
        if (sets[t * k + j] == e) {
          perm_src[p] = (int32_t)(t * k + j);
          if (pos) pos[t * k + j] = (int32_t)p;
          ++p;
        }
  return HYO_OK;
}

/* -------------------------------------------------------- expert FFN ----- */

static double silu(double z) { return z / (1.0 + exp(-z)); }

typedef struct {
  const uint16_t *x, *wg, *wu, *wd;
  int64_t d, I;
  double* h; /* [I] of the current row */
  double* y; /* [d] of the current row */
} ffn_ctx;

static void ffn_hidden(void* p, int64_t i0, int64_t i1) {
  ffn_ctx* c = (ffn_ctx*)p;
  for (int64_t i = i0; i < i1; ++i) {
    const uint16_t* g = c->wg + i * c->d;
    const uint16_t* u = c->wu + i * c->d;
    double sg = 0.0, su = 0.0;
    for (int64_t j = 0; j < c->d; ++j) {
      double xj = bf16_value(c->x[j]);
      sg += bf16_value(g[j]) * xj;
      su += bf16_value(u[j]) * xj;
    }
    c->h[i] = silu(sg) * su;
  }
}

static void ffn_out(void* p, int64_t m0, int64_t m1) {
  ffn_ctx* c = (ffn_ctx*)p;
  for (int64_t m = m0; m < m1; ++m) {
    const uint16_t* dn = c->wd + m * c->I;
    double s = 0.0;
    for (int64_t i = 0; i < c->I; ++i) s += bf16_value(dn[i]) * c->h[i];
    c->y[m] = s;
  }
}

/* One expert applied to n token rows: for each row r,
 *   h = silu(W_gate x_r) * (W_up x_r),   y_r = W_down h.
 * x_rows: bf16 [n][d]; wg, wu: bf16 [I][d]; wd: bf16 [d][I]; y: fp64 [n][d]. */
int hyo_ffn(const uint16_t* x_rows, int64_t n, const uint16_t* wg, const uint16_t* wu,
            const uint16_t* wd, int64_t d, int64_t I, double* y, int nthreads) {
  if (n < 0 || d <= 0 || I <= 0 || (n > 0 && (!x_rows || !wg || !wu || !wd || !y))) return HYO_ERR_ARG;
  double* h = (double*)malloc(sizeof(double) * (size_t)I);
  if (!h) return HYO_ERR_ARG;
  for (int64_t r = 0; r < n; ++r) {
    ffn_ctx c = {x_rows + r * d, wg, wu, wd, d, I, h, y + r * d};
    parallel_for(I, ffn_hidden, &c, nthreads);
    parallel_for(d, ffn_out, &c, nthreads);
  }
  free(h);
  return HYO_OK;
}

/* ----------------------------------------------------------- combine ----- */

/* out[t] = ys[t] + sum_j w[t][j] * yr[t][j], j ascending.
 * ys: fp64 [T][d]; yr: fp64 [T][k][d]; w: fp64 [T][k]; out: fp64 [T][d]. */
int hyo_combine(const double* ys, const double* yr, const double* w, int64_t T, int64_t k, int64_t d,
                double* out) {
  if (T < 0 || k < 1 || d <= 0 || (T > 0 && (!ys || !yr || !w || !out))) return HYO_ERR_ARG;
  for (int64_t t = 0; t < T; ++t)
    for (int64_t c = 0; c < d; ++c) {
      double s = ys[t * d + c];
      for (int64_t j = 0; j < k; ++j) s += w[t * k + j] * yr[(t * k + j) * d + c];
      out[t * d + c] = s;
    }
  return HYO_OK;
}

/* ------------------------------------------------------ Sherry decode ---- */

/* Bit b (0-based) of the little-endian word sequence w. */
static unsigned bit_at(const uint32_t* w, int64_t b) { return (w[b >> 5] >> (b & 31)) & 1u; }

/* Ternary values of one packed matrix: codes [rows][cols/128*5] -> tern [rows][cols]
 * in {-1,0,+1}; if scale (bf16 [rows]) and w (bf16 [rows][cols]) are given, also
 * writes the weights scale[r]*tern[r][c] as bf16 (exact: +-scale or 0). */
int hyo_sherry_decode(const uint32_t* packed, const uint16_t* scale, int64_t rows, int64_t cols,
                      int8_t* tern, uint16_t* w) {
  if (rows < 0 || cols <= 0 || cols % 128 != 0 || (rows > 0 && !packed)) return HYO_ERR_ARG;
  if (!tern && !(w && scale)) return HYO_ERR_ARG;
  int64_t words = cols / 128 * 5;
  for (int64_t r = 0; r < rows; ++r) {
    const uint32_t* row = packed + r * words;
    for (int64_t g = 0; g < cols / 4; ++g) {
      const uint32_t* blk = row + (g / 32) * 5;
      int64_t base = (g % 32) * 5;
      unsigned code = 0;
      for (int b = 0; b < 5; ++b) code |= bit_at(blk, base + b) << b;
      unsigned zero_pos = code & 3u;
      int nz = 0;
      for (int q = 0; q < 4; ++q) {
        int v = 0;
        if ((unsigned)q != zero_pos) {
          v = ((code >> (2 + nz)) & 1u) ? -1 : 1;
          ++nz;
        }
        int64_t c = g * 4 + q;
        if (tern) tern[r * cols + c] = (int8_t)v;
        if (w && scale) w[r * cols + c] = v == 0 ? 0 : (uint16_t)(scale[r] ^ (v < 0 ? 0x8000u : 0u));
      }
    }
  }
  return HYO_OK;
}

/* ------------------------------------------------------- FP8 E4M3 ------- */

/* Value of one E4M3 code, from the encoding's definition. */
static double e4m3_value(uint8_t c) {
  int neg = c >> 7, e = (c >> 3) & 15, m = c & 7;
  if (e == 15 && m == 7) return NAN;
  double v = e == 0 ? ldexp((double)m / 8.0, -6) : ldexp(1.0 + (double)m / 8.0, e - 7);
  return neg ? -v : v;
}

/* Weights of one FP8 matrix: q [rows][cols] E4M3 codes, scale fp32 [rows] or
 * NULL (taken as 1) -> w fp64 [rows][cols] = scale[r] * value(q[r][c]). */
int hyo_fp8_decode(const uint8_t* q, const float* scale, int64_t rows, int64_t cols, double* w) {
  if (rows < 0 || cols <= 0 || (rows > 0 && (!q || !w))) return HYO_ERR_ARG;
  for (int64_t r = 0; r < rows; ++r) {
    double s = scale ? (double)scale[r] : 1.0;
    for (int64_t c = 0; c < cols; ++c) w[r * cols + c] = s * e4m3_value(q[r * cols + c]);
  }
  return HYO_OK;
}

/* The same expert FFN with fp64 weights (bf16 token rows):
 *   h = silu(W_gate x_r) * (W_up x_r),   y_r = W_down h.
 * x_rows: bf16 [n][d]; wg, wu: fp64 [I][d]; wd: fp64 [d][I]; y: fp64 [n][d]. */
typedef struct {
  const uint16_t* x;
  const double *wg, *wu, *wd;
  int64_t d, I;
  double* h;
  double* y;
} ffn64_ctx;

static void ffn64_hidden(void* p, int64_t i0, int64_t i1) {
  ffn64_ctx* c = (ffn64_ctx*)p;
  for (int64_t i = i0; i < i1; ++i) {
    const double* g = c->wg + i * c->d;
    const double* u = c->wu + i * c->d;
    double sg = 0.0, su = 0.0;
    for (int64_t j = 0; j < c->d; ++j) {
      double xj = bf16_value(c->x[j]);
      sg += g[j] * xj;
      su += u[j] * xj;
    }
    c->h[i] = silu(sg) * su;
  }
}

static void ffn64_out(void* p, int64_t m0, int64_t m1) {
  ffn64_ctx* c = (ffn64_ctx*)p;
  for (int64_t m = m0; m < m1; ++m) {
    const double* dn = c->wd + m * c->I;
    double s = 0.0;
    for (int64_t i = 0; i < c->I; ++i) s += dn[i] * c->h[i];
    c->y[m] = s;
  }
}

int hyo_ffn_w64(const uint16_t* x_rows, int64_t n, const double* wg, const double* wu, const double* wd,
                int64_t d, int64_t I, double* y, int nthreads) {
  if (n < 0 || d <= 0 || I <= 0 || (n > 0 && (!x_rows || !wg || !wu || !wd || !y))) return HYO_ERR_ARG;
  double* h = (double*)malloc(sizeof(double) * (size_t)I);
  if (!h) return HYO_ERR_ARG;
  for (int64_t r = 0; r < n; ++r) {
    ffn64_ctx c = {x_rows + r * d, wg, wu, wd, d, I, h, y + r * d};
    parallel_for(I, ffn64_hidden, &c, nthreads);
    parallel_for(d, ffn64_out, &c, nthreads);
  }
  free(h);
  return HYO_OK;
}

/* ------------------------------------- FP8 activations (MXFP8) -------- */

/* x rounded to the nearest integer, ties to the even one (exact for |x| < 2^52). */
static double round_half_even(double x) {
  double f = floor(x), r = x - f;
  if (r > 0.5) return f + 1.0;
  if (r < 0.5) return f;
  return fmod(f, 2.0) == 0.0 ? f : f + 1.0;
}

/* E4M3 code of the value nearest to v (ties to the even mantissa), saturated to
 * +-448; the sign of zero is kept. From the encoding's definition: normals are
 * (1 + m/8) 2^(E) for E in [-6, 8], subnormals m/8 * 2^-6. */
static uint8_t e4m3_encode(double v) {
  const uint8_t sign = signbit(v) ? 0x80 : 0x00;
  const double a = fabs(v);
  if (a == 0.0) return sign;
  int ex;
  frexp(a, &ex);
  int E = ex - 1; /* floor(log2 a) */
  if (E < -6) {   /* subnormal range: multiples of 2^-9 */
    const double n = round_half_even(ldexp(a, 9));
    return n >= 8.0 ? (uint8_t)(sign | 0x08) : (uint8_t)(sign | (uint8_t)n);
  }
  double m = round_half_even(ldexp(a, 3 - E)); /* 8..16: the significand in eighths */
  if (m == 16.0) {
    m = 8.0;
    E += 1;
  }
  if (E > 8 || (E == 8 && m > 14.0)) return (uint8_t)(sign | 0x7E); /* 448 */
  return (uint8_t)(sign | (uint8_t)(((E + 7) << 3) | ((int)m - 8)));
}

/* MXFP8 quantization of rows of fp32 values, blocks of 32 along a row:
 * v [rows][cols] (cols % 32 == 0) -> codes uint8 [rows][cols] (E4M3),
 * scales uint8 [rows][cols / 32] (E8M0: the block's scale is 2^(byte - 127)). */
int hyo_mx_quantize(const float* v, int64_t rows, int64_t cols, uint8_t* codes, uint8_t* scales) {
  if (rows < 0 || cols <= 0 || cols % 32 != 0 || (rows > 0 && (!v || !codes || !scales))) return HYO_ERR_ARG;
  const int64_t nb = cols / 32;
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t b = 0; b < nb; ++b) {
      const float* blk = v + r * cols + 32 * b;
      double amax = 0.0;
      for (int i = 0; i < 32; ++i) amax = fmax(amax, fabs((double)blk[i]));
      int e = -127;
      if (amax > 0.0) {
        int ex;
        frexp(amax, &ex);
        e = ex - 1 - 8;
        if (e < -127) e = -127;
        if (e > 127) e = 127;
      }
      scales[r * nb + b] = (uint8_t)(e + 127);
      for (int i = 0; i < 32; ++i) codes[r * cols + 32 * b + i] = e4m3_encode(ldexp((double)blk[i], -e));
    }
  return HYO_OK;
}

/* The values an MXFP8 row stands for: code value * 2^(scale - 127). */
static void mx_values(const uint8_t* codes, const uint8_t* scales, int64_t cols, double* out) {
  for (int64_t c = 0; c < cols; ++c) out[c] = ldexp(e4m3_value(codes[c]), (int)scales[c / 32] - 127);
}

/* A row quantized to MXFP8 and read back: fp32 in, fp64 values out. */
static int mx_round_trip(const float* v, int64_t cols, double* out) {
  uint8_t* q = (uint8_t*)malloc((size_t)cols);
  uint8_t* sc = (uint8_t*)malloc((size_t)(cols / 32));
  if (!q || !sc) {
    free(q);
    free(sc);
    return HYO_ERR_ARG;
  }
  int rc = hyo_mx_quantize(v, 1, cols, q, sc);
  if (rc == HYO_OK) mx_values(q, sc, cols, out);
  free(q);
  free(sc);
  return rc;
}

typedef struct {
  const double *x, *wg, *wu, *wd; /* x: the row's MXFP8 values [d] */
  int64_t d, I;
  double* h; /* [I]: silu(g) * u, then its MXFP8 values */
  double* y; /* [d] */
} ffn8_ctx;

static void ffn8_hidden(void* p, int64_t i0, int64_t i1) {
  ffn8_ctx* c = (ffn8_ctx*)p;
  for (int64_t i = i0; i < i1; ++i) {
    const double* g = c->wg + i * c->d;
    const double* u = c->wu + i * c->d;
    double sg = 0.0, su = 0.0;
    for (int64_t j = 0; j < c->d; ++j) {
      sg += g[j] * c->x[j];
      su += u[j] * c->x[j];
    }
    c->h[i] = silu(sg) * su;
  }
}

static void ffn8_out(void* p, int64_t m0, int64_t m1) {
  ffn8_ctx* c = (ffn8_ctx*)p;
  for (int64_t m = m0; m < m1; ++m) {
    const double* dn = c->wd + m * c->I;
    double s = 0.0;
    for (int64_t i = 0; i < c->I; ++i) s += dn[i] * c->h[i];
    c->y[m] = s;
  }
}

/* One routed expert with fp64 (decoded FP8) weights and MXFP8 activations:
 *   x~ = MXFP8(x_r), h = silu(W_gate x~) * (W_up x~), h~ = MXFP8(fp32(h)),
 *   y_r = W_down h~.
 * x_rows: bf16 [n][d]; wg, wu: fp64 [I][d]; wd: fp64 [d][I]; y: fp64 [n][d];
 * d % 32 == 0, I % 32 == 0. h32_out (fp32 [n][I], or NULL) receives fp32(h). If hq_in and
 * hs_in are given (E4M3 codes [n][I] and E8M0 scales [n][I / 32]), h~ is read from them
 * instead of quantized from h: the substitution of a hidden code that lies on the other
 * side of a rounding boundary (the test decides which codes are admissible). */
int hyo_ffn_w8a8_ex(const uint16_t* x_rows, int64_t n, const double* wg, const double* wu, const double* wd,
                    int64_t d, int64_t I, const uint8_t* hq_in, const uint8_t* hs_in, float* h32_out, double* y,
                    int nthreads) {
  if (n < 0 || d <= 0 || I <= 0 || d % 32 || I % 32 || (n > 0 && (!x_rows || !wg || !wu || !wd || !y)))
    return HYO_ERR_ARG;
  if ((hq_in == NULL) != (hs_in == NULL)) return HYO_ERR_ARG;
  int rc = HYO_OK;
  float* xf = (float*)malloc(sizeof(float) * (size_t)d);
  double* xq = (double*)malloc(sizeof(double) * (size_t)d);
  double* h = (double*)malloc(sizeof(double) * (size_t)I);
  float* hf = (float*)malloc(sizeof(float) * (size_t)I);
  if (!xf || !xq || !h || !hf) {
    rc = HYO_ERR_ARG;
    goto done;
  }
  for (int64_t r = 0; r < n; ++r) {
    for (int64_t j = 0; j < d; ++j) xf[j] = (float)bf16_value(x_rows[r * d + j]);
    if ((rc = mx_round_trip(xf, d, xq))) goto done;
    ffn8_ctx c = {xq, wg, wu, wd, d, I, h, y + r * d};
    parallel_for(I, ffn8_hidden, &c, nthreads);
    for (int64_t i = 0; i < I; ++i) hf[i] = (float)h[i];
    if (h32_out) memcpy(h32_out + r * I, hf, sizeof(float) * (size_t)I);
    if (hq_in)
      mx_values(hq_in + r * I, hs_in + r * (I / 32), I, h);
    else if ((rc = mx_round_trip(hf, I, h)))
      goto done;
    parallel_for(d, ffn8_out, &c, nthreads);
  }
done:
  free(xf); free(xq); free(h); free(hf);
  return rc;
}

int hyo_ffn_w8a8(const uint16_t* x_rows, int64_t n, const double* wg, const double* wu, const double* wd,
                 int64_t d, int64_t I, double* y, int nthreads) {
  return hyo_ffn_w8a8_ex(x_rows, n, wg, wu, wd, d, I, NULL, NULL, NULL, y, nthreads);
}

/* ------------------------------------------------------- whole layer ----- */

/* The whole layer; routed experts' weights as bf16 (wg..wd) or as fp64 (fg..fd, the
 * other set NULL). */
static int forward_impl(const uint16_t* x, const uint16_t* wr, const float* bias, const uint16_t* wg,
                        const uint16_t* wu, const uint16_t* wd, const double* fg, const double* fu,
                        const double* fd, int a8, const uint16_t* sg, const uint16_t* su, const uint16_t* sd,
                        int64_t T, int64_t d, int64_t E, int64_t k, int64_t I, const int32_t* sets_in,
                        double* out, int32_t* sets_out, double* w_out, double* margin_out, double* logits_out,
                        int nthreads) {
  if (T < 0 || d <= 0 || E <= 0 || k < 1 || k > E || I <= 0) return HYO_ERR_ARG;
  if (T == 0) return HYO_OK;
  const int f64 = fg != NULL;
  if (!x || !wr || !sg || !su || !sd || !out) return HYO_ERR_ARG;
  if (f64 ? (!fu || !fd) : (!wg || !wu || !wd)) return HYO_ERR_ARG;
  int rc = HYO_OK;
  double* logits = (double*)malloc(sizeof(double) * (size_t)(T * E));
  int32_t* sets = (int32_t*)malloc(sizeof(int32_t) * (size_t)(T * k));
  double* w = (double*)malloc(sizeof(double) * (size_t)(T * k));
  double* ys = (double*)malloc(sizeof(double) * (size_t)(T * d));
  double* yr = (double*)malloc(sizeof(double) * (size_t)(T * k * d));
  if (!logits || !sets || !w || !ys || !yr) { rc = HYO_ERR_ARG; goto done; }
  if ((rc = hyo_logits(x, wr, bias, T, d, E, logits, nthreads))) goto done;
  if ((rc = hyo_select(logits, T, E, k, sets, margin_out))) goto done;
  if (sets_in) memcpy(sets, sets_in, sizeof(int32_t) * (size_t)(T * k));
  if ((rc = hyo_weights(logits, sets, T, E, k, w))) goto done;
  if ((rc = hyo_ffn(x, T, sg, su, sd, d, I, ys, nthreads))) goto done;
  for (int64_t t = 0; t < T; ++t)
    for (int64_t j = 0; j < k; ++j) {
      int64_t e = sets[t * k + j];
      if (a8)
        rc = hyo_ffn_w8a8(x + t * d, 1, fg + e * I * d, fu + e * I * d, fd + e * d * I, d, I, yr + (t * k + j) * d,
                          nthreads);
      else if (f64)
        rc = hyo_ffn_w64(x + t * d, 1, fg + e * I * d, fu + e * I * d, fd + e * d * I, d, I, yr + (t * k + j) * d,
                         nthreads);
      else
        rc = hyo_ffn(x + t * d, 1, wg + e * I * d, wu + e * I * d, wd + e * d * I, d, I, yr + (t * k + j) * d,
                     nthreads);
      if (rc) goto done;
    }
  rc = hyo_combine(ys, yr, w, T, k, d, out);
  if (sets_out) memcpy(sets_out, sets, sizeof(int32_t) * (size_t)(T * k));
  if (w_out) memcpy(w_out, w, sizeof(double) * (size_t)(T * k));
  if (logits_out) memcpy(logits_out, logits, sizeof(double) * (size_t)(T * E));
done:
  free(logits); free(sets); free(w); free(ys); free(yr);
  return rc;
}

/* Forward pass of the whole layer for small shapes (bf16 routed experts).
 *   x [T][d], wr [E][d], bias [E] fp32 or NULL,
 *   wg, wu [E][I][d], wd [E][d][I], sg, su [I][d], sd [d][I]   (bf16)
 * Outputs: out fp64 [T][d]; optional sets int32 [T][k], w fp64 [T][k],
 * margin fp64 [T], logits fp64 [T][E]. If sets_in is non-NULL it replaces the
 * top-k selection (used to substitute an admissible set for a near-tie token). */
int hyo_forward(const uint16_t* x, const uint16_t* wr, const float* bias, const uint16_t* wg,
                const uint16_t* wu, const uint16_t* wd, const uint16_t* sg, const uint16_t* su,
                const uint16_t* sd, int64_t T, int64_t d, int64_t E, int64_t k, int64_t I,
                const int32_t* sets_in, double* out, int32_t* sets_out, double* w_out,
                double* margin_out, double* logits_out, int nthreads) {
  return forward_impl(x, wr, bias, wg, wu, wd, NULL, NULL, NULL, 0, sg, su, sd, T, d, E, k, I, sets_in, out,
                      sets_out, w_out, margin_out, logits_out, nthreads);
}

/* The same with fp64 routed weights fg, fu [E][I][d], fd [E][d][I] (e.g. decoded
 * FP8 experts); the shared expert stays bf16. */
int hyo_forward_w64(const uint16_t* x, const uint16_t* wr, const float* bias, const double* fg,
                    const double* fu, const double* fd, const uint16_t* sg, const uint16_t* su,
                    const uint16_t* sd, int64_t T, int64_t d, int64_t E, int64_t k, int64_t I,
                    const int32_t* sets_in, double* out, int32_t* sets_out, double* w_out,
                    double* margin_out, double* logits_out, int nthreads) {
  if (!fg) return HYO_ERR_ARG;
  return forward_impl(x, wr, bias, NULL, NULL, NULL, fg, fu, fd, 0, sg, su, sd, T, d, E, k, I, sets_in, out,
                      sets_out, w_out, margin_out, logits_out, nthreads);
}

/* The same with the routed experts on MXFP8 activations (hyo_ffn_w8a8); the router
 * and the shared expert stay bf16. d % 32 == 0, I % 32 == 0. */
int hyo_forward_w8a8(const uint16_t* x, const uint16_t* wr, const float* bias, const double* fg,
                     const double* fu, const double* fd, const uint16_t* sg, const uint16_t* su,
                     const uint16_t* sd, int64_t T, int64_t d, int64_t E, int64_t k, int64_t I,
                     const int32_t* sets_in, double* out, int32_t* sets_out, double* w_out,
                     double* margin_out, double* logits_out, int nthreads) {
  if (!fg || d % 32 || I % 32) return HYO_ERR_ARG;
  return forward_impl(x, wr, bias, NULL, NULL, NULL, fg, fu, fd, 1, sg, su, sd, T, d, E, k, I, sets_in, out,
                      sets_out, w_out, margin_out, logits_out, nthreads);
}

/* ------------------------------------------------------- indexer --------- */

/* Scores of B queries, each against its own S keys:
 * q bf16 [B][H][D], w fp32 [B][H], keys bf16 [B][S][D] -> scores fp64 [B][S]. */
int hyo_indexer_scores(const uint16_t* q, const float* w, const uint16_t* keys, int64_t B, int64_t H, int64_t D,
                       int64_t S, double* scores) {
  if (B < 0 || H <= 0 || D <= 0 || S < 0 || (B > 0 && S > 0 && (!q || !w || !keys || !scores))) return HYO_ERR_ARG;
  for (int64_t b = 0; b < B; ++b)
    for (int64_t s = 0; s < S; ++s) {
      const uint16_t* kv = keys + (b * S + s) * D;
      double acc = 0.0;
      for (int64_t h = 0; h < H; ++h) {
        const uint16_t* qv = q + (b * H + h) * D;
        double dot = 0.0;
        for (int64_t i = 0; i < D; ++i) dot += bf16_value(qv[i]) * bf16_value(kv[i]);
        acc += (double)w[b * H + h] * (dot > 0.0 ? dot : 0.0);
      }
      scores[b * S + s] = acc;
    }
  return HYO_OK;
}

typedef struct {
  double v;
  int64_t i;
} scored;

/* by score descending, then key index ascending */
static int by_score_desc_then_index(const void* a, const void* b) {
  const scored* x = (const scored*)a;
  const scored* y = (const scored*)b;
  if (x->v != y->v) return x->v > y->v ? -1 : 1;
  return x->i < y->i ? -1 : (x->i > y->i);
}

static int by_key_index(const void* a, const void* b) {
  const int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
  return (x > y) - (x < y);
}

/* Top-K selection per row: scores fp64 [B][S] -> idx int32 [B][min(K, S)], the K
 * highest scores (ties to the lower index), in ascending index order; kth fp64 [B]
 * (optional) gets the K-th highest score and margin fp64 [B] (optional) its lead over
 * the (K+1)-th (+inf when S <= K). */
int hyo_topk_indices(const double* scores, int64_t B, int64_t S, int64_t K, int32_t* idx, double* kth,
                     double* margin) {
  if (B < 0 || S < 0 || K < 1 || (B > 0 && S > 0 && (!scores || !idx))) return HYO_ERR_ARG;
  const int64_t n = S < K ? S : K;
  scored* tmp = (scored*)malloc(sizeof(scored) * (size_t)(S > 0 ? S : 1));
  if (!tmp) return HYO_ERR_ARG;
  for (int64_t b = 0; b < B; ++b) {
    for (int64_t s = 0; s < S; ++s) tmp[s] = (scored){scores[b * S + s], s};
    qsort(tmp, (size_t)S, sizeof(scored), by_score_desc_then_index);
    for (int64_t j = 0; j < n; ++j) idx[b * n + j] = (int32_t)tmp[j].i;
    qsort(idx + b * n, (size_t)n, sizeof(int32_t), by_key_index);
    if (kth) kth[b] = n > 0 ? tmp[n - 1].v : NAN;
    if (margin) margin[b] = S > K ? tmp[K - 1].v - tmp[K].v : INFINITY;
  }
  free(tmp);
  return HYO_OK;
}
