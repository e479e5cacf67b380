/*
 * moe_oracle.c -- CPU reference of one sparsely-gated MoE FFN layer forward.
 *
 * TEST INFRASTRUCTURE ONLY (see moe_oracle.h).  Written from the pages'
 * definitions, step by step; no blocking, fusion or reordering beyond what a
 * definition states.  Reductions are in double, in ascending index order.
 */
#include "moe_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---- element access ----------------------------------------------------- */

static inline double bf16_bits_to_double(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* element i of a bf16 or fp32 array, widened exactly to double */
static inline double elem(const void* p, int32_t bf16, int64_t i) {
  return bf16 ? bf16_bits_to_double(((const uint16_t*)p)[i]) : (double)((const float*)p)[i];
}

double orc_fp8_e4m3(uint8_t c) {
  /* OCP FP8 E4M3: sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent
   * field 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN; no infinities. */
  const int sgn = c >> 7, e = (c >> 3) & 15, m = c & 7;
  if (e == 15 && m == 7) return NAN;
  const double v = e == 0 ? ldexp((double)m / 8.0, -6) : ldexp(1.0 + (double)m / 8.0, e - 7);
  return sgn ? -v : v;
}

/* element i of an expert weight: wdt 0 fp32, 1 bf16, 2 FP8 E4M3 code times
 * the per-row scale scale[i / row_len] */
static inline double welem(const void* p, int32_t wdt, int64_t i, const float* scale, int64_t row_len) {
  if (wdt == 2) return orc_fp8_e4m3(((const uint8_t*)p)[i]) * (double)scale[i / row_len];
  return elem(p, wdt, i);
}

/* ---- a1: router logits  [TD §3.1 step 1; BD §3.2] ------------------------ */

void orc_logits(const orc_layer* L, const void* x, const float* Wg, const float* logit_bias, float* logits) {
  const int64_t T = L->T, d = L->d, E = L->E;
#pragma omp parallel for schedule(dynamic, 4)
  for (int64_t t = 0; t < T; ++t) {
    for (int64_t e = 0; e < E; ++e) {
      double acc = 0.0;
      for (int64_t i = 0; i < d; ++i) acc += elem(x, L->bf16, t * d + i) * (double)Wg[e * d + i];
      if (logit_bias) acc += (double)logit_bias[e];
      logits[t * E + e] = (float)acc;
    }
  }
}

/* ---- a2 + a3: gate, key, Top-K, weights ----------------------------------- */

/* "a ranks before b": larger key first, ties to the lower expert index.  Keys
 * are compared as IEEE values, so -0 and +0 are equal. */
static inline int ranks_before(float ka, int64_t ea, float kb, int64_t eb) {
  if (ka != kb) return ka > kb;
  return ea < eb;
}

/* Selection key and gate score of every expert for one token's logits. */
static void token_scores(const orc_layer* L, const float* l, const float* sel_bias, float* key, double* score) {
  const int64_t E = L->E;
  if (L->gate == ORC_GATE_SOFTMAX) {
    /* p_i = e^{l_i} / sum_j e^{l_j}  [TD §3.2], evaluated with the max
     * subtracted; softmax is monotone, so the key is the logit itself. */
    double m = -INFINITY;
    for (int64_t e = 0; e < E; ++e) m = fmax(m, (double)l[e]);
    double z = 0.0;
    for (int64_t e = 0; e < E; ++e) z += exp((double)l[e] - m);
    for (int64_t e = 0; e < E; ++e) {
      score[e] = exp((double)l[e] - m) / z;
      key[e] = l[e];
    }
  } else {
    /* s = Sigmoid(u^T e_i)  [TD §3.5]; selection on s + b_i, weights on s
     * alone  [TD §4.3; §9.2].  The key is formed in fp32. */
    for (int64_t e = 0; e < E; ++e) {
      double s = 1.0 / (1.0 + exp(-(double)l[e]));
      float sf = (float)s;
      float b = sel_bias ? sel_bias[e] : 0.0f;
      score[e] = s;
      key[e] = sf + b;
    }
  }
}

/* order[0 .. n) = the n best experts by repeated maximum under the total
 * order above [TD §3.1 KeepTopK]; order[n ..) holds the rest. */
static void top_n(const float* key, int64_t E, int64_t n, int64_t* order) {
  for (int64_t e = 0; e < E; ++e) order[e] = e;
  for (int64_t k = 0; k < n && k < E; ++k) {
    int64_t best = k;
    for (int64_t j = k + 1; j < E; ++j)
      if (ranks_before(key[order[j]], order[j], key[order[best]], order[best])) best = j;
    int64_t tmp = order[k];
    order[k] = order[best];
    order[best] = tmp;
  }
}

void orc_select(const orc_layer* L, const float* logits, const float* sel_bias, int32_t* idx, double* w,
                double* gap) {
  const int64_t T = L->T, E = L->E, K = L->K;
#pragma omp parallel
  {
    float* key = (float*)malloc(sizeof(float) * (size_t)E);
    double* score = (double*)malloc(sizeof(double) * (size_t)E);
    int64_t* order = (int64_t*)malloc(sizeof(int64_t) * (size_t)E);
#pragma omp for schedule(dynamic, 16)
    for (int64_t t = 0; t < T; ++t) {
      token_scores(L, logits + t * E, sel_bias, key, score);
      top_n(key, E, K, order);
      double sum = 0.0;
      for (int64_t k = 0; k < K; ++k) sum += score[order[k]];
      for (int64_t k = 0; k < K; ++k) {
        idx[t * K + k] = (int32_t)order[k];
        /* renormalised Top-K weights  [TD §9.1] */
        w[t * K + k] = L->renorm ? score[order[k]] / sum : score[order[k]];
      }
      if (gap) {
        if (K >= E) {
          gap[t] = INFINITY;
        } else {
          /* the (K+1)-th key is the largest among the unselected ones */
          float next = key[order[K]];
          for (int64_t j = K + 1; j < E; ++j)
            if (key[order[j]] > next) next = key[order[j]];
          gap[t] = (double)key[order[K - 1]] - (double)next;
        }
      }
    }
    free(key);
    free(score);
    free(order);
  }
}

void orc_select_ranked(const orc_layer* L, const float* logits, const float* sel_bias, int64_t n, int32_t* idx,
                       double* w) {
  const int64_t T = L->T, E = L->E, K = L->K;
#pragma omp parallel
  {
    float* key = (float*)malloc(sizeof(float) * (size_t)E);
    double* score = (double*)malloc(sizeof(double) * (size_t)E);
    int64_t* order = (int64_t*)malloc(sizeof(int64_t) * (size_t)E);
#pragma omp for schedule(dynamic, 16)
    for (int64_t t = 0; t < T; ++t) {
      token_scores(L, logits + t * E, sel_bias, key, score);
      top_n(key, E, n, order);
      double sum = 0.0;
      for (int64_t k = 0; k < K; ++k) sum += score[order[k]];
      for (int64_t r = 0; r < n; ++r) {
        idx[t * n + r] = (int32_t)order[r];
        w[t * n + r] = L->renorm ? score[order[r]] / sum : score[order[r]];
      }
    }
    free(key);
    free(score);
    free(order);
  }
}

/* ---- a4: capacity, histogram, stable permutation  [TD §3.2] -------------- */

int64_t orc_capacity(const orc_layer* L) {
  if (!(L->capacity_factor > 0.0)) return -1;
  /* K_max = floor(C * N_tokens / N_experts), with N_tokens counted in
   * (token, choice) assignments so the formula also covers K > 1. */
  return (int64_t)floor(L->capacity_factor * (double)(L->T * L->K) / (double)L->E);
}

void orc_permute(const orc_layer* L, const int32_t* idx, int32_t* counts, int32_t* offsets, int32_t* dest,
                 int32_t* row_src, uint8_t* dropped) {
  const int64_t E = L->E, N = L->T * L->K;
  const int64_t cap = orc_capacity(L);
  int64_t* pos = (int64_t*)malloc(sizeof(int64_t) * (size_t)(N > 0 ? N : 1));
  for (int64_t e = 0; e < E; ++e) counts[e] = 0;
  /* pos(f): arrivals in flat order; the first `cap` arrivals are kept and
   * the rest overflow and are dropped. */
  for (int64_t f = 0; f < N; ++f) pos[f] = counts[idx[f]]++;
  offsets[0] = 0;
  for (int64_t e = 0; e < E; ++e) {
    int64_t kept = counts[e];
    if (cap >= 0 && kept > cap) kept = cap;
    offsets[e + 1] = offsets[e] + (int32_t)kept;
  }
  for (int64_t r = 0; r < N; ++r) row_src[r] = -1;
  for (int64_t f = 0; f < N; ++f) {
    int keep = (cap < 0) || (pos[f] < cap);
    dest[f] = keep ? (int32_t)(offsets[idx[f]] + pos[f]) : -1;
    dropped[f] = (uint8_t)!keep;
    if (keep) row_src[dest[f]] = (int32_t)f;
  }
  free(pos);
}

/* ---- a4 variants: which overflow assignments drop ----------------------- */

typedef struct aff_item {
  float a;
  int64_t f;
} aff_item;

/* higher affinity first, then the lower flat index */
static int aff_cmp(const void* pa, const void* pb) {
  const aff_item* x = (const aff_item*)pa;
  const aff_item* y = (const aff_item*)pb;
  if (x->a != y->a) return x->a > y->a ? -1 : 1;
  return x->f < y->f ? -1 : (x->f > y->f ? 1 : 0);
}

void orc_permute_affinity(const orc_layer* L, const int32_t* idx, const float* aff, int32_t* counts,
                          int32_t* offsets, int32_t* dest, int32_t* row_src, uint8_t* dropped) {
  const int64_t E = L->E, N = L->T * L->K;
  const int64_t cap = orc_capacity(L);
  uint8_t* keep = (uint8_t*)malloc((size_t)(N > 0 ? N : 1));
  aff_item* items = (aff_item*)malloc(sizeof(aff_item) * (size_t)(N > 0 ? N : 1));
  for (int64_t e = 0; e < E; ++e) counts[e] = 0;
  for (int64_t f = 0; f < N; ++f) counts[idx[f]]++;
  /* each expert over capacity keeps its `cap` highest-affinity assignments
   * and drops the rest, in descending-affinity order  [TD §5.2, V2 token
   * dropping]; ties go to the earlier assignment */
  for (int64_t e = 0; e < E; ++e) {
    int64_t n = 0;
    for (int64_t f = 0; f < N; ++f)
      if (idx[f] == e) {
        items[n].a = aff[f];
        items[n].f = f;
        ++n;
      }
    if (n > 1) qsort(items, (size_t)n, sizeof(aff_item), aff_cmp);
    for (int64_t i = 0; i < n; ++i) keep[items[i].f] = (uint8_t)(cap < 0 || i < cap);
  }
  offsets[0] = 0;
  for (int64_t e = 0; e < E; ++e) {
    int64_t kept = counts[e];
    if (cap >= 0 && kept > cap) kept = cap;
    offsets[e + 1] = offsets[e] + (int32_t)kept;
  }
  /* kept rows of an expert stay in flat order */
  int32_t* run = (int32_t*)calloc((size_t)E, sizeof(int32_t));
  for (int64_t r = 0; r < N; ++r) row_src[r] = -1;
  for (int64_t f = 0; f < N; ++f) {
    const int32_t e = idx[f];
    dest[f] = keep[f] ? offsets[e] + run[e]++ : -1;
    dropped[f] = (uint8_t)!keep[f];
    if (keep[f]) row_src[dest[f]] = (int32_t)f;
  }
  free(run);
  free(items);
  free(keep);
}

void orc_permute_reroute(const orc_layer* L, const int32_t* idx, const double* w, const int32_t* alt_idx,
                         const double* alt_w, int64_t n_alt, int32_t* counts, int32_t* offsets, int32_t* dest,
                         int32_t* row_src, uint8_t* dropped, int32_t* idx_out, double* w_out) {
  const int64_t E = L->E, T = L->T, K = L->K, N = T * K;
  const int64_t cap = orc_capacity(L);
  int64_t* pos = (int64_t*)malloc(sizeof(int64_t) * (size_t)(N > 0 ? N : 1));
  int32_t* cand = (int32_t*)malloc(sizeof(int32_t) * (size_t)(N > 0 ? N : 1));
  int64_t* first = (int64_t*)calloc((size_t)E, sizeof(int64_t));
  int64_t* second = (int64_t*)calloc((size_t)E, sizeof(int64_t));
  /* first pass: the first-come rule of orc_permute */
  for (int64_t e = 0; e < E; ++e) counts[e] = 0;
  for (int64_t f = 0; f < N; ++f) pos[f] = counts[idx[f]]++;
  for (int64_t e = 0; e < E; ++e) first[e] = (cap >= 0 && counts[e] > cap) ? cap : counts[e];
  /* an overflowing assignment is sent to the token's next-best expert
   * [LN §3.2]: the j-th overflowing choice of token t (in k order) takes the
   * token's rank K + j expert, if there is one */
  for (int64_t t = 0; t < T; ++t) {
    int64_t j = 0;
    for (int64_t k = 0; k < K; ++k) {
      const int64_t f = t * K + k;
      idx_out[f] = idx[f];
      w_out[f] = w[f];
      cand[f] = -1;
      if (cap >= 0 && pos[f] >= cap) {
        if (j < n_alt && alt_idx[t * n_alt + j] >= 0) {
          cand[f] = alt_idx[t * n_alt + j];
          idx_out[f] = cand[f];
          w_out[f] = alt_w[t * n_alt + j];
        }
        ++j;
      }
    }
  }
  /* second pass: re-routed assignments, in flat order, take what capacity
   * their new expert has left after the first pass */
  for (int64_t f = 0; f < N; ++f)
    if (cand[f] >= 0) pos[f] = second[cand[f]]++;
  /* with no capacity limit nothing overflows and nothing is re-routed: the
   * result is the first-come permutation */
  offsets[0] = 0;
  for (int64_t e = 0; e < E; ++e) {
    const int64_t room = cap < 0 ? 0 : cap - first[e];
    const int64_t extra = second[e] < room ? second[e] : room;
    offsets[e + 1] = offsets[e] + (int32_t)(first[e] + extra);
  }
  /* rows of an expert: its first-pass assignments, then its re-routed ones,
   * each in flat order */
  for (int64_t r = 0; r < N; ++r) row_src[r] = -1;
  for (int64_t f = 0; f < N; ++f) {
    int64_t row = -1;
    if (cap < 0 || (cand[f] < 0 && pos[f] < cap)) {
      row = offsets[idx[f]] + pos[f];
    } else if (cand[f] >= 0 && pos[f] < cap - first[cand[f]]) {
      row = offsets[cand[f]] + first[cand[f]] + pos[f];
    }
    dest[f] = (int32_t)row;
    dropped[f] = (uint8_t)(row < 0);
    if (row >= 0) row_src[row] = (int32_t)f;
  }
  free(second);
  free(first);
  free(cand);
  free(pos);
}

/* ---- a6 + a7: one SwiGLU expert on one row  [LN §2.2] -------------------- */

double orc_bf16_round(double v) {
  /* bf16 keeps 8 significant bits and fp32's exponent range: round v to
   * that grid, ties to even (the default rounding mode of nearbyint). */
  if (v == 0.0 || !isfinite(v)) return v;
  const double min_normal = ldexp(1.0, -126);
  if (fabs(v) < min_normal) return ldexp(nearbyint(ldexp(v, 133)), -133); /* subnormal spacing 2^-133 */
  int e;
  const double m = frexp(v, &e); /* v = m * 2^e, 0.5 <= |m| < 1 */
  return ldexp(nearbyint(ldexp(m, 8)), e - 8);
}

void orc_swiglu(int64_t d, int64_t F, int32_t wdt, int32_t round_h, const void* W1, const void* W3,
                const void* W2, const float* s1, const float* s3, const float* s2, const double* x, double* out,
                int32_t threads) {
  double* h = (double*)malloc(sizeof(double) * (size_t)F);
  int nt = threads > 1 ? threads : 1;
#pragma omp parallel for schedule(static) num_threads(nt) if (nt > 1)
  for (int64_t j = 0; j < F; ++j) {
    double a = 0.0, b = 0.0;
    for (int64_t i = 0; i < d; ++i) {
      a += welem(W1, wdt, j * d + i, s1, d) * x[i];
      b += welem(W3, wdt, j * d + i, s3, d) * x[i];
    }
    double silu = a / (1.0 + exp(-a));
    h[j] = silu * b;
    /* a bf16 layer holds its activations, h included, in bf16 */
    if (round_h) h[j] = orc_bf16_round(h[j]);
  }
#pragma omp parallel for schedule(static) num_threads(nt) if (nt > 1)
  for (int64_t m = 0; m < d; ++m) {
    double o = 0.0;
    for (int64_t j = 0; j < F; ++j) o += welem(W2, wdt, m * F + j, s2, F) * h[j];
    out[m] = o;
  }
  free(h);
}

/* ---- a6-a9: routed experts, shared experts, weighted combine ------------- */

void orc_forward_rows(const orc_layer* L, const void* x, const int32_t* idx, const double* w, const int32_t* dest,
                      const void* const* W1e, const void* const* W3e, const void* const* W2e, const void* Ws1,
                      const void* Ws3, const void* Ws2, const float* const* S1e, const float* const* S3e,
                      const float* const* S2e, const float* Ss1, const float* Ss3, const float* Ss2,
                      const int64_t* tokens, int64_t n_tokens, double* y) {
  const int64_t d = L->d, K = L->K, F = L->F, Fs = L->Fs;
  const int32_t wdt = L->w_fp8 ? 2 : L->bf16;
  const size_t esz = L->w_fp8 ? 1 : (L->bf16 ? 2 : 4);
  int max_threads = 1;
#ifdef _OPENMP
  max_threads = omp_get_max_threads();
#endif
  /* Few tokens: split each expert's output loops across threads instead. */
  const int inner = (n_tokens < 2 * max_threads) ? max_threads : 1;
#pragma omp parallel for schedule(dynamic, 1) if (inner == 1)
  for (int64_t j = 0; j < n_tokens; ++j) {
    const int64_t t = tokens[j];
    double* xt = (double*)malloc(sizeof(double) * (size_t)d);
    double* o = (double*)malloc(sizeof(double) * (size_t)d);
    double* acc = y + j * d;
    for (int64_t i = 0; i < d; ++i) {
      xt[i] = elem(x, L->bf16, t * d + i);
      acc[i] = 0.0;
    }
    /* y = sum_i G_i E_i(x) over the chosen experts  [TD §3.1 step 4]; an
     * assignment dropped for capacity contributes nothing  [TD §3.2]. */
    for (int64_t k = 0; k < K; ++k) {
      if (dest && dest[t * K + k] < 0) continue;
      const int32_t e = idx[t * K + k];
      orc_swiglu(d, F, wdt, L->round_h, W1e[e], W3e[e], W2e[e], S1e ? S1e[e] : NULL, S3e ? S3e[e] : NULL,
                 S2e ? S2e[e] : NULL, xt, o, inner);
      for (int64_t i = 0; i < d; ++i) acc[i] += w[t * K + k] * o[i];
    }
    /* always-active shared experts, added unweighted  [TD §3.4; §9.1] */
    for (int64_t s = 0; s < L->n_shared; ++s) {
      const char* p1 = (const char*)Ws1 + (size_t)(s * Fs * d) * esz;
      const char* p3 = (const char*)Ws3 + (size_t)(s * Fs * d) * esz;
      const char* p2 = (const char*)Ws2 + (size_t)(s * d * Fs) * esz;
      orc_swiglu(d, Fs, wdt, L->round_h, p1, p3, p2, Ss1 ? Ss1 + s * Fs : NULL, Ss3 ? Ss3 + s * Fs : NULL,
                 Ss2 ? Ss2 + s * d : NULL, xt, o, inner);
      for (int64_t i = 0; i < d; ++i) acc[i] += o[i];
    }
    /* residual Add of the MoE block  [TD §2.1] */
    if (L->residual)
      for (int64_t i = 0; i < d; ++i) acc[i] += xt[i];
    free(xt);
    free(o);
  }
}

/* ---- a9 alone ------------------------------------------------------------ */

void orc_combine(const orc_layer* L, const float* yp, const double* w, const int32_t* dest, const float* shared,
                 const void* x, double* y) {
  const int64_t T = L->T, d = L->d, K = L->K;
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    double* acc = y + t * d;
    for (int64_t i = 0; i < d; ++i) acc[i] = 0.0;
    for (int64_t k = 0; k < K; ++k) {
      const int32_t r = dest[t * K + k];
      if (r < 0) continue;
      for (int64_t i = 0; i < d; ++i) acc[i] += w[t * K + k] * (double)yp[(int64_t)r * d + i];
    }
    if (shared)
      for (int64_t i = 0; i < d; ++i) acc[i] += (double)shared[t * d + i];
    if (L->residual)
      for (int64_t i = 0; i < d; ++i) acc[i] += elem(x, L->bf16, t * d + i);
  }
}

/* ---- router statistics  [TD §4.2, §4.4, §9.1] ---------------------------- */

void orc_router_stats(const orc_layer* L, const float* logits, const int32_t* idx, double* out) {
  const int64_t T = L->T, E = L->E, K = L->K;
  double* P = (double*)calloc((size_t)E, sizeof(double));
  double* f = (double*)calloc((size_t)E, sizeof(double));
  double z = 0.0;
  for (int64_t t = 0; t < T; ++t) {
    const float* l = logits + t * E;
    double m = -INFINITY;
    for (int64_t e = 0; e < E; ++e) m = fmax(m, (double)l[e]);
    double se = 0.0;
    for (int64_t e = 0; e < E; ++e) se += exp((double)l[e] - m);
    const double lse = m + log(se);
    z += lse * lse;
    if (L->gate == ORC_GATE_SOFTMAX) {
      for (int64_t e = 0; e < E; ++e) P[e] += exp((double)l[e] - m) / se;
    } else {
      double ss = 0.0;
      for (int64_t e = 0; e < E; ++e) ss += 1.0 / (1.0 + exp(-(double)l[e]));
      for (int64_t e = 0; e < E; ++e) P[e] += (1.0 / (1.0 + exp(-(double)l[e]))) / ss;
    }
  }
  for (int64_t q = 0; q < T * K; ++q) f[idx[q]] += 1.0;
  double bal = 0.0, fmaxv = 0.0, fmean = 0.0, hP = 0.0, hf = 0.0;
  for (int64_t e = 0; e < E; ++e) {
    P[e] /= (double)T;
    f[e] /= (double)(T * K);
    bal += f[e] * P[e];
    fmaxv = fmax(fmaxv, f[e]);
    fmean += f[e];
    if (P[e] > 0) hP -= P[e] * log(P[e]);
    if (f[e] > 0) hf -= f[e] * log(f[e]);
  }
  fmean /= (double)E;
  double var = 0.0;
  for (int64_t e = 0; e < E; ++e) var += (f[e] - fmean) * (f[e] - fmean);
  var /= (double)E;
  for (int64_t e = 0; e < E; ++e) out[e] = P[e];
  out[E + 0] = (double)E * bal;
  out[E + 1] = z / (double)T;
  out[E + 2] = (double)E * fmaxv;
  out[E + 3] = sqrt(var) / fmean;
  out[E + 4] = hP;
  out[E + 5] = hf;
  free(P);
  free(f);
}

/* ---- expert-choice routing  [TD §3.3] ------------------------------------ */

void orc_expert_choice(const orc_layer* L, const float* logits, int64_t cap, int32_t* tok, double* g) {
  const int64_t T = L->T, E = L->E;
#pragma omp parallel
  {
    int64_t* order = (int64_t*)malloc(sizeof(int64_t) * (size_t)(T > 0 ? T : 1));
#pragma omp for schedule(dynamic, 1)
    for (int64_t e = 0; e < E; ++e) {
      for (int64_t t = 0; t < T; ++t) order[t] = t;
      for (int64_t c = 0; c < cap && c < T; ++c) {
        int64_t best = c;
        for (int64_t j = c + 1; j < T; ++j) {
          float a = logits[order[j] * E + e], b = logits[order[best] * E + e];
          if (a > b || (a == b && order[j] < order[best])) best = j;
        }
        int64_t tmp = order[c];
        order[c] = order[best];
        order[best] = tmp;
        const int64_t t = order[c];
        const float* l = logits + t * E;
        double m = -INFINITY, z = 0.0;
        for (int64_t q = 0; q < E; ++q) m = fmax(m, (double)l[q]);
        for (int64_t q = 0; q < E; ++q) z += exp((double)l[q] - m);
        tok[e * cap + c] = (int32_t)t;
        g[e * cap + c] = exp((double)l[e] - m) / z;
      }
    }
    free(order);
  }
}

int32_t orc_threads(void) {
#ifdef _OPENMP
  return (int32_t)omp_get_max_threads();
#else
  return 1;
#endif
}
