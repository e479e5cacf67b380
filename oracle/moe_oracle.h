/*
 * moe_oracle.h -- plain, slow, obviously-correct CPU reference of one
 * sparsely-gated Mixture-of-Experts FFN layer forward.
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The product path (the
 * HIP library under mixture_experts_sparse_route_amd/) never calls it, and the
 * two share no code, header, table or constant.
 *
 * Conventions
 *   - All pointers are host pointers, row-major, caller-owned.
 *   - "bf16" tensors are raw bf16 bit patterns (uint16); they are widened to
 *     fp32 exactly, then to double.
 *   - Every floating-point reduction runs in double, in ascending index order,
 *     one accumulator per output, so results do not depend on the thread count.
 *
 * Sources (pages of the reference set, cited by title and section):
 *   [TD]  "技术日报 2026-04-14" (jsqmd.com): §2.1 MoE block, §3.1 Top-K
 *         routing (Shazeer), §3.2 Switch top-1 and capacity factor, §3.4
 *         shared experts, §3.5 sigmoid gate, §4.3 selection-only bias, §9.1
 *         MoELayer code, §9.2 AuxFreeRouter code.
 *   [BD]  "MoE稀疏架构：定义、原理与工程实践" (cloud.baidu.com): §3.2 gating
 *         network, §4 six-step forward workflow.
 *   [LN]  lnwmold.com article on GPT-4-class sparse activation: §2.2 expert
 *         FFN with W1/W2/W3, §3.2 capacity example and re-routing, §5.5 toy
 *         MoE layer.
 *   [TD]  §5.2 also gives DeepSeek-V2's affinity-ordered token dropping.
 *
 * Parity pins: every function here is pinned by the CPU test suite against
 * library routines, brute force, closed forms or the pages' worked numbers;
 * none is "parity unpinned".
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_GATE_SOFTMAX = 0, ORC_GATE_SIGMOID = 1 };

typedef struct orc_layer {
  int64_t T;        /* tokens */
  int64_t d;        /* d_model */
  int64_t F;        /* routed expert d_ff */
  int64_t E;        /* routed experts */
  int64_t K;        /* experts per token */
  int32_t gate;     /* ORC_GATE_* */
  int32_t renorm;   /* renormalise the K selected weights */
  int32_t residual; /* add x to the output (the block's residual Add) */
  int32_t bf16;     /* 1: x, expert weights and y are bf16; 0: fp32 */
  double capacity_factor; /* <= 0: no capacity limit */
  int64_t n_shared; /* always-active shared experts */
  int64_t Fs;       /* shared expert d_ff */
  /* 0 (the definition): h stays in double.  1: the SwiGLU output h is
   * stored in bf16 (rounded to nearest even) before the down projection, the
   * way a bf16 layer stores its activations; a tighter second reference for
   * kernels that do so, never the definition */
  int32_t round_h;
  /* 1: the expert weights (routed and shared) are OCP FP8 E4M3 codes, each
   * row with an fp32 scale (weight = decoded code * scale of its row); x
   * and y keep the `bf16` setting */
  int32_t w_fp8;
} orc_layer;

/* a1. logits[t][e] = fp32( sum_i x[t][i] * Wg[e][i] + logit_bias[e] )  [TD §3.1 step 1]
 * logit_bias may be NULL. */
void orc_logits(const orc_layer* L, const void* x, const float* Wg, const float* logit_bias, float* logits);

/* a2 + a3.  Gate, selection key, Top-K and weights for every token.
 *   softmax gate: key = logit; p = softmax over all E logits (double)
 *   sigmoid gate: s = fp32(sigmoid(logit)); key = fp32(s + sel_bias[e])
 *   Top-K = the K largest keys, ties to the lower expert, in key-descending order.
 *   w[t][k] = p (or s) of the chosen expert; renormalised to sum 1 if L->renorm.
 *   gap[t] = key of the K-th choice minus key of the (K+1)-th (+inf if K == E).
 * sel_bias may be NULL (treated as 0); it never enters w.  gap may be NULL. */
void orc_select(const orc_layer* L, const float* logits, const float* sel_bias, int32_t* idx, double* w,
                double* gap);

/* Per-expert capacity: floor(cf * T * K / E) when cf > 0, else -1 (no limit).  [TD §3.2] */
int64_t orc_capacity(const orc_layer* L);

/* a4.  Histogram, capacity and stable permutation of the T*K assignments
 * f = t*K + k.  pos(f) = number of earlier f' (in f order) with the same
 * expert; kept iff pos < capacity.  counts[e] = demand; offsets = exclusive
 * scan of min(counts, capacity) with offsets[E] = R; dest[f] = offsets[e] +
 * pos(f) or -1 when dropped; row_src[dest[f]] = f for kept f (entries >= R
 * are set to -1); dropped[f] = (dest[f] < 0). */
void orc_permute(const orc_layer* L, const int32_t* idx, int32_t* counts, int32_t* offsets, int32_t* dest,
                 int32_t* row_src, uint8_t* dropped);

/* The n best experts of every token (n <= E), ranked as orc_select ranks
 * them; weights normalised as orc_select normalises the first K (with
 * renorm, every rank is divided by the sum over the K selected).
 * idx, w: [T][n]. */
void orc_select_ranked(const orc_layer* L, const float* logits, const float* sel_bias, int64_t n, int32_t* idx,
                       double* w);

/* a4 with the affinity-descending drop rule [TD §5.2, DeepSeek-V2 token
 * dropping]: an expert over capacity keeps its `capacity` assignments of
 * highest affinity aff[f] (ties to the lower f) and drops the others; the
 * kept rows of each expert are in flat order.  Outputs as orc_permute. */
void orc_permute_affinity(const orc_layer* L, const int32_t* idx, const float* aff, int32_t* counts,
                          int32_t* offsets, int32_t* dest, int32_t* row_src, uint8_t* dropped);

/* a4 with overflow re-routing [LN §3.2: over-capacity tokens go to the
 * next-best expert].  First pass: the first-come rule of orc_permute
 * (counts = this pass's demand).  The j-th overflowing choice of token t (in
 * k order) is re-routed to alt_idx[t][j] (the token's rank-(K+j) expert)
 * with weight alt_w[t][j], when j < n_alt and alt_idx[t][j] >= 0; otherwise
 * it is dropped.  Second pass: re-routed assignments, in flat order, are kept
 * while their new expert has room left (capacity minus its first-pass kept
 * count).  Rows of an expert: first-pass kept, then re-routed kept, each in
 * flat order.  idx_out / w_out: the final expert and weight of every
 * assignment (the new expert and weight when re-routed). */
void orc_permute_reroute(const orc_layer* L, const int32_t* idx, const double* w, const int32_t* alt_idx,
                         const double* alt_w, int64_t n_alt, int32_t* counts, int32_t* offsets, int32_t* dest,
                         int32_t* row_src, uint8_t* dropped, int32_t* idx_out, double* w_out);

/* v rounded to the nearest bf16 value (8 significant bits, fp32 exponent
 * range), ties to even. */
double orc_bf16_round(double v);

/* The value of an OCP FP8 E4M3 code (NaN for the two NaN codes). */
double orc_fp8_e4m3(uint8_t c);

/* a6 + a7 for one row and one expert:
 *   out[m] = sum_j W2[m][j] * h_j,   h_j = SiLU(a_j) * b_j,  SiLU(z) = z / (1 + e^-z),
 *   a_j = sum_i W1[j][i] x[i],  b_j = sum_i W3[j][i] x[i].          [LN §2.2]
 * W1, W3: [F][d]; W2: [d][F]; wdt 0 fp32, 1 bf16, 2 FP8 E4M3 codes with
 * row scales s1, s3 [F] and s2 [d] (ignored otherwise); x, out in double;
 * h_j replaced by orc_bf16_round(h_j) when round_h.
 * If `threads` > 1 the output loops are split across OpenMP threads. */
void orc_swiglu(int64_t d, int64_t F, int32_t wdt, int32_t round_h, const void* W1, const void* W3,
                const void* W2, const float* s1, const float* s3, const float* s2, const double* x, double* out,
                int32_t threads);

/* a6-a9 for the listed tokens:
 *   y[j] = sum_{k ascending, dest[t][k] >= 0} w[t][k] * E_{idx[t][k]}(x_t)
 *        + sum_s Shared_s(x_t)  (+ x_t if L->residual),   t = tokens[j].
 * [TD §3.1 step 4, §3.4, §9.1; BD §4]
 * W1e/W3e/W2e: E pointers, one per expert ([F][d], [F][d], [d][F]); entries
 * for experts no listed token uses may be NULL.  Ws1/Ws3/Ws2: the shared
 * experts, [S][Fs][d], [S][Fs][d], [S][d][Fs] (NULL when n_shared == 0).
 * dest may be NULL (every assignment kept).  y: [n_tokens][d] double.
 * With L->w_fp8: S1e/S3e [F] and S2e [d] per expert, Ss1/Ss3 [S][Fs] and
 * Ss2 [S][d] are the row scales (NULL otherwise). */
void orc_forward_rows(const orc_layer* L, const void* x, const int32_t* idx, const double* w, const int32_t* dest,
                      const void* const* W1e, const void* const* W3e, const void* const* W2e, const void* Ws1,
                      const void* Ws3, const void* Ws2, const float* const* S1e, const float* const* S3e,
                      const float* const* S2e, const float* Ss1, const float* Ss3, const float* Ss2,
                      const int64_t* tokens, int64_t n_tokens, double* y);

/* a9 alone: y[t] = sum_{k ascending, dest[t][k] >= 0} w[t][k] * yp[dest[t][k]]
 *                 + shared[t]  (+ x[t] if L->residual)            [TD §3.1 step 4]
 * yp: [R][d] fp32 expert-output rows; w: [T][K] double; shared: [T][d] fp32,
 * may be NULL; y: [T][d] double. */
void orc_combine(const orc_layer* L, const float* yp, const double* w, const int32_t* dest, const float* shared,
                 const void* x, double* y);

/* Expert-choice routing [TD §3.3]: the affinity matrix is S = logits [T][E];
 * each expert e takes the `cap` tokens with the largest S[:, e] (ties to the
 * lower token), in descending-affinity order.  tok[e][c] = chosen token;
 * g[e][c] = the softmax-over-experts probability of that token for e (double;
 * the page names no combine weight, the token-choice softmax gate of §3.2 is
 * used).  Requires cap <= T. */
void orc_expert_choice(const orc_layer* L, const float* logits, int64_t cap, int32_t* tok, double* g);

/* Router statistics  [TD §4.2 auxiliary losses; §4.4 load diagnostics; §9.1].
 * Router distribution p[t][e]: softmax gate -> softmax of the logits;
 * sigmoid gate -> sigmoid scores normalised over all E experts.
 * f_e = counts_e / (T*K) (demand before capacity), P_e = mean_t p[t][e],
 * lse_t = log sum_e exp(l[t][e]).
 * out[e] = P_e (e < E), then out[E+0] = E * sum_e f_e P_e (Switch balance term
 * without alpha), out[E+1] = mean_t lse_t^2 (router z-loss),
 * out[E+2] = E * max_e f_e (load imbalance factor), out[E+3] = std(f)/mean(f)
 * (population std), out[E+4] = -sum_e P_e ln P_e, out[E+5] = -sum_e f_e ln f_e
 * (0 ln 0 = 0).  All in double. */
void orc_router_stats(const orc_layer* L, const float* logits, const int32_t* idx, double* out);

/* Number of OpenMP threads the oracle's parallel loops use. */
int32_t orc_threads(void);

#ifdef __cplusplus
}
#endif
#endif
