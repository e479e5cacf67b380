/*
 * moe.h -- C ABI of the MI355X (gfx950) sparse Mixture-of-Experts FFN layer.
 *
 * One sparsely-gated MoE FFN layer forward on one GPU, in the order the
 * pages give it:
 *   router logits -> softmax or sigmoid gate -> per-token Top-K (optionally
 *   with a per-expert capacity; overflow assignments are dropped) ->
 *   dispatch (permute tokens into expert-contiguous rows) -> each expert's
 *   SwiGLU FFN -> gate-weighted combine back to token order.
 *
 * Sources, cited by page title and section:
 *   [TD] "技术日报 2026-04-14" (jsqmd.com)
 *   [BD] "MoE稀疏架构：定义、原理与工程实践" (cloud.baidu.com)
 *   [LN] lnwmold.com article on GPT-4-class sparse activation
 *
 * General rules for every entry point
 *   - Pointers named as device pointers must be device memory of the current
 *     HIP device (or be NULL where a parameter says "nullable").  Every array
 *     is dense row-major; the caller owns all memory.  The library never
 *     allocates device memory: scratch lives in the caller's workspace
 *     (size from moe_workspace_size), 256-byte aligned.
 *   - Activation, weight, scale and output arrays (x, Wg, W*, Ws*, scales,
 *     xp, yp, shared_out, x_residual, y) must be 16-byte aligned (hipMalloc
 *     and torch allocations are); others return MOE_ERR_INVALID_ARG.  Bias
 *     and routing arrays need only their element alignment.
 *   - Configs and routing descriptors are host structs, read during the call.
 *   - All GPU work is enqueued on `stream` (NULL = the default stream) and is
 *     asynchronous.  Argument validation is synchronous, happens on the host
 *     before any launch, and returns MOE_ERR_INVALID_ARG / MOE_ERR_UNSUPPORTED /
 *     MOE_ERR_WORKSPACE without touching the GPU.  A failed launch returns
 *     MOE_ERR_HIP.  moe_last_error() gives a thread-local detail string.
 *   - The number of kept rows R is computed on the device and never read
 *     back, so no call synchronises with the host.
 *   - Calls are stateless; calls sharing a workspace must be stream-ordered.
 *   - Results are deterministic: no floating-point atomics; every reduction
 *     has a fixed order.  Behaviour on non-finite inputs is undefined.
 *   - Tile plans are chosen from the shapes.  For tuning only, and only when
 *     MOE_TUNING=1 is set in the environment, environment variables read at
 *     each call override them (MOE_GEMM_K64, MOE_GEMM_K64_DOWN, MOE_GEMM_BM,
 *     MOE_GEMM_BM_DOWN, MOE_GEMM_BNB_UP, MOE_GEMM_NS_UP, MOE_GEMM_BNB_DOWN,
 *     MOE_GEMM_NS_DOWN, MOE_GEMM_WGS, MOE_GEMM_EVEN_UP, MOE_GEMM_STREAM,
 *     MOE_GEMM_STREAM_UP, MOE_GEMM_STREAM_DOWN, MOE_GEMM_STREAM_U,
 *     MOE_GEMM_XCD_CHUNK, MOE_GEMM_XCD_CHUNK_UP, MOE_GEMM_XCD_CHUNK_DOWN,
 *     MOE_GEMM_NT_UP, MOE_GEMM_NT_DOWN, MOE_GEMM_NT_ROWS_UP,
 *     MOE_GEMM_NT_ROWS_DOWN, MOE_GATHER; MOE_ROUTER_WGS, read once); a set
 *     that names no compiled
 *     configuration is ignored.  Results do not depend on the plan: every
 *     output element sums its 32-wide MFMA k-steps in k order whatever the
 *     tile shape, tile order or kernel.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same type as hipStream_t. */
typedef struct ihipStream_t* moe_stream_t;

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1, /* a size, pointer or enum is out of range */
  MOE_ERR_UNSUPPORTED = 2, /* valid, but this library does not implement it */
  MOE_ERR_WORKSPACE = 3,   /* workspace NULL or smaller than moe_workspace_size */
  MOE_ERR_HIP = 4          /* a HIP launch or runtime call failed */
} moe_status;

/* Element types.  Router weights and logits are always fp32.
 * MOE_FP8_E4M3 (expert weights only, with bf16 activations): OCP FP8 E4M3
 * codes, one byte per weight, each weight row with an fp32 scale
 * (moe_scales): weight[row][k] = E4M3(code[row][k]) * scale[row]
 * [TD §7.4 FP8 expert GEMMs; LN §4.2 E4M3]. */
typedef enum moe_dtype { MOE_F32 = 0, MOE_BF16 = 1, MOE_FP8_E4M3 = 2 } moe_dtype;

/* Per-row fp32 scales of MOE_FP8_E4M3 expert weights (device pointers): a
 * scale per output channel, i.e. per row of W1, W3 ([E, F] each), W2
 * ([E, d]) and of the shared Ws1, Ws3 ([n_shared, d_ff_shared]) and Ws2
 * ([n_shared, d]).  Ignored for bf16 / fp32 weights (the pointer to the
 * struct may then be NULL). */
typedef struct moe_scales {
  const float* w1;
  const float* w3;
  const float* w2;
  const float* ws1;
  const float* ws3;
  const float* ws2;
} moe_scales;

/* Gate [TD §3.2 softmax; TD §3.5 sigmoid]. */
typedef enum moe_gate { MOE_GATE_SOFTMAX = 0, MOE_GATE_SIGMOID = 1 } moe_gate;

/* Which assignments an expert over capacity drops (moe_config.drop_policy;
 * only used when capacity_factor > 0). */
typedef enum moe_drop_policy {
  /* the first K_max arrivals in flat order f = t*K + k are kept [TD §3.2] */
  MOE_DROP_FIRST_COME = 0,
  /* the K_max assignments of highest affinity are kept, the rest dropped
   * in descending-affinity order [TD §5.2, DeepSeek-V2]; the affinity is
   * the assignment's gate weight topk_w, ties to the lower f */
  MOE_DROP_AFFINITY = 1,
  /* overflow goes to the token's next-best expert [LN §3.2]: after a
   * first-come pass, the j-th overflowing choice of a token (in k order) is
   * re-routed to its rank-(K+j) expert (the best ones it did not choose),
   * with that expert's gate weight normalised like the token's other
   * weights; re-routed assignments, in flat order, take what capacity their
   * new expert has left and are dropped when it is full.  Rows of an expert
   * hold its first-pass assignments, then its re-routed ones.  topk_idx /
   * topk_w then give the final expert and weight of each assignment;
   * counts stays the first-pass demand. */
  MOE_DROP_REROUTE = 2
} moe_drop_policy;

/* Flags (moe_config.flags). */
enum {
  /* Renormalise the K selected gate values to sum to 1 [TD §9.1]. */
  MOE_F_RENORM = 1u,
  /* Add x to y: the MoE block's residual Add [TD §2.1].  Dropped
   * assignments then pass x through unchanged [TD §3.2]. */
  MOE_F_RESIDUAL = 2u,
  /* moe_route / moe_forward read the caller's fp32 logits from
   * routing->logits instead of computing x . Wg. */
  MOE_F_LOGITS_IN = 4u,
  /* moe_route / moe_forward read the caller's Top-K choice from
   * routing->topk_idx and routing->topk_w and skip logits and gate. */
  MOE_F_TOPK_IN = 8u,
  /* moe_route / moe_forward also write the router statistics to
   * routing->stats (see below); not with MOE_F_TOPK_IN. */
  MOE_F_STATS = 16u,
  /* Expert-choice routing [TD §3.3]: the affinity matrix is the logits
   * S [T, E]; expert e takes the cap = min(floor(C * T * top_k / E), T)
   * tokens with the largest S[:, e] (C = capacity_factor, 1 when <= 0; ties
   * to the lower token), so each expert processes exactly cap rows and a
   * token may be taken by 0 .. E experts.  The routing arrays then have the
   * K = E form: topk_idx / topk_w / dest / row_src / dropped are [T, E],
   * entry (t, e) = expert e with weight p = the token's softmax over all E
   * logits [TD §3.2], dest = e * cap + (rank of t among the tokens e took,
   * ascending t) or -1; counts[e] = cap, offsets[e] = e * cap; every other
   * entry point then takes K = E.  Softmax gate only; not with
   * MOE_F_TOPK_IN, MOE_F_STATS or MOE_F_RENORM. */
  MOE_F_EXPERT_CHOICE = 32u,
  /* Expert weights in the packed layout that moe_pack_weights writes
   * instead of the nn.Linear row-major one, per GEMM: W1 and W3 (and the
   * shared expert's Ws1, Ws3) with MOE_F_PACKED_UP, W2 (and Ws2) with
   * MOE_F_PACKED_DOWN.  The same values, so every result is bit for bit that
   * of the row-major weights; which layout streams faster depends on the
   * GEMM's tile plan, so a caller chooses per matrix once, when it loads
   * the weights.  bf16 or E4M3 weights (MOE_ERR_UNSUPPORTED for fp32); the
   * E4M3 row scales stay [groups, N]. */
  MOE_F_PACKED_UP = 64u,
  MOE_F_PACKED_DOWN = 128u
};

/* Router statistics, written to routing->stats (E + MOE_N_STATS doubles)
 * with MOE_F_STATS [TD §4.2 auxiliary losses; TD §4.4 load diagnostics].
 * p[t][e] is the router distribution: the softmax of the logits (softmax
 * gate) or the sigmoid scores normalised over all E experts (sigmoid gate).
 * f_e = counts[e] / (T*K), the share of assignments each expert is asked to
 * take before capacity (for K = 1 the argmax fraction of the Switch loss;
 * E * f_e is DeepSeek's N'/(K'T) count).  lse_t = log sum_e exp(logit[t][e]).
 *   stats[e], e < E       P_e = (1/T) sum_t p[t][e]
 *   stats[E + BALANCE]    E * sum_e f_e P_e   (Switch / expert-balance term without alpha)
 *   stats[E + Z_LOSS]     (1/T) sum_t lse_t^2 (router z-loss)
 *   stats[E + LIF]        E * max_e f_e       (load imbalance factor, 1 = balanced)
 *   stats[E + CV]         std(f) / mean(f)    (population std; 0 = balanced)
 *   stats[E + ENTROPY_P]  -sum_e P_e ln P_e   (router entropy)
 *   stats[E + ENTROPY_F]  -sum_e f_e ln f_e   (entropy of the load)
 * Sums are taken in double in a fixed order.  Nothing is written for T = 0. */
enum {
  MOE_STAT_BALANCE = 0,
  MOE_STAT_Z_LOSS = 1,
  MOE_STAT_LIF = 2,
  MOE_STAT_CV = 3,
  MOE_STAT_ENTROPY_P = 4,
  MOE_STAT_ENTROPY_F = 5,
  MOE_N_STATS = 6
};

/* Layer description.  T = tokens, d = d_model, F = d_ff, E = n_experts,
 * K = top_k. */
typedef struct moe_config {
  int64_t tokens;          /* T >= 0; T == 0 makes every call a no-op */
  int64_t d_model;         /* d >= 1; bf16: multiple of 64 */
  int64_t d_ff;            /* F >= 1; bf16: multiple of 64 */
  int64_t n_experts;       /* 1 <= E <= 1024 */
  int64_t top_k;           /* 1 <= K <= min(E, 32) */
  int32_t gate;            /* moe_gate */
  uint32_t flags;          /* MOE_F_* */
  /* Capacity factor C [TD §3.2].  C > 0: each expert keeps at most
   * K_max = floor(C * T * K / E) assignments (T*K counts (token, choice)
   * pairs, which is T for top-1); drop_policy says which are kept (by
   * default the first K_max in flat order f = t*K + k).  C <= 0: no limit. */
  double capacity_factor;
  int64_t n_shared;        /* always-active shared experts, 0 or 1 [TD §3.4] */
  int64_t d_ff_shared;     /* shared expert d_ff; bf16: multiple of 64 */
  int32_t act_dtype;       /* moe_dtype of x and the expert activations (xp, h) */
  int32_t w_dtype;         /* moe_dtype of the expert weights: act_dtype, or MOE_FP8_E4M3 with bf16 act_dtype */
  /* moe_dtype of y: act_dtype, or MOE_F32 for a bf16 layer (the fp32 sum
   * before its final rounding; the bf16 output is exactly its
   * round-to-nearest-even image). */
  int32_t out_dtype;
  int32_t drop_policy;     /* moe_drop_policy; MOE_DROP_REROUTE needs the logits (not MOE_F_TOPK_IN) */
} moe_config;

/* Routing arrays, all DEVICE pointers.  Sizes are in elements. */
typedef struct moe_routing {
  float* logits;     /* [T, E]  fp32 router logits (input with MOE_F_LOGITS_IN) */
  int32_t* topk_idx; /* [T, K]  chosen experts, key-descending, ties to the lower index */
  float* topk_w;     /* [T, K]  gate weights of the chosen experts */
  int32_t* counts;   /* [E]     assignments per expert before capacity (demand) */
  int32_t* offsets;  /* [E+1]   exclusive scan of kept counts; offsets[E] = R */
  int32_t* dest;     /* [T*K]   row of assignment f = t*K + k in xp / yp, or -1 if dropped */
  int32_t* row_src;  /* [T*K]   assignment f held by row r (r < R); rows >= R are not written */
  uint8_t* dropped;  /* [T*K]   1 if assignment f was dropped for capacity */
  double* stats;     /* [E + MOE_N_STATS] router statistics; used only with MOE_F_STATS */
} moe_routing;

/* Bytes of workspace any entry point needs for `cfg` (the same figure is
 * enough for all of them).  Host only. */
moe_status moe_workspace_size(const moe_config* cfg, size_t* bytes);

/* Upper bound of the kept-row count R for `cfg`: min(T*K, E*K_max), or T*K
 * without capacity.  Host only; size xp / yp with it. */
moe_status moe_max_rows(const moe_config* cfg, int64_t* rows);

/* a1-a4: router logits, gate, Top-K and weights, per-expert histogram,
 * capacity and stable permutation.
 *   logits[t][e] = x[t] . Wg[e] (+ logit_bias[e])                  [TD §3.1]
 *   softmax gate: key = logit; p = softmax over all E logits        [TD §3.2]
 *   sigmoid gate: s = sigmoid(logit) (fp32); key = s + sel_bias[e]  [TD §3.5, §4.3]
 *   topk_idx = the K largest keys, ties to the lower expert index (keys are
 *   compared as IEEE values, -0 equal to +0), in key-descending order;
 *   topk_w = p (or s) of each choice, divided by their sum with MOE_F_RENORM.
 *   counts / offsets / dest / row_src / dropped as described in moe_routing,
 *   with the capacity rule of cfg->drop_policy.          [TD §3.2, §5.2; LN §3.2]
 * x:          device, [T, d] act_dtype
 * Wg:         device, [E, d] fp32 (unused with MOE_F_LOGITS_IN / MOE_F_TOPK_IN)
 * logit_bias: device, [E] fp32, nullable; added to the logits (enters both
 *             selection and weights)
 * sel_bias:   device, [E] fp32, nullable; sigmoid gate only; enters the
 *             selection key, never the weights
 * r:          every pointer required (r->stats only with MOE_F_STATS).  With
 *             MOE_F_TOPK_IN, r->logits is not touched and topk_idx / topk_w
 *             are inputs (idx in [0, E), distinct per token, not checked on
 *             the device).
 */
moe_status moe_route(const moe_config* cfg, const void* x, const float* Wg, const float* logit_bias,
                     const float* sel_bias, const moe_routing* r, void* ws, size_t ws_bytes, moe_stream_t stream);

/* a5: dispatch.  xp[row][:] = x[row_src[row] / K][:] for every kept row
 * (R = offsets[E] rows, read on the device) [BD §4 step 3; TD §9.1].
 * x: device [T, d]; xp: device [max_rows, d], act_dtype.  Uses r->row_src and
 * r->offsets only. */
moe_status moe_dispatch(const moe_config* cfg, const void* x, const moe_routing* r, void* xp, moe_stream_t stream);

/* a6-a7: grouped SwiGLU experts [LN §2.2]. For each group g < n_groups, rows
 * offsets[g] .. offsets[g+1]-1 of xp go through expert g:
 *   yp[row] = W2[g] . ( SiLU(W1[g] . xp[row]) * (W3[g] . xp[row]) ),  SiLU(z) = z / (1 + e^-z)
 * xp:      device [max_rows, d] act_dtype
 * offsets: device [n_groups + 1] int32, offsets[0] = 0, non-decreasing,
 *          offsets[n_groups] <= max_rows (not checked on the device)
 * W1, W3:  device [n_groups, F, d] w_dtype (nn.Linear out x in layout)
 * W2:      device [n_groups, d, F] w_dtype
 * scales:  host struct of device pointers; required (w1, w3, w2) for
 *          MOE_FP8_E4M3 weights, else nullable
 * yp:      device [max_rows, d] fp32
 * The intermediate h = SiLU(.) * (.) is kept in act_dtype in the workspace.
 * max_rows: host upper bound on offsets[n_groups], at most moe_max_rows(cfg);
 * 1 <= n_groups <= n_experts. */
moe_status moe_expert_ffn(const moe_config* cfg, const void* xp, const int32_t* offsets, int64_t n_groups,
                          int64_t max_rows, const void* W1, const void* W3, const void* W2, const moe_scales* scales,
                          float* yp, void* ws, size_t ws_bytes, moe_stream_t stream);

/* Weight packing, done once when a layer's weights are loaded (not part of
 * the forward).  The expert GEMMs [LN §2.2; TD §7.4] reduce every weight row
 * along its length (d for W1 / W3, F for W2) in steps of 64 elements, and a
 * workgroup reads one step of 64-row blocks of rows at a time; in the
 * row-major layout those are 128-byte pieces of rows 2 d or 2 F bytes apart.
 * The packed layout cuts each group's rows into panels of 64 rows and stores
 * a panel's 64-element steps one after the other, each as one run of
 * 64 x 64 elements (8 KB of bf16, 4 KB of E4M3):
 *   src: device [groups, N, K] row-major (nn.Linear out x in), elements of
 *        w_dtype (MOE_BF16 or MOE_FP8_E4M3)
 *   dst: device [groups, N/64, K/64, 64, 64], same elements: element
 *        (g, n, k) of src at
 *        dst[(((g * (N/64) + n/64) * (K/64) + k/64) * 64 + n % 64) * 64 + k % 64]
 * W1 / W3 are packed with (N, K) = (F, d) and W2 with (d, F) (the shared
 * expert's likewise with Fs); the result is then passed with
 * MOE_F_PACKED_UP / MOE_F_PACKED_DOWN.  groups >= 1; N and K positive multiples of 64 (as
 * every bf16 layer's d, F and Fs are); src and dst 16-byte aligned and not
 * overlapping, owned by the caller.  Enqueued on `stream`;
 * MOE_ERR_INVALID_ARG on a bad size or pointer, before any launch. */
moe_status moe_pack_weights(const void* src, void* dst, int64_t groups, int64_t N, int64_t K, int32_t w_dtype,
                            moe_stream_t stream);

/* a9: weighted combine [TD §3.1 step 4; BD §4 step 5]:
 *   y[t] = sum_{k ascending, dest[t*K+k] >= 0} topk_w[t][k] * yp[dest[t*K+k]]
 *          + shared_out[t] + (x[t] if MOE_F_RESIDUAL)
 * accumulated in fp32 in that order and rounded once to out_dtype.
 * yp: device [max_rows, d] fp32; shared_out: device [T, d] fp32, nullable;
 * x_residual: device [T, d] act_dtype, required iff MOE_F_RESIDUAL;
 * y: device [T, d] out_dtype.  Uses r->topk_w and r->dest. */
moe_status moe_combine(const moe_config* cfg, const float* yp, const moe_routing* r, const float* shared_out,
                       const void* x_residual, void* y, moe_stream_t stream);

/* The whole layer: moe_route, moe_dispatch, moe_expert_ffn, the shared
 * expert (a SwiGLU over all T rows with Ws1, Ws3 [1, Fs, d], Ws2 [1, d, Fs],
 * added unweighted [TD §3.4, §9.1]) and moe_combine, in one stream-ordered
 * sequence with no host synchronisation.  With a shared expert, and `stream`
 * on the current device, the shared expert runs on a second stream of that
 * device that the library creates once (default priority) and orders with
 * `stream` through events: it starts after the work enqueued on `stream`
 * before the call, and the combine waits for it, so the call keeps plain
 * stream semantics.
 * r: nullable; when NULL the routing arrays live in the workspace.  When
 * given, the routing results are written there (and MOE_F_LOGITS_IN /
 * MOE_F_TOPK_IN inputs read from there).  Required with MOE_F_*_IN and
 * MOE_F_STATS.
 * Ws1/Ws3/Ws2: required iff n_shared == 1.  scales: as for moe_expert_ffn,
 * plus ws1, ws3, ws2 when n_shared == 1.  y: device [T, d] out_dtype. */
moe_status moe_forward(const moe_config* cfg, const void* x, const float* Wg, const float* logit_bias,
                       const float* sel_bias, const void* W1, const void* W3, const void* W2, const void* Ws1,
                       const void* Ws3, const void* Ws2, const moe_scales* scales, void* y, const moe_routing* r,
                       void* ws, size_t ws_bytes, moe_stream_t stream);

/* ---- The same forward without any allocation -----------------------------
 * For callers that cannot allocate device memory or create streams or events
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * it): moe_forward with the same arguments and results, minus the workspace.
 * Its scratch is a built-in device array of MOE_NOALLOC_SCRATCH_BYTES per
 * GPU (held from the library's load on that GPU until the process ends); a
 * layer whose moe_workspace_size exceeds it returns MOE_ERR_WORKSPACE before
 * any launch.  The call allocates nothing (no hipMalloc / hipFree, no stream
 * or event creation): the shared expert runs in order on `stream`, and the
 * per-kernel timing facility is not applied.  `stream` must belong to the
 * current device (else MOE_ERR_INVALID_ARG).  Every call on one GPU uses that
 * GPU's one array and leaves its contents behind (no part of it needs to
 * start at zero): calls that overlap on one GPU -- on different streams
 * without ordering, or from different threads -- race and corrupt each
 * other's results; order them on one stream. */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
moe_status moe_forward_noalloc(const moe_config* cfg, const void* x, const float* Wg, const float* logit_bias,
                               const float* sel_bias, const void* W1, const void* W3, const void* W2, const void* Ws1,
                               const void* Ws3, const void* Ws2, const moe_scales* scales, void* y,
                               const moe_routing* r, moe_stream_t stream);

/* Static string for a status code. */
const char* moe_status_string(moe_status s);

/* Detail of the calling thread's last failed call ("" if none). */
const char* moe_last_error(void);

/* ---- Per-kernel timing (diagnostics) --------------------------------------
 * When enabled for a kernel (bit `kernel_id` of `kernel_mask`), every launch
 * of that kernel is bracketed by a pair of HIP events recorded on the launch
 * stream.  moe_profile_read synchronises on the recorded events and returns
 * the summed duration in milliseconds and the launch count since the last
 * reset.  kernel_mask = 0 turns timing off.  Not thread-safe across
 * concurrent callers; intended for benchmarks. */
moe_status moe_profile_enable(uint32_t kernel_mask);
moe_status moe_profile_reset(void);
moe_status moe_profile_read(int kernel_id, double* total_ms, int64_t* launches);
/* Name of kernel id `kernel_id` (NULL past the last id). */
const char* moe_kernel_name(int kernel_id);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
