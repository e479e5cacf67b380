// C-ABI layer of the MoE layer: argument validation (host only, before any
// HIP call), workspace layout, and the stream-ordered launch sequence.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdlib>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <initializer_list>
#include <mutex>
#include <string>
#include <vector>

#include "api_internal.h"
#include "internal.h"
#include "moe.h"

namespace moe {
namespace {

thread_local std::string g_err;

moe_status fail(moe_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

moe_status hip_fail(hipError_t e, const char* where) {
  return fail(MOE_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

#define MOE_HIP(call)                                       \
  do {                                                      \
    hipError_t e_ = (call);                                 \
    if (e_ != hipSuccess) return hip_fail(e_, #call);      \
  } while (0)

constexpr uint32_t kKnownFlags =
    MOE_F_RENORM | MOE_F_RESIDUAL | MOE_F_LOGITS_IN | MOE_F_TOPK_IN | MOE_F_STATS | MOE_F_EXPERT_CHOICE |
    MOE_F_PACKED_UP | MOE_F_PACKED_DOWN;

// Everything the launches need, derived from a validated config.
struct Shape {
  bool bf16;
  bool out_bf16;
  bool stats;  // router statistics requested
  bool w8;     // expert weights are E4M3 bytes with per-row scales
  bool packed_up, packed_down;  // W1 / W3 and W2 in the packed layout (moe_pack_weights)
  int policy;  // moe_drop_policy in effect (first-come when there is no capacity)
  int64_t K2;  // re-routing alternates per token
  bool ec;     // expert-choice routing: K is E (the K = E form), cap the tokens per expert
  int64_t T, d, F, E, K, S, Fs;
  int64_t cap;       // -1: no limit
  int64_t max_rows;  // upper bound of kept rows R
  int64_t n_chunks;  // router_topk workgroups / histogram chunks
  size_t esz;
  // moe_forward: one assignment per token and no shared expert (bf16): the
  // routed rows are copied into a k-blocked xp and GEMM2 writes y itself;
  // other bf16 layers read the routed rows from a k-blocked copy of x
  // through the routing (no per-row copy)
  bool fused;
};

moe_status validate(const moe_config* c, Shape* sh) {
  if (!c) return fail(MOE_ERR_INVALID_ARG, "config is NULL");
  if (c->tokens < 0) return fail(MOE_ERR_INVALID_ARG, "tokens = %lld < 0", (long long)c->tokens);
  if (c->d_model < 1 || c->d_ff < 1) return fail(MOE_ERR_INVALID_ARG, "d_model and d_ff must be >= 1");
  if (c->n_experts < 1 || c->n_experts > 1024)
    return fail(MOE_ERR_INVALID_ARG, "n_experts = %lld outside [1, 1024]", (long long)c->n_experts);
  if (c->top_k < 1 || c->top_k > c->n_experts || c->top_k > 32)
    return fail(MOE_ERR_INVALID_ARG, "top_k = %lld outside [1, min(n_experts, 32)]", (long long)c->top_k);
  if (c->gate != MOE_GATE_SOFTMAX && c->gate != MOE_GATE_SIGMOID)
    return fail(MOE_ERR_INVALID_ARG, "unknown gate %d", (int)c->gate);
  if (c->flags & ~kKnownFlags) return fail(MOE_ERR_INVALID_ARG, "unknown flag bits 0x%x", c->flags & ~kKnownFlags);
  if ((c->flags & MOE_F_STATS) && (c->flags & MOE_F_TOPK_IN))
    return fail(MOE_ERR_INVALID_ARG, "MOE_F_STATS needs logits; it cannot be combined with MOE_F_TOPK_IN");
  if (c->drop_policy < MOE_DROP_FIRST_COME || c->drop_policy > MOE_DROP_REROUTE)
    return fail(MOE_ERR_INVALID_ARG, "unknown drop_policy %d", (int)c->drop_policy);
  if (c->drop_policy == MOE_DROP_REROUTE && (c->flags & MOE_F_TOPK_IN))
    return fail(MOE_ERR_INVALID_ARG, "MOE_DROP_REROUTE ranks experts from the logits; not with MOE_F_TOPK_IN");
  const bool ec = c->flags & MOE_F_EXPERT_CHOICE;
  if (ec && (c->flags & (MOE_F_TOPK_IN | MOE_F_STATS | MOE_F_RENORM)))
    return fail(MOE_ERR_INVALID_ARG, "MOE_F_EXPERT_CHOICE excludes MOE_F_TOPK_IN, MOE_F_STATS and MOE_F_RENORM");
  if (ec && c->gate != MOE_GATE_SOFTMAX)
    return fail(MOE_ERR_UNSUPPORTED, "expert-choice routing is implemented for the softmax gate");
  if (!std::isfinite(c->capacity_factor)) return fail(MOE_ERR_INVALID_ARG, "capacity_factor is not finite");
  if (c->n_shared < 0 || c->n_shared > 1) return fail(MOE_ERR_INVALID_ARG, "n_shared must be 0 or 1");
  if (c->n_shared == 1 && c->d_ff_shared < 1) return fail(MOE_ERR_INVALID_ARG, "d_ff_shared must be >= 1");
  if (c->act_dtype != MOE_F32 && c->act_dtype != MOE_BF16)
    return fail(MOE_ERR_INVALID_ARG, "unknown act_dtype %d", (int)c->act_dtype);
  if (c->w_dtype != MOE_F32 && c->w_dtype != MOE_BF16 && c->w_dtype != MOE_FP8_E4M3)
    return fail(MOE_ERR_INVALID_ARG, "unknown w_dtype %d", (int)c->w_dtype);
  if (c->w_dtype == MOE_FP8_E4M3 ? c->act_dtype != MOE_BF16 : c->w_dtype != c->act_dtype)
    return fail(MOE_ERR_UNSUPPORTED, "w_dtype must equal act_dtype, or be MOE_FP8_E4M3 with bf16 activations");
  if (c->out_dtype != MOE_F32 && c->out_dtype != MOE_BF16)
    return fail(MOE_ERR_INVALID_ARG, "unknown out_dtype %d", (int)c->out_dtype);
  if (c->act_dtype == MOE_F32 && c->out_dtype != MOE_F32)
    return fail(MOE_ERR_UNSUPPORTED, "an fp32 layer has an fp32 output");
  if ((c->flags & (MOE_F_PACKED_UP | MOE_F_PACKED_DOWN)) && c->w_dtype == MOE_F32)
    return fail(MOE_ERR_UNSUPPORTED, "packed weights (MOE_F_PACKED_UP / _DOWN) are bf16 or E4M3");
  const bool bf16 = c->act_dtype == MOE_BF16;
  if (bf16) {
    if (c->d_model % 64 || c->d_ff % 64 || (c->n_shared && c->d_ff_shared % 64))
      return fail(MOE_ERR_UNSUPPORTED, "bf16 needs d_model, d_ff and d_ff_shared to be multiples of 64");
  }
  const int64_t T = c->tokens, d = c->d_model, F = c->d_ff, E = c->n_experts;
  const int64_t K = ec ? c->n_experts : c->top_k;  // expert choice: the K = E form
  const int64_t Fs = c->n_shared ? c->d_ff_shared : 0;
  if (T > (int64_t)INT32_MAX / K) return fail(MOE_ERR_UNSUPPORTED, "tokens * top_k exceeds 2^31 - 1");
  if (T > (int64_t)INT32_MAX / E) return fail(MOE_ERR_UNSUPPORTED, "tokens * n_experts exceeds 2^31 - 1");
  if (F > (int64_t)INT32_MAX / d || Fs > (int64_t)INT32_MAX / d)
    return fail(MOE_ERR_UNSUPPORTED, "d_ff * d_model exceeds 2^31 - 1");
  int64_t cap = -1;
  if (ec) {
    // tokens per expert: floor(C * T * top_k / E), C = 1 when not given, at most T
    const double C = c->capacity_factor > 0.0 ? c->capacity_factor : 1.0;
    const double v = std::floor(C * (double)(T * c->top_k) / (double)E);
    cap = v > (double)T ? T : (int64_t)v;
  } else if (c->capacity_factor > 0.0) {
    // K_max = floor(C * N_tokens / N_experts) with N_tokens = T * K assignments
    const double v = std::floor(c->capacity_factor * (double)(T * K) / (double)E);
    cap = v > (double)(T * K) ? T * K : (int64_t)v;
  }
  sh->bf16 = bf16;
  sh->out_bf16 = c->out_dtype == MOE_BF16;
  sh->stats = c->flags & MOE_F_STATS;
  sh->w8 = c->w_dtype == MOE_FP8_E4M3;
  sh->packed_up = c->flags & MOE_F_PACKED_UP;
  sh->packed_down = c->flags & MOE_F_PACKED_DOWN;
  sh->policy = cap >= 0 ? c->drop_policy : MOE_DROP_FIRST_COME;
  sh->K2 = sh->policy == MOE_DROP_REROUTE ? std::min(K, E - K) : 0;
  sh->T = T;
  sh->d = d;
  sh->F = F;
  sh->E = E;
  sh->K = K;
  sh->S = c->n_shared;
  sh->Fs = Fs;
  sh->cap = cap;
  sh->max_rows = cap >= 0 ? std::min(T * K, E * cap) : T * K;
  sh->ec = ec;
  sh->n_chunks = (T + chunk_tokens(E, K) - 1) / chunk_tokens(E, K);
  sh->esz = bf16 ? 2 : 4;
  sh->fused = bf16 && K == 1 && c->n_shared == 0 && !ec;
  return MOE_OK;
}

// ---- workspace layout ----
struct Layout {
  size_t router_part, blk_count, blk_base, blk_P, blk_z, dem_off, seg, alt_idx, alt_w, pos1, cand, cand_w,
      blk_count2, blk_base2, counts2, tab_up, tab_down, counts, sh_range, sh_tab_up, sh_tab_down, sh_counts;
  size_t h, xp, xkb, yp, sh_h, sh_out;
  size_t r_logits, r_idx, r_w, r_counts, r_offsets, r_dest, r_row_src, r_dropped;
  size_t total;
};

Layout layout(const Shape& s) {
  Layout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += (bytes + 255) / 256 * 256;
    return at;
  };
  const size_t TK = (size_t)(s.T * s.K);
  const int S = router_splits(s.T, s.d, s.E, s.bf16);
  L.router_part = take(S > 1 ? (size_t)S * s.T * s.E * 4 : 0);
  L.blk_count = take((size_t)(s.n_chunks * s.E) * 4);
  L.blk_base = take((size_t)(s.n_chunks * s.E) * 4);
  L.blk_P = take(s.stats ? (size_t)(s.n_chunks * s.E) * 4 : 0);
  L.blk_z = take(s.stats ? (size_t)s.n_chunks * 4 : 0);
  const bool aff = s.policy == MOE_DROP_AFFINITY, rr = s.policy == MOE_DROP_REROUTE;
  L.dem_off = take(aff ? (size_t)(s.E + 1) * 4 : 0);
  L.seg = take(aff || s.ec ? TK * 8 : 0);
  L.alt_idx = take(rr ? (size_t)(s.T * s.K2) * 4 : 0);
  L.alt_w = take(rr ? (size_t)(s.T * s.K2) * 4 : 0);
  L.pos1 = take(rr ? TK * 4 : 0);
  L.cand = take(rr ? TK * 4 : 0);
  L.cand_w = take(rr ? TK * 4 : 0);
  L.blk_count2 = take(rr ? (size_t)(s.n_chunks * s.E) * 4 : 0);
  L.blk_base2 = take(rr ? (size_t)(s.n_chunks * s.E) * 4 : 0);
  L.counts2 = take(rr ? (size_t)s.E * 4 : 0);
  L.tab_up = take((size_t)ffn_table_entries(s.bf16, s.max_rows, s.E, s.F, true) * 16);
  L.tab_down = take((size_t)ffn_table_entries(s.bf16, s.max_rows, s.E, s.d, false) * 16);
  L.counts = take(2 * 4);
  L.sh_range = take(2 * 4);
  L.sh_tab_up = take(s.S ? (size_t)ffn_table_entries(s.bf16, s.T, 1, s.Fs, true) * 16 : 0);
  L.sh_tab_down = take(s.S ? (size_t)ffn_table_entries(s.bf16, s.T, 1, s.d, false) * 16 : 0);
  L.sh_counts = take(2 * 4);
  L.h = take((size_t)s.max_rows * s.F * s.esz);
  // xp: the routed rows (fp32 layers row-major; bf16 k-blocked: the fused
  // path, or the dispatch when the gather is turned off for tuning); xkb: x
  // k-blocked [d/kbw][T][kbw] (the other bf16 layers)
  L.xp = take((size_t)s.max_rows * s.d * s.esz);
  L.xkb = take(s.bf16 && !s.fused ? (size_t)s.T * s.d * s.esz : 0);
  L.yp = take((size_t)s.max_rows * s.d * 4);
  L.sh_h = take((size_t)(s.S ? s.T * s.Fs : 0) * s.esz);
  L.sh_out = take((size_t)(s.S ? s.T * s.d : 0) * 4);
  L.r_logits = take((size_t)(s.T * s.E) * 4);
  L.r_idx = take(TK * 4);
  L.r_w = take(TK * 4);
  L.r_counts = take((size_t)s.E * 4);
  L.r_offsets = take((size_t)(s.E + 1) * 4);
  L.r_dest = take(TK * 4);
  L.r_row_src = take(TK * 4);
  L.r_dropped = take(TK);
  L.total = off;
  return L;
}

moe_status check_ws(const Shape& s, const void* ws, size_t ws_bytes, Layout* L) {
  *L = layout(s);
  if (!ws) return fail(MOE_ERR_WORKSPACE, "workspace is NULL");
  if ((uintptr_t)ws % 256) return fail(MOE_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (ws_bytes < L->total)
    return fail(MOE_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, L->total);
  return MOE_OK;
}

// Activation, weight, scale and output arrays are read and written with
// 16-byte vector accesses.
moe_status check_aligned(std::initializer_list<const void*> ptrs) {
  for (const void* q : ptrs)
    if ((uintptr_t)q % 16) return fail(MOE_ERR_INVALID_ARG, "activation, weight, scale and output arrays must be 16-byte aligned");
  return MOE_OK;
}

template <typename T>
T* at(void* ws, size_t off) {
  return (T*)((char*)ws + off);
}

moe_status check_routing(const moe_routing* r, bool need_logits, bool need_stats) {
  if (!r) return fail(MOE_ERR_INVALID_ARG, "routing is NULL");
  if ((need_logits && !r->logits) || !r->topk_idx || !r->topk_w || !r->counts || !r->offsets || !r->dest ||
      !r->row_src || !r->dropped)
    return fail(MOE_ERR_INVALID_ARG, "a routing pointer is NULL");
  if (need_stats && !r->stats) return fail(MOE_ERR_INVALID_ARG, "MOE_F_STATS needs routing->stats");
  return MOE_OK;
}

// a1-a4 on a validated shape.
// drop_y non-null (first-come drops, one assignment per token, no shared
// expert): the scatter also writes the dropped tokens' output rows (x or 0
// when drop_x is null) and *drop_done says it did.
// disp_xp non-null (same layers, bf16): the scatter also copies the kept
// tokens' rows of x to the k-blocked xp (disp_rows rows per k-block), the
// dispatch's work, under the same *drop_done.  tiles non-null: the scatter
// that runs on the final offsets also writes those GEMM tile tables, and
// *tiles_done says whether it did (expert-choice routing has no scatter).
moe_status do_route(const moe_config* c, const Shape& s, const Layout& L, const void* x, const float* Wg,
                    const float* logit_bias, const float* sel_bias, const moe_routing& r, void* ws, hipStream_t st,
                    void* drop_y = nullptr, const void* drop_x = nullptr, bool* drop_done = nullptr,
                    void* disp_xp = nullptr, int64_t disp_rows = 0, const TileJob* tiles = nullptr,
                    bool* tiles_done = nullptr) {
  if (drop_done) *drop_done = false;
  if (tiles_done) *tiles_done = false;
  int32_t* blk_count = at<int32_t>(ws, L.blk_count);
  int32_t* blk_base = at<int32_t>(ws, L.blk_base);
  const bool topk_in = c->flags & MOE_F_TOPK_IN;
  const float* sb = c->gate == MOE_GATE_SIGMOID ? sel_bias : nullptr;
  float* blk_P = s.stats ? at<float>(ws, L.blk_P) : nullptr;
  float* blk_z = s.stats ? at<float>(ws, L.blk_z) : nullptr;
  const bool rr = s.policy == MOE_DROP_REROUTE, aff = s.policy == MOE_DROP_AFFINITY;
  int32_t* alt_idx = rr ? at<int32_t>(ws, L.alt_idx) : nullptr;
  float* alt_w = rr ? at<float>(ws, L.alt_w) : nullptr;
  if (s.ec) {
    int S = 1;
    float* part = at<float>(ws, L.router_part);
    if (!(c->flags & MOE_F_LOGITS_IN)) {
      S = router_splits(s.T, s.d, s.E, s.bf16);
      MOE_HIP(launch_router_logits(s.bf16, x, Wg, logit_bias, r.logits, part, s.T, s.d, s.E, st));
    }
    MOE_HIP(launch_expert_choice(r.logits, part, S, logit_bias, r.topk_idx, r.topk_w, at<uint64_t>(ws, L.seg),
                                 r.counts, r.offsets, r.dest, r.row_src, r.dropped, s.T, s.E, s.cap, st));
    return MOE_OK;
  }
  if (!topk_in) {
    int S = 1;
    float* part = at<float>(ws, L.router_part);
    if (!(c->flags & MOE_F_LOGITS_IN)) {
      S = router_splits(s.T, s.d, s.E, s.bf16);
      MOE_HIP(launch_router_logits(s.bf16, x, Wg, logit_bias, r.logits, part, s.T, s.d, s.E, st));
    }
    MOE_HIP(launch_router_topk(r.logits, part, S, logit_bias, sb, r.topk_idx, r.topk_w, blk_count, blk_P, blk_z,
                               alt_idx, alt_w, s.K2, s.T, s.E, s.K, c->gate, c->flags & MOE_F_RENORM, false, st));
  } else {
    MOE_HIP(launch_router_topk(nullptr, nullptr, 1, nullptr, nullptr, r.topk_idx, nullptr, blk_count, nullptr,
                               nullptr, nullptr, nullptr, 0, s.T, s.E, s.K, c->gate, false, true, st));
  }
  int32_t* dem_off = aff ? at<int32_t>(ws, L.dem_off) : nullptr;
  // one chunk with first-come drops and no statistics (decode-sized batches):
  // the scatter does the capacity scan itself, one launch fewer
  const bool one = s.n_chunks == 1 && !aff && !rr && !s.stats;
  if (!one)
    MOE_HIP(launch_route_scan(blk_count, blk_base, r.counts, r.offsets, s.n_chunks, s.E, s.cap, blk_P, blk_z,
                              s.stats ? r.stats : nullptr, s.T, s.K, nullptr, dem_off, st));
  RouteScatter sc{};
  sc.idx = r.topk_idx;
  sc.blk_base = blk_base;
  sc.offsets = r.offsets;
  sc.dest = r.dest;
  sc.row_src = r.row_src;
  sc.dropped = r.dropped;
  if (aff) {
    uint64_t* seg = at<uint64_t>(ws, L.seg);
    sc.mode = kAffinity;
    if (tiles) sc.tiles = *tiles;
    sc.counts = r.counts;
    sc.dem_off = dem_off;
    sc.aff = r.topk_w;
    sc.seg = seg;
    MOE_HIP(launch_route_scatter(sc, s.T, s.K, s.E, s.cap, st));
    MOE_HIP(launch_route_affinity(seg, r.counts, dem_off, r.offsets, r.dest, r.row_src, r.dropped, s.E, s.cap, st));
  } else if (rr) {
    int32_t* blk_count2 = at<int32_t>(ws, L.blk_count2);
    int32_t* blk_base2 = at<int32_t>(ws, L.blk_base2);
    sc.mode = kReroute1;
    sc.alt_idx = alt_idx;
    sc.alt_w = alt_w;
    sc.K2 = (int)s.K2;
    sc.pos1 = at<int32_t>(ws, L.pos1);
    sc.cand = at<int32_t>(ws, L.cand);
    sc.cand_w = at<float>(ws, L.cand_w);
    sc.blk_count2 = blk_count2;
    MOE_HIP(launch_route_scatter(sc, s.T, s.K, s.E, s.cap, st));
    // second pass: final offsets from the first-pass kept and the candidates that fit
    MOE_HIP(launch_route_scan(blk_count2, blk_base2, at<int32_t>(ws, L.counts2), r.offsets, s.n_chunks, s.E, s.cap,
                              nullptr, nullptr, nullptr, s.T, s.K, r.counts, nullptr, st));
    sc.mode = kReroute2;
    if (tiles) sc.tiles = *tiles;
    sc.idx = sc.cand;
    sc.blk_base = blk_base2;
    sc.first_counts = r.counts;
    sc.topk_idx = r.topk_idx;
    sc.topk_w = r.topk_w;
    MOE_HIP(launch_route_scatter(sc, s.T, s.K, s.E, s.cap, st));
  } else {
    sc.mode = kFirstCome;
    if (tiles) sc.tiles = *tiles;
    if (one) {
      sc.one_count = blk_count;
      sc.one_counts = r.counts;
      sc.one_offsets = r.offsets;
    }
    if (drop_y && s.K == 1 && s.S == 0 && s.bf16 && s.d % 8 == 0) {
      sc.drop_y = drop_y;
      sc.drop_x = (const uint16_t*)drop_x;
      sc.drop_y_bf16 = s.out_bf16;
      sc.drop_d = (int)s.d;
      if (disp_xp) {
        sc.disp_xp = (uint4*)disp_xp;
        sc.disp_x = (const uint4*)x;
        sc.disp_n_kb = (int)(s.d / 32);
        sc.disp_blk_rows = disp_rows;
      }
    }
    MOE_HIP(launch_route_scatter(sc, s.T, s.K, s.E, s.cap, st));
    if (drop_done) *drop_done = sc.drop_y != nullptr;
  }
  if (tiles_done) *tiles_done = tiles != nullptr;
  return MOE_OK;
}

// The GEMM plan of an FFN of the layer, with its weights' layout.
FfnPlan plan_of(const Shape& s, int64_t max_rows, int64_t group_max, int64_t n_groups, int64_t F) {
  FfnPlan p = ffn_plan(s.bf16, s.w8, max_rows, group_max, n_groups, F, s.d, s.packed_up, s.packed_down);
  p.packed_up = s.packed_up;
  p.packed_down = s.packed_down;
  return p;
}

// s1 / s3 / s2: row scales of E4M3 weights (s.w8), else unused.
// group_max: bound of any group's rows; A: GEMM1's A operand (fp32 layers:
// row-major A.ptr).  plan_in: the plan (else computed here); tiles_ready:
// its tile tables are already written (by the routing scatter).
moe_status do_ffn(const Shape& s, const AOperand& A, const int32_t* offsets, int64_t n_groups,
                  int64_t max_rows, int64_t group_max,
                  const void* W1, const void* W3, const void* W2, const float* s1, const float* s3, const float* s2,
                  void* h, float* yp, int4* tab_up, int4* tab_down, int32_t* counts, int64_t F, hipStream_t st,
                  const CombineFuse* fuse = nullptr, const FfnPlan* plan_in = nullptr, bool tiles_ready = false,
                  bool shared = false) {
  const FfnPlan plan = plan_in ? *plan_in : plan_of(s, max_rows, group_max, n_groups, F);
  if (!tiles_ready && !(s.bf16 && plan.stream_up && plan.stream_down))
    MOE_HIP(launch_ffn_tiles(plan, offsets, n_groups, max_rows, F, s.d, tab_up, tab_down, counts, st));
  MOE_HIP(launch_gemm_gate_up(s.bf16, plan, A, tab_up, counts, offsets, n_groups, max_rows, W1, W3, s1, s3, h, F, s.d,
                              st, shared ? K_SHARED_GATE_UP : K_GEMM_GATE_UP));
  MOE_HIP(launch_gemm_down(s.bf16, plan, h, tab_down, counts + 1, offsets, n_groups, max_rows, W2, s2, yp, fuse, F,
                           s.d, st, shared ? K_SHARED_DOWN : K_GEMM_DOWN));
  return MOE_OK;
}

// ---- per-kernel timing ----
struct ProfRec {
  int id;
  hipEvent_t a, b;
};
uint32_t g_prof = 0;  // bit k: time kernel id k
std::mutex g_prof_mu;
std::vector<ProfRec> g_recs;
std::vector<hipEvent_t> g_pool;
hipEvent_t g_open = nullptr;
double g_ms[K_COUNT];
int64_t g_n[K_COUNT];

hipEvent_t get_event() {
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  // timing-only events: no system-scope fence (cache writeback and
  // invalidate) when recorded, so the bracketed kernel and its neighbours run
  // as they would unobserved
  hipEvent_t e = nullptr;
  if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
  return e;
}

moe_status resolve_records() {
  for (const ProfRec& r : g_recs) {
    MOE_HIP(hipEventSynchronize(r.b));
    float ms = 0.f;
    MOE_HIP(hipEventElapsedTime(&ms, r.a, r.b));
    g_ms[r.id] += ms;
    g_n[r.id] += 1;
    g_pool.push_back(r.a);
    g_pool.push_back(r.b);
  }
  g_recs.clear();
  return MOE_OK;
}

// ---- side stream for the shared expert ----
// The shared expert reads only x, so moe_forward runs it on a second stream
// of the same device (default priority), forked from the caller's stream at
// entry and joined before the combine: its GEMMs overlap the routing kernels
// and the routed FFN.  One per device, created on first use; g_side_mu is
// held while a call enqueues, so concurrent callers do not interleave their
// fork / join records.
struct Side {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
constexpr int kMaxDevices = 64;
std::mutex g_side_mu;
Side g_side[kMaxDevices];

// The side stream of device `dev` (the current device), created on first use.
moe_status side_of(int dev, Side** out) {
  if (dev < 0 || dev >= kMaxDevices) return fail(MOE_ERR_UNSUPPORTED, "device id %d out of range", dev);
  Side& sd = g_side[dev];
  if (!sd.s) {
    // cross-stream ordering on one device needs no timing and no
    // system-scope (host-visible) fence
    MOE_HIP(hipEventCreateWithFlags(&sd.fork, hipEventDisableTiming | hipEventDisableSystemFence));
    MOE_HIP(hipEventCreateWithFlags(&sd.join, hipEventDisableTiming | hipEventDisableSystemFence));
    MOE_HIP(hipStreamCreateWithFlags(&sd.s, hipStreamNonBlocking));
  }
  *out = &sd;
  return MOE_OK;
}

// moe_forward after validation.  allow_side: the shared expert may run on
// the device's side stream (created on first use); otherwise every launch is
// in order on hs.
moe_status forward_impl(const moe_config* cfg, const Shape& s, const void* x, const float* Wg,
                        const float* logit_bias, const float* sel_bias, const void* W1, const void* W3, const void* W2,
                        const void* Ws1, const void* Ws3, const void* Ws2, const moe_scales* scales, void* y,
                        const moe_routing* r, void* ws, size_t ws_bytes, hipStream_t hs, bool allow_side) {
  moe_status st;
  const bool topk_in = cfg->flags & MOE_F_TOPK_IN;
  const bool logits_in = cfg->flags & MOE_F_LOGITS_IN;
  if (!x || !y || !W1 || !W3 || !W2) return fail(MOE_ERR_INVALID_ARG, "x, y, W1, W3, W2 are required");
  if (!topk_in && !logits_in && !Wg) return fail(MOE_ERR_INVALID_ARG, "Wg is required");
  if (s.S && (!Ws1 || !Ws3 || !Ws2)) return fail(MOE_ERR_INVALID_ARG, "shared expert weights are required");
  if (s.w8 && (!scales || !scales->w1 || !scales->w3 || !scales->w2 ||
               (s.S && (!scales->ws1 || !scales->ws3 || !scales->ws2))))
    return fail(MOE_ERR_INVALID_ARG, "MOE_FP8_E4M3 weights need their scales");
  if ((st = check_aligned({x, Wg, W1, W3, W2, Ws1, Ws3, Ws2, y})) != MOE_OK) return st;
  if (s.w8 && (st = check_aligned({scales->w1, scales->w3, scales->w2, scales->ws1, scales->ws3, scales->ws2})) != MOE_OK)
    return st;
  const moe_scales none{};
  const moe_scales& sc = s.w8 ? *scales : none;
  if ((topk_in || logits_in || s.stats) && !r)
    return fail(MOE_ERR_INVALID_ARG, "MOE_F_*_IN and MOE_F_STATS need the routing arrays");
  if (r && (st = check_routing(r, !topk_in, s.stats)) != MOE_OK) return st;
  Layout L;
  if ((st = check_ws(s, ws, ws_bytes, &L)) != MOE_OK) return st;
  if (s.T == 0) return MOE_OK;
  // the shared expert on the device's side stream when allowed and the
  // caller's stream belongs to the current device (else in order on the
  // caller's stream)
  std::unique_lock<std::mutex> side_lk;
  Side* sd = nullptr;
  if (s.S && allow_side) {
    int cur = -1, sdev = -2;
    if (hipGetDevice(&cur) == hipSuccess && hipStreamGetDevice(hs, &sdev) == hipSuccess && sdev == cur) {
      side_lk = std::unique_lock<std::mutex>(g_side_mu);
      if ((st = side_of(cur, &sd)) != MOE_OK) return st;
    }
  }
  moe_routing rr;
  if (r) {
    rr = *r;
  } else {
    rr.logits = at<float>(ws, L.r_logits);
    rr.topk_idx = at<int32_t>(ws, L.r_idx);
    rr.topk_w = at<float>(ws, L.r_w);
    rr.counts = at<int32_t>(ws, L.r_counts);
    rr.offsets = at<int32_t>(ws, L.r_offsets);
    rr.dest = at<int32_t>(ws, L.r_dest);
    rr.row_src = at<int32_t>(ws, L.r_row_src);
    rr.dropped = at<uint8_t>(ws, L.r_dropped);
    rr.stats = nullptr;
  }
  // x k-blocked once for the bf16 layers that read it through the routing
  // (and for the shared expert), before the shared expert forks off: in
  // blocks of 64 k when every GEMM1 reading it takes stages of 64 k (a
  // gathered row's piece of a stage is then one whole 128-byte line), else 32
  const int64_t group_max = s.cap >= 0 ? std::min(s.T, s.cap) : s.T;
  FfnPlan plan = plan_of(s, s.max_rows, group_max, s.E, s.F);
  if (s.fused) plan.stream_down = false;  // the fused GEMM2 epilogue is the tile kernel's
  // decode-sized batches (at most 64 tokens) read the rows from x itself,
  // row-major (x is then a few hundred KB and stays in L2; the copy would
  // cost a launch); tuning: MOE_GATHER=0 dispatches a per-row copy instead,
  // =1 always copies, =2 always reads x row-major
  const int gather_env = tuning_enabled() && getenv("MOE_GATHER") ? atoi(getenv("MOE_GATHER")) : -1;
  const bool gather = s.bf16 && !s.fused && gather_env != 0;
  const bool gather_row = gather && (gather_env == 2 || (gather_env == -1 && s.T <= 64));
  int kbw = 0;  // 0: x is not k-blocked (fp32 layers, the fused path)
  if (s.bf16 && !s.fused) {
    // the weight-streaming kernels read A in blocks of 32 k
    auto wants64 = [](const FfnPlan& q) { return q.k64_up && !q.stream_up; };
    const bool sh64 = !s.S || wants64(plan_of(s, s.T, s.T, 1, s.Fs));
    kbw = (wants64(plan) || !gather) && sh64 && s.d % 64 == 0 ? 64 : 32;
    if ((!gather || gather_row) && !s.S) kbw = 0;  // nothing reads x k-blocked
    if (gather_row) kbw = 0;
  }
  void* xkb = at<void>(ws, L.xkb);
  if (kbw) MOE_HIP(launch_kblock_copy(x, xkb, s.T, s.d * (int64_t)s.esz, kbw, hs));
  // a8: the shared expert over all T rows of x
  float* sh_out = s.S ? at<float>(ws, L.sh_out) : nullptr;
  auto shared_ffn = [&](hipStream_t q) -> moe_status {
    int32_t* range = at<int32_t>(ws, L.sh_range);
    MOE_HIP(launch_set_range(range, s.T, q));
    const AOperand xa = kbw ? AOperand{xkb, s.T, nullptr, 1, kbw} : AOperand{x, 0, nullptr, 1, 32};
    return do_ffn(s, xa, range, 1, s.T, s.T, Ws1, Ws3, Ws2, sc.ws1, sc.ws3, sc.ws2, at<void>(ws, L.sh_h), sh_out,
                  at<int4>(ws, L.sh_tab_up), at<int4>(ws, L.sh_tab_down), at<int32_t>(ws, L.sh_counts), s.Fs, q,
                  nullptr, nullptr, false, true);
  };
  if (sd) {
    MOE_HIP(hipEventRecord(sd->fork, hs));
    MOE_HIP(hipStreamWaitEvent(sd->s, sd->fork, 0));
    if ((st = shared_ffn(sd->s)) != MOE_OK) return st;
    MOE_HIP(hipEventRecord(sd->join, sd->s));
  }
  const bool residual = cfg->flags & MOE_F_RESIDUAL;
  // one assignment per token and no shared expert (bf16): GEMM2 writes the
  // kept tokens' outputs itself, and the dropped tokens' rows are written by
  // the capacity scatter (first-come drops) or else by the combine
  const bool fused = s.fused;
  bool drop_done = false;
  void* xp = at<void>(ws, L.xp);
  // the routed FFN's plan (above) is known before routing: the scatter that
  // runs on the final offsets writes its tile tables (one launch fewer); an
  // expert holds at most one row per token, and at most its capacity
  const TileJob tj = tile_job(plan, s.F, s.d, at<int4>(ws, L.tab_up), at<int4>(ws, L.tab_down),
                              at<int32_t>(ws, L.counts));
  bool tiles_done = false;
  // on the fused path the scatter also does the dispatch (one row per kept token)
  if ((st = do_route(cfg, s, L, x, Wg, logit_bias, sel_bias, rr, ws, hs, fused ? y : nullptr,
                     residual ? x : nullptr, &drop_done, fused && s.max_rows > 0 ? xp : nullptr, s.max_rows,
                     s.max_rows > 0 && !(plan.stream_up && plan.stream_down) ? &tj : nullptr, &tiles_done)) != MOE_OK)
    return st;
  float* yp = at<float>(ws, L.yp);
  const CombineFuse fuse{rr.row_src, rr.topk_w, residual ? x : nullptr, y, s.bf16, s.out_bf16};
  if (s.max_rows > 0) {
    // A of the routed GEMM1: the fused path's xp (k-blocked, each k-step of a
    // tile one contiguous run), written by the scatter or the dispatch; the
    // other bf16 layers read x k-blocked through row_src (the a5 gather is
    // folded into GEMM1's loads); fp32 layers dispatch row-major rows
    AOperand xa{xp, 0, nullptr, 1, 32};
    if (gather_row) {
      xa = AOperand{x, 0, rr.row_src, (int)s.K, 32};
    } else if (gather) {
      xa = AOperand{xkb, s.T, rr.row_src, (int)s.K, kbw};
    } else {
      if (!drop_done)
        MOE_HIP(launch_dispatch(x, rr.row_src, rr.offsets + s.E, xp, s.max_rows, s.K, s.d * (int64_t)s.esz, s.bf16,
                                hs));
      if (s.bf16) xa.blk_rows = s.max_rows;
    }
    if ((st = do_ffn(s, xa, rr.offsets, s.E, s.max_rows, group_max, W1, W3, W2, sc.w1, sc.w3, sc.w2, at<void>(ws, L.h), yp,
                     at<int4>(ws, L.tab_up), at<int4>(ws, L.tab_down), at<int32_t>(ws, L.counts), s.F, hs,
                     fused ? &fuse : nullptr, &plan, tiles_done)) != MOE_OK)
      return st;
  }
  if (s.S && !sd && (st = shared_ffn(hs)) != MOE_OK) return st;
  if (sd) MOE_HIP(hipStreamWaitEvent(hs, sd->join, 0));
  if (!drop_done)
    MOE_HIP(launch_combine(s.bf16, s.out_bf16, yp, rr.topk_w, rr.dest, sh_out, residual ? x : nullptr, y, s.T, s.d,
                           s.K, fused, hs));
  return MOE_OK;
}


const char* const kNames[K_COUNT] = {"router_logits", "router_topk",  "route_scan", "route_scatter",
                                     "dispatch",      "ffn_tiles",    "gemm_gate_up", "gemm_down",
                                     "combine",       "shared_gate_up", "shared_down"};

}  // namespace

const char* kernel_name(int id) { return (id >= 0 && id < K_COUNT) ? kNames[id] : nullptr; }

// Set while the calling thread is inside moe_forward_noalloc: the timing
// facility creates events on demand, which that entry point must not do.
thread_local bool g_no_timing = false;

void prof_begin(int id, hipStream_t s) {
  if (!(g_prof >> id & 1u) || g_no_timing) return;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_open = get_event();
  if (g_open) (void)hipEventRecord(g_open, s);
}

void prof_end(int id, hipStream_t s) {
  if (!(g_prof >> id & 1u) || g_no_timing) return;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (!g_open) return;
  hipEvent_t b = get_event();
  if (!b) return;
  (void)hipEventRecord(b, s);
  g_recs.push_back(ProfRec{id, g_open, b});
  g_open = nullptr;
}

moe_status forward_in_scratch(const moe_config* cfg, const void* x, const float* Wg, const float* logit_bias,
                              const float* sel_bias, const void* W1, const void* W3, const void* W2,
                              const void* Ws1, const void* Ws3, const void* Ws2, const moe_scales* scales, void* y,
                              const moe_routing* r, void* ws, size_t ws_bytes, hipStream_t hs) {
  Shape s;
  moe_status st = validate(cfg, &s);
  if (st != MOE_OK) return st;
  const size_t need = layout(s).total;
  if (need > ws_bytes)
    return fail(MOE_ERR_WORKSPACE, "this layer needs %zu bytes of scratch, more than the %zu available; call "
                "moe_forward with a workspace", need, ws_bytes);
  g_no_timing = true;
  st = forward_impl(cfg, s, x, Wg, logit_bias, sel_bias, W1, W3, W2, Ws1, Ws3, Ws2, scales, y, r, ws, ws_bytes, hs,
                    false);
  g_no_timing = false;
  return st;
}

moe_status fail_detail(moe_status s, const char* msg) { return fail(s, "%s", msg); }

}  // namespace moe

using namespace moe;

extern "C" {

moe_status moe_workspace_size(const moe_config* cfg, size_t* bytes) {
  Shape s;
  moe_status st = validate(cfg, &s);
  if (st != MOE_OK) return st;
  if (!bytes) return fail(MOE_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = layout(s).total;
  return MOE_OK;
}

moe_status moe_max_rows(const moe_config* cfg, int64_t* rows) {
  Shape s;
  moe_status st = validate(cfg, &s);
  if (st != MOE_OK) return st;
  if (!rows) return fail(MOE_ERR_INVALID_ARG, "rows is NULL");
  *rows = s.max_rows;
  return MOE_OK;
}

moe_status moe_route(const moe_config* cfg, const void* x, const float* Wg, const float* logit_bias,
                     const float* sel_bias, const moe_routing* r, void* ws, size_t ws_bytes, moe_stream_t stream) {
  Shape s;
  moe_status st = validate(cfg, &s);
  if (st != MOE_OK) return st;
  const bool topk_in = cfg->flags & MOE_F_TOPK_IN;
  const bool logits_in = cfg->flags & MOE_F_LOGITS_IN;
  if ((st = check_routing(r, !topk_in, s.stats)) != MOE_OK) return st;
  if (!topk_in && !logits_in && (!x || !Wg)) return fail(MOE_ERR_INVALID_ARG, "x and Wg are required");
  if ((st = check_aligned({x, Wg})) != MOE_OK) return st;
  Layout L;
  if ((st = check_ws(s, ws, ws_bytes, &L)) != MOE_OK) return st;
  if (s.T == 0) return MOE_OK;
  return do_route(cfg, s, L, x, Wg, logit_bias, sel_bias, *r, ws, (hipStream_t)stream);
}

moe_status moe_dispatch(const moe_config* cfg, const void* x, const moe_routing* r, void* xp, moe_stream_t stream) {
  Shape s;
  moe_status st = validate(cfg, &s);
  if (st != MOE_OK) return st;
  if (!r || !r->row_src || !r->offsets) return fail(MOE_ERR_INVALID_ARG, "routing row_src / offsets required");
  if (!x || !xp) return fail(MOE_ERR_INVALID_ARG, "x and xp are required");
  if ((st = check_aligned({x, xp})) != MOE_OK) return st;
  if (s.T == 0) return MOE_OK;
  MOE_HIP(launch_dispatch(x, r->row_src, r->offsets + s.E, xp, s.max_rows, s.K, s.d * (int64_t)s.esz, false,
                          (hipStream_t)stream));
  return MOE_OK;
}

moe_status moe_expert_ffn(const moe_config* cfg, const void* xp, const int32_t* offsets, int64_t n_groups,
                          int64_t max_rows, const void* W1, const void* W3, const void* W2, const moe_scales* scales,
                          float* yp, void* ws, size_t ws_bytes, moe_stream_t stream) {
  Shape s;
  moe_status st = validate(cfg, &s);
  if (st != MOE_OK) return st;
  if (n_groups < 1 || n_groups > s.E) return fail(MOE_ERR_INVALID_ARG, "n_groups must be in [1, n_experts]");
  if (max_rows < 0 || max_rows > s.max_rows)
    return fail(MOE_ERR_INVALID_ARG, "max_rows = %lld outside [0, %lld]", (long long)max_rows,
                (long long)s.max_rows);
  if (!xp || !offsets || !W1 || !W3 || !W2 || !yp) return fail(MOE_ERR_INVALID_ARG, "a required pointer is NULL");
  if (s.w8 && (!scales || !scales->w1 || !scales->w3 || !scales->w2))
    return fail(MOE_ERR_INVALID_ARG, "MOE_FP8_E4M3 weights need scales->w1, w3, w2");
  if ((st = check_aligned({xp, W1, W3, W2, yp})) != MOE_OK) return st;
  if (s.w8 && (st = check_aligned({scales->w1, scales->w3, scales->w2})) != MOE_OK) return st;
  Layout L;
  if ((st = check_ws(s, ws, ws_bytes, &L)) != MOE_OK) return st;
  if (max_rows == 0) return MOE_OK;
  const moe_scales none{};
  const moe_scales& sc = s.w8 ? *scales : none;
  // the plan assumes the routed bound of a group's rows (any rows stay correct)
  const int64_t group_max = s.cap >= 0 ? std::min(s.T, s.cap) : s.T;
  return do_ffn(s, AOperand{xp, 0, nullptr, 1, 32}, offsets, n_groups, max_rows, group_max, W1, W3, W2, sc.w1, sc.w3, sc.w2,
                at<void>(ws, L.h), yp,
                at<int4>(ws, L.tab_up), at<int4>(ws, L.tab_down), at<int32_t>(ws, L.counts), s.F,
                (hipStream_t)stream);
}

moe_status moe_pack_weights(const void* src, void* dst, int64_t groups, int64_t N, int64_t K, int32_t w_dtype,
                            moe_stream_t stream) {
  if (!src || !dst) return fail(MOE_ERR_INVALID_ARG, "src and dst are required");
  if (w_dtype != MOE_BF16 && w_dtype != MOE_FP8_E4M3)
    return fail(MOE_ERR_INVALID_ARG, "w_dtype %d: packing takes MOE_BF16 or MOE_FP8_E4M3 weights", (int)w_dtype);
  const int64_t esz = w_dtype == MOE_BF16 ? 2 : 1;
  if (groups < 1 || N < 64 || N % 64 || K < 64 || K % 64)
    return fail(MOE_ERR_INVALID_ARG, "groups = %lld must be >= 1, N = %lld and K = %lld positive multiples of 64",
                (long long)groups, (long long)N, (long long)K);
  if (N > (int64_t)INT32_MAX || groups > (int64_t)INT32_MAX / N || K > (int64_t)INT32_MAX / 8)
    return fail(MOE_ERR_UNSUPPORTED, "groups * N or K exceeds the supported range");
  moe_status st;
  if ((st = check_aligned({src, dst})) != MOE_OK) return st;
  const uintptr_t a = (uintptr_t)src, b = (uintptr_t)dst, n = (uintptr_t)(groups * N * K * esz);
  if (a < b + n && b < a + n) return fail(MOE_ERR_INVALID_ARG, "src and dst overlap");
  // N is a multiple of 64, so the panels of all groups' rows are the groups' panels
  MOE_HIP(launch_pack_weights(src, dst, groups * N, K, (int)esz, (hipStream_t)stream));
  return MOE_OK;
}

moe_status moe_combine(const moe_config* cfg, const float* yp, const moe_routing* r, const float* shared_out,
                       const void* x_residual, void* y, moe_stream_t stream) {
  Shape s;
  moe_status st = validate(cfg, &s);
  if (st != MOE_OK) return st;
  if (!r || !r->topk_w || !r->dest) return fail(MOE_ERR_INVALID_ARG, "routing topk_w / dest required");
  if (!yp || !y) return fail(MOE_ERR_INVALID_ARG, "yp and y are required");
  const bool residual = cfg->flags & MOE_F_RESIDUAL;
  if (residual && !x_residual) return fail(MOE_ERR_INVALID_ARG, "MOE_F_RESIDUAL needs x_residual");
  if ((st = check_aligned({yp, y, shared_out, residual ? x_residual : nullptr})) != MOE_OK) return st;
  if (s.T == 0) return MOE_OK;
  MOE_HIP(launch_combine(s.bf16, s.out_bf16, yp, r->topk_w, r->dest, shared_out, residual ? x_residual : nullptr, y, s.T, s.d,
                         s.K, false, (hipStream_t)stream));
  return MOE_OK;
}

moe_status moe_forward(const moe_config* cfg, const void* x, const float* Wg, const float* logit_bias,
                       const float* sel_bias, const void* W1, const void* W3, const void* W2, const void* Ws1,
                       const void* Ws3, const void* Ws2, const moe_scales* scales, void* y, const moe_routing* r,
                       void* ws, size_t ws_bytes, moe_stream_t stream) {
  Shape s;
  moe_status st = validate(cfg, &s);
  if (st != MOE_OK) return st;
  return forward_impl(cfg, s, x, Wg, logit_bias, sel_bias, W1, W3, W2, Ws1, Ws3, Ws2, scales, y, r, ws, ws_bytes,
                      (hipStream_t)stream, true);
}

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
  }
  return "MOE_ERR_UNKNOWN";
}

const char* moe_last_error(void) { return g_err.c_str(); }

moe_status moe_profile_enable(uint32_t kernel_mask) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof = kernel_mask;
  return MOE_OK;
}

moe_status moe_profile_reset(void) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  moe_status st = resolve_records();
  for (int i = 0; i < K_COUNT; ++i) {
    g_ms[i] = 0.0;
    g_n[i] = 0;
  }
  return st;
}

moe_status moe_profile_read(int kernel_id, double* total_ms, int64_t* launches) {
  if (kernel_id < 0 || kernel_id >= K_COUNT || !total_ms || !launches)
    return fail(MOE_ERR_INVALID_ARG, "bad kernel id or NULL output");
  std::lock_guard<std::mutex> lk(g_prof_mu);
  moe_status st = resolve_records();
  if (st != MOE_OK) return st;
  *total_ms = g_ms[kernel_id];
  *launches = g_n[kernel_id];
  return MOE_OK;
}

const char* moe_kernel_name(int kernel_id) { return kernel_name(kernel_id); }

}  // extern "C"
