// Host-side interface between the C-ABI layer (api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Kernel ids for the per-kernel timing facility (order = moe_kernel_name).
enum KernelId {
  K_ROUTER_LOGITS = 0,
  K_ROUTER_TOPK,
  K_ROUTE_SCAN,
  K_ROUTE_SCATTER,
  K_DISPATCH,
  K_FFN_TILES,
  K_GEMM_GATE_UP,    // grouped GEMM1 + SiLU*gate epilogue
  K_GEMM_DOWN,       // grouped GEMM2
  K_COMBINE,
  K_SHARED_GATE_UP,  // the shared expert's GEMM1 (+ SiLU*gate) and GEMM2
  K_SHARED_DOWN,
  K_COUNT
};
const char* kernel_name(int id);

// Records a timing event pair around a launch when profiling is on.
void prof_begin(int id, hipStream_t s);
void prof_end(int id, hipStream_t s);

// Tokens per router_topk workgroup, which is also the histogram chunk of the
// capacity scan and scatter: at most kTopkTokens.  Layers with a costly
// selection (E * K >= 512) take chunks of 16 tokens, so the Top-K kernel has
// twice the workgroups; the others 32 (fewer chunks for the scan).
constexpr int kTopkTokens = 32;
inline int chunk_tokens(int64_t E, int64_t K) { return E * K >= 512 ? 16 : 32; }

// ---- router (a1-a3) ----
// Number of d-slices the logits GEMM is cut into (1 = logits written directly).
int router_splits(int64_t T, int64_t d, int64_t E, bool bf16);
// part: [S, T, E] fp32 partial sums (unused when S == 1).
hipError_t launch_router_logits(bool bf16, const void* x, const float* Wg, const float* bias, float* logits,
                                float* part, int64_t T, int64_t d, int64_t E, hipStream_t s);
// S > 1: logits = sum of the S slices of `part` (in order) + bias, written to
// `logits` before selection; S == 1: `logits` is read as is.
// topk_in: idx is an input; only the per-chunk histogram is produced.
// blk_P / blk_z non-null (never with topk_in): per-chunk router-distribution
// sums [n_chunks, E] and logsumexp^2 sums [n_chunks] for the statistics.
// K2 > 0: also the ranks K .. K+K2-1 of every token (alt_idx / alt_w [T, K2],
// weights normalised like the first K) for re-routing.
hipError_t launch_router_topk(float* logits, const float* part, int S, const float* bias, const float* sel_bias,
                              int32_t* idx, float* w, int32_t* blk_count, float* blk_P, float* blk_z, int32_t* alt_idx,
                              float* alt_w, int64_t K2, int64_t T, int64_t E, int64_t K, int gate, bool renorm,
                              bool topk_in, hipStream_t s);

// ---- permutation (a4) and dispatch (a5) ----
// stats non-null: also folds blk_P / blk_z into the router statistics
// (E + 6 doubles).
// first_counts non-null: second scan of re-routing (kept = first-pass kept +
// what fits of this pass's demand).  dem_off non-null: also the exclusive
// scan of the demand (segments of the affinity drop).
hipError_t launch_route_scan(const int32_t* blk_count, int32_t* blk_base, int32_t* counts, int32_t* offsets,
                             int64_t n_chunks, int64_t E, int64_t cap, const float* blk_P, const float* blk_z,
                             double* stats, int64_t T, int64_t K, const int32_t* first_counts, int32_t* dem_off,
                             hipStream_t s);

// Tile tables of one FFN's two GEMMs (as launch_ffn_tiles writes them), for
// a routing kernel to write once the final offsets exist.  tab_up ==
// nullptr: none.
struct TileJob {
  int bm_up, nt_up, bn_up, bm_down, nt_down, bn_down;
  int even_up;  // GEMM1 m-tiles split evenly (FfnPlan::even_up)
  int4* tab_up;
  int4* tab_down;
  int32_t* counts;
};

// Capacity drop policy of the scatter (kernel comments give each mode).
enum ScatterMode { kFirstCome = 0, kAffinity = 1, kReroute1 = 2, kReroute2 = 3 };

// Arrays of one scatter launch; unused ones may be null.
struct RouteScatter {
  int mode;                 // ScatterMode
  const int32_t* idx;       // the expert ranked for each assignment (-1 or >= E: none)
  const int32_t* blk_base;  // [chunks, E] rank base of each chunk
  const int32_t* offsets;   // [E + 1] final row offsets (unused by kReroute1)
  int32_t* dest;
  int32_t* row_src;
  uint8_t* dropped;
  const int32_t* counts;    // kAffinity: demand per expert
  const int32_t* dem_off;   // kAffinity: exclusive scan of the demand
  const float* aff;         // kAffinity: affinity of each assignment (its gate weight)
  uint64_t* seg;            // kAffinity: [T*K] keys, expert e's segment at dem_off[e]
  const int32_t* alt_idx;   // kReroute1: [T, K2] rank-(K+j) expert of each token
  const float* alt_w;       // kReroute1: [T, K2] its weight
  int K2;
  int32_t* pos1;            // first-pass rank of kept assignments, -1 when overflowing
  int32_t* cand;            // re-routing candidate expert of each assignment or -1
  float* cand_w;            // its weight
  int32_t* blk_count2;      // kReroute1: [chunks, E] candidates per chunk
  const int32_t* first_counts;  // kReroute2: first-pass demand
  int32_t* topk_idx;        // kReroute2: re-routed assignments get their new expert
  float* topk_w;            //            and weight
  // kFirstCome with one assignment per token and no shared expert: the
  // layer output rows of the dropped tokens, y[t] = 0 + x[t] (x nullable:
  // 0), rounded once to y's type (the combine's arithmetic for such a row),
  // are written here.  drop_y == nullptr: not written.
  void* drop_y;
  const uint16_t* drop_x;   // bf16 residual rows
  bool drop_y_bf16;         // y is bf16, else fp32
  int drop_d;               // row length (a multiple of 8)
  // kFirstCome with one assignment per token: the kept tokens' rows of x
  // (bf16, disp_n_kb 64-byte k-blocks each) are also copied to their rows of
  // the k-blocked xp ([n_kb][disp_blk_rows][32]), the dispatch's output.
  // disp_xp == nullptr: not copied.
  uint4* disp_xp;
  const uint4* disp_x;
  int disp_n_kb;
  int64_t disp_blk_rows;
  // a scatter that runs on the final offsets (kFirstCome, kAffinity,
  // kReroute2) may also write the GEMM tile tables
  TileJob tiles;
  // kFirstCome with a single chunk (decode-sized batches): the scatter first
  // does the capacity scan itself from the chunk's histogram one_count [E],
  // writing one_counts (= counts) and one_offsets (= offsets), and the scan
  // launch is skipped.  one_count == nullptr: not done here.
  const int32_t* one_count;
  int32_t* one_counts;
  int32_t* one_offsets;
};
hipError_t launch_route_scatter(const RouteScatter& r, int64_t T, int64_t K, int64_t E, int64_t cap, hipStream_t s);
hipError_t launch_route_affinity(const uint64_t* seg, const int32_t* counts, const int32_t* dem_off,
                                 const int32_t* offsets, int32_t* dest, int32_t* row_src, uint8_t* dropped, int64_t E,
                                 int64_t cap, hipStream_t s);
// Expert-choice routing in the K = E form: w / idx / dest / dropped are
// [T, E]; seg: [E, T] key scratch; cap tokens per expert (0 <= cap <= T).
// S > 1: logits = sum of the router's d-slices in `part` (+ bias), written.
hipError_t launch_expert_choice(float* logits, const float* part, int S, const float* bias, int32_t* idx, float* w,
                                uint64_t* seg, int32_t* counts, int32_t* offsets, int32_t* dest, int32_t* row_src,
                                uint8_t* dropped, int64_t T, int64_t E, int64_t cap, hipStream_t s);
// blocked: xp is k-blocked bf16 [d/32][max_rows][32] (row_bytes = 2 d), else
// row-major.
hipError_t launch_dispatch(const void* x, const int32_t* row_src, const int32_t* R_ptr, void* xp, int64_t max_rows,
                           int64_t K, int64_t row_bytes, bool blocked, hipStream_t s);
// x [T, d] bf16 -> k-blocked [d/kbw][T][kbw], kbw = 32 or 64 (row_bytes = 2 d,
// a multiple of 2 kbw).
hipError_t launch_kblock_copy(const void* x, void* xkb, int64_t T, int64_t row_bytes, int kbw, hipStream_t s);
// moe_pack_weights: rows [rows, K] of esz-byte elements (bf16: 2, E4M3: 1;
// rows a multiple of 64) into panels [rows/64][K/64][64][64].
hipError_t launch_pack_weights(const void* src, void* dst, int64_t rows, int64_t K, int esz, hipStream_t s);

// ---- grouped expert FFN (a6-a7) ----
struct FfnPlan {
  int bm;           // rows per m-tile
  int bnb_up;       // bf16: weight rows per GEMM1 tile (W1 and W3 rows together)
  int ns_up;        // bf16: LDS stages of GEMM1
  int bnb_down;     // bf16: weight rows per GEMM2 tile
  int ns_down;      // bf16: LDS stages of GEMM2
  int wg_per_cu;    // bf16: persistent workgroups per CU (0 = one workgroup per tile)
  int bn_out_up;    // h columns per GEMM1 tile
  int bn_out_down;  // yp columns per GEMM2 tile
  bool w8;          // expert weights are E4M3 bytes with per-row scales
  int bm_down;      // rows per m-tile of GEMM2 (bm: GEMM1)
  bool k64_up;      // GEMM1 in stages of 64 k (else 32)
  bool k64_down;    // GEMM2 in stages of 64 k (else 32)
  // GEMM1 m-tiles of a group split evenly in 32-row units instead of full
  // bm-row tiles and a remainder, so the m-tiles that share a weight tile
  // stay in step (MFMA-bound groups of 512 rows or more on average)
  bool even_up = false;
  // bf16 weights, at most 32 rows in any group: GEMM1 / GEMM2 are the
  // weight-streaming kernels (gemm_stream.hip; they need no tile table)
  bool stream_up = false;
  bool stream_down = false;
  int stream_u = 8;  // GEMM2's 32-k steps per load batch (8 or 4)
  // tile kernels: > 0 deals tiles to the XCDs in chunks of this many
  // consecutive tiles, round-robin (one tile per workgroup)
  int xcd_chunk_up = 0;
  int xcd_chunk_down = 0;
  // bf16 weights of GEMM1 / GEMM2 packed in 64-row panels
  // [groups][N/64][K/64][64][64] (moe_pack_weights), else row-major
  bool packed_up = false;
  bool packed_down = false;
  // GEMM1 / GEMM2 weight loads with the non-temporal cache policy
  bool nt_up = false;
  bool nt_down = false;
  // > 0: the tiles that hold a whole group of at most this many rows also
  // load their weights non-temporally (no other m-tile reads them)
  int nt_rows_up = 0;
  int nt_rows_down = 0;
};
// Compute units of the current device (queried once).
int device_cus();
// Tile-plan overrides from the environment (MOE_GEMM_*, MOE_ROUTER_WGS) are
// honoured only when MOE_TUNING=1 is set, so an inherited variable cannot
// change what a production caller launches.
bool tuning_enabled();
// group_max: upper bound of any group's rows (the expert capacity when there
// is one); max_rows: of all groups together.
// packed_up / packed_down: W1, W3 / W2 in moe_pack_weights' layout, which
// some plans stream faster.
FfnPlan ffn_plan(bool bf16, bool w8, int64_t max_rows, int64_t group_max, int64_t n_groups, int64_t F, int64_t d,
                 bool packed_up = false, bool packed_down = false);
// Whether the bf16-activation GEMM is compiled for (m-tile rows, weight-tile
// rows, stages), with bf16 (w8 false) or E4M3 (w8 true) weights in stages of
// 32 k or (k64) 64 k.
bool gemm_bf16_has_config(bool w8, bool k64, int bm, int bnb, int ns);
// The smallest m-tile and weight tile (rows) of any compiled bf16 GEMM
// configuration; the tile tables are sized for them (checked at compile time
// against every configuration).
constexpr int kMinTileRows = 64;
constexpr int kMinWeightTileRows = 128;
// Worst-case m-tiles for `bm`-row tiles.
int64_t ffn_max_mtiles(int bm, int64_t max_rows, int64_t n_groups);
// Entries the tile tables need for any plan of this dtype.
int64_t ffn_table_entries(bool bf16, int64_t max_rows, int64_t n_groups, int64_t n_cols, bool gate_up);
// Builds both GEMMs' tile tables (int4 {group, first row, rows, first column};
// m-tiles of p.bm rows for gate_up, p.bm_down for down)
// and their entry counts counts[0] (gate_up) and counts[1] (down).
// The tile-table job of plan p (F: GEMM1 output columns, d: GEMM2's).
TileJob tile_job(const FfnPlan& p, int64_t F, int64_t d, int4* tab_up, int4* tab_down, int32_t* counts);
hipError_t launch_ffn_tiles(const FfnPlan& p, const int32_t* offsets, int64_t n_groups, int64_t max_rows, int64_t F,
                            int64_t d, int4* tab_up, int4* tab_down, int32_t* counts, hipStream_t s);
// Combine fused into GEMM2 for one assignment per token (K == 1, no shared
// expert): the epilogue writes y[t] = w[t] * yp_row (+ x[t]) for the token t
// = row_src[row] of each kept row, in the combine's arithmetic; the combine
// then only writes the dropped tokens.
struct CombineFuse {
  const int32_t* row_src;  // [R] flat assignment (= token) of each row
  const float* w;          // [T] gate weight
  const void* xres;        // residual x [T, d] or null
  void* y;                 // [T, d] output
  bool x_bf16, y_bf16;
};

// The A operand of GEMM1: row-major [rows, Kdim] (blk_rows = 0) or k-blocked
// [Kdim/kbw][blk_rows][kbw] with kbw = 32 or 64 (the kbw columns of all rows
// are one contiguous run).  gather non-null: GEMM row r reads A row
// gather[r] / gather_div -- the routed rows read x (k-blocked or row-major)
// through the routing's row_src (gather_div = K), so no per-row copy of x is
// made.
struct AOperand {
  const void* ptr;
  int64_t blk_rows;
  const int32_t* gather;
  int gather_div;
  int kbw;
};

// Weight-streaming GEMMs (gemm_stream.hip) for plans with p.stream_*: groups
// from offsets directly; A k-blocked in blocks of 32 k or row-major; h
// k-blocked with h_blk rows; yp row-major fp32.  packed: the weights are in
// the packed layout of moe_pack_weights, else row-major.
hipError_t stream_gate_up(const AOperand& A, const int32_t* offsets, int64_t n_groups, const void* W1, const void* W3,
                          void* h, int64_t h_blk, int64_t F, int64_t d, bool packed, bool nt, hipStream_t s);
// u_max: 32-k steps per load batch of GEMM2 (8 or 4; fewer when K / 32 is
// not a multiple).
hipError_t stream_down(const void* h, int64_t h_blk, const int32_t* offsets, int64_t n_groups, const void* W2,
                       float* yp, int64_t F, int64_t d, int u_max, bool packed, bool nt, hipStream_t s);

// bf16 MFMA path (gemm_bf16.hip); called through the launchers below.
// s1 / s3 / s2: [groups, N] row scales of E4M3 weights (p.w8), else unused.
// a_blk / h_blk: the row count R of a k-blocked operand ([cols/32][R][32]:
// the 32 columns of a k-step of R rows are one contiguous run), 0 = row-major.
hipError_t gemm_bf16_gate_up(const FfnPlan& p, const AOperand& A, const int4* tab, const int32_t* count,
                             const int32_t* offsets, int64_t grid, const void* W1, const void* W3, const float* s1,
                             const float* s3, void* h, int64_t h_blk, int64_t F, int64_t d, hipStream_t s);
hipError_t gemm_bf16_down(const FfnPlan& p, const void* h, int64_t h_blk, const int4* tab, const int32_t* count,
                          const int32_t* offsets, int64_t grid, const void* W2, const float* s2, float* yp,
                          const CombineFuse* fuse, int64_t F, int64_t d, hipStream_t s);
// bf16: h is k-blocked with max_rows rows; A as AOperand says; fp32:
// everything row-major (A.ptr only).
// prof_id: the timing facility's kernel id of the launch (the routed or the
// shared expert's GEMM).
hipError_t launch_gemm_gate_up(bool bf16, const FfnPlan& p, const AOperand& A, const int4* tab,
                               const int32_t* count, const int32_t* offsets, int64_t n_groups, int64_t max_rows,
                               const void* W1, const void* W3,
                               const float* s1, const float* s3, void* h, int64_t F, int64_t d, hipStream_t s,
                               int prof_id = K_GEMM_GATE_UP);
// fuse (bf16 only, nullable): write y instead of yp.
hipError_t launch_gemm_down(bool bf16, const FfnPlan& p, const void* h, const int4* tab, const int32_t* count,
                            const int32_t* offsets, int64_t n_groups, int64_t max_rows, const void* W2, const float* s2,
                            float* yp,
                            const CombineFuse* fuse, int64_t F, int64_t d, hipStream_t s,
                            int prof_id = K_GEMM_DOWN);

// dst[0] = 0, dst[1] = n (row range of the shared expert).
hipError_t launch_set_range(int32_t* dst, int64_t n, hipStream_t s);

// ---- combine (a9) ----
// only_dropped: write only the tokens none of whose assignments was kept
// (the others were written by a fused GEMM2 epilogue).
hipError_t launch_combine(bool x_bf16, bool y_bf16, const float* yp, const float* w, const int32_t* dest, const float* shared,
                          const void* xres, void* y, int64_t T, int64_t d, int64_t K, bool only_dropped, hipStream_t s);

}  // namespace moe
