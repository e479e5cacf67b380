// Grouped expert GEMMs on bf16 MFMA (gfx950 v_mfma_f32_16x16x32_bf16).
//
// The expert is the SwiGLU FFN y = W2 (SiLU(W1 x) * (W3 x)) of the lnwmold.com
// article on GPT-4-class sparse activation, §2.2 (three matrices W1, W2, W3);
// "技术日报 2026-04-14" §7.4 names them Gate / Up / Down.
//
// Rows are grouped by expert (group g owns rows offsets[g] .. offsets[g+1]-1
// of A).  A workgroup computes one (group, m-tile, n-tile) output tile:
//   gate_up: h[rows, n0:n0+128] = SiLU(A W1[g]^T) * (A W3[g]^T), bf16 out
//   down:    yp[rows, n0:n0+256] = h W2[g]^T, fp32 out
// Both read a 256-row weight tile per k-step; for gate_up its rows are
// W1[n0..+63], W3[n0..+63], W1[n0+64..+127], W3[n0+64..+127], so each wave
// holds the W1 and W3 results of the same h columns and the SiLU*gate product
// is formed in registers.
//
// Data movement: k-steps of 32 (one MFMA k) move through a ring of NS LDS
// stages, filled by direct global->LDS 16-byte loads (no staging registers).
// Each wave issues the same number of loads per stage, so "stage kt has
// landed" is an exact vmcnt wait; NS-1 stages are in flight while one is
// multiplied.  LDS rows are 64 bytes; the 16-byte chunk c of row r sits at
// position c ^ ((r >> 1) & 3): the DMA writes stay 1 KB contiguous per wave,
// and the 8 rows that a 16-byte-per-lane fragment read covers in one LDS
// cycle (rows 8m .. 8m+7, one chunk) fall on 8 distinct 16-byte bank groups
// (with c ^ ((r >> 2) & 3), rows r and r + 2 collided: measured as half of
// all LDS cycles lost to bank conflicts in the prefill GEMM).
//
// FP8 weights (E4M3, two stage widths).  Stages of 32 k: the weight tile is
// staged as E4M3 bytes in 32-byte LDS rows (16-byte chunk c of row r at
// c ^ ((r >> 2) & 1)), one MFMA k-step per stage.  Stages of 64 k: the weight
// tile is staged as OCP E4M3
// bytes in the 64-byte rows of the bf16 layout (so the weight loads are the
// bf16 ones), the A tile as 128-byte rows (chunk c of row r at
// c ^ (r & 7)).  Each stage is two MFMA k-steps in k order, the same sums as
// two bf16 stages.  E4M3 values are bf16 values, so the conversion at
// fragment read is exact; the MFMAs are the bf16 ones, and the per-row weight scale
// multiplies the fp32 sums in the epilogue (weight = code * scale[row], so
// sum_k a_k w_k = scale * sum_k a_k code_k).
//
// Compute: 4 waves, 2 (M) x 2 (N); each wave owns BNB/2 weight rows (MFMA
// column blocks of 16) and the 16-row MFMA row blocks 2i + wm of the m-tile.
// The weight fragment is the MFMA's first operand and the row fragment its
// second, so the accumulator of a lane runs along the output columns (four
// consecutive ones), which makes the output stores 8 or 16 bytes wide.  Row
// blocks past the group's last row are skipped, so a part-filled m-tile costs
// in proportion to its rows.  A rows past the end are loaded clamped to the
// last row (their results are never stored).
#pragma once

#include "common.h"
#include "internal.h"

namespace moe {
namespace {

constexpr int BKS = 32;   // k per stage
constexpr int kCpolNT = 2;  // cache-policy operand of a load: the nt (non-temporal) bit
constexpr int RB = 64;    // LDS bytes per tile row
constexpr int LDS_BYTES = 160 * 1024;

typedef __attribute__((address_space(3))) void* lds_ptr_t;

struct GemmArgs {
  const uint16_t* A;       // [rows, Kdim]
  const void* B0;          // [groups, N, Kdim]  W1 or W2 (bf16, or E4M3 bytes)
  const void* B1;          // [groups, N, Kdim]  W3 (gate_up only)
  const float* S0;         // E4M3 weights: [groups, N] row scales of B0
  const float* S1;         // E4M3 weights: [groups, N] row scales of B1
  void* C;                 // gate_up: bf16 [rows, N]; down: fp32 [rows, N]
  const int4* tab;         // tile table {group, first row, rows, first column}
  const int32_t* count;    // entries in tab
  int N, Kdim;
  // element (row, k) of A at row * a_rs + (k / 32) * a_ks + k % 32, and
  // element (row, n) of C at row * c_rs + (n / 32) * c_bs + n % 32: row-major
  // (a_rs = Kdim, a_ks = 32) or k-blocked [Kdim/32][rows][32] (a_rs = 32,
  // a_ks = 32 * rows), where a k-step's A tile is one contiguous run
  int64_t a_rs, a_ks, c_rs, c_bs;
  // A rows gathered (A mode AM_GATHER): GEMM row r reads A row
  // gather[r] / gather_div (the token of the row's assignment)
  const int32_t* gather;
  int gather_div;
  CombineFuse fuse;        // down: y written through it when fuse.y is set
  // > 0: tiles go to the XCDs in chunks of xcd_chunk consecutive tiles,
  // round-robin (one tile per workgroup), instead of one contiguous range
  // per XCD
  int xcd_chunk;
  // weights (elements of e = 2 bytes for bf16, 1 for E4M3) row-major
  // [groups][N][Kdim], or packed (w_packed) in panels of 64 rows
  // [groups][N/64][Kdim/64][64][64]: element (g, n, k) at byte
  // e (g N Kdim + (n / 64) 64 Kdim + (k / 64) 4096 + (n % 64) 64 + k % 64),
  // so the 64-k steps of a panel follow each other in memory and a stage
  // reads whole runs of 4096 e bytes.  w_bs = bytes between a row's
  // consecutive 64-k steps (64 e row-major, 4096 e packed).
  int w_packed;
  int64_t w_bs;
  // nonzero: the weight DMA loads carry the non-temporal cache policy (for
  // plans whose weight tiles are each read by one m-tile)
  int w_nt;
  // > 0: also for the tiles that hold a whole group of at most w_nt_rows
  // rows (groups from offsets), whose weight tiles no other m-tile reads
  int w_nt_rows;
  const int32_t* offsets;
};

// A operand modes: row-major; k-blocked in blocks of 32 k ([Kdim/32][rows][32])
// or 64 k ([Kdim/64][rows][64]); either k-blocked layout with the GEMM's rows
// gathered from A's rows through GemmArgs::gather.  With 64-k blocks a
// gathered row's piece of a 64-k stage is one whole 128-byte line (with
// 32-k blocks it is two half lines in blocks far apart); or row-major with
// the rows gathered (a 64-k stage's piece of a row is then also one line).
enum { AM_ROW = 0, AM_KB = 1, AM_GATHER = 2, AM_KB64 = 3, AM_GATHER64 = 4, AM_GATHER_ROW = 5 };

__device__ __forceinline__ int lds_pos(int row, int chunk) { return row * RB + ((chunk ^ ((row >> 1) & 3)) << 4); }

// two floats -> two bf16 (round to nearest even), lo in the low half
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// 8 E4M3 bytes (k order, little-endian in lo, hi) -> 8 bf16, exactly
__device__ __forceinline__ bf16x8_t fp8x8_to_bf16(uint32_t lo, uint32_t hi) {
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
  const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  const bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  const bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  bf16x8_t r;
  r[0] = a.x;
  r[1] = a.y;
  r[2] = b.x;
  r[3] = b.y;
  r[4] = c.x;
  r[5] = c.y;
  r[6] = d.x;
  r[7] = d.y;
  return r;
}

// Weight kinds: bf16 in stages of 32 k (64-byte A and weight rows); E4M3 in
// stages of 32 k (64-byte A rows, 32-byte weight rows) or of 64 k (128-byte A
// rows, 64-byte weight rows).
// bf16 weights may also take stages of 64 k (128-byte A and weight rows).
enum { WK_BF16 = 0, WK_E4M3_32 = 1, WK_E4M3_64 = 2, WK_BF16_64 = 3 };
template <int WK>
constexpr int stage_bytes(int bm, int bnb) {
  return WK == WK_BF16_64 ? (bm + bnb) * 2 * RB
                          : (WK == WK_E4M3_64 ? bm * 2 * RB + bnb * RB
                                              : (WK == WK_E4M3_32 ? bm * RB + bnb * 32 : bm * RB + bnb * RB));
}
template <int WK>
constexpr int k_per_stage() {
  return WK == WK_E4M3_64 || WK == WK_BF16_64 ? 2 * BKS : BKS;
}

// byte offset of E4M3 bytes k = 8*lk .. 8*lk+7 of a 32-byte weight row
// (stages of 32 k): chunk c of row r at c ^ ((r >> 2) & 1)
__device__ __forceinline__ int lds_pos8(int row, int lk) {
  return row * 32 + ((((lk >> 1) ^ ((row >> 2) & 1))) << 4) + (lk & 1) * 8;
}

// byte offset of the 16-byte chunk c (bf16 k = 8c .. 8c+7) of a 128-byte A
// row of a 64-k stage: chunk c sits at position c ^ (row & 7)
__device__ __forceinline__ int lds_pos128(int row, int chunk) { return row * 2 * RB + ((chunk ^ (row & 7)) << 4); }

// s_waitcnt vmcnt(N) with N an immediate.
template <int N>
__device__ __forceinline__ void vm_wait() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Wait until at most min(ahead, MAXA) stages of LPS loads each are still
// outstanding (loads complete in issue order).
template <int LPS, int MAXA>
__device__ __forceinline__ void vm_wait_stages(int ahead) {
  if constexpr (MAXA > 0) {
    if (ahead >= MAXA) {
      vm_wait<MAXA * LPS>();
      return;
    }
    vm_wait_stages<LPS, MAXA - 1>(ahead);
  } else {
    vm_wait<0>();
  }
}

// DMA issue state of one workgroup: the table entry of the tile whose
// k-steps are being issued, and of the tile after it.
struct TileRef {
  int g, row_first, rows, n0;  // group, first row, rows, first column
};

// The entry is uniform: it is moved to scalar registers at once, so the wait
// for it happens here (at a tile's start) and no later copy of the issue
// state waits on vector loads in flight (which would drain the DMA ring).
__device__ __forceinline__ TileRef load_tile(const int4* tab, int64_t L) {
  const int4 v = tab[L];
  return TileRef{__builtin_amdgcn_readfirstlane(v.x), __builtin_amdgcn_readfirstlane(v.y),
                 __builtin_amdgcn_readfirstlane(v.z), __builtin_amdgcn_readfirstlane(v.w)};
}

// Per-workgroup constants of the tile sequence.
struct Seq {
  int64_t lbase;    // table index of the first tile
  int lstride;      // table stride between consecutive tiles of this workgroup
  int n_tiles;      // tiles of this workgroup
  int nk;           // k-steps per tile
  int total_steps;  // n_tiles * nk
};

// DMA issue state of one wave: the table entries of the tile whose k-steps
// are being issued and of the tile after it, and this lane's source address
// of every load of a stage, at k-step 0 of the current tile (set when the
// issue crosses into a tile; a stage then only adds k-step x stride).
//
// Lane mapping (chunk swizzles as in lds_pos / lds_pos128 / lds_pos8):
// 64-byte rows: lane -> (row lane/4 of a 16-row group, chunk (lane%4) ^
// ((row >> 1) & 3)); 128-byte rows: (row lane/8 of an 8-row group, chunk
// (lane%8) ^ row); 32-byte E4M3 rows: (row lane/2 of a 32-row group, chunk
// (lane%2) ^ ((row >> 2) & 1)).  A rows past the tile's end are loaded
// clamped to its last row (their results are never stored); weight rows past
// N likewise.
template <int BM, int BNB, int NS, bool GATE_UP, int WK, int AM>
struct Issuer {
  static constexpr bool K64 = k_per_stage<WK>() == 2 * BKS;
  static constexpr int NA = K64 ? BM / 32 : BM / 16 / 4;  // A loads per wave per stage
  static constexpr int NB = WK == WK_BF16_64 ? BNB / 32 : (WK == WK_E4M3_32 ? BNB / 32 / 4 : BNB / 16 / 4);
  static constexpr int HALF = BNB / 4;  // gate_up: rows of one matrix in each quarter of the weight tile
  static constexpr int STAGE = stage_bytes<WK>(BM, BNB);

  static constexpr bool KB64 = AM == AM_KB64 || AM == AM_GATHER64;  // A in blocks of 64 k
  // A row stride: the block width for a k-blocked A (known at compile time),
  // else the caller's
  __device__ __forceinline__ static int64_t a_rs(const GemmArgs& p) {
    return (AM == AM_ROW || AM == AM_GATHER_ROW) ? p.a_rs : (int64_t)(KB64 ? 2 * BKS : BKS);
  }
  // the A row that GEMM row r reads
  __device__ __forceinline__ static int64_t a_row(const GemmArgs& p, int r) {
    if constexpr (AM == AM_GATHER || AM == AM_GATHER64 || AM == AM_GATHER_ROW)
      return (int64_t)(p.gather[r] / p.gather_div);
    return (int64_t)r;
  }

  TileRef cur;   // tile whose k-steps are being issued
  int nt;        // cur's weight loads take the non-temporal policy
  TileRef next;  // the following tile
  int tile;      // position of `cur` in this workgroup's tile sequence
  int64_t aks;   // A bytes per stage along k
  const char* ab[NA];
  const char* wb[NB];

  // weight row (table column) of tile-relative weight row rt, and its matrix
  __device__ __forceinline__ const char* wrow(const GemmArgs& p, int rt, int64_t esz, int64_t off) const {
    const char* base = (const char*)p.B0;
    int col;
    if (GATE_UP) {
      // quarters of the weight tile: W1 half 0, W3 half 0, W1 half 1, W3 half 1
      const int qb = rt / HALF;
      if (qb & 1) base = (const char*)p.B1;
      col = cur.n0 + (qb >> 1) * HALF + rt % HALF;
    } else {
      col = cur.n0 + rt;
    }
    col = min(col, p.N - 1);
    if (p.w_packed)
      return base + ((int64_t)cur.g * p.N * p.Kdim + (int64_t)(col >> 6) * 64 * p.Kdim + (col & 63) * 64) * esz + off;
    return base + (((int64_t)cur.g * p.N + col) * p.Kdim) * esz + off;
  }

  __device__ __forceinline__ void setup(const GemmArgs& p, int wave, int lane) {
    nt = p.w_nt;
    if (!nt && p.w_nt_rows > 0 && cur.rows <= p.w_nt_rows)
      nt = cur.row_first == p.offsets[cur.g] && cur.row_first + cur.rows == p.offsets[cur.g + 1];
    const int rows = cur.rows, row_first = cur.row_first;
    if constexpr (!K64) {
      // 32 k per stage; with 64-k blocks a stage is the half (kt & 1) of
      // block kt >> 1 (issue adds the half's 64 bytes)
      const int r_l = lane >> 2, c_l = (lane & 3) ^ ((r_l >> 1) & 3);
      aks = p.a_ks * 2;
#pragma unroll
      for (int j = 0; j < NA; ++j) {
        const int row = min((wave + 4 * j) * 16 + r_l, rows - 1);
        ab[j] = (const char*)(p.A + a_row(p, row_first + row) * a_rs(p) + c_l * 8);
      }
    } else {
      const int r8 = lane >> 3, ch = (lane & 7) ^ r8;
      aks = KB64 ? p.a_ks * 2 : p.a_ks * 4;
#pragma unroll
      for (int j = 0; j < NA; ++j) {
        const int row = min((wave + 4 * j) * 8 + r8, rows - 1);
        const int64_t kofs = KB64 ? (int64_t)ch * 8 : (int64_t)(ch >> 2) * p.a_ks + (ch & 3) * 8;
        ab[j] = (const char*)(p.A + a_row(p, row_first + row) * a_rs(p) + kofs);
      }
    }
    if constexpr (WK == WK_BF16_64) {
      const int r8 = lane >> 3, ch = (lane & 7) ^ r8;
#pragma unroll
      for (int j = 0; j < NB; ++j) wb[j] = wrow(p, (wave + 4 * j) * 8 + r8, 2, ch * 16);
    } else if constexpr (WK == WK_E4M3_32) {
      const int r2 = lane >> 1, c8 = (lane & 1) ^ ((r2 >> 2) & 1);
#pragma unroll
      for (int j = 0; j < NB; ++j) wb[j] = wrow(p, (wave + 4 * j) * 32 + r2, 1, c8 * 16);
    } else {
      const int r_l = lane >> 2, c_l = (lane & 3) ^ ((r_l >> 1) & 3);
#pragma unroll
      for (int j = 0; j < NB; ++j) wb[j] = wrow(p, (wave + 4 * j) * 16 + r_l, WK == WK_BF16 ? 2 : 1, c_l * 16);
    }
  }

  // Issues the DMA of global step s (tile s / nk, k-step s % nk) into stage s % NS.
  __device__ __forceinline__ void issue(const GemmArgs& p, const Seq& q, char* lds, int s, int wave, int lane) {
    const int ti = s / q.nk, kt = s - ti * q.nk;
    if (ti != tile) {  // crossed into the next tile of the sequence
      tile = ti;
      cur = next;
      if (ti + 1 < q.n_tiles) next = load_tile(p.tab, q.lbase + (int64_t)(ti + 1) * q.lstride);
      setup(p, wave, lane);
    }
    char* const st = lds + (s % NS) * STAGE;
    const int64_t ao = (!K64 && KB64) ? (int64_t)(kt >> 1) * aks + (kt & 1) * 2 * BKS : (int64_t)kt * aks;
    // weight offset of k-step kt: 64-k stage kt is block kt; a 32-k stage
    // is the half (kt & 1) of block kt >> 1
    constexpr int E = (WK == WK_BF16 || WK == WK_BF16_64) ? 2 : 1;  // weight element bytes
    const int64_t wo = K64 ? (int64_t)kt * p.w_bs : (int64_t)(kt >> 1) * p.w_bs + (kt & 1) * 32 * E;
#pragma unroll
    for (int j = 0; j < NA; ++j)
      __builtin_amdgcn_global_load_lds(ab[j] + ao, (lds_ptr_t)(st + (wave + 4 * j) * (K64 ? 8 * 2 * RB : 16 * RB)), 16,
                                       0, 0);
    constexpr int WOFF = BM * (K64 ? 2 * RB : RB);  // weight tile offset in the stage
    constexpr int WLOAD = WK == WK_BF16_64 ? 8 * 2 * RB : (WK == WK_E4M3_32 ? 32 * 32 : 16 * RB);  // bytes per load
    if (nt) {
#pragma unroll
      for (int j = 0; j < NB; ++j)
        __builtin_amdgcn_global_load_lds(wb[j] + wo, (lds_ptr_t)(st + WOFF + (wave + 4 * j) * WLOAD), 16, 0, kCpolNT);
    } else {
#pragma unroll
      for (int j = 0; j < NB; ++j)
        __builtin_amdgcn_global_load_lds(wb[j] + wo, (lds_ptr_t)(st + WOFF + (wave + 4 * j) * WLOAD), 16, 0, 0);
    }
  }
};

// k-loop and epilogue of one tile for a wave that owns NBW active 16-row
// blocks.  `step` is the global step of the tile's first k-step.
template <int BM, int BNB, int NS, bool GATE_UP, int WK, int AM, int NBW>
__device__ __forceinline__ void gemm_tile(Issuer<BM, BNB, NS, GATE_UP, WK, AM>& is, const GemmArgs& p, const Seq& q,
                                          char* lds, const TileRef te,
                                          const int step0, const int wave, const int lane) {
  constexpr bool W8 = WK == WK_E4M3_32 || WK == WK_E4M3_64;  // E4M3 codes: row scales in the epilogue
  constexpr bool K64 = k_per_stage<WK>() == 2 * BKS;
  constexpr int AG = K64 ? BM / 32 : BM / 16 / 4;  // A loads per wave per stage
  constexpr int BG = WK == WK_BF16_64 ? BNB / 32 : (WK == WK_E4M3_32 ? BNB / 32 / 4 : BNB / 16 / 4);  // weight loads
  constexpr int CB = BNB / 32;  // 16-column MFMA blocks per N-wave
  constexpr int LPS = AG + BG;  // loads per wave per stage
  static_assert((NS - 2) * LPS <= 63, "vmcnt counts at most 63 outstanding loads");
  constexpr int STAGE = stage_bytes<WK>(BM, BNB);
  const int wm = wave & 1, wn = wave >> 1;
  const int lr = lane & 15, lk = lane >> 4;

  constexpr int NA = NBW > 0 ? NBW : 1;  // array extent (NBW may be 0)
  f32x4_t acc[NA][CB];
#pragma unroll
  for (int i = 0; i < NBW; ++i)
#pragma unroll
    for (int j = 0; j < CB; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int kt = 0; kt < q.nk; ++kt) {
    const int s = step0 + kt;
    // stage s has landed once at most min(NS-2, total_steps-1-s) later stages are outstanding
    vm_wait_stages<LPS, NS - 2>(q.total_steps - 1 - s);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    const char* st = lds + (s % NS) * STAGE;
    if constexpr (K64) {
      // 64-k stage, two MFMA k-steps in k order (those of two bf16 stages):
      // in step u lane (lr, lk) takes k = 32 u + 8 lk + 0..7, i.e. bytes
      // 32 u + 8 lk .. +7 of its 64-byte E4M3 row and chunk 4 u + lk of its
      // 128-byte A row
      bf16x8_t b0[CB], b1[CB];
#pragma unroll
      for (int j = 0; j < CB; ++j) {
        const int row = wn * (BNB / 2) + j * 16 + lr;
        if constexpr (WK == WK_BF16_64) {
          b0[j] = *(const bf16x8_t*)(st + BM * 2 * RB + lds_pos128(row, lk));
          b1[j] = *(const bf16x8_t*)(st + BM * 2 * RB + lds_pos128(row, 4 + lk));
        } else {
          const uint2 r0 = *(const uint2*)(st + BM * 2 * RB + lds_pos(row, lk >> 1) + (lk & 1) * 8);
          const uint2 r1 = *(const uint2*)(st + BM * 2 * RB + lds_pos(row, 2 + (lk >> 1)) + (lk & 1) * 8);
          b0[j] = fp8x8_to_bf16(r0.x, r0.y);
          b1[j] = fp8x8_to_bf16(r1.x, r1.y);
        }
      }
      bf16x8_t a0[NA], a1[NA];
#pragma unroll
      for (int i = 0; i < NBW; ++i) {
        a0[i] = *(const bf16x8_t*)(st + lds_pos128((2 * i + wm) * 16 + lr, lk));
        a1[i] = *(const bf16x8_t*)(st + lds_pos128((2 * i + wm) * 16 + lr, 4 + lk));
      }
      asm volatile("" ::: "memory");
      if (s + NS - 1 < q.total_steps) is.issue(p, q, lds, s + NS - 1, wave, lane);
#pragma unroll
      for (int i = 0; i < NBW; ++i)
#pragma unroll
        for (int j = 0; j < CB; ++j) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b0[j], a0[i], acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b1[j], a1[i], acc[i][j], 0, 0, 0);
        }
    } else {
      bf16x8_t bfr[CB];
      if constexpr (WK == WK_E4M3_32) {
#pragma unroll
        for (int j = 0; j < CB; ++j) {
          const uint2 raw = *(const uint2*)(st + BM * RB + lds_pos8(wn * (BNB / 2) + j * 16 + lr, lk));
          bfr[j] = fp8x8_to_bf16(raw.x, raw.y);
        }
      } else {
#pragma unroll
        for (int j = 0; j < CB; ++j)
          bfr[j] = *(const bf16x8_t*)(st + BM * RB + lds_pos(wn * (BNB / 2) + j * 16 + lr, lk));
      }
      bf16x8_t afr[NA];
#pragma unroll
      for (int i = 0; i < NBW; ++i) afr[i] = *(const bf16x8_t*)(st + lds_pos((2 * i + wm) * 16 + lr, lk));
      asm volatile("" ::: "memory");
      // refill the stage consumed in the previous step (every wave has passed
      // this step's barrier, so nobody reads it any more); near the end of a
      // tile this already fetches the next tile's first k-steps
      if (s + NS - 1 < q.total_steps) is.issue(p, q, lds, s + NS - 1, wave, lane);
#pragma unroll
      for (int i = 0; i < NBW; ++i)
#pragma unroll
        for (int j = 0; j < CB; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bfr[j], afr[i], acc[i][j], 0, 0, 0);
    }
  }

  // ---- epilogue.  The weight fragment is the MFMA's first operand, so for
  // row block i and column block j lane (lr, lk) holds row (2i+wm)*16 + lr
  // and the four consecutive weight rows lk*4 .. lk*4+3 of block j: one
  // 8-byte store of bf16 h, or one 16-byte store of fp32 yp.
  const int rows = te.rows, n0 = te.n0;
#pragma unroll
  for (int i = 0; i < NBW; ++i) {
    const int r = (2 * i + wm) * 16 + lr;
    if (r >= rows) continue;
    const int64_t orow = (int64_t)(te.row_first + r) * p.c_rs;
    if (GATE_UP) {
      // column blocks j < CB/2 hold W1 results, j + CB/2 the W3 results of the same h columns
      uint16_t* C = (uint16_t*)p.C + orow;
#pragma unroll
      for (int j = 0; j < CB / 2; ++j) {
        const int col = n0 + wn * (BNB / 4) + j * 16 + lk * 4;
        if (col >= p.N) continue;
        f32x4_t g = acc[i][j], u = acc[i][j + CB / 2];
        if constexpr (W8) {
          g *= *(const f32x4_t*)(p.S0 + (int64_t)te.g * p.N + col);
          u *= *(const f32x4_t*)(p.S1 + (int64_t)te.g * p.N + col);
        }
        uint2 o;
        o.x = pack_bf16x2(silu(g[0]) * u[0], silu(g[1]) * u[1]);
        o.y = pack_bf16x2(silu(g[2]) * u[2], silu(g[3]) * u[3]);
        *(uint2*)(C + (int64_t)(col >> 5) * p.c_bs + (col & 31)) = o;
      }
    } else if (p.fuse.y) {
      // combine fused (one assignment per token): y[t] = w[t] * yp_row (+ x[t]),
      // the combine's arithmetic (fmaf(w, yp, 0), then + x, one rounding)
      const int64_t t = p.fuse.row_src[te.row_first + r];
      const float wt = p.fuse.w[t];
#pragma unroll
      for (int j = 0; j < CB; ++j) {
        const int col = n0 + wn * (BNB / 2) + j * 16 + lk * 4;
        if (col >= p.N) continue;
        f32x4_t o = acc[i][j];
        if constexpr (W8) o *= *(const f32x4_t*)(p.S0 + (int64_t)te.g * p.N + col);
        const int64_t yo = t * p.N + col;
        float v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = fmaf(wt, o[u], 0.f);
        if (p.fuse.xres) {
          if (p.fuse.x_bf16) {
            const uint2 xv = *(const uint2*)((const uint16_t*)p.fuse.xres + yo);
            v[0] += bf16_to_f32((uint16_t)xv.x);
            v[1] += bf16_to_f32((uint16_t)(xv.x >> 16));
            v[2] += bf16_to_f32((uint16_t)xv.y);
            v[3] += bf16_to_f32((uint16_t)(xv.y >> 16));
          } else {
            const f32x4_t xv = *(const f32x4_t*)((const float*)p.fuse.xres + yo);
#pragma unroll
            for (int u = 0; u < 4; ++u) v[u] += xv[u];
          }
        }
        if (p.fuse.y_bf16)
          *(uint2*)((uint16_t*)p.fuse.y + yo) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
        else
          *(f32x4_t*)((float*)p.fuse.y + yo) = f32x4_t{v[0], v[1], v[2], v[3]};
      }
    } else {
      float* C = (float*)p.C + orow;
#pragma unroll
      for (int j = 0; j < CB; ++j) {
        const int col = n0 + wn * (BNB / 2) + j * 16 + lk * 4;
        if (col >= p.N) continue;
        f32x4_t o = acc[i][j];
        if constexpr (W8) o *= *(const f32x4_t*)(p.S0 + (int64_t)te.g * p.N + col);
        *(f32x4_t*)(C + (int64_t)(col >> 5) * p.c_bs + (col & 31)) = o;
      }
    }
  }
}

// Persistent grouped GEMM.  The tiles of the table are cut into 8 contiguous
// ranges, one per XCD; the G workgroups of an XCD take its tiles round-robin,
// so the tiles in flight on an XCD at any time are neighbours (same weight
// tile, same rows).  A workgroup's tiles form one stream of k-steps for the
// LDS ring, so the next tile's first stages load while the current tile
// finishes and writes its output.  With one workgroup per tile this is the
// plain one-tile-per-workgroup GEMM.
template <int BM, int BNB, int NS, bool GATE_UP, int WK, int AM>
__global__ __launch_bounds__(256, NS* stage_bytes<WK>(BM, BNB) <= LDS_BYTES / 2 ? 2 : 1) void gemm_bf16_kernel(
    const GemmArgs p) {
  constexpr int MI = BM / 32;  // MFMA row blocks per M-wave
  constexpr int STAGE = stage_bytes<WK>(BM, BNB);
  static_assert(NS * STAGE <= LDS_BYTES, "LDS stages exceed 160 KB");
  __shared__ __attribute__((aligned(1024))) char lds[NS * STAGE];

  const int total = *p.count;
  const int per_xcd = (total + kXcds - 1) / kXcds;
  const int g8 = gridDim.x / kXcds;
  const int xcd = blockIdx.x % kXcds, j = blockIdx.x / kXcds;
  Seq q;
  if (p.xcd_chunk > 0) {
    // chunk k of XCD x is the table's chunk 8 k + x (the launcher sizes the
    // grid to a multiple of 8 chunks covering every tile)
    const int C = p.xcd_chunk;
    const int t = ((j / C) * kXcds + xcd) * C + j % C;
    if (t >= total) return;
    q.lbase = t;
    q.lstride = 1;
    q.n_tiles = 1;
  } else {
    const int begin = xcd * per_xcd, end = min(total, begin + per_xcd);
    if (begin + j >= end) return;
    q.lbase = begin + j;
    q.lstride = g8;
    q.n_tiles = (end - begin - j + g8 - 1) / g8;
  }
  q.nk = p.Kdim / k_per_stage<WK>();
  q.total_steps = q.n_tiles * q.nk;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;

  Issuer<BM, BNB, NS, GATE_UP, WK, AM> is;
  is.tile = 0;
  is.cur = load_tile(p.tab, q.lbase);
  is.next = q.n_tiles > 1 ? load_tile(p.tab, q.lbase + q.lstride) : is.cur;
  is.setup(p, wave, lane);
#pragma unroll
  for (int s = 0; s < NS - 1; ++s)
    if (s < q.total_steps) is.issue(p, q, lds, s, wave, lane);

  for (int t = 0; t < q.n_tiles; ++t) {
    // k-steps issued so far end inside tile t (nk >= NS - 1), so the issue
    // state's current entry is tile t's
    const TileRef te = is.cur;
    const int nbm = (te.rows + 15) >> 4;
    const int nbw = min(MI, (nbm - (wave & 1) + 1) >> 1);
    switch (nbw) {
#define GG_CASE(n)                                                                        \
  case n:                                                                                 \
    if constexpr (n <= MI) gemm_tile<BM, BNB, NS, GATE_UP, WK, AM, n>(is, p, q, lds, te, t * q.nk, wave, lane); \
    break;
      GG_CASE(1) GG_CASE(2) GG_CASE(3) GG_CASE(4) GG_CASE(5) GG_CASE(6) GG_CASE(7) GG_CASE(8)
#undef GG_CASE
      default:
        // no rows in this M half: still take part in the barriers and loads
        gemm_tile<BM, BNB, NS, GATE_UP, WK, AM, 0>(is, p, q, lds, te, t * q.nk, wave, lane);
        break;
    }
  }
}

}  // namespace

// (m-tile rows, weight-tile rows, LDS stages) compiled below: bf16 weights,
// E4M3 weights in stages of 32 k, E4M3 weights in stages of 64 k.  The k-loop
// needs K >= (k per stage) * (NS - 1); the launchers check it.
#define MOE_GEMM_CONFIGS(X) X(128, 256, 3) X(128, 256, 6) X(64, 256, 4) \
  X(128, 128, 4) X(128, 128, 3) X(64, 128, 8) X(64, 128, 6) X(64, 128, 3) X(192, 128, 4) X(192, 128, 3) X(192, 256, 3) \
  X(256, 128, 3)
#define MOE_GEMM8_CONFIGS(X) X(128, 256, 5) X(128, 256, 3) X(128, 128, 6) X(128, 128, 3) X(64, 128, 10) \
  X(64, 128, 3)
#define MOE_GEMM8K64_CONFIGS(X) X(64, 256, 3) X(128, 128, 3) X(128, 128, 2) X(64, 128, 5) X(64, 128, 4) X(64, 128, 2) \
  X(192, 128, 2) X(192, 128, 3)
#define MOE_GEMM16K64_CONFIGS(X) X(192, 128, 3) X(192, 128, 2) X(128, 128, 3) X(128, 128, 2) X(64, 128, 3) \
  X(64, 128, 2) X(64, 256, 3) X(128, 256, 2) X(64, 128, 5) X(64, 256, 2) X(256, 128, 2) X(192, 128, 4) \
  X(128, 256, 3) X(96, 128, 5)

// every configuration fits the tile tables' sizing
#define MOE_FITS_TABLES(B, W, N) \
  static_assert(B >= kMinTileRows && W >= kMinWeightTileRows, "tile tables are sized for larger tiles");
MOE_GEMM_CONFIGS(MOE_FITS_TABLES)
MOE_GEMM8_CONFIGS(MOE_FITS_TABLES)
MOE_GEMM8K64_CONFIGS(MOE_FITS_TABLES)
MOE_GEMM16K64_CONFIGS(MOE_FITS_TABLES)
#undef MOE_FITS_TABLES

// Workgroups to launch: one per tile (upper bound `grid`), or with
// pl.wg_per_cu > 0 a persistent grid of wg_per_cu workgroups per CU.
static inline int64_t launch_grid(const FfnPlan& pl, int64_t grid, int xcd_chunk) {
  if (xcd_chunk > 0 && pl.wg_per_cu <= 0) {
    const int64_t c8 = (int64_t)kXcds * xcd_chunk;
    return (grid + c8 - 1) / c8 * c8;
  }
  if (pl.wg_per_cu <= 0) return grid;
  const int64_t pg = (int64_t)device_cus() * pl.wg_per_cu / kXcds * kXcds;
  return pg < grid ? pg : grid;
}

// a_blk / c_blk: rows of a k-blocked A / h ([cols/kbw][rows][kbw], kbw = 32
// or 64 for A, 32 for h), 0 = row-major.
static inline void set_layout(GemmArgs& a, int64_t a_blk, int64_t c_blk, int kbw = BKS) {
  a.a_rs = a_blk ? kbw : a.Kdim;
  a.a_ks = a_blk ? kbw * a_blk : BKS;
  a.c_rs = c_blk ? 32 : a.N;
  a.c_bs = c_blk ? 32 * c_blk : 32;
}

// weights of esz-byte elements row-major [groups][N][Kdim] or packed in
// 64-row panels [groups][N/64][Kdim/64][64][64]
static inline void set_weight_layout(GemmArgs& a, bool packed, bool nt, int esz) {
  a.w_nt = nt ? 1 : 0;
  a.w_packed = packed ? 1 : 0;
  a.w_bs = (packed ? 64 * 64 : 64) * (int64_t)esz;
}

// the configuration list of the weight kind (pl.w8, k64), each entry expanded by LAUNCH
#define MOE_DISPATCH_KIND(k64, LAUNCH) \
  if (pl.w8 && k64) {                  \
    constexpr int WKV = WK_E4M3_64;    \
    MOE_GEMM8K64_CONFIGS(LAUNCH)       \
  } else if (k64) {                    \
    constexpr int WKV = WK_BF16_64;    \
    MOE_GEMM16K64_CONFIGS(LAUNCH)      \
  } else if (pl.w8) {                  \
    constexpr int WKV = WK_E4M3_32;    \
    MOE_GEMM8_CONFIGS(LAUNCH)          \
  } else {                             \
    constexpr int WKV = WK_BF16;       \
    MOE_GEMM_CONFIGS(LAUNCH)           \
  }

}  // namespace moe
