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
// position c ^ ((r >> 2) & 3), which makes both the DMA writes (1 KB
// contiguous per wave) and the MFMA fragment reads bank-conflict free.
//
// Compute: 4 waves, 2 (M) x 2 (N); each wave owns 128 weight rows (8 MFMA
// column blocks) and the 16-row MFMA row blocks 2i + wm of the m-tile.  Row
// blocks past the group's last row are skipped, so a part-filled m-tile costs
// in proportion to its rows.  A rows past the end are loaded clamped to the
// last row (their results are never stored).
#include "common.h"
#include "internal.h"

namespace moe {
namespace {

constexpr int BKS = 32;   // k per stage
constexpr int RB = 64;    // LDS bytes per tile row
constexpr int BNB = 256;  // weight rows per tile
constexpr int LDS_BYTES = 160 * 1024;

typedef __attribute__((address_space(3))) void* lds_ptr_t;

struct GemmArgs {
  const uint16_t* A;       // [rows, Kdim]
  const uint16_t* B0;      // [groups, N, Kdim]  W1 or W2
  const uint16_t* B1;      // [groups, N, Kdim]  W3 (gate_up only)
  void* C;                 // gate_up: bf16 [rows, N]; down: fp32 [rows, N]
  const int4* tab;         // tile table {group, first row, rows, first column}
  const int32_t* count;    // entries in tab
  int N, Kdim;
};

__device__ __forceinline__ int lds_pos(int row, int chunk) { return row * RB + ((chunk ^ ((row >> 2) & 3)) << 4); }

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

// Per-tile state handed from the kernel's set-up to the k-loop.
struct TileCtx {
  char* lds;
  const uint16_t* a_src[4];
  const uint16_t* b_src[4];
  void* C;
  int64_t out_row0;
  int rows, n0, N, nk, wave, lane;
};

// k-loop and epilogue for a wave that owns NBW active 16-row blocks.
template <int BM, int NS, bool GATE_UP, int NBW>
__device__ __forceinline__ void gemm_tile(const TileCtx& t) {
  constexpr int AG = BM / 16 / 4;   // A 16-row groups loaded per wave per stage
  constexpr int BG = BNB / 16 / 4;  // B 16-row groups loaded per wave per stage
  constexpr int LPS = AG + BG;      // loads per wave per stage
  static_assert((NS - 2) * LPS <= 63, "vmcnt counts at most 63 outstanding loads");
  constexpr int STAGE = (BM + BNB) * RB;
  const int wave = t.wave, lane = t.lane;
  const int wm = wave & 1, wn = wave >> 1;
  const int lr = lane & 15, lk = lane >> 4;
  char* const lds_wave_a = t.lds + wave * 16 * RB;
  char* const lds_wave_b = t.lds + BM * RB + wave * 16 * RB;

#define GG_ISSUE(kt_)                                                                                   \
  do {                                                                                                  \
    const int st_ = (kt_) % NS;                                                                         \
    const int64_t ko_ = (int64_t)(kt_) * BKS;                                                           \
    _Pragma("unroll") for (int j = 0; j < AG; ++j) __builtin_amdgcn_global_load_lds(                   \
        t.a_src[j] + ko_, (lds_ptr_t)(lds_wave_a + st_ * STAGE + j * 4 * 16 * RB), 16, 0, 0);           \
    _Pragma("unroll") for (int j = 0; j < BG; ++j) __builtin_amdgcn_global_load_lds(                   \
        t.b_src[j] + ko_, (lds_ptr_t)(lds_wave_b + st_ * STAGE + j * 4 * 16 * RB), 16, 0, 0);           \
  } while (0)

  constexpr int NA = NBW > 0 ? NBW : 1;  // array extent (NBW may be 0)
  f32x4_t acc[NA][8];
#pragma unroll
  for (int i = 0; i < NBW; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int nk = t.nk;
#pragma unroll
  for (int s = 0; s < NS - 1; ++s)
    if (s < nk) GG_ISSUE(s);

  for (int kt = 0; kt < nk; ++kt) {
    // stage kt has landed once at most min(NS-2, nk-1-kt) later stages are outstanding
    vm_wait_stages<LPS, NS - 2>(nk - 1 - kt);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");

    const char* st = t.lds + (kt % NS) * STAGE;
    bf16x8_t bfr[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      bfr[j] = *(const bf16x8_t*)(st + BM * RB + lds_pos(wn * 128 + j * 16 + lr, lk));
    bf16x8_t afr[NA];
#pragma unroll
    for (int i = 0; i < NBW; ++i) afr[i] = *(const bf16x8_t*)(st + lds_pos((2 * i + wm) * 16 + lr, lk));
    asm volatile("" ::: "memory");
    // refill the stage consumed in the previous iteration (every wave has
    // passed this iteration's barrier, so nobody reads it any more)
    if (kt + NS - 1 < nk) GG_ISSUE(kt + NS - 1);
#pragma unroll
    for (int i = 0; i < NBW; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr[i], bfr[j], acc[i][j], 0, 0, 0);
  }
#undef GG_ISSUE

  // ---- epilogue: lane holds rows (2i+wm)*16 + lk*4 + v, column block j, column lr
#pragma unroll
  for (int i = 0; i < NBW; ++i) {
    const int rb_ = (2 * i + wm) * 16 + lk * 4;
    if (GATE_UP) {
      uint16_t* C = (uint16_t*)t.C;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col = t.n0 + wn * 64 + j * 16 + lr;
        if (col >= t.N) continue;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int rr = rb_ + v;
          if (rr < t.rows) C[(t.out_row0 + rr) * t.N + col] = f32_to_bf16(silu(acc[i][j][v]) * acc[i][j + 4][v]);
        }
      }
    } else {
      float* C = (float*)t.C;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int col = t.n0 + wn * 128 + j * 16 + lr;
        if (col >= t.N) continue;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int rr = rb_ + v;
          if (rr < t.rows) C[(t.out_row0 + rr) * t.N + col] = acc[i][j][v];
        }
      }
    }
  }
}

template <int BM, int NS, bool GATE_UP>
__global__ __launch_bounds__(256, NS*(BM + BNB) * RB <= LDS_BYTES / 2 ? 2 : 1) void gemm_bf16_kernel(const GemmArgs p) {
  constexpr int MI = BM / 32;        // MFMA row blocks per M-wave
  constexpr int AG = BM / 16 / 4;
  constexpr int BG = BNB / 16 / 4;
  static_assert(AG <= 4 && BG <= 4, "TileCtx holds at most 4 source rows per wave");
  constexpr int STAGE = (BM + BNB) * RB;
  static_assert(NS * STAGE <= LDS_BYTES, "LDS stages exceed 160 KB");
  __shared__ __attribute__((aligned(1024))) char lds[NS * STAGE];

  // ---- which tile: one table entry
  const int64_t L = xcd_tile(blockIdx.x, *p.count);
  if (L < 0) return;
  const int4 te = p.tab[L];
  const int g = te.x, row_first = te.y;

  TileCtx t;
  t.lds = lds;
  t.rows = te.z;
  t.n0 = te.w;
  t.N = p.N;
  t.nk = p.Kdim / BKS;
  t.C = p.C;
  t.out_row0 = row_first;
  t.wave = threadIdx.x >> 6;
  t.lane = threadIdx.x & 63;
  const int64_t Kd = p.Kdim;

  // ---- DMA sources: lane -> (row r_l of a 16-row group, chunk c_l)
  const int r_l = t.lane >> 2;
  const int c_l = (t.lane & 3) ^ ((r_l >> 2) & 3);
#pragma unroll
  for (int j = 0; j < AG; ++j) {
    const int row = min((t.wave + 4 * j) * 16 + r_l, t.rows - 1);
    t.a_src[j] = p.A + (int64_t)(row_first + row) * Kd + c_l * 8;
  }
  const int64_t gbase = (int64_t)g * p.N * Kd;
#pragma unroll
  for (int j = 0; j < BG; ++j) {
    const int q16 = t.wave + 4 * j;
    int col;
    const uint16_t* base = p.B0;
    if (GATE_UP) {
      const int qb = q16 >> 2;
      if (qb & 1) base = p.B1;
      col = t.n0 + (qb >> 1) * 64 + (q16 & 3) * 16 + r_l;
    } else {
      col = t.n0 + q16 * 16 + r_l;
    }
    col = min(col, p.N - 1);
    t.b_src[j] = base + gbase + (int64_t)col * Kd + c_l * 8;
  }

  // active 16-row blocks of this wave's M half: blocks 2i + wm
  const int nbm = (t.rows + 15) >> 4;
  const int nbw = min(MI, (nbm - (t.wave & 1) + 1) >> 1);
  switch (nbw) {
#define GG_CASE(n) \
  case n:          \
    if constexpr (n <= MI) gemm_tile<BM, NS, GATE_UP, n>(t); \
    break;
    GG_CASE(1) GG_CASE(2) GG_CASE(3) GG_CASE(4) GG_CASE(5) GG_CASE(6) GG_CASE(7) GG_CASE(8)
#undef GG_CASE
    default:
      // no rows in this M half: still take part in the barriers and loads
      gemm_tile<BM, NS, GATE_UP, 0>(t);
      break;
  }
}

}  // namespace

// (bm, stages) pairs compiled below
#define MOE_GEMM_CONFIGS(X) X(256, 5) X(256, 4) X(128, 6) X(128, 3) X(64, 8) X(64, 4)

int gemm_bf16_default_stages(int bm) { return bm == 256 ? 5 : bm == 128 ? 3 : 4; }

bool gemm_bf16_has_config(int bm, int ns) {
#define MOE_HAS(B, N) \
  if (bm == B && ns == N) return true;
  MOE_GEMM_CONFIGS(MOE_HAS)
#undef MOE_HAS
  return false;
}

hipError_t gemm_bf16_gate_up(const FfnPlan& pl, const void* A, const int4* tab, const int32_t* count, int64_t grid,
                             const void* W1, const void* W3, void* h, int64_t F, int64_t d, hipStream_t s) {
  GemmArgs a{(const uint16_t*)A, (const uint16_t*)W1, (const uint16_t*)W3, h, tab, count, (int)F, (int)d};
#define MOE_LAUNCH(B, N)                                                                     \
  if (pl.bm == B && pl.ns == N) {                                                            \
    gemm_bf16_kernel<B, N, true><<<(unsigned)grid, 256, 0, s>>>(a);                          \
    return hipGetLastError();                                                                \
  }
  MOE_GEMM_CONFIGS(MOE_LAUNCH)
#undef MOE_LAUNCH
  return hipErrorInvalidValue;
}

hipError_t gemm_bf16_down(const FfnPlan& pl, const void* h, const int4* tab, const int32_t* count, int64_t grid,
                          const void* W2, float* yp, int64_t F, int64_t d, hipStream_t s) {
  GemmArgs a{(const uint16_t*)h, (const uint16_t*)W2, nullptr, yp, tab, count, (int)d, (int)F};
#define MOE_LAUNCH(B, N)                                                                     \
  if (pl.bm == B && pl.ns == N) {                                                            \
    gemm_bf16_kernel<B, N, false><<<(unsigned)grid, 256, 0, s>>>(a);                         \
    return hipGetLastError();                                                                \
  }
  MOE_GEMM_CONFIGS(MOE_LAUNCH)
#undef MOE_LAUNCH
  return hipErrorInvalidValue;
}

}  // namespace moe
