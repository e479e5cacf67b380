// Weight-streaming grouped expert GEMMs for decode-sized groups (at most 32
// rows per expert): the lnwmold.com article on GPT-4-class sparse activation,
// §2.1, notes that with few tokens the expert FFN's time is the loading of its
// weights, and §2.2 gives the expert's three matrices (W1, W3, W2).
//
// With so few rows the tile kernels' LDS rings buy nothing (every weight
// element meets at most two 16-row MFMA blocks), while their stage structure
// reads only 64-128 bytes of each weight row per barrier; on rows of 14-28 KB
// that spreads every stage over many DRAM pages.  Here each wave owns 16
// weight rows of one expert and streams them straight into registers, U
// consecutive 32-k steps (U * 64 bytes of each row, U = 8 for GEMM2, 4 for
// GEMM1) per load batch, two batches in flight, with no LDS and no barrier;
// the expert's (at most 32) rows of A are read from L2 by every wave that
// needs them.
//
// The MFMAs, their operand fragments and their order over k are those of the
// tile kernels (one v_mfma_f32_16x16x32_bf16 per 32-k step, in k order, the
// weight fragment first), and the epilogues are the same arithmetic, so the
// outputs are bit-identical to the tile kernels'.
#include "common.h"
#include "internal.h"

namespace moe {
namespace {

struct StreamArgs {
  const uint16_t* A;        // element (row, k) at row * a_rs + (k / 32) * a_ks + k % 32
  int64_t a_rs, a_ks;
  const int32_t* gather;    // non-null: GEMM row r reads A row gather[r] / gather_div
  int gather_div;
  const int32_t* offsets;   // [groups + 1] row offsets of the groups
  const uint16_t* B0;       // [groups, N, K] W1 or W2
  const uint16_t* B1;       // [groups, N, K] W3 (gate_up)
  void* C;                  // gate_up: bf16 h, element (row, n) at row * c_rs + (n / 32) * c_bs + n % 32;
                            // down: fp32 yp, the same addressing
  int64_t c_rs, c_bs;
  int N, K;
  // weights packed in 64-row panels [groups][N/64][K/64][64][64] (the tile
  // kernels' packed layout), else row-major
  int w_packed;
  int w_nt;  // weight loads non-temporal
};

__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// Wave w of workgroup (x, g) computes output columns n0 .. n0 + 15, n0 =
// 16 (4x + w), for all rows of group g, in chunks of two 16-row blocks (a
// group of more than 32 rows streams the weights once per chunk).  Lane (lr, lk)
// loads weight row n0 + lr and A row lr of each block, k = 32 kt + 8 lk .. +7
// of step kt, the tile kernels' fragment layout.
template <bool GATE_UP, int U>
__global__ __launch_bounds__(256) void stream_gemm_kernel(const StreamArgs p) {
  const int g = blockIdx.y;
  const int r0 = p.offsets[g], rows = p.offsets[g + 1] - r0;
  if (rows <= 0) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, lr = lane & 15, lk = lane >> 4;
  const int n0 = (blockIdx.x * 4 + wave) * 16;
  if (n0 >= p.N) return;
  // weight element (n, k) of group g: row-major at (g N + n) K + k; packed at
  // g N K + (n / 64) 64 K + (k / 64) 4096 + (n % 64) 64 + k % 64, so 32-k
  // step kt of a row is at (kt / 2) * w_bs + (kt % 2) * 32 from its start
  const int n = min(n0 + lr, p.N - 1);
  const int64_t wofs = p.w_packed ? (int64_t)g * p.N * p.K + (int64_t)(n >> 6) * 64 * p.K + (n & 63) * 64
                                  : ((int64_t)g * p.N + n) * p.K;
  const int64_t w_bs = p.w_packed ? 4096 : 64;
  const uint16_t* b0 = p.B0 + wofs + lk * 8;
  const uint16_t* b1 = GATE_UP ? p.B1 + wofs + lk * 8 : nullptr;
  // A rows past the group's end are loaded clamped to its last row (their
  // results are never stored)
  auto arow = [&](int r) -> int64_t {
    const int rr = r0 + min(r, rows - 1);
    return p.gather ? (int64_t)(p.gather[rr] / p.gather_div) : (int64_t)rr;
  };
  constexpr int NB = GATE_UP ? 2 : 1;  // weight matrices
  struct Batch {
    bf16x8_t w[NB][U];
    bf16x8_t a[2][U];
  };
  const int nk = p.K / 32;  // a multiple of U (checked by the launcher)
  const int col = n0 + lk * 4;

  // rows in chunks of 32 (two 16-row blocks); decode-sized groups are one chunk
  for (int c0 = 0; c0 < rows; c0 += 32) {
    const bool two = rows - c0 > 16;  // a second 16-row block (uniform)
    const uint16_t* a0 = p.A + arow(c0 + lr) * p.a_rs + lk * 8;
    const uint16_t* a1 = p.A + arow(c0 + 16 + lr) * p.a_rs + lk * 8;
    f32x4_t acc[2][NB];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    auto load = [&](Batch& bt, int kt) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t wk = (int64_t)((kt + u) >> 1) * w_bs + ((kt + u) & 1) * 32;
        if (p.w_nt) {
          bt.w[0][u] = __builtin_nontemporal_load((const bf16x8_t*)(b0 + wk));
          if constexpr (GATE_UP) bt.w[1][u] = __builtin_nontemporal_load((const bf16x8_t*)(b1 + wk));
        } else {
          bt.w[0][u] = *(const bf16x8_t*)(b0 + wk);
          if constexpr (GATE_UP) bt.w[1][u] = *(const bf16x8_t*)(b1 + wk);
        }
        bt.a[0][u] = *(const bf16x8_t*)(a0 + (int64_t)(kt + u) * p.a_ks);
      }
      if (two) {
#pragma unroll
        for (int u = 0; u < U; ++u) bt.a[1][u] = *(const bf16x8_t*)(a1 + (int64_t)(kt + u) * p.a_ks);
      }
    };
    auto mma = [&](const Batch& bt) {
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int j = 0; j < NB; ++j)
          acc[0][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bt.w[j][u], bt.a[0][u], acc[0][j], 0, 0, 0);
      if (two) {
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int j = 0; j < NB; ++j)
            acc[1][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bt.w[j][u], bt.a[1][u], acc[1][j], 0, 0, 0);
      }
    };

    // two batches in flight: batch X holds steps kt .. kt+U-1, batch Y the next U
    Batch X, Y;
    load(X, 0);
    for (int kt = 0; kt < nk; kt += 2 * U) {
      const bool y = kt + U < nk;
      if (y) load(Y, kt + U);
      mma(X);
      if (kt + 2 * U < nk) load(X, kt + 2 * U);
      if (y) mma(Y);
    }

    // epilogue: lane (lr, lk) holds row lr of each block and the four
    // consecutive columns n0 + 4 lk .. +3
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = c0 + i * 16 + lr;
      if (r >= rows) continue;
      const int64_t o = (int64_t)(r0 + r) * p.c_rs + (int64_t)(col >> 5) * p.c_bs + (col & 31);
      if constexpr (GATE_UP) {
        const f32x4_t gt = acc[i][0], up = acc[i][1];
        uint2 h;
        h.x = pack2(silu(gt[0]) * up[0], silu(gt[1]) * up[1]);
        h.y = pack2(silu(gt[2]) * up[2], silu(gt[3]) * up[3]);
        *(uint2*)((uint16_t*)p.C + o) = h;
      } else {
        *(f32x4_t*)((float*)p.C + o) = acc[i][0];
      }
    }
  }
}

// U: 32-k steps per load batch, the largest of u_max, 4, 2 that divides K / 32
template <bool GATE_UP>
hipError_t launch_stream(const StreamArgs& a, int64_t n_groups, int u_max, hipStream_t s) {
  const int nk = a.K / 32;
  if (a.K % 64 || a.N % 16 || n_groups < 1 || n_groups > 65535) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((a.N + 63) / 64), (unsigned)n_groups);
  if (!GATE_UP && u_max >= 8 && nk % 8 == 0)
    stream_gemm_kernel<GATE_UP, 8><<<grid, 256, 0, s>>>(a);
  else if (nk % 4 == 0)
    stream_gemm_kernel<GATE_UP, 4><<<grid, 256, 0, s>>>(a);
  else
    stream_gemm_kernel<GATE_UP, 2><<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t stream_gate_up(const AOperand& A, const int32_t* offsets, int64_t n_groups, const void* W1, const void* W3,
                          void* h, int64_t h_blk, int64_t F, int64_t d, bool packed, bool nt, hipStream_t s) {
  if (A.blk_rows && A.kbw != 32) return hipErrorInvalidValue;
  if (A.gather && A.gather_div < 1) return hipErrorInvalidValue;
  StreamArgs a{};
  a.A = (const uint16_t*)A.ptr;
  a.a_rs = A.blk_rows ? 32 : d;
  a.a_ks = A.blk_rows ? 32 * A.blk_rows : 32;
  a.gather = A.gather;
  a.gather_div = A.gather_div;
  a.offsets = offsets;
  a.B0 = (const uint16_t*)W1;
  a.B1 = (const uint16_t*)W3;
  a.C = h;
  a.c_rs = 32;
  a.c_bs = 32 * h_blk;
  a.N = (int)F;
  a.K = (int)d;
  a.w_packed = packed ? 1 : 0;
  a.w_nt = nt ? 1 : 0;
  return launch_stream<true>(a, n_groups, 4, s);
}

hipError_t stream_down(const void* h, int64_t h_blk, const int32_t* offsets, int64_t n_groups, const void* W2,
                       float* yp, int64_t F, int64_t d, int u_max, bool packed, bool nt, hipStream_t s) {
  StreamArgs a{};
  a.A = (const uint16_t*)h;
  a.a_rs = 32;
  a.a_ks = 32 * h_blk;
  a.gather = nullptr;
  a.gather_div = 1;
  a.offsets = offsets;
  a.B0 = (const uint16_t*)W2;
  a.B1 = nullptr;
  a.C = yp;
  a.c_rs = d;
  a.c_bs = 32;
  a.N = (int)d;
  a.K = (int)F;
  a.w_packed = packed ? 1 : 0;
  a.w_nt = nt ? 1 : 0;
  return launch_stream<false>(a, n_groups, u_max, s);
}

}  // namespace moe
