// fp32 grouped expert GEMMs (the fp32 layer), the FFN tile plan, and the
// dispatch between the fp32 and bf16 paths.
//
// Same SwiGLU expert as the bf16 path (lnwmold.com article, §2.2): vector
// FMA, 32 x 32 output tiles, k-tiles of 32 staged through LDS, any sizes.
#include <stdlib.h>

#include "common.h"
#include "internal.h"

namespace moe {
namespace {

constexpr int FB = 32;  // rows, columns and k per fp32 tile

struct F32Args {
  const float* A;
  const float* B0;
  const float* B1;
  float* C;
  const int4* tab;       // {group, first row, rows, first column}
  const int32_t* count;  // entries in tab
  int N, Kdim;
};

template <bool GATE_UP>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const F32Args p) {
  __shared__ float as[FB][FB + 1];
  __shared__ float b0s[FB][FB + 1];
  __shared__ float b1s[GATE_UP ? FB : 1][FB + 1];
  const int64_t L = xcd_tile(blockIdx.x, *p.count);
  if (L < 0) return;
  const int4 te = p.tab[L];
  const int g = te.x, row0 = te.y, rows = te.z, n0 = te.w;
  const int m0 = 0;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int64_t gb = (int64_t)g * p.N * p.Kdim;
  float a00 = 0, a01 = 0, a10 = 0, a11 = 0;
  float c00 = 0, c01 = 0, c10 = 0, c11 = 0;
  for (int k0 = 0; k0 < p.Kdim; k0 += FB) {
    for (int q = threadIdx.x; q < FB * FB; q += 256) {
      const int rr = q / FB, kk = q % FB, k = k0 + kk;
      as[rr][kk] = (rr < rows && k < p.Kdim) ? p.A[(int64_t)(row0 + m0 + rr) * p.Kdim + k] : 0.f;
      const int col = n0 + rr;
      const bool ok = col < p.N && k < p.Kdim;
      b0s[rr][kk] = ok ? p.B0[gb + (int64_t)col * p.Kdim + k] : 0.f;
      if (GATE_UP) b1s[rr][kk] = ok ? p.B1[gb + (int64_t)col * p.Kdim + k] : 0.f;
    }
    __syncthreads();
#pragma unroll 8
    for (int kk = 0; kk < FB; ++kk) {
      const float x0 = as[ty * 2][kk], x1 = as[ty * 2 + 1][kk];
      const float w0 = b0s[tx * 2][kk], w1 = b0s[tx * 2 + 1][kk];
      a00 = fmaf(x0, w0, a00);
      a01 = fmaf(x0, w1, a01);
      a10 = fmaf(x1, w0, a10);
      a11 = fmaf(x1, w1, a11);
      if (GATE_UP) {
        const float u0 = b1s[tx * 2][kk], u1 = b1s[tx * 2 + 1][kk];
        c00 = fmaf(x0, u0, c00);
        c01 = fmaf(x0, u1, c01);
        c10 = fmaf(x1, u0, c10);
        c11 = fmaf(x1, u1, c11);
      }
    }
    __syncthreads();
  }
  const float av[2][2] = {{a00, a01}, {a10, a11}};
  const float cv[2][2] = {{c00, c01}, {c10, c11}};
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int rr = ty * 2 + i;
    if (rr >= rows) continue;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = n0 + tx * 2 + j;
      if (col >= p.N) continue;
      const float v = GATE_UP ? silu(av[i][j]) * cv[i][j] : av[i][j];
      p.C[(int64_t)(row0 + m0 + rr) * p.N + col] = v;
    }
  }
}

}  // namespace

int device_cus() {
  static int n_cu = 0;
  if (n_cu == 0) {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
      n_cu = v;
    else
      n_cu = 256;
  }
  return n_cu;
}

bool tuning_enabled() {
  const char* e = getenv("MOE_TUNING");
  return e && e[0] == '1' && e[1] == 0;
}

// a tuning override, or `def` when none is set or tuning is off
static int env_int(const char* name, int def) {
  const char* e = tuning_enabled() ? getenv(name) : nullptr;
  return e ? atoi(e) : def;
}

FfnPlan ffn_plan(bool bf16, bool w8, int64_t max_rows, int64_t group_max, int64_t n_groups, int64_t F, int64_t d,
                 bool packed_up, bool packed_down) {
  if (!bf16) return FfnPlan{FB, 0, 1, 0, 1, 0, FB, FB, false, FB, false, false};
  // Fields: bm, bnb_up, ns_up, bnb_down, ns_down, wg_per_cu, bn_out_up,
  // bn_out_down, w8, bm_down, k64_up, k64_down.
  //
  // bf16 weights: 128-row m-tiles with a 3-stage ring of 256-row weight tiles
  // in stages of 32 k (72 KB of LDS): two workgroups per CU, so one tile's
  // pipeline fill and epilogue overlap the other's main loop.  A GEMM that
  // would have fewer than two such tiles per CU uses 128-row weight tiles (4
  // stages, 64 KB).  Decode-sized groups (at most 64 rows on average): 64-row
  // m-tiles, 128-row weight tiles, 5 stages of 64 k (120 KB).
  // E4M3 weights, always in stages of 64 k (the same weight bytes per stage
  // as bf16 in half the stages): where groups are small (at most 96 rows on
  // average, or an expert capacity of at most 192 rows) the weight stream
  // dominates: 64 x 256 tiles, 3 stages (72 KB), or 64 x 128 tiles, 5 stages,
  // for decode-sized groups; larger groups 192 x 128 tiles, 2 stages.  Stages
  // of 32 k remain available through the tuning overrides.
  const int64_t avg = n_groups > 0 ? max_rows / n_groups : 0;
  const bool small = n_groups > 0 && avg <= 64;
  const bool w8k64 = w8 && n_groups > 0 && (avg <= 96 || group_max <= 192);
  FfnPlan p{128, 256, w8 ? 5 : 3, 256, w8 ? 5 : 3, 0, 128, 256, w8, 128, false, false};
  if (small) {
    // 5 stages (120 KB, one workgroup per CU) for bf16 too: same box,
    // decode 0.532 -> 0.523 ms against 3 stages at two workgroups per CU
    p = w8 ? FfnPlan{64, 128, 5, 128, 5, 0, 64, 128, true, 64, true, true}
           : FfnPlan{64, 128, 5, 128, 5, 0, 64, 128, false, 64, true, true};
    // every weight tile is read by one m-tile: bf16 W1 / W3 stream faster
    // with the non-temporal load policy (same box: Mixtral-shaped decode
    // gate_up 290-293 -> 270-273 us; the DeepSeek-style layer at 512 tokens
    // 2171-2176 -> 1934-1949 us on packed weights), and so do packed E4M3
    // ones (decode 0.396-0.399 -> 0.381-0.385 ms), whose stages then read
    // whole lines; row-major E4M3 weights (225 -> 236 us), the streaming
    // GEMM2 (no change) and the plans whose weight tiles several m-tiles
    // share (DeepSeek-style, prefill, Switch: 5-40% slower) keep the
    // default policy
    p.nt_up = !w8 || packed_up;
  } else if (w8k64) {
    p = FfnPlan{64, 256, 3, 256, 3, 0, 128, 256, true, 64, true, true};
  } else if (w8) {
    // larger E4M3 groups: 192 x 128 tiles, 2 stages of 64 k (64 KB), both
    // GEMMs (same box: FP8 prefill 3.27 -> 2.84 ms, DeepSeek 5.54 -> 5.46 ms
    // against stages of 32 k)
    p = FfnPlan{192, 128, 2, 128, 2, 0, 64, 128, true, 192, true, true};
    // packed W1 / W3: the tiles that hold a whole expert load them
    // non-temporally (same box, DeepSeek-style FP8 layer 4.99-5.02 ->
    // 4.94-4.95 ms)
    if (packed_up) p.nt_rows_up = p.bm;
  } else {
    const int ns_narrow = w8 ? 6 : 4;
    const int64_t mtiles = max_rows / 128 > n_groups ? max_rows / 128 : n_groups;  // rough m-tile count
    const int64_t want = 2 * (int64_t)device_cus();
    if (mtiles * ((F + 127) / 128) < want) {
      p.bnb_up = 128;
      p.ns_up = ns_narrow;
    }
    if (mtiles * ((d + 255) / 256) < want) {
      p.bnb_down = 128;
      p.ns_down = ns_narrow;
    }
  }
  // bf16 GEMM2 m-tiles of 192 rows: when no group can exceed 192 rows but
  // some may exceed 128 (an expert capacity in (128, 192]), every group is
  // one m-tile, so each W2 tile is streamed once and the tile count is
  // E * d / 128 (stages of 32 k, 4 deep); when groups average 512 rows or
  // more (MFMA-bound), stages of 64 k, 2 deep (80 KB): two MFMA k-steps per
  // barrier and each weight fragment reused over 192 rows.
  // Otherwise (groups neither decode-sized nor bounded by such a capacity)
  // GEMM1 takes 192 x 128 tiles in 2 stages of 64 k as well (same box:
  // DeepSeek 6.79 -> 6.46 ms, prefill 3.03 -> 2.95 ms; Switch, whose groups
  // the capacity bounds, is slower with them).
  if (!w8 && p.bm == 128) {
    if (group_max > 128 && group_max <= 192) {
      p.bm_down = 192;
      p.bnb_down = 128;
      p.ns_down = 4;
      // packed W1 / W3: GEMM1 in 192 x 128 tiles, 2 stages of 64 k, as for
      // unbounded groups (same box, Switch: gate_up 235 us on row-major
      // weights in 128 x 256 x 3 of 32 k, 243 packed, 228 packed in these)
      if (packed_up) {
        p.bm = 192;
        p.bnb_up = 128;
        p.ns_up = 2;
        p.k64_up = true;
      }
    } else {
      p.bm_down = p.bm;
      p.bm = 192;
      p.bnb_up = 128;
      p.ns_up = 2;
      p.k64_up = true;
      // the tiles that hold a whole expert read weight tiles that no other
      // m-tile reads: their weight loads take the non-temporal policy (same
      // box, DeepSeek-style gate_up 3.46-3.47 -> 3.41-3.42 ms; GEMM2 and the
      // plans in stages of 32 k, which read each 128-byte line in two
      // stages, gain nothing or lose: Switch down 135 -> 180 us)
      p.nt_rows_up = p.bm;
      // packed W2: GEMM2 in 192 x 128 tiles, 2 stages of 64 k (same box,
      // DeepSeek-style: down 1.93 ms on row-major weights in 128 x 256 x 3 of
      // 32 k, 1.94 packed, 1.89 packed in these)
      if (packed_down) {
        p.bm_down = 192;
        p.bnb_down = 128;
        p.ns_down = 2;
        p.k64_down = true;
      }
      if (avg >= 512) {
        // GEMM1's m-tiles split evenly (same box: prefill gate_up
        // 1.83 -> 1.80 ms; the same split of GEMM2's measured 0.94 -> 0.95)
        p.even_up = true;
        p.nt_rows_up = 0;  // groups of 512 rows and more share every weight tile
        p.bm_down = 192;
        p.bnb_down = 128;
        p.ns_down = 2;
        p.k64_down = true;
      }
    }
  }
  // A ring deeper than the reduction dimension's stages + 1 cannot be
  // filled.  bf16: such a GEMM takes stages of 32 k, 3 deep (every bf16 size
  // is at least 2 of them); E4M3 in stages of 64 k: 2 stages of 128-row
  // weight tiles (every size is at least 1 stage); E4M3 in stages of 32 k:
  // 3 stages.
  auto shallow = [&](int64_t K, bool& k64, int& ns, int& bnb) {
    if (K / (k64 ? 64 : 32) >= ns - 1) return;
    if (!w8 && k64) {
      k64 = false;
      ns = 3;
    } else if (k64) {
      ns = 2;
      bnb = 128;
    } else {
      ns = 3;
    }
  };
  shallow(d, p.k64_up, p.ns_up, p.bnb_up);
  shallow(F, p.k64_down, p.ns_down, p.bnb_down);
  if (!p.k64_up) p.nt_rows_up = 0, p.nt_up = false;  // stages of 32 k read a line in two halves
  if (!p.k64_down) p.nt_rows_down = 0, p.nt_down = false;
  // bf16 weights and at most 32 rows in any group (decode-sized batches):
  // GEMM2 is the weight-streaming kernel, which reads 512 bytes of each
  // weight row per load batch instead of 128 per LDS stage (same box, Mixtral
  // decode: down 196-197 -> 179-182 us on its 28 KB rows; 185-189 with
  // 256-byte batches); GEMM1 keeps the tile kernel (its 8 KB rows stream at
  // 6.1-6.4 TB/s there; the streaming GEMM1 measured 351-370 against
  // 307-317 us on the same box)
  if (!w8 && n_groups > 0 && group_max <= 32) p.stream_down = true;
  // bf16 tile plans other than the decode-sized one deal their tiles to the
  // XCDs in chunks of 16 consecutive tiles, round-robin, instead of one
  // contiguous range per XCD, so every XCD works through every expert's
  // tiles (m-tiles of one weight tile stay together).  Same box, same
  // process: Switch 0.420-0.440 -> 0.403-0.410 ms, prefill 2.82-2.97 ->
  // 2.78-2.80 ms; GEMM2 with 256-row weight tiles (the DeepSeek-style
  // layer's) was slower (1.91 -> 1.96-1.98 ms) and keeps the ranges, and
  // decode's GEMM1 was slower (292-297 -> 322-329 us).
  if (!w8 && !small) {
    p.xcd_chunk_up = 16;
    p.xcd_chunk_down = p.bnb_down == 128 ? 16 : 0;
  }
  // overrides for tuning, honoured with MOE_TUNING=1 only: MOE_GEMM_K64
  // (both GEMMs in stages of 64 k, 0 or 1), MOE_GEMM_K64_DOWN, MOE_GEMM_BM, MOE_GEMM_BM_DOWN,
  // MOE_GEMM_{BNB,NS}_{UP,DOWN}, MOE_GEMM_WGS, MOE_GEMM_EVEN_UP, MOE_GEMM_STREAM{,_UP,_DOWN},
  // MOE_GEMM_STREAM_U, MOE_GEMM_XCD_CHUNK{,_UP,_DOWN}, MOE_GEMM_NT_{UP,DOWN}, MOE_GEMM_NT_ROWS_{UP,DOWN};
  // a set that names no compiled
  // configuration leaves the plan as it was
  const FfnPlan def = p;
  const int k64_env = env_int("MOE_GEMM_K64", -1);
  if (k64_env >= 0) p.k64_up = p.k64_down = k64_env != 0;
  p.k64_down = env_int("MOE_GEMM_K64_DOWN", p.k64_down ? 1 : 0) != 0;
  p.bm = env_int("MOE_GEMM_BM", p.bm);
  p.bm_down = env_int("MOE_GEMM_BM_DOWN", p.bm_down == def.bm ? p.bm : p.bm_down);
  p.bnb_up = env_int("MOE_GEMM_BNB_UP", p.bnb_up);
  p.ns_up = env_int("MOE_GEMM_NS_UP", p.ns_up);
  p.bnb_down = env_int("MOE_GEMM_BNB_DOWN", p.bnb_down);
  p.ns_down = env_int("MOE_GEMM_NS_DOWN", p.ns_down);
  p.wg_per_cu = env_int("MOE_GEMM_WGS", p.wg_per_cu);
  p.even_up = env_int("MOE_GEMM_EVEN_UP", p.even_up ? 1 : 0) != 0;
  const int st_env = env_int("MOE_GEMM_STREAM", -1);  // both GEMMs
  if (st_env >= 0) p.stream_up = p.stream_down = st_env != 0;
  p.stream_up = env_int("MOE_GEMM_STREAM_UP", p.stream_up ? 1 : 0) != 0 && !w8;
  p.stream_down = env_int("MOE_GEMM_STREAM_DOWN", p.stream_down ? 1 : 0) != 0 && !w8;
  p.stream_u = env_int("MOE_GEMM_STREAM_U", p.stream_u);
  const int xc_env = env_int("MOE_GEMM_XCD_CHUNK", -1);  // both GEMMs
  if (xc_env >= 0) p.xcd_chunk_up = p.xcd_chunk_down = xc_env;
  p.xcd_chunk_up = env_int("MOE_GEMM_XCD_CHUNK_UP", p.xcd_chunk_up);
  p.xcd_chunk_down = env_int("MOE_GEMM_XCD_CHUNK_DOWN", p.xcd_chunk_down);
  p.nt_up = env_int("MOE_GEMM_NT_UP", p.nt_up ? 1 : 0) != 0;
  p.nt_rows_up = env_int("MOE_GEMM_NT_ROWS_UP", p.nt_rows_up);
  p.nt_rows_down = env_int("MOE_GEMM_NT_ROWS_DOWN", p.nt_rows_down);
  p.nt_down = env_int("MOE_GEMM_NT_DOWN", p.nt_down ? 1 : 0) != 0;
  if (!gemm_bf16_has_config(w8, p.k64_up, p.bm, p.bnb_up, p.ns_up) ||
      !gemm_bf16_has_config(w8, p.k64_down, p.bm_down, p.bnb_down, p.ns_down) ||
      d / (p.k64_up ? 64 : 32) < p.ns_up - 1 || F / (p.k64_down ? 64 : 32) < p.ns_down - 1)
    p = def;
  p.bn_out_up = p.bnb_up / 2;
  p.bn_out_down = p.bnb_down;
  return p;
}

int64_t ffn_max_mtiles(int bm, int64_t max_rows, int64_t n_groups) {
  // sum over groups of ceil(rows_g / bm) <= floor(max_rows / bm) + n_groups
  return max_rows / bm + n_groups;
}

int64_t ffn_table_entries(bool bf16, int64_t max_rows, int64_t n_groups, int64_t n_cols, bool gate_up) {
  const int bm = bf16 ? kMinTileRows : FB;  // the smallest m-tile any plan uses
  // the narrowest output tiles any plan uses (GEMM1: half the weight rows)
  const int bn = bf16 ? (gate_up ? kMinWeightTileRows / 2 : kMinWeightTileRows) : FB;
  return ffn_max_mtiles(bm, max_rows, n_groups) * ((n_cols + bn - 1) / bn);
}

static int64_t grid_of(int bm, int64_t max_rows, int64_t n_groups, int64_t n_cols, int bn) {
  const int64_t tiles = ffn_max_mtiles(bm, max_rows, n_groups) * ((n_cols + bn - 1) / bn);
  return (tiles + kXcds - 1) / kXcds * kXcds;
}

hipError_t launch_gemm_gate_up(bool bf16, const FfnPlan& p, const AOperand& A, const int4* tab,
                               const int32_t* count, const int32_t* offsets, int64_t n_groups, int64_t max_rows,
                               const void* W1, const void* W3,
                               const float* s1, const float* s3, void* h, int64_t F, int64_t d, hipStream_t s,
                               int prof_id) {
  const int64_t grid = grid_of(p.bm, max_rows, n_groups, F, p.bn_out_up);
  if (grid == 0) return hipSuccess;
  prof_begin(prof_id, s);
  hipError_t err;
  if (p.packed_up && !bf16) return hipErrorInvalidValue;  // packed weights are bf16
  if (bf16 && p.stream_up) {
    err = stream_gate_up(A, offsets, n_groups, W1, W3, h, max_rows, F, d, p.packed_up, p.nt_up, s);
  } else if (bf16) {
    err = gemm_bf16_gate_up(p, A, tab, count, offsets, grid, W1, W3, s1, s3, h, max_rows, F, d, s);
  } else {
    F32Args a{(const float*)A.ptr, (const float*)W1, (const float*)W3, (float*)h, tab, count, (int)F, (int)d};
    gemm_f32_kernel<true><<<(unsigned)grid, 256, 0, s>>>(a);
    err = hipGetLastError();
  }
  prof_end(prof_id, s);
  return err;
}

hipError_t launch_gemm_down(bool bf16, const FfnPlan& p, const void* h, const int4* tab, const int32_t* count,
                            const int32_t* offsets, int64_t n_groups, int64_t max_rows, const void* W2, const float* s2,
                            float* yp, const CombineFuse* fuse, int64_t F, int64_t d, hipStream_t s, int prof_id) {
  if ((fuse && !bf16) || (fuse && p.stream_down)) return hipErrorInvalidValue;
  const int64_t grid = grid_of(p.bm_down, max_rows, n_groups, d, p.bn_out_down);
  if (grid == 0) return hipSuccess;
  prof_begin(prof_id, s);
  hipError_t err;
  if (p.packed_down && !bf16) return hipErrorInvalidValue;
  if (bf16 && p.stream_down) {
    err = stream_down(h, max_rows, offsets, n_groups, W2, yp, F, d, p.stream_u, p.packed_down, p.nt_down, s);
  } else if (bf16) {
    err = gemm_bf16_down(p, h, max_rows, tab, count, offsets, grid, W2, s2, yp, fuse, F, d, s);
  } else {
    F32Args a{(const float*)h, (const float*)W2, nullptr, yp, tab, count, (int)d, (int)F};
    gemm_f32_kernel<false><<<(unsigned)grid, 256, 0, s>>>(a);
    err = hipGetLastError();
  }
  prof_end(prof_id, s);
  return err;
}

}  // namespace moe
