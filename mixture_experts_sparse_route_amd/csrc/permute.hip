// Capacity and stable permutation (a4), dispatch gather (a5), and the tile
// list of the grouped expert GEMMs.
//
// Capacity rule: "技术日报 2026-04-14" (jsqmd.com) §3.2 -- each expert keeps at
// most K_max = floor(C * N_tokens / N_experts) assignments; overflow is dropped.
// The first K_max arrivals in flat (token, choice) order are kept.
#include <limits.h>

#include <algorithm>

#include "common.h"
#include "internal.h"
#include "radix_select.h"

namespace moe {
namespace {

// ------------------------------------------------------------ a4: scan
// One workgroup.  For every expert e: blk_base[b][e] = sum of blk_count[b'][e]
// over chunks b' < b; counts[e] = total demand; offsets = exclusive scan of
// min(counts, cap) with offsets[E] = R.  S threads share each expert's chunk
// range.
//
// With `stats` (router statistics, [TD §4.2 auxiliary losses, §4.4 load
// diagnostics]) the kernel also folds the Top-K kernel's per-chunk sums,
// in double and in chunk order, into
//   stats[e]   = P_e = (1/T) sum_t p[t][e]
//   stats[E+0] = E * sum_e f_e P_e        (Switch balance term, no alpha)
//   stats[E+1] = (1/T) sum_t lse_t^2      (router z-loss)
//   stats[E+2] = E * max_e f_e            (load imbalance factor)
//   stats[E+3] = std(f) / mean(f)         (population std; mean f = 1/E)
//   stats[E+4] = -sum_e P_e ln P_e        (router entropy)
//   stats[E+5] = -sum_e f_e ln f_e
// where f_e = counts[e] / (T*K) is the demand before capacity.
__device__ __forceinline__ double wave_sum(double v) {
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

__device__ __forceinline__ double wave_max(double v) {
  for (int off = 32; off > 0; off >>= 1) v = fmax(v, __shfl_xor(v, off, 64));
  return v;
}

__global__ __launch_bounds__(1024) void route_scan_kernel(const int32_t* __restrict__ blk_count,
                                                          int32_t* __restrict__ blk_base, int32_t* __restrict__ counts,
                                                          int32_t* __restrict__ offsets, int NB, int E, int Epad,
                                                          int cap, const float* __restrict__ blk_P,
                                                          const float* __restrict__ blk_z, double* __restrict__ stats,
                                                          int T, int K, const int32_t* __restrict__ first_counts,
                                                          int32_t* __restrict__ dem_off) {
  __shared__ int part[1024];
  __shared__ int kept[1024];
  __shared__ int dem[1024];
  __shared__ int total[1024];
  __shared__ double dpart[1024];
  __shared__ double red[7][16];
  const int S = 1024 / Epad;
  const int e = threadIdx.x % Epad, sub = threadIdx.x / Epad;
  const int per = (NB + S - 1) / S;
  const int b0 = min(NB, sub * per), b1 = min(NB, b0 + per);
  int sum = 0;
  double psum = 0.0;
  if (e < E) {
    if (stats) {
#pragma unroll 8
      for (int b = b0; b < b1; ++b) {
        sum += blk_count[(int64_t)b * E + e];
        psum += (double)blk_P[(int64_t)b * E + e];
      }
    } else {
#pragma unroll 8
      for (int b = b0; b < b1; ++b) sum += blk_count[(int64_t)b * E + e];
    }
  }
  part[sub * Epad + e] = sum;
  dpart[sub * Epad + e] = psum;
  __syncthreads();
  if (e < E) {
    int run = 0;
    for (int q = 0; q < sub; ++q) run += part[q * Epad + e];
#pragma unroll 8
    for (int b = b0; b < b1; ++b) {
      blk_base[(int64_t)b * E + e] = run;
      run += blk_count[(int64_t)b * E + e];
    }
    if (sub == S - 1) {
      counts[e] = run;
      if (first_counts) {
        // second pass of re-routing: room left after the first pass
        const int k1 = min(first_counts[e], cap);
        kept[e] = k1 + min(run, cap - k1);
      } else {
        kept[e] = min(run, cap);
      }
      total[e] = run;
      dem[e] = run;
    }
  } else if (sub == S - 1) {
    kept[e] = 0;
    dem[e] = 0;
  }
  __syncthreads();
  if (stats) {
    // thread i < E: expert i; every thread adds the chunks' z sums i, i+1024, ...
    const int i = threadIdx.x, wave = i >> 6, lane = i & 63;
    double z = 0.0;
    for (int b = i; b < NB; b += 1024) z += (double)blk_z[b];
    double v[6] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
    if (i < E) {
      double P = 0.0;
      for (int q = 0; q < S; ++q) P += dpart[q * Epad + i];
      P /= (double)T;
      const double f = (double)total[i] / ((double)T * (double)K);
      const double df = f - 1.0 / (double)E;
      stats[i] = P;
      v[0] = f * P;
      v[1] = f;
      v[2] = df * df;
      v[3] = P > 0.0 ? -P * log(P) : 0.0;
      v[4] = f > 0.0 ? -f * log(f) : 0.0;
    }
    v[5] = z;
#pragma unroll
    for (int q = 0; q < 6; ++q) {
      const double r = q == 1 ? wave_max(v[q]) : wave_sum(v[q]);
      if (lane == 0) red[q][wave] = r;
    }
    __syncthreads();
    if (i == 0) {
      double a[6] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
      for (int w = 0; w < 16; ++w)
        for (int q = 0; q < 6; ++q) a[q] = q == 1 ? fmax(a[q], red[q][w]) : a[q] + red[q][w];
      const double En = (double)E;
      stats[E + 0] = En * a[0];
      stats[E + 1] = a[5] / (double)T;
      stats[E + 2] = En * a[1];
      stats[E + 3] = sqrt(a[2] / En) * En;
      stats[E + 4] = a[3];
      stats[E + 5] = a[4];
    }
  }
  // inclusive Hillis-Steele scans of kept[0 .. Epad) (and of the demand for
  // dem_off) with the first Epad threads
  for (int off = 1; off < Epad; off <<= 1) {
    int v = 0, w = 0;
    if (threadIdx.x < Epad && threadIdx.x >= off) {
      v = kept[threadIdx.x - off];
      w = dem[threadIdx.x - off];
    }
    __syncthreads();
    if (threadIdx.x < Epad) {
      kept[threadIdx.x] += v;
      dem[threadIdx.x] += w;
    }
    __syncthreads();
  }
  if (threadIdx.x < E) offsets[threadIdx.x + 1] = kept[threadIdx.x];
  if (threadIdx.x == 0) offsets[0] = 0;
  if (dem_off) {
    if (threadIdx.x < E) dem_off[threadIdx.x + 1] = dem[threadIdx.x];
    if (threadIdx.x == 0) dem_off[0] = 0;
  }
}

// ------------------------------------------------------------ a4: scatter
// Chunk b (ct <= kTopkTokens tokens = ct*K assignments) is ranked in passes
// of 256 assignments.  Within a wave, lanes holding the same expert find each
// other with one ballot per expert-id bit; a lane's rank is the number of
// lower lanes in its peer set.  Per-wave counts are then scanned across the
// four waves in LDS, and a running per-expert count carries across passes.
// pos(f) = blk_base[b][e] + (earlier passes) + (earlier waves) + rank, which
// is the number of assignments before f in flat order with the same expert.
//
// What happens to an assignment past its expert's capacity depends on MODE:
//   kFirstCome   it is dropped [TD §3.2];
//   kAffinity    an expert over capacity has all its assignments written,
//                in flat order, to its segment of `seg` as 64-bit keys
//                (affinity, then the earlier assignment); route_affinity
//                decides them [TD §5.2];
//   kReroute1    first pass of re-routing [LN §3.2]: within-expert ranks of
//                the kept ones go to pos1; the j-th overflowing choice of a
//                token becomes a candidate for the token's rank-(K+j) expert
//                (cand, cand_w), counted per chunk in blk_count2;
//   kReroute2    second pass: candidates (idx = cand) ranked the same way
//                take the room their expert has left; every dest is final.
__device__ __forceinline__ uint64_t affinity_key(float a, int64_t f) {
  uint32_t u = __float_as_uint(a + 0.0f);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)u << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)f);
}

// Rows of m-tile mm of a group of `rows` rows that is cut into `mtiles`
// tiles of at most bm rows (mtiles = ceil(rows / bm), bm a multiple of 32):
// the group's 32-row units (one 16-row MFMA block for each of a tile's two
// M-waves) are dealt out as evenly as possible (the first u % mtiles tiles
// take one unit more), so the m-tiles of one weight tile take about equally
// long and stay in step through k, sharing the weight tile's k-slices in L2.
// u / mtiles <= bm / 32, so no tile exceeds bm rows; every tile holds at
// least one unit, and only the last can be part-filled.
// Returns {first row relative to the group, rows}.
__device__ __forceinline__ int2 mtile_span(int rows, int mtiles, int mm) {
  const int u = (rows + 31) >> 5;
  const int q = u / mtiles, extra = u % mtiles;
  const int r0 = 32 * (mm * q + min(mm, extra));
  return make_int2(r0, min(32 * (q + (mm < extra ? 1 : 0)), rows - r0));
}

// m-tile mm of a group: evenly split (mtile_span) or bm rows from row mm * bm
__device__ __forceinline__ int2 mtile_rows(int rows, int mtiles, int mm, int bm, bool even) {
  return even ? mtile_span(rows, mtiles, mm) : make_int2(mm * bm, min(bm, rows - mm * bm));
}

// The GEMM tile tables (the entries ffn_tiles_kernel writes) from the final
// offsets, by a grid of 256-thread workgroups: every workgroup scans the
// m-tile counts of the G <= 1024 groups in LDS (thread t owns groups 4t ..
// 4t+3), then one wave per group writes that group's contiguous range of
// entries [mstart[g] * nt, mstart[g+1] * nt) with coalesced stores.
__device__ void scatter_tiles(const int32_t* __restrict__ offsets, int G, const TileJob& j) {
  __shared__ int mst[2][1025];
  __shared__ int2 wtot[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int2 m[4];
  int2 tot = make_int2(0, 0);
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int g = 4 * tid + u;
    const int rows = g < G ? offsets[g + 1] - offsets[g] : 0;
    m[u] = rows > 0 ? make_int2((rows + j.bm_up - 1) / j.bm_up, (rows + j.bm_down - 1) / j.bm_down) : make_int2(0, 0);
    tot.x += m[u].x;
    tot.y += m[u].y;
  }
  // inclusive scan of the per-thread totals: within the wave, then over waves
  int2 v = tot;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int ux = __shfl_up(v.x, o), uy = __shfl_up(v.y, o);
    if (lane >= o) {
      v.x += ux;
      v.y += uy;
    }
  }
  if (lane == 63) wtot[wave] = v;
  __syncthreads();
  for (int w = 0; w < wave; ++w) {
    v.x += wtot[w].x;
    v.y += wtot[w].y;
  }
  int2 run = make_int2(v.x - tot.x, v.y - tot.y);
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int g = 4 * tid + u;
    if (g < G) {
      mst[0][g] = run.x;
      mst[1][g] = run.y;
    }
    run.x += m[u].x;
    run.y += m[u].y;
  }
  if (tid == 255) {  // threads past G add nothing: the last inclusive value is the total
    mst[0][G] = v.x;
    mst[1][G] = v.y;
  }
  __syncthreads();
  if (blockIdx.x == 0 && tid == 0) {
    j.counts[0] = mst[0][G] * j.nt_up;
    j.counts[1] = mst[1][G] * j.nt_down;
  }
  for (int pass = 0; pass < 2; ++pass) {
    const int nt = pass == 0 ? j.nt_up : j.nt_down;
    const int bn = pass == 0 ? j.bn_up : j.bn_down;
    const int bm = pass == 0 ? j.bm_up : j.bm_down;
    const bool even = pass == 0 && j.even_up;
    const int* ms = mst[pass];
    int4* tab = pass == 0 ? j.tab_up : j.tab_down;
    for (int gg = blockIdx.x * 4 + wave; gg < G; gg += gridDim.x * 4) {
      const int mtiles = ms[gg + 1] - ms[gg];
      const int cnt = mtiles * nt, base = ms[gg] * nt;
      const int g0 = offsets[gg], g1 = offsets[gg + 1];
      for (int r = lane; r < cnt; r += 64) {
        const int n = r / mtiles, mm = r % mtiles;
        const int2 sp = mtile_rows(g1 - g0, mtiles, mm, bm, even);
        tab[base + r] = make_int4(gg, g0 + sp.x, sp.y, n * bn);
      }
    }
  }
}

// The capacity scan of one chunk (route_scan_kernel with a single chunk and
// no statistics) by one 256-thread workgroup: thread t owns experts 4t ..
// 4t+3; counts[e] = the demand, offsets = exclusive scan of min(demand, cap),
// offsets[E] = R.
__device__ void one_chunk_scan(const int32_t* __restrict__ hist, int32_t* counts, int32_t* offsets, int E, int cap) {
  __shared__ int wtot[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int kept[4], tot = 0;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int e = 4 * tid + u;
    const int c = e < E ? hist[e] : 0;
    if (e < E) counts[e] = c;
    kept[u] = min(c, cap);
    tot += kept[u];
  }
  int v = tot;  // inclusive scan: within the wave, then over the waves
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(v, o);
    if (lane >= o) v += u;
  }
  if (lane == 63) wtot[wave] = v;
  __syncthreads();
  for (int w = 0; w < wave; ++w) v += wtot[w];
  int run = v - tot;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int e = 4 * tid + u;
    if (e < E) offsets[e] = run;
    run += kept[u];
  }
  if (tid == 255) offsets[E] = v;  // threads past E add nothing: the last inclusive value is R
}

template <int MODE>
__global__ __launch_bounds__(256) void route_scatter_kernel(const RouteScatter a, const int T, const int K,
                                                            const int E, const int nbits, const int cap, const int ct) {
  __shared__ int running[1024];
  __shared__ int wcnt[4][1024];
  __shared__ uint8_t ovf[MODE == kReroute1 ? kTopkTokens * 32 : 1];
  __shared__ int hist2[MODE == kReroute1 ? 1024 : 1];
  __shared__ uint8_t dropl[MODE == kFirstCome ? kTopkTokens : 1];  // K == 1: dropped tokens of the chunk
  __shared__ int32_t keptd[MODE == kFirstCome ? kTopkTokens : 1];  // K == 1: their rows (kept tokens)
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t f_begin = (int64_t)blockIdx.x * ct * K;
  const int64_t f_end = min((int64_t)T * K, f_begin + (int64_t)ct * K);
  if (MODE == kFirstCome && a.one_count) {
    // a single chunk: the capacity scan here (every chunk base is 0); the
    // offsets it writes are read back below after a barrier
    one_chunk_scan(a.one_count, a.one_counts, a.one_offsets, E, cap);
    for (int e = threadIdx.x; e < E; e += 256) running[e] = 0;
  } else {
    for (int e = threadIdx.x; e < E; e += 256) {
      running[e] = a.blk_base[(int64_t)blockIdx.x * E + e];
      if constexpr (MODE == kReroute1) hist2[e] = 0;
    }
  }
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int64_t pass = f_begin; pass < f_end; pass += 256) {
    for (int q = threadIdx.x; q < 4 * E; q += 256) wcnt[q / E][q % E] = 0;
    __syncthreads();
    const int64_t f = pass + threadIdx.x;
    int e = f < f_end ? a.idx[f] : -1;
    const bool valid = e >= 0 && e < E;  // out-of-range choices are dropped
    if (!valid) e = 0;
    uint64_t peers = __ballot(valid);
    for (int bit = 0; bit < nbits; ++bit) {
      const bool mine = (e >> bit) & 1;
      const uint64_t bal = __ballot(mine);
      peers &= mine ? bal : ~bal;
    }
    const int rank = __popcll(peers & lt_mask);
    // the highest lane of each peer set publishes the set size
    if (valid && (peers >> lane) == 1ull) wcnt[wave][e] = __popcll(peers);
    __syncthreads();
    int pos = 0;
    if (valid) {
      pos = running[e] + rank;
      for (int q = 0; q < wave; ++q) pos += wcnt[q][e];
    }
    __syncthreads();
    for (int q = threadIdx.x; q < E; q += 256) running[q] += wcnt[0][q] + wcnt[1][q] + wcnt[2][q] + wcnt[3][q];
    if (f < f_end) {
      if constexpr (MODE == kFirstCome) {
        const bool keep = valid && pos < cap;
        const int32_t d = keep ? a.offsets[e] + pos : -1;
        a.dest[f] = d;
        a.dropped[f] = keep ? 0 : 1;
        if (keep) a.row_src[d] = (int32_t)f;
        if (K == 1) {
          dropl[f - f_begin] = keep ? 0 : 1;
          keptd[f - f_begin] = d;
        }
      } else if constexpr (MODE == kAffinity) {
        if (valid && a.counts[e] > cap) {
          a.seg[a.dem_off[e] + pos] = affinity_key(a.aff[f], f);
        } else {
          const int32_t d = valid ? a.offsets[e] + pos : -1;
          a.dest[f] = d;
          a.dropped[f] = valid ? 0 : 1;
          if (valid) a.row_src[d] = (int32_t)f;
        }
      } else if constexpr (MODE == kReroute1) {
        const bool keep = valid && pos < cap;
        a.pos1[f] = keep ? pos : -1;
        ovf[f - f_begin] = keep ? 0 : 1;
      } else {
        const int32_t p1 = a.pos1[f];
        int32_t d = -1;
        if (p1 >= 0) {
          d = a.offsets[a.topk_idx[f]] + p1;
        } else if (valid) {
          const int k1 = min(a.first_counts[e], cap);
          if (pos < cap - k1) d = a.offsets[e] + k1 + pos;
          a.topk_idx[f] = e;
          a.topk_w[f] = a.cand_w[f];
        }
        a.dest[f] = d;
        a.dropped[f] = d >= 0 ? 0 : 1;
        if (d >= 0) a.row_src[d] = (int32_t)f;
      }
    }
    __syncthreads();
  }
  if constexpr (MODE == kFirstCome) {
    if (a.disp_xp && K == 1) {
      // one wave per kept token: its x row, k-block kb (64 bytes = 4 lanes)
      // to row keptd of xp's k-block kb
      const int n = (int)(f_end - f_begin), nkb = a.disp_n_kb;
      const int64_t kb_stride = a.disp_blk_rows * 4;
      const int c = lane & 3;
      for (int i = wave; i < n; i += 4) {
        if (dropl[i]) continue;
        const uint4* src = a.disp_x + (f_begin + i) * (int64_t)nkb * 4 + c;
        uint4* dst = a.disp_xp + (int64_t)keptd[i] * 4 + c;
        for (int kb0 = 0; kb0 < nkb; kb0 += 32) {
          // 32 k-blocks per pass: two loads per lane in flight before the stores
          const int kb1 = kb0 + (lane >> 2), kb2 = kb1 + 16;
          uint4 v1 = make_uint4(0, 0, 0, 0), v2 = v1;
          if (kb1 < nkb) v1 = src[kb1 * 4];
          if (kb2 < nkb) v2 = src[kb2 * 4];
          if (kb1 < nkb) dst[kb1 * kb_stride] = v1;
          if (kb2 < nkb) dst[kb2 * kb_stride] = v2;
        }
      }
    }
    if (a.drop_y && K == 1) {
      // one wave per dropped token of the chunk (token t = assignment f),
      // 8 elements per lane and step (bf16 layers: d is a multiple of 64)
      const int n = (int)(f_end - f_begin), d = a.drop_d;
      for (int i = wave; i < n; i += 4) {
        if (!dropl[i]) continue;
        const int64_t o = (f_begin + i) * (int64_t)d;
        for (int c = lane * 8; c < d; c += 512) {
          float v[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) v[u] = 0.f;
          if (a.drop_x) {
            const uint4 xv = *(const uint4*)(a.drop_x + o + c);
            const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              v[2 * u] += bf16_to_f32((uint16_t)xw[u]);
              v[2 * u + 1] += bf16_to_f32((uint16_t)(xw[u] >> 16));
            }
          }
          if (a.drop_y_bf16) {
            uint32_t yw[4];
#pragma unroll
            for (int u = 0; u < 4; ++u)
              yw[u] = (uint32_t)f32_to_bf16(v[2 * u]) | ((uint32_t)f32_to_bf16(v[2 * u + 1]) << 16);
            *(uint4*)((uint16_t*)a.drop_y + o + c) = make_uint4(yw[0], yw[1], yw[2], yw[3]);
          } else {
            float* yr = (float*)a.drop_y + o + c;
            *(float4*)yr = make_float4(v[0], v[1], v[2], v[3]);
            *(float4*)(yr + 4) = make_float4(v[4], v[5], v[6], v[7]);
          }
        }
      }
    }
  }
  if constexpr (MODE != kReroute1) {
    if (a.tiles.tab_up) scatter_tiles(a.offsets, E, a.tiles);
  }
  if constexpr (MODE == kReroute1) {
    // the j-th overflowing choice of token t (in k order) is offered to the
    // token's rank-(K+j) expert
    for (int64_t f = f_begin + threadIdx.x; f < f_end; f += 256) {
      int32_t c = -1;
      float cw = 0.0f;
      if (ovf[f - f_begin]) {
        const int64_t t = f / K;
        int j = 0;
        for (int64_t q = t * K; q < f; ++q) j += ovf[q - f_begin];
        if (j < a.K2) {
          c = a.alt_idx[t * a.K2 + j];
          cw = a.alt_w[t * a.K2 + j];
        }
        if (c >= 0 && c < E) atomicAdd(&hist2[c], 1);
        else c = -1;
      }
      a.cand[f] = c;
      a.cand_w[f] = cw;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += 256) a.blk_count2[(int64_t)blockIdx.x * E + e] = hist2[e];
  }
}

// ------------------------------------------------------- a4: affinity drop
// One workgroup per expert.  An expert over capacity keeps its `cap`
// largest keys (affinity, then the earlier assignment) [TD §5.2]: a
// most-significant-digit radix select (8 passes of 8 bits over the
// expert's segment) finds the cap-th largest key, then one ordered pass
// gives the kept assignments consecutive rows in flat order.  Experts within
// capacity were finished by the scatter.
__global__ __launch_bounds__(256) void route_affinity_kernel(const uint64_t* __restrict__ seg,
                                                             const int32_t* __restrict__ counts,
                                                             const int32_t* __restrict__ dem_off,
                                                             const int32_t* __restrict__ offsets,
                                                             int32_t* __restrict__ dest, int32_t* __restrict__ row_src,
                                                             uint8_t* __restrict__ dropped, int cap) {
  __shared__ int hist[256];
  __shared__ int sel[2];
  __shared__ int wtot[4];
  const int e = blockIdx.x;
  const int n = counts[e];
  if (n <= cap) return;
  const uint64_t* s = seg + dem_off[e];
  // keep iff key >= thr; cap == 0 keeps none
  const uint64_t thr = cap > 0 ? radix_select_desc<256>(s, n, cap, hist, sel) : 0ull;
  const int base = offsets[e];
  int run = 0;
  for (int i0 = 0; i0 < n; i0 += 256) {
    const int i = i0 + threadIdx.x;
    const bool in = i < n;
    const uint64_t k = in ? s[i] : 0ull;
    const bool keep = in && cap > 0 && k >= thr;
    int tot;
    const int rank = block_rank<256>(keep, wtot, &tot);
    if (in) {
      const int32_t f = (int32_t)(0xFFFFFFFFu - (uint32_t)(k & 0xFFFFFFFFull));
      const int32_t row = keep ? base + run + rank : -1;
      dest[f] = row;
      dropped[f] = keep ? 0 : 1;
      if (keep) row_src[row] = f;
    }
    run += tot;
  }
}

// ------------------------------------------------------------ a5: dispatch
// xp[r] = x[row_src[r] / K] for r < R; R = offsets[E] read on the device.
template <typename V>
__global__ __launch_bounds__(256) void dispatch_kernel(const V* __restrict__ x, const int32_t* __restrict__ row_src,
                                                       const int32_t* __restrict__ R_ptr, V* __restrict__ xp, int K,
                                                       int row_vecs, int rows_per_block) {
  const int R = *R_ptr;
  const int r0 = blockIdx.x * rows_per_block;
  for (int rr = 0; rr < rows_per_block; ++rr) {
    const int r = r0 + rr;
    if (r >= R) return;
    const int64_t t = row_src[r] / K;
    const V* src = x + t * row_vecs;
    V* dst = xp + (int64_t)r * row_vecs;
    for (int c = threadIdx.x; c < row_vecs; c += 256) dst[c] = src[c];
  }
}

// The same into a k-blocked xp (bf16, [d/32][blk_rows][32]): workgroup b
// moves rows 16b .. 16b+15; in each instruction a wave writes one 64-byte
// k-block of those 16 rows, 1 KB contiguous (lane: row lane/4, 16-byte chunk
// lane%4), reading 64 bytes of each row's token.
__global__ __launch_bounds__(256) void dispatch_blocked_kernel(const uint4* __restrict__ x,
                                                               const int32_t* __restrict__ row_src,
                                                               const int32_t* __restrict__ R_ptr,
                                                               uint4* __restrict__ xp, int K, int n_kb,
                                                               int64_t blk_rows) {
  const int R = *R_ptr;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = blockIdx.x * 16 + (lane >> 2), c = lane & 3;
  if (blockIdx.x * 16 >= R) return;
  if (r >= R) return;
  const uint4* src = x + (int64_t)(row_src[r] / K) * n_kb * 4 + c;
  uint4* dst = xp + (int64_t)r * 4 + c;
  const int64_t kb_stride = blk_rows * 4;
  int kb = wave;
  for (; kb + 12 < n_kb; kb += 16) {  // four k-blocks in flight per lane
    const uint4 v0 = src[kb * 4], v1 = src[(kb + 4) * 4], v2 = src[(kb + 8) * 4], v3 = src[(kb + 12) * 4];
    dst[kb * kb_stride] = v0;
    dst[(kb + 4) * kb_stride] = v1;
    dst[(kb + 8) * kb_stride] = v2;
    dst[(kb + 12) * kb_stride] = v3;
  }
  for (; kb < n_kb; kb += 4) dst[kb * kb_stride] = src[kb * 4];
}

// x itself k-blocked: [T, d] -> [d/kbw][T][kbw] with CPB = kbw / 8 16-byte
// chunks per row and block.  Workgroup b takes rows 64/CPB * b onward; in each
// instruction a wave writes one block of those rows, 1 KB contiguous (lane:
// row lane / CPB, chunk lane % CPB), reading 2 kbw bytes of each row.
template <int CPB>
__global__ __launch_bounds__(256) void kblock_copy_kernel(const uint4* __restrict__ x, uint4* __restrict__ xkb, int T,
                                                          int n_kb) {
  constexpr int RPW = 64 / CPB;  // rows per workgroup
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = blockIdx.x * RPW + lane / CPB, c = lane % CPB;
  if (r >= T) return;
  const uint4* src = x + (int64_t)r * n_kb * CPB + c;
  uint4* dst = xkb + (int64_t)r * CPB + c;
  const int64_t kb_stride = (int64_t)T * CPB;
  int kb = wave;
  for (; kb + 12 < n_kb; kb += 16) {  // four blocks in flight per lane
    const uint4 v0 = src[kb * CPB], v1 = src[(kb + 4) * CPB], v2 = src[(kb + 8) * CPB], v3 = src[(kb + 12) * CPB];
    dst[kb * kb_stride] = v0;
    dst[(kb + 4) * kb_stride] = v1;
    dst[(kb + 8) * kb_stride] = v2;
    dst[(kb + 12) * kb_stride] = v3;
  }
  for (; kb < n_kb; kb += 4) dst[kb * kb_stride] = src[kb * CPB];
}

// Weight packing (moe_pack_weights): rows [rows, K] into panels of 64
// rows, [rows/64][K/64][64][64] elements.  CPS = 16-byte chunks in a 64-element
// step of a row (8 for bf16, 4 for E4M3).  A workgroup moves 64 / CPS rows
// (lane: row lane / CPS, chunk lane % CPS); wave w copies the 64-k steps w,
// w + 4, ...
template <int CPS>
__global__ __launch_bounds__(256) void pack_weights_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                           int64_t rows, int n_kb) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t r = (int64_t)blockIdx.x * (64 / CPS) + lane / CPS;
  const int c = lane % CPS;
  if (r >= rows) return;
  const uint4* s = src + r * n_kb * CPS + c;
  uint4* d = dst + (r >> 6) * (int64_t)n_kb * 64 * CPS + (r & 63) * CPS + c;  // a panel step: 64 rows x CPS chunks
  for (int kb = wave; kb < n_kb; kb += 4) d[(int64_t)kb * 64 * CPS] = s[(int64_t)kb * CPS];
}

// ------------------------------------------------------------ FFN tiles
// Tile list of both expert GEMMs (each workgroup scans the m-tile counts and
// writes its share of the entries): for group g with rows(g) rows,
// ceil(rows(g) / bm) m-tiles (bm of that GEMM; GEMM1's split by mtile_span
// when even_up is set) times its n-tiles, in the order
// (group, n-tile, m-tile) with the m-tile fastest, so the m-tiles of one
// weight tile are neighbours.  Entry L = {group, first row, rows, first
// column}; counts[0] / counts[1] = entries of the gate_up / down tables.
__global__ __launch_bounds__(1024) void ffn_tiles_kernel(const int32_t* __restrict__ offsets, int G, int bm_up,
                                                         int nt_up, int bn_up, int bm_down, int nt_down, int bn_down,
                                                         int even_up, int4* __restrict__ tab_up,
                                                         int4* __restrict__ tab_down, int32_t* __restrict__ counts) {
  __shared__ int mstart[2][1025];  // exclusive scans of m-tiles per group (G <= 1024), per GEMM
  __shared__ int2 wsum[16];
  const int g = threadIdx.x, lane = g & 63, wave = g >> 6;
  const int rows = g < G ? offsets[g + 1] - offsets[g] : 0;
  const int2 mt = rows > 0 ? make_int2((rows + bm_up - 1) / bm_up, (rows + bm_down - 1) / bm_down) : make_int2(0, 0);
  // both inclusive scans at once: within the wave, then over the wave totals
  int2 v = mt;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int ux = __shfl_up(v.x, o), uy = __shfl_up(v.y, o);
    if (lane >= o) {
      v.x += ux;
      v.y += uy;
    }
  }
  if (lane == 63) wsum[wave] = v;
  __syncthreads();
  for (int w = 0; w < wave; ++w) {
    v.x += wsum[w].x;
    v.y += wsum[w].y;
  }
  if (g < G) {
    mstart[0][g] = v.x - mt.x;
    mstart[1][g] = v.y - mt.y;
  }
  if (g == 1023) {  // threads past G add nothing: the last inclusive value is the total
    mstart[0][G] = v.x;
    mstart[1][G] = v.y;
  }
  __syncthreads();
  const int tot_up = mstart[0][G] * nt_up, tot_down = mstart[1][G] * nt_down;
  if (g == 0 && blockIdx.x == 0) {
    counts[0] = tot_up;
    counts[1] = tot_down;
  }
  // every workgroup computes the scan; workgroup b writes entries b*1024 + i
  // (+ multiples of the grid's threads)
  for (int pass = 0; pass < 2; ++pass) {
    const int nt = pass == 0 ? nt_up : nt_down;
    const int bn = pass == 0 ? bn_up : bn_down;
    const int tot = pass == 0 ? tot_up : tot_down;
    const int bm = pass == 0 ? bm_up : bm_down;
    const bool even = pass == 0 && even_up;
    const int* ms = mstart[pass];
    int4* tab = pass == 0 ? tab_up : tab_down;
    for (int L = blockIdx.x * 1024 + threadIdx.x; L < tot; L += gridDim.x * 1024) {
      // group of entry L: largest gg with mstart[gg] * nt <= L
      int lo = 0, hi = G;
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (ms[mid] * nt <= L) lo = mid; else hi = mid;
      }
      const int mtiles = ms[lo + 1] - ms[lo];
      const int r = L - ms[lo] * nt;
      const int n = r / mtiles, m = r % mtiles;
      const int2 sp = mtile_rows(offsets[lo + 1] - offsets[lo], mtiles, m, bm, even);
      tab[L] = make_int4(lo, offsets[lo] + sp.x, sp.y, n * bn);
    }
  }
}

}  // namespace

hipError_t launch_route_scan(const int32_t* blk_count, int32_t* blk_base, int32_t* counts, int32_t* offsets,
                             int64_t n_chunks, int64_t E, int64_t cap, const float* blk_P, const float* blk_z,
                             double* stats, int64_t T, int64_t K, const int32_t* first_counts, int32_t* dem_off,
                             hipStream_t s) {
  int Epad = 1;
  while (Epad < E) Epad <<= 1;
  const int capi = cap < 0 || cap > INT_MAX ? INT_MAX : (int)cap;
  prof_begin(K_ROUTE_SCAN, s);
  route_scan_kernel<<<1, 1024, 0, s>>>(blk_count, blk_base, counts, offsets, (int)n_chunks, (int)E, Epad, capi,
                                       blk_P, blk_z, stats, (int)T, (int)K, first_counts, dem_off);
  prof_end(K_ROUTE_SCAN, s);
  return hipGetLastError();
}

hipError_t launch_route_scatter(const RouteScatter& r, int64_t T, int64_t K, int64_t E, int64_t cap, hipStream_t s) {
  int nbits = 0;
  while ((1ll << nbits) < E) ++nbits;
  const int capi = cap < 0 || cap > INT_MAX ? INT_MAX : (int)cap;
  const int ct = chunk_tokens(E, K);
  const unsigned nb = (unsigned)((T + ct - 1) / ct);
  const int Ti = (int)T, Ki = (int)K, Ei = (int)E;
  if (r.one_count && (r.mode != kFirstCome || nb != 1 || E > 1024)) return hipErrorInvalidValue;
  prof_begin(K_ROUTE_SCATTER, s);
  switch (r.mode) {
    case kFirstCome: route_scatter_kernel<kFirstCome><<<nb, 256, 0, s>>>(r, Ti, Ki, Ei, nbits, capi, ct); break;
    case kAffinity: route_scatter_kernel<kAffinity><<<nb, 256, 0, s>>>(r, Ti, Ki, Ei, nbits, capi, ct); break;
    case kReroute1: route_scatter_kernel<kReroute1><<<nb, 256, 0, s>>>(r, Ti, Ki, Ei, nbits, capi, ct); break;
    default: route_scatter_kernel<kReroute2><<<nb, 256, 0, s>>>(r, Ti, Ki, Ei, nbits, capi, ct); break;
  }
  prof_end(K_ROUTE_SCATTER, s);
  return hipGetLastError();
}

hipError_t launch_route_affinity(const uint64_t* seg, const int32_t* counts, const int32_t* dem_off,
                                 const int32_t* offsets, int32_t* dest, int32_t* row_src, uint8_t* dropped, int64_t E,
                                 int64_t cap, hipStream_t s) {
  const int capi = cap < 0 || cap > INT_MAX ? INT_MAX : (int)cap;
  prof_begin(K_ROUTE_SCATTER, s);
  route_affinity_kernel<<<(unsigned)E, 256, 0, s>>>(seg, counts, dem_off, offsets, dest, row_src, dropped, capi);
  prof_end(K_ROUTE_SCATTER, s);
  return hipGetLastError();
}

hipError_t launch_dispatch(const void* x, const int32_t* row_src, const int32_t* R_ptr, void* xp, int64_t max_rows,
                           int64_t K, int64_t row_bytes, bool blocked, hipStream_t s) {
  if (blocked) {
    if (row_bytes % 64) return hipErrorInvalidValue;
    const unsigned nb = (unsigned)((max_rows + 15) / 16);
    if (nb == 0) return hipSuccess;
    prof_begin(K_DISPATCH, s);
    dispatch_blocked_kernel<<<nb, 256, 0, s>>>((const uint4*)x, row_src, R_ptr, (uint4*)xp, (int)K,
                                               (int)(row_bytes / 64), max_rows);
    prof_end(K_DISPATCH, s);
    return hipGetLastError();
  }
  int rpb = row_bytes >= 4096 ? 1 : (int)(4096 / row_bytes);
  if (rpb > 64) rpb = 64;
  const unsigned nb = (unsigned)((max_rows + rpb - 1) / rpb);
  if (nb == 0) return hipSuccess;
  prof_begin(K_DISPATCH, s);
  if (row_bytes % 16 == 0)
    dispatch_kernel<uint4><<<nb, 256, 0, s>>>((const uint4*)x, row_src, R_ptr, (uint4*)xp, (int)K,
                                              (int)(row_bytes / 16), rpb);
  else if (row_bytes % 4 == 0)
    dispatch_kernel<uint32_t><<<nb, 256, 0, s>>>((const uint32_t*)x, row_src, R_ptr, (uint32_t*)xp, (int)K,
                                                 (int)(row_bytes / 4), rpb);
  else
    dispatch_kernel<uint16_t><<<nb, 256, 0, s>>>((const uint16_t*)x, row_src, R_ptr, (uint16_t*)xp, (int)K,
                                                 (int)(row_bytes / 2), rpb);
  prof_end(K_DISPATCH, s);
  return hipGetLastError();
}

TileJob tile_job(const FfnPlan& p, int64_t F, int64_t d, int4* tab_up, int4* tab_down, int32_t* counts) {
  TileJob j{};
  j.bm_up = p.bm;
  j.nt_up = (int)((F + p.bn_out_up - 1) / p.bn_out_up);
  j.bn_up = p.bn_out_up;
  j.bm_down = p.bm_down;
  j.nt_down = (int)((d + p.bn_out_down - 1) / p.bn_out_down);
  j.bn_down = p.bn_out_down;
  j.even_up = p.even_up ? 1 : 0;
  j.tab_up = tab_up;
  j.tab_down = tab_down;
  j.counts = counts;
  return j;
}

hipError_t launch_kblock_copy(const void* x, void* xkb, int64_t T, int64_t row_bytes, int kbw, hipStream_t s) {
  if ((kbw != 32 && kbw != 64) || row_bytes % (2 * kbw) || T > INT32_MAX) return hipErrorInvalidValue;
  const int rpw = kbw == 64 ? 8 : 16;
  const unsigned nb = (unsigned)((T + rpw - 1) / rpw);
  if (nb == 0) return hipSuccess;
  const int n_kb = (int)(row_bytes / (2 * kbw));
  prof_begin(K_DISPATCH, s);
  if (kbw == 64)
    kblock_copy_kernel<8><<<nb, 256, 0, s>>>((const uint4*)x, (uint4*)xkb, (int)T, n_kb);
  else
    kblock_copy_kernel<4><<<nb, 256, 0, s>>>((const uint4*)x, (uint4*)xkb, (int)T, n_kb);
  prof_end(K_DISPATCH, s);
  return hipGetLastError();
}

hipError_t launch_pack_weights(const void* src, void* dst, int64_t rows, int64_t K, int esz, hipStream_t s) {
  if (rows % 64 || K % 64 || rows < 64 || K < 64 || (esz != 1 && esz != 2)) return hipErrorInvalidValue;
  if (esz == 2)
    pack_weights_kernel<8><<<(unsigned)(rows / 8), 256, 0, s>>>((const uint4*)src, (uint4*)dst, rows, (int)(K / 64));
  else
    pack_weights_kernel<4><<<(unsigned)(rows / 16), 256, 0, s>>>((const uint4*)src, (uint4*)dst, rows, (int)(K / 64));
  return hipGetLastError();
}

hipError_t launch_ffn_tiles(const FfnPlan& p, const int32_t* offsets, int64_t n_groups, int64_t max_rows, int64_t F,
                            int64_t d, int4* tab_up, int4* tab_down, int32_t* counts, hipStream_t s) {
  const int nt_up = (int)((F + p.bn_out_up - 1) / p.bn_out_up);
  const int nt_down = (int)((d + p.bn_out_down - 1) / p.bn_out_down);
  // enough workgroups for the largest table this plan can produce, at most 32
  const int64_t most = std::max(ffn_max_mtiles(p.bm, max_rows, n_groups) * nt_up,
                                ffn_max_mtiles(p.bm_down, max_rows, n_groups) * nt_down);
  const unsigned grid = (unsigned)std::min<int64_t>(32, std::max<int64_t>(1, (most + 1023) / 1024));
  prof_begin(K_FFN_TILES, s);
  ffn_tiles_kernel<<<grid, 1024, 0, s>>>(offsets, (int)n_groups, p.bm, nt_up, p.bn_out_up, p.bm_down, nt_down,
                                         p.bn_out_down, p.even_up ? 1 : 0, tab_up, tab_down, counts);
  prof_end(K_FFN_TILES, s);
  return hipGetLastError();
}

}  // namespace moe
