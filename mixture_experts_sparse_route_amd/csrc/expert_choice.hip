// Expert-choice routing: each expert takes its top tokens by affinity
// ("技术日报 2026-04-14" (jsqmd.com), §3.3: S = X W_r^T, expert e takes the
// Top-k of S[:, e]).  The result is written in the K = E form of the routing
// arrays: assignment (t, e) is expert e with the token's softmax gate weight
// [TD §3.2], kept iff e chose t, so dispatch, the expert GEMMs and the combine
// run unchanged.
#include <limits.h>

#include "common.h"
#include "internal.h"
#include "radix_select.h"

namespace moe {
namespace {

// One wave per token: logits (summing the router's S d-slices when S > 1),
// softmax weights w[t][e] = exp(l_e - m) / sum_e' exp(l_e' - m) over all E,
// idx[t][e] = e, and the selection keys of the token for every expert,
// seg[e][t] = order-preserving image of S[t][e] (high word), ~t (low word),
// so a larger key is a larger affinity and equal affinities favour the
// lower token.
__global__ __launch_bounds__(256) void ec_weights_kernel(float* __restrict__ logits, const float* __restrict__ part,
                                                         int S, const float* __restrict__ bias,
                                                         int32_t* __restrict__ idx, float* __restrict__ w,
                                                         uint64_t* __restrict__ seg, int T, int E) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wave;
  if (t >= T) return;
  float* lt = logits + (int64_t)t * E;
  float m = -INFINITY;
  for (int e = lane; e < E; e += 64) {
    float l;
    if (S > 1) {
      // the d-slices' partial sums in slice order, loads issued together
      l = part[(int64_t)t * E + e];
      int q = 1;
      for (; q + 8 <= S; q += 8) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = part[((int64_t)(q + u) * T + t) * E + e];
#pragma unroll
        for (int u = 0; u < 8; ++u) l += v[u];
      }
      for (; q < S; ++q) l += part[((int64_t)q * T + t) * E + e];
      if (bias) l += bias[e];
      lt[e] = l;
    } else {
      l = lt[e];
    }
    m = fmaxf(m, l);
    uint32_t u = __float_as_uint(l + 0.0f);
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    seg[(int64_t)e * T + t] = ((uint64_t)u << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)t);
  }
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  float z = 0.0f;
  for (int e = lane; e < E; e += 64) z += expf(lt[e] - m);
  for (int off = 32; off > 0; off >>= 1) z += __shfl_xor(z, off, 64);
  for (int e = lane; e < E; e += 64) {
    w[(int64_t)t * E + e] = expf(lt[e] - m) / z;
    idx[(int64_t)t * E + e] = e;
  }
}

// One workgroup per expert: the cap-th largest key of the expert's T keys by
// radix select, then the chosen tokens in ascending order get rows
// e*cap .. e*cap + cap - 1.  dest / dropped of every (t, e), counts, offsets.
constexpr int kEcThreads = 1024;

__global__ __launch_bounds__(kEcThreads) void ec_select_kernel(const uint64_t* __restrict__ seg,
                                                               int32_t* __restrict__ counts,
                                                               int32_t* __restrict__ offsets,
                                                               int32_t* __restrict__ dest,
                                                               int32_t* __restrict__ row_src,
                                                               uint8_t* __restrict__ dropped, int T, int E, int cap) {
  __shared__ int hist[256];
  __shared__ int sel[2];
  __shared__ int wtot[kEcThreads / 64];
  const int e = blockIdx.x;
  const uint64_t* s = seg + (int64_t)e * T;
  const uint64_t thr = cap > 0 ? radix_select_desc<kEcThreads>(s, T, cap, hist, sel) : 0ull;
  int run = 0;
  for (int t0 = 0; t0 < T; t0 += kEcThreads) {
    const int t = t0 + threadIdx.x;
    const bool in = t < T;
    const bool keep = in && cap > 0 && s[in ? t : 0] >= thr;
    int tot;
    const int rank = block_rank<kEcThreads>(keep, wtot, &tot);
    if (in) {
      const int64_t f = (int64_t)t * E + e;
      const int32_t row = keep ? e * cap + run + rank : -1;
      dest[f] = row;
      dropped[f] = keep ? 0 : 1;
      if (keep) row_src[row] = (int32_t)f;
    }
    run += tot;
  }
  if (threadIdx.x == 0) {
    counts[e] = cap;
    offsets[e + 1] = (e + 1) * cap;
    if (e == 0) offsets[0] = 0;
  }
}

}  // namespace

hipError_t launch_expert_choice(float* logits, const float* part, int S, const float* bias, int32_t* idx, float* w,
                                uint64_t* seg, int32_t* counts, int32_t* offsets, int32_t* dest, int32_t* row_src,
                                uint8_t* dropped, int64_t T, int64_t E, int64_t cap, hipStream_t s) {
  prof_begin(K_ROUTER_TOPK, s);
  ec_weights_kernel<<<(unsigned)((T + 3) / 4), 256, 0, s>>>(logits, part, S, bias, idx, w, seg, (int)T, (int)E);
  prof_end(K_ROUTER_TOPK, s);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  prof_begin(K_ROUTE_SCATTER, s);
  ec_select_kernel<<<(unsigned)E, kEcThreads, 0, s>>>(seg, counts, offsets, dest, row_src, dropped, (int)T, (int)E,
                                                      (int)cap);
  prof_end(K_ROUTE_SCATTER, s);
  return hipGetLastError();
}

}  // namespace moe
