// Router: logits (a1), gate (a2), Top-K and weights (a3), per-chunk expert
// histogram (input of the capacity scan).
//
// Gate and selection follow "技术日报 2026-04-14" (jsqmd.com): §3.1 Top-K
// (KeepTopK), §3.2 softmax gate, §3.5 sigmoid gate, §4.3 and §9.2 selection-only
// bias, §9.1 renormalised Top-K weights.
#include "common.h"
#include "internal.h"

namespace moe {
namespace {

// ---------------------------------------------------------------- a1 logits
// logits[t][e] = sum_i x[t][i] * Wg[e][i] (+ bias[e]); fp32 FMA in ascending i.
// 64 tokens x 64 experts per workgroup, k-tiles of 32 staged through LDS.
constexpr int LG_T = 64, LG_E = 64, LG_K = 32;

template <typename XT>
__global__ __launch_bounds__(256) void router_logits_kernel(const XT* __restrict__ x, const float* __restrict__ Wg,
                                                            const float* __restrict__ bias, float* __restrict__ logits,
                                                            int T, int d, int E) {
  __shared__ float xs[LG_K][LG_T + 4];
  __shared__ float ws[LG_K][LG_E + 4];
  const int ne = (E + LG_E - 1) / LG_E;
  const int t0 = (blockIdx.x / ne) * LG_T, e0 = (blockIdx.x % ne) * LG_E;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;

  for (int k0 = 0; k0 < d; k0 += LG_K) {
    for (int q = threadIdx.x; q < LG_T * LG_K; q += 256) {
      const int r = q / LG_K, c = q % LG_K;
      const int t = t0 + r, k = k0 + c;
      xs[c][r] = (t < T && k < d) ? load_act(x, (int64_t)t * d + k) : 0.0f;
      const int e = e0 + r;
      ws[c][r] = (e < E && k < d) ? Wg[(int64_t)e * d + k] : 0.0f;
    }
    __syncthreads();
#pragma unroll 8
    for (int c = 0; c < LG_K; ++c) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = xs[c][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = ws[c][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = t0 + ty * 4 + i;
    if (t >= T) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = e0 + tx * 4 + j;
      if (e < E) logits[(int64_t)t * E + e] = acc[i][j] + (bias ? bias[e] : 0.0f);
    }
  }
}

// ------------------------------------------------------- a2 + a3 Top-K
// A token's E experts are spread over a group of L lanes (L = E rounded up to
// a power of two, at most 64); each lane holds P = ceil(E / L) experts.  K
// rounds of a group-wide maximum over packed 64-bit keys select the experts:
// high word = order-preserving image of the fp32 key, low word = ~expert, so
// equal keys resolve to the lower expert.  Each workgroup covers
// kTopkTokens consecutive tokens and also counts its assignments per expert.

__device__ __forceinline__ uint64_t pack_key(float key, int e) {
  uint32_t u = __float_as_uint(key + 0.0f);  // -0 -> +0: signed zeros tie
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)u << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)e);
}

__device__ __forceinline__ uint64_t group_max(uint64_t v, int L) {
  for (int off = L >> 1; off > 0; off >>= 1) {
    const uint64_t o = __shfl_xor(v, off, 64);
    v = o > v ? o : v;
  }
  return v;
}

__device__ __forceinline__ float group_sum(float v, int L) {
  for (int off = L >> 1; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

template <int P>
__global__ __launch_bounds__(256) void router_topk_kernel(const float* __restrict__ logits,
                                                          const float* __restrict__ sel_bias, int32_t* __restrict__ idx,
                                                          float* __restrict__ w, int32_t* __restrict__ blk_count, int T,
                                                          int E, int K, int L, int gate, int renorm, int topk_in) {
  __shared__ int hist[1024];
  for (int e = threadIdx.x; e < E; e += 256) hist[e] = 0;
  __syncthreads();

  const int t_begin = blockIdx.x * kTopkTokens;
  const int t_end = min(T, t_begin + kTopkTokens);
  if (topk_in) {
    for (int f = t_begin * K + threadIdx.x; f < t_end * K; f += 256) {
      const int e = idx[f];
      if (e >= 0 && e < E) atomicAdd(&hist[e], 1);  // out-of-range choices are dropped by the scatter
    }
  } else {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int G = 64 / L;            // tokens per wave per pass
    const int slot = lane / L, ll = lane % L;
    for (int base = t_begin; base < t_end; base += 4 * G) {
      const int t = base + wave * G + slot;
      const bool valid = t < t_end;
      const float* lt = logits + (int64_t)(valid ? t : t_begin) * E;
      uint64_t pk[P];
      float lv[P];
#pragma unroll
      for (int p = 0; p < P; ++p) {
        const int e = ll + L * p;
        pk[p] = 0;
        lv[p] = -INFINITY;
        if (valid && e < E) {
          const float l = lt[e];
          lv[p] = l;
          float key;
          if (gate == 0) {
            key = l;  // softmax is monotone: select on the logit
          } else {
            // sigmoid formed in double and rounded once, then the selection bias
            const float s = (float)(1.0 / (1.0 + exp(-(double)l)));
            key = s + (sel_bias ? sel_bias[e] : 0.0f);
          }
          pk[p] = pack_key(key, e);
        }
      }
      // K rounds of group max; lane ll == k keeps choice k.
      int my_e = -1;
      for (int k = 0; k < K; ++k) {
        uint64_t m = 0;
#pragma unroll
        for (int p = 0; p < P; ++p) m = pk[p] > m ? pk[p] : m;
        m = group_max(m, L);
        const int e = (int)(0xFFFFFFFFu - (uint32_t)(m & 0xFFFFFFFFu));
#pragma unroll
        for (int p = 0; p < P; ++p)
          if (pk[p] == m) pk[p] = 0;
        if (ll == k) my_e = e;
      }
      // weights
      float contrib = 0.0f, mine = 0.0f;
      if (gate == 0) {
        // p_e = exp(l_e - m) / sum; m = the largest logit = the first choice
        const float top = __shfl(my_e >= 0 ? lt[my_e] : -INFINITY, slot * L, 64);
        float zs = 0.0f;
#pragma unroll
        for (int p = 0; p < P; ++p) zs += (lv[p] == -INFINITY) ? 0.0f : expf(lv[p] - top);
        const float z_all = group_sum(zs, L);
        if (my_e >= 0) mine = expf(lt[my_e] - top);
        contrib = mine;
        const float z_sel = group_sum(contrib, L);
        if (valid && my_e >= 0) {
          w[(int64_t)t * K + ll] = mine / (renorm ? z_sel : z_all);
        }
      } else {
        if (my_e >= 0) mine = (float)(1.0 / (1.0 + exp(-(double)lt[my_e])));
        contrib = mine;
        const float z_sel = group_sum(contrib, L);
        if (valid && my_e >= 0) w[(int64_t)t * K + ll] = renorm ? mine / z_sel : mine;
      }
      if (valid && my_e >= 0) {
        idx[(int64_t)t * K + ll] = my_e;
        atomicAdd(&hist[my_e], 1);
      }
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) blk_count[(int64_t)blockIdx.x * E + e] = hist[e];
}

}  // namespace

hipError_t launch_router_logits(bool bf16, const void* x, const float* Wg, const float* bias, float* logits, int64_t T,
                                int64_t d, int64_t E, hipStream_t s) {
  const unsigned grid = (unsigned)(((E + LG_E - 1) / LG_E) * ((T + LG_T - 1) / LG_T));
  prof_begin(K_ROUTER_LOGITS, s);
  if (bf16)
    router_logits_kernel<uint16_t><<<grid, 256, 0, s>>>((const uint16_t*)x, Wg, bias, logits, (int)T, (int)d, (int)E);
  else
    router_logits_kernel<float><<<grid, 256, 0, s>>>((const float*)x, Wg, bias, logits, (int)T, (int)d, (int)E);
  prof_end(K_ROUTER_LOGITS, s);
  return hipGetLastError();
}

hipError_t launch_router_topk(const float* logits, const float* sel_bias, int32_t* idx, float* w, int32_t* blk_count,
                              int64_t T, int64_t E, int64_t K, int gate, bool renorm, bool topk_in, hipStream_t s) {
  int L = 1;
  while (L < E && L < 64) L <<= 1;
  const int P = (int)((E + L - 1) / L);
  const unsigned nb = (unsigned)((T + kTopkTokens - 1) / kTopkTokens);
  prof_begin(K_ROUTER_TOPK, s);
#define MOE_TOPK(PP)                                                                                          \
  router_topk_kernel<PP><<<nb, 256, 0, s>>>(logits, sel_bias, idx, w, blk_count, (int)T, (int)E, (int)K, L, gate, \
                                            renorm ? 1 : 0, topk_in ? 1 : 0)
  if (P <= 1)
    MOE_TOPK(1);
  else if (P <= 2)
    MOE_TOPK(2);
  else if (P <= 4)
    MOE_TOPK(4);
  else if (P <= 8)
    MOE_TOPK(8);
  else
    MOE_TOPK(16);
#undef MOE_TOPK
  prof_end(K_ROUTER_TOPK, s);
  return hipGetLastError();
}

}  // namespace moe
