// Router: logits (a1), gate (a2), Top-K and weights (a3), per-chunk expert
// histogram (input of the capacity scan).
//
// Gate and selection follow "技术日报 2026-04-14" (jsqmd.com): §3.1 Top-K
// (KeepTopK), §3.2 softmax gate, §3.5 sigmoid gate, §4.3 and §9.2 selection-only
// bias, §9.1 renormalised Top-K weights.
#include <stdlib.h>

#include "common.h"
#include "internal.h"

namespace moe {
namespace {

// ---------------------------------------------------------------- a1 logits
// logits[t][e] = sum_i x[t][i] * Wg[e][i] (+ bias[e]).
//
// bf16 x: bf16 MFMA.  Each fp32 router weight is split exactly into three
// bf16 parts, w = hi + mid + lo (hi = bf16(w), mid = bf16(w - hi),
// lo = w - hi - mid, each difference exact in fp32), so every product
// x * part is exact in fp32 and the fp32 MFMA accumulation gives an fp32 dot
// product of the unrounded operands.  Work is cut into 64-token x EW-expert
// tiles and S slices of d; slice s writes its partial sums to part[s] and the
// Top-K kernel adds the S slices in order.  With S == 1 the tile writes the
// logits (plus bias) directly.
// fp32 x: the same tiling with fp32 FMA.
constexpr int LG_T = 64, LG_K = 32;

// 16-byte chunk c of 64-byte row r at c ^ ((r >> 1) & 3): the 8 rows a
// 16-byte-per-lane read covers in one LDS cycle fall on 8 distinct 16-byte
// bank groups
__device__ __forceinline__ int lg_pos(int row, int chunk) { return row * 64 + ((chunk ^ ((row >> 1) & 3)) << 4); }

__device__ __forceinline__ void split3(float w, uint16_t& hi, uint16_t& mid, uint16_t& lo) {
  hi = f32_to_bf16(w);
  const float r1 = w - bf16_to_f32(hi);
  mid = f32_to_bf16(r1);
  const float r2 = r1 - bf16_to_f32(mid);
  lo = f32_to_bf16(r2);
}

template <int EW>
__global__ __launch_bounds__(256) void router_logits_mfma_kernel(const uint16_t* __restrict__ x,
                                                                 const float* __restrict__ Wg,
                                                                 const float* __restrict__ bias, float* __restrict__ out,
                                                                 int T, int d, int E, int S) {
  constexpr int WE = EW == 64 ? 2 : 1;     // waves along experts
  constexpr int WT = 4 / WE;               // waves along tokens
  constexpr int TB = LG_T / WT / 16;       // 16-token blocks per wave
  constexpr int EB = EW / WE / 16;         // 16-expert blocks per wave
  __shared__ __attribute__((aligned(16))) char xs[2][LG_T * 64];
  __shared__ __attribute__((aligned(16))) char ws[2][3][EW * 64];

  const int ne = (E + EW - 1) / EW, nt = (T + LG_T - 1) / LG_T;
  const int b = blockIdx.x;
  const int s = b / (ne * nt);
  const int et = (b / nt) % ne, tt = b % nt;
  const int t0 = tt * LG_T, e0 = et * EW;
  const int kr = d / S, kbeg = s * kr;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;

  // staging: one 16-byte chunk of x per thread; EW*8 float4 chunks of Wg
  const int xr = tid >> 2, xc = tid & 3;
  const bool x_ok = t0 + xr < T;
  const uint16_t* xsrc = x + (int64_t)(x_ok ? t0 + xr : 0) * d + kbeg + xc * 8;
  constexpr int WL = EW * 8 / 256 > 0 ? EW * 8 / 256 : 1;  // float4 loads per thread
  // two register sets: k-step kt+2 loads while kt+1 waits to be staged
  uint4 xregA, xregB;
  float4 wregA[WL], wregB[WL];
  // Loads are unconditional (rows past T or E are clamped and zeroed when
  // staged): straight-line loads let the compiler wait for exactly the
  // register set being staged instead of draining every load in flight.
  const float* wsrc[WL];
  bool w_ok[WL];
#pragma unroll
  for (int i = 0; i < WL; ++i) {
    const int q = (tid + 256 * i) % (EW * 8);
    const int er = q >> 3, c4 = q & 7;
    w_ok[i] = tid + 256 * i < EW * 8 && e0 + er < E;
    wsrc[i] = Wg + (int64_t)min(e0 + er, E - 1) * d + kbeg + c4 * 4;
  }
  auto gload = [&](uint4& xreg, float4 (&wreg)[WL], int k0) {
    xreg = *(const uint4*)(xsrc + k0);
#pragma unroll
    for (int i = 0; i < WL; ++i) wreg[i] = *(const float4*)(wsrc[i] + k0);
  };
  auto lstore = [&](const uint4& xreg, const float4 (&wreg)[WL], int st) {
    *(uint4*)(xs[st] + lg_pos(xr, xc)) = x_ok ? xreg : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < WL; ++i) {
      const int q = tid + 256 * i;
      if (q >= EW * 8) continue;
      const int er = q >> 3, c4 = q & 7;
      const float4 wv = w_ok[i] ? wreg[i] : make_float4(0.f, 0.f, 0.f, 0.f);
      const float f[4] = {wv.x, wv.y, wv.z, wv.w};
      uint16_t hi[4], mi[4], lo[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) split3(f[u], hi[u], mi[u], lo[u]);
      const int off = lg_pos(er, c4 >> 1) + (c4 & 1) * 8;
      *(uint2*)(ws[st][0] + off) = make_uint2(hi[0] | (uint32_t)hi[1] << 16, hi[2] | (uint32_t)hi[3] << 16);
      *(uint2*)(ws[st][1] + off) = make_uint2(mi[0] | (uint32_t)mi[1] << 16, mi[2] | (uint32_t)mi[3] << 16);
      *(uint2*)(ws[st][2] + off) = make_uint2(lo[0] | (uint32_t)lo[1] << 16, lo[2] | (uint32_t)lo[3] << 16);
    }
  };

  const int wt = wave / WE, we = wave % WE;
  const int lr = lane & 15, lk = lane >> 4;
  f32x4_t acc[TB][EB];
#pragma unroll
  for (int i = 0; i < TB; ++i)
#pragma unroll
    for (int j = 0; j < EB; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int cur) {
    bf16x8_t af[TB];
#pragma unroll
    for (int i = 0; i < TB; ++i) af[i] = *(const bf16x8_t*)(xs[cur] + lg_pos((wt * TB + i) * 16 + lr, lk));
#pragma unroll
    for (int p = 0; p < 3; ++p) {
#pragma unroll
      for (int j = 0; j < EB; ++j) {
        const bf16x8_t bfr = *(const bf16x8_t*)(ws[cur][p] + lg_pos((we * EB + j) * 16 + lr, lk));
#pragma unroll
        for (int i = 0; i < TB; ++i) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr, acc[i][j], 0, 0, 0);
      }
    }
  };

  // LDS buffer kt % 2 holds k-step kt; register set A holds even k-steps,
  // B odd ones, loaded two k-steps before they are staged.  The barriers
  // wait only for this thread's LDS traffic (lgkmcnt), not for the global
  // loads in flight (a plain __syncthreads would drain those every k-step);
  // a register set is waited for where lstore reads it.
  auto lds_barrier = [] {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  // Every load is issued (k-steps past the end reload the last one and are
  // never multiplied), so the loop has no branch around a load.
  const int nk = kr / LG_K;
  auto kofs = [&](int kt) { return min(kt, nk - 1) * LG_K; };
  gload(xregA, wregA, 0);
  gload(xregB, wregB, kofs(1));
  lstore(xregA, wregA, 0);
  lds_barrier();
  for (int kt = 0; kt < nk; kt += 2) {
    gload(xregA, wregA, kofs(kt + 2));
    compute(0);
    lstore(xregB, wregB, 1);
    lds_barrier();
    if (kt + 1 < nk) compute(1);
    gload(xregB, wregB, kofs(kt + 3));
    lstore(xregA, wregA, 0);
    lds_barrier();
  }
  // lane holds tokens (block*16 + lk*4 + v), expert (block*16 + lr)
#pragma unroll
  for (int i = 0; i < TB; ++i)
#pragma unroll
    for (int j = 0; j < EB; ++j) {
      const int e = e0 + (we * EB + j) * 16 + lr;
      if (e >= E) continue;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int t = t0 + (wt * TB + i) * 16 + lk * 4 + v;
        if (t >= T) continue;
        if (S == 1)
          out[(int64_t)t * E + e] = acc[i][j][v] + (bias ? bias[e] : 0.0f);
        else
          out[((int64_t)s * T + t) * E + e] = acc[i][j][v];
      }
    }
}

// fp32 x: 64 tokens x 64 experts per workgroup, fp32 FMA, same slices.
__global__ __launch_bounds__(256) void router_logits_f32_kernel(const float* __restrict__ x,
                                                                const float* __restrict__ Wg,
                                                                const float* __restrict__ bias, float* __restrict__ out,
                                                                int T, int d, int E, int S) {
  constexpr int LE = 64;
  __shared__ float xs[LG_K][LG_T + 4];
  __shared__ float wsh[LG_K][LE + 4];
  const int ne = (E + LE - 1) / LE, nt = (T + LG_T - 1) / LG_T;
  const int b = blockIdx.x;
  const int s = b / (ne * nt);
  const int et = (b / nt) % ne, tt = b % nt;
  const int t0 = tt * LG_T, e0 = et * LE;
  const int kr = (d + S - 1) / S, kbeg = s * kr, kend = min(d, kbeg + kr);
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;
  for (int k0 = kbeg; k0 < kend; k0 += LG_K) {
    for (int q = threadIdx.x; q < LG_T * LG_K; q += 256) {
      const int r = q / LG_K, c = q % LG_K;
      const int t = t0 + r, k = k0 + c;
      xs[c][r] = (t < T && k < kend) ? x[(int64_t)t * d + k] : 0.0f;
      const int e = e0 + r;
      wsh[c][r] = (e < E && k < kend) ? Wg[(int64_t)e * d + k] : 0.0f;
    }
    __syncthreads();
#pragma unroll 8
    for (int c = 0; c < LG_K; ++c) {
      float a[4], bb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = xs[c][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) bb[j] = wsh[c][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], bb[j], acc[i][j]);
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
      if (e >= E) continue;
      if (S == 1)
        out[(int64_t)t * E + e] = acc[i][j] + (bias ? bias[e] : 0.0f);
      else
        out[((int64_t)s * T + t) * E + e] = acc[i][j];
    }
  }
}

// ------------------------------------------------------- a2 + a3 Top-K
// A token's E experts are spread over a group of L lanes (L = E rounded up to
// a power of two, at most 64); each lane holds P = ceil(E / L) experts.  K
// rounds of a group-wide maximum over packed 64-bit keys select the experts:
// high word = order-preserving image of the fp32 key, low word = ~expert, so
// equal keys resolve to the lower expert.  Each workgroup covers
// ct <= kTopkTokens consecutive tokens and also counts its assignments per
// expert.

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

// part[0][i] + part[1][i] + ... + part[S-1][i], added in slice order; the
// loads are issued 32 at a time so they overlap instead of forming one
// dependent chain of S loads.
__device__ __forceinline__ float sum_slices(const float* __restrict__ part, int S, int64_t stride, int64_t i) {
  float l = part[i];
  int q = 1;
  for (; q + 32 <= S; q += 32) {
    float v[32];
#pragma unroll
    for (int u = 0; u < 32; ++u) v[u] = part[(int64_t)(q + u) * stride + i];
#pragma unroll
    for (int u = 0; u < 32; ++u) l += v[u];
  }
  for (; q + 8 <= S; q += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = part[(int64_t)(q + u) * stride + i];
#pragma unroll
    for (int u = 0; u < 8; ++u) l += v[u];
  }
  for (; q < S; ++q) l += part[(int64_t)q * stride + i];
  return l;
}

__device__ __forceinline__ float group_maxf(float v, int L) {
  for (int off = L >> 1; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

// With STATS the kernel also writes, per workgroup b, the router distribution
// summed over its tokens, blk_P[b][e] = sum_t p[t][e], and blk_z[b] =
// sum_t lse_t^2 with lse_t = log sum_e exp(logit[t][e])  ([TD §4.2] P_i and
// the z-loss).  p is the softmax over all E logits (softmax gate) or the
// sigmoid scores normalised over all E experts (sigmoid gate).  Each lane
// keeps its running sums in registers; the tokens of a wave are then added
// by a butterfly and the four waves in wave order, so the sums have a fixed
// order.
template <int P, bool STATS>
__global__ __launch_bounds__(256) void router_topk_kernel(float* __restrict__ logits, const float* __restrict__ part,
                                                          int S, const float* __restrict__ bias,
                                                          const float* __restrict__ sel_bias, int32_t* __restrict__ idx,
                                                          float* __restrict__ w, int32_t* __restrict__ blk_count,
                                                          float* __restrict__ blk_P, float* __restrict__ blk_z,
                                                          int32_t* __restrict__ alt_idx, float* __restrict__ alt_w,
                                                          int K2, int T, int E, int K, int L, int gate, int renorm,
                                                          int topk_in, int ct) {
  __shared__ int hist[1024];
  __shared__ float wsum[STATS ? 4 : 1][STATS ? 1024 : 1];
  __shared__ float wz[4];
  for (int e = threadIdx.x; e < E; e += 256) hist[e] = 0;
  __syncthreads();
  float pacc[P];
  float zacc = 0.0f;
#pragma unroll
  for (int p = 0; p < P; ++p) pacc[p] = 0.0f;

  const int t_begin = blockIdx.x * ct;
  const int t_end = min(T, t_begin + ct);
  // Many d-slices (small T): the chunk's logits first, all threads over its
  // (token, expert) pairs, so the long slice sums run in parallel; with few
  // slices each lane sums its own experts' slices in the selection loop.
  const bool presum = !topk_in && S >= 8;
  if (presum) {
    // the d-slices' partial sums in slice order, then the bias
    const int n = (t_end - t_begin) * E;
    for (int i = threadIdx.x; i < n; i += 256) {
      const int64_t te = (int64_t)t_begin * E + i;
      float l = sum_slices(part, S, (int64_t)T * E, te);
      if (bias) l += bias[i % E];
      logits[te] = l;
    }
    __syncthreads();  // the selection below reads them back (same workgroup)
  }
  if (topk_in) {
    for (int f = t_begin * K + threadIdx.x; f < t_end * K; f += 256) {
      const int e = idx[f];
      if (e >= 0 && e < E) atomicAdd(&hist[e], 1);  // out-of-range choices are dropped by the scatter
    }
  } else {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int G = 64 / L;            // tokens per wave per pass
    const int slot = lane / L, ll = lane % L;
    // This lane's logits of token t (its experts ll + L*p): with d-slices,
    // their partial sums added in slice order, then the bias.  Every load of
    // a block of slices (and the bias) is issued before the first add, so a
    // pass waits for about one load latency rather than one per expert.
    const bool sliced = S > 1 && !presum;
    auto gather = [&](int t, bool valid, float (&l)[P]) {
      int64_t off[P];
      float b[P];
#pragma unroll
      for (int p = 0; p < P; ++p) {
        const int e = ll + L * p;
        const bool ok = valid && e < E;
        off[p] = ok ? (int64_t)t * E + e : (int64_t)t_begin * E;  // unused lanes read an in-range element
        b[p] = (sliced && bias) ? bias[ok ? e : 0] : 0.0f;
      }
      if (sliced) {
        const int64_t stride = (int64_t)T * E;
#pragma unroll
        for (int p = 0; p < P; ++p) l[p] = part[off[p]];
        int q = 1;
        for (; q + 4 <= S; q += 4) {
          float v[4][P];
#pragma unroll
          for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int p = 0; p < P; ++p) v[u][p] = part[(int64_t)(q + u) * stride + off[p]];
#pragma unroll
          for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int p = 0; p < P; ++p) l[p] += v[u][p];
        }
        for (; q < S; ++q) {
          float v[P];
#pragma unroll
          for (int p = 0; p < P; ++p) v[p] = part[(int64_t)q * stride + off[p]];
#pragma unroll
          for (int p = 0; p < P; ++p) l[p] += v[p];
        }
        if (bias) {
#pragma unroll
          for (int p = 0; p < P; ++p) l[p] += b[p];
        }
      } else {
#pragma unroll
        for (int p = 0; p < P; ++p) l[p] = logits[off[p]];
      }
    };
    // the next pass's logits load while this pass selects
    float lcur[P], lnext[P];
#pragma unroll
    for (int p = 0; p < P; ++p) lnext[p] = 0.0f;
    gather(t_begin + wave * G + slot, t_begin + wave * G + slot < t_end, lcur);
    for (int base = t_begin; base < t_end; base += 4 * G) {
      const int t = base + wave * G + slot;
      const bool valid = t < t_end;
      if (base + 4 * G < t_end) {
        const int tn = t + 4 * G;
        gather(tn, tn < t_end, lnext);
      }
      uint64_t pk[P];
      float lv[P], sv[P];
#pragma unroll
      for (int p = 0; p < P; ++p) {
        const int e = ll + L * p;
        pk[p] = 0;
        lv[p] = -INFINITY;
        sv[p] = 0.0f;
        if (valid && e < E) {
          const float l = lcur[p];
          if (sliced) logits[(int64_t)t * E + e] = l;
          lv[p] = l;
          float key;
          if (gate == 0) {
            key = l;  // softmax is monotone: select on the logit
          } else {
            // sigmoid formed in double and rounded once, then the selection bias
            const float s = (float)(1.0 / (1.0 + exp(-(double)l)));
            sv[p] = s;
            key = s + (sel_bias ? sel_bias[e] : 0.0f);
          }
          pk[p] = pack_key(key, e);
        }
      }
      // K rounds of group max; lane ll == k keeps choice k and its logit,
      // fetched from the lane that holds that expert.  K2 more rounds give
      // the re-routing alternates (ranks K .. K+K2-1), kept by lane k - K.
      int my_e = -1, alt_e = -1;
      float my_l = -INFINITY, alt_l = -INFINITY;
      for (int k = 0; k < K + K2; ++k) {
        uint64_t m = 0;
#pragma unroll
        for (int p = 0; p < P; ++p) m = pk[p] > m ? pk[p] : m;
        m = group_max(m, L);
        const int e = (int)(0xFFFFFFFFu - (uint32_t)(m & 0xFFFFFFFFu));
#pragma unroll
        for (int p = 0; p < P; ++p)
          if (pk[p] == m) pk[p] = 0;
        const int pe = e >= 0 ? e / L : 0, oe = e >= 0 ? e % L : 0;
        float v = lv[0];
#pragma unroll
        for (int p = 1; p < P; ++p)
          if (p == pe) v = lv[p];
        const float le = __shfl(v, slot * L + oe, 64);
        if (k < K) {
          if (ll == k) {
            my_e = e;
            my_l = le;
          }
        } else if (ll == k - K) {
          alt_e = e;
          alt_l = le;
        }
      }
      // weights
      float contrib = 0.0f, mine = 0.0f;
      float top = 0.0f, z_all = 1.0f;
      float ez[P];
      if (gate == 0) {
        // p_e = exp(l_e - m) / sum; m = the largest logit = the first choice
        top = __shfl(my_l, slot * L, 64);
        float zs = 0.0f;
#pragma unroll
        for (int p = 0; p < P; ++p) {
          ez[p] = (lv[p] == -INFINITY) ? 0.0f : expf(lv[p] - top);
          zs += ez[p];
        }
        z_all = group_sum(zs, L);
        if (my_e >= 0) mine = expf(my_l - top);
        contrib = mine;
        const float z_sel = group_sum(contrib, L);
        if (valid && my_e >= 0) {
          w[(int64_t)t * K + ll] = mine / (renorm ? z_sel : z_all);
        }
        if (valid && alt_e >= 0) {
          alt_idx[(int64_t)t * K2 + ll] = alt_e;
          alt_w[(int64_t)t * K2 + ll] = expf(alt_l - top) / (renorm ? z_sel : z_all);
        }
      } else {
        if (my_e >= 0) mine = (float)(1.0 / (1.0 + exp(-(double)my_l)));
        contrib = mine;
        const float z_sel = group_sum(contrib, L);
        if (valid && my_e >= 0) w[(int64_t)t * K + ll] = renorm ? mine / z_sel : mine;
        if (valid && alt_e >= 0) {
          const float sa = (float)(1.0 / (1.0 + exp(-(double)alt_l)));
          alt_idx[(int64_t)t * K2 + ll] = alt_e;
          alt_w[(int64_t)t * K2 + ll] = renorm ? sa / z_sel : sa;
        }
      }
      if (valid && my_e >= 0) {
        idx[(int64_t)t * K + ll] = my_e;
        atomicAdd(&hist[my_e], 1);
      }
      if constexpr (STATS) {
        float lse;
        if (gate == 0) {
          lse = top + logf(z_all);
#pragma unroll
          for (int p = 0; p < P; ++p) ez[p] = ez[p] / z_all;
        } else {
          float ss = 0.0f, mx = -INFINITY;
#pragma unroll
          for (int p = 0; p < P; ++p) {
            ss += sv[p];
            mx = fmaxf(mx, lv[p]);
          }
          ss = group_sum(ss, L);
          mx = group_maxf(mx, L);
          float es = 0.0f;
#pragma unroll
          for (int p = 0; p < P; ++p) es += (lv[p] == -INFINITY) ? 0.0f : expf(lv[p] - mx);
          lse = mx + logf(group_sum(es, L));
#pragma unroll
          for (int p = 0; p < P; ++p) ez[p] = sv[p] / ss;
        }
        if (valid) {
#pragma unroll
          for (int p = 0; p < P; ++p)
            if (ll + L * p < E) pacc[p] += ez[p];
          if (ll == 0) zacc += lse * lse;
        }
      }
#pragma unroll
      for (int p = 0; p < P; ++p) lcur[p] = lnext[p];
    }
  }
  if constexpr (STATS) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    // add the wave's token slots (lanes with equal ll) and its z terms
    for (int off = 64 >> 1; off > 0; off >>= 1) zacc += __shfl_xor(zacc, off, 64);
    for (int off = L; off < 64; off <<= 1) {
#pragma unroll
      for (int p = 0; p < P; ++p) pacc[p] += __shfl_xor(pacc[p], off, 64);
    }
    if (lane < L) {
#pragma unroll
      for (int p = 0; p < P; ++p)
        if (lane + L * p < E) wsum[wave][lane + L * p] = pacc[p];
    }
    if (lane == 0) wz[wave] = zacc;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) {
    blk_count[(int64_t)blockIdx.x * E + e] = hist[e];
    if constexpr (STATS) blk_P[(int64_t)blockIdx.x * E + e] = ((wsum[0][e] + wsum[1][e]) + wsum[2][e]) + wsum[3][e];
  }
  if constexpr (STATS)
    if (threadIdx.x == 0) blk_z[blockIdx.x] = ((wz[0] + wz[1]) + wz[2]) + wz[3];
}

}  // namespace

int router_splits(int64_t T, int64_t d, int64_t E, bool bf16) {
  const int64_t ew = (!bf16 || E > 16) ? 64 : 16;
  const int64_t tiles = ((T + LG_T - 1) / LG_T) * ((E + ew - 1) / ew);
  // split d until there is a workgroup per CU and no slice is longer than
  // 4096 (a slice is one workgroup's serial chain of 32-wide k-steps; more
  // slices cost the Top-K kernel their partial sums).  Tuning override
  // (read once, with MOE_TUNING=1 only): MOE_ROUTER_WGS, a workgroup count to
  // reach instead.
  static const int64_t want_env = [] {
    const char* v = tuning_enabled() ? getenv("MOE_ROUTER_WGS") : nullptr;
    const long n = v ? atol(v) : 0;
    return n > 0 ? (int64_t)n : (int64_t)0;
  }();
  const int64_t want = want_env > 0 ? want_env : (int64_t)device_cus();
  int S = 1;
  while ((tiles * S < want || (want_env == 0 && d / S > 4096)) && S < 64 && d % ((int64_t)S * 2 * LG_K) == 0) S *= 2;
  return S;
}

hipError_t launch_router_logits(bool bf16, const void* x, const float* Wg, const float* bias, float* logits,
                                float* part, int64_t T, int64_t d, int64_t E, hipStream_t s) {
  const int S = router_splits(T, d, E, bf16);
  float* out = S == 1 ? logits : part;
  prof_begin(K_ROUTER_LOGITS, s);
  if (bf16) {
    if (E <= 16) {
      const unsigned grid = (unsigned)(((T + LG_T - 1) / LG_T) * S);
      router_logits_mfma_kernel<16><<<grid, 256, 0, s>>>((const uint16_t*)x, Wg, bias, out, (int)T, (int)d, (int)E, S);
    } else {
      const unsigned grid = (unsigned)(((T + LG_T - 1) / LG_T) * ((E + 63) / 64) * S);
      router_logits_mfma_kernel<64><<<grid, 256, 0, s>>>((const uint16_t*)x, Wg, bias, out, (int)T, (int)d, (int)E, S);
    }
  } else {
    const unsigned grid = (unsigned)(((T + LG_T - 1) / LG_T) * ((E + 63) / 64) * S);
    router_logits_f32_kernel<<<grid, 256, 0, s>>>((const float*)x, Wg, bias, out, (int)T, (int)d, (int)E, S);
  }
  prof_end(K_ROUTER_LOGITS, s);
  return hipGetLastError();
}

hipError_t launch_router_topk(float* logits, const float* part, int S, const float* bias, const float* sel_bias,
                              int32_t* idx, float* w, int32_t* blk_count, float* blk_P, float* blk_z, int32_t* alt_idx,
                              float* alt_w, int64_t K2, int64_t T, int64_t E, int64_t K, int gate, bool renorm,
                              bool topk_in, hipStream_t s) {
  // lanes per token: a power of two with at most 4 experts per lane and at
  // least K lanes (lane k keeps choice k, and re-routing alternate k, K2 <= K);
  // fewer lanes per token = more tokens per wave pass
  int L = 1;
  while (L < 64 && (L * 4 < E || L < K)) L <<= 1;
  const int P = (int)((E + L - 1) / L);
  const int ct = chunk_tokens(E, K);
  const unsigned nb = (unsigned)((T + ct - 1) / ct);
  prof_begin(K_ROUTER_TOPK, s);
#define MOE_TOPK(PP)                                                                                             \
  do {                                                                                                           \
    if (blk_P)                                                                                                   \
      router_topk_kernel<PP, true><<<nb, 256, 0, s>>>(logits, part, S, bias, sel_bias, idx, w, blk_count, blk_P,  \
                                                      blk_z, alt_idx, alt_w, (int)K2, (int)T, (int)E, (int)K, L,  \
                                                      gate, renorm ? 1 : 0, topk_in ? 1 : 0, ct);                 \
    else                                                                                                         \
      router_topk_kernel<PP, false><<<nb, 256, 0, s>>>(logits, part, S, bias, sel_bias, idx, w, blk_count,        \
                                                       nullptr, nullptr, alt_idx, alt_w, (int)K2, (int)T, (int)E, \
                                                       (int)K, L, gate, renorm ? 1 : 0, topk_in ? 1 : 0, ct);     \
  } while (0)
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
