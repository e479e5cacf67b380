// Gate-weighted combine back to token order (a9):
//   y[t] = sum_{k ascending, dest >= 0} w[t][k] * yp[dest[t*K+k]] + shared[t] (+ x[t])
// "技术日报 2026-04-14" (jsqmd.com) §3.1 step 4 (y = sum_i G_i E_i(x)), §3.4
// (shared experts added unweighted), §3.2 (a dropped assignment contributes
// nothing; the token passes on the residual).  Gather form: each thread owns
// VEC columns of one token and reads its K expert rows, so the sum order is
// fixed and no atomics are needed.  fp32 accumulation, one final rounding.
#include "common.h"
#include "internal.h"

namespace moe {
namespace {

template <typename XT, typename OUT, int VEC>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ yp, const float* __restrict__ w,
                                                      const int32_t* __restrict__ dest,
                                                      const float* __restrict__ shared, const XT* __restrict__ xres,
                                                      OUT* __restrict__ y, int T, int d, int K, int only_dropped) {
  const int vecs = d / VEC;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  // vecs % 64 == 0: all 64 lanes of a wave serve one token (the grid is a
  // whole number of waves, so such a wave never straddles the end)
  const bool wave_token = vecs % 64 == 0;
  if (!wave_token && gid >= (int64_t)T * vecs) return;
  const int t = (int)(gid / vecs);
  const int c = (int)(gid % vecs) * VEC;
  float acc[VEC];
#pragma unroll
  for (int v = 0; v < VEC; ++v) acc[v] = 0.f;
  auto add_row = [&](int r, float wk) {
    const float* src = yp + (int64_t)r * d + c;
    if (VEC == 4) {
      const float4 q = *(const float4*)src;
      acc[0] = fmaf(wk, q.x, acc[0]);
      acc[1] = fmaf(wk, q.y, acc[1]);
      acc[2] = fmaf(wk, q.z, acc[2]);
      acc[3] = fmaf(wk, q.w, acc[3]);
    } else {
#pragma unroll
      for (int v = 0; v < VEC; ++v) acc[v] = fmaf(wk, src[v], acc[v]);
    }
  };
  if (wave_token) {
    if (t >= T) return;
    // the wave loads the token's K (row, weight) pairs, one per lane, and
    // visits the kept ones in ascending k
    const int lane = threadIdx.x & 63;
    for (int k0 = 0; k0 < K; k0 += 64) {
      const int k = k0 + lane;
      const int r = k < K ? dest[(int64_t)t * K + k] : -1;
      const float wk = k < K ? w[(int64_t)t * K + k] : 0.f;
      uint64_t kept = __ballot(r >= 0);
      if (only_dropped && kept) return;  // written by the fused GEMM2 epilogue (K <= 64 here)
      while (kept) {
        const int j = __ffsll((unsigned long long)kept) - 1;
        kept &= kept - 1;
        add_row(__shfl(r, j, 64), __shfl(wk, j, 64));
      }
    }
  } else {
    for (int k = 0; k < K; ++k) {
      const int r = dest[(int64_t)t * K + k];
      if (r < 0) continue;
      if (only_dropped) return;  // written by the fused GEMM2 epilogue
      add_row(r, w[(int64_t)t * K + k]);
    }
  }
  const int64_t o = (int64_t)t * d + c;
  if (shared) {
#pragma unroll
    for (int v = 0; v < VEC; ++v) acc[v] += shared[o + v];
  }
  if (xres) {
#pragma unroll
    for (int v = 0; v < VEC; ++v) acc[v] += load_act(xres, o + v);
  }
#pragma unroll
  for (int v = 0; v < VEC; ++v) store_act(y, o + v, acc[v]);
}

__global__ void set_range_kernel(int32_t* dst, int n) {
  dst[0] = 0;
  dst[1] = n;
}

}  // namespace

hipError_t launch_combine(bool x_bf16, bool y_bf16, const float* yp, const float* w, const int32_t* dest,
                          const float* shared, const void* xres, void* y, int64_t T, int64_t d, int64_t K,
                          bool only_dropped, hipStream_t s) {
  if (only_dropped && (K > 64 || shared)) return hipErrorInvalidValue;
  const int VEC = (d % 4 == 0) ? 4 : 1;
  const int64_t threads = T * (d / VEC);
  const unsigned nb = (unsigned)((threads + 255) / 256);
  if (nb == 0) return hipSuccess;
  prof_begin(K_COMBINE, s);
#define MOE_COMBINE(XT, YT, V)                                                                                 \
  combine_kernel<XT, YT, V><<<nb, 256, 0, s>>>(yp, w, dest, shared, (const XT*)xres, (YT*)y, (int)T, (int)d, \
                                               (int)K, only_dropped ? 1 : 0)
  if (x_bf16 && y_bf16) {
    if (VEC == 4) MOE_COMBINE(uint16_t, uint16_t, 4); else MOE_COMBINE(uint16_t, uint16_t, 1);
  } else if (x_bf16) {
    if (VEC == 4) MOE_COMBINE(uint16_t, float, 4); else MOE_COMBINE(uint16_t, float, 1);
  } else {
    if (VEC == 4) MOE_COMBINE(float, float, 4); else MOE_COMBINE(float, float, 1);
  }
#undef MOE_COMBINE
  prof_end(K_COMBINE, s);
  return hipGetLastError();
}

hipError_t launch_set_range(int32_t* dst, int64_t n, hipStream_t s) {
  set_range_kernel<<<1, 1, 0, s>>>(dst, (int)n);
  return hipGetLastError();
}

}  // namespace moe
