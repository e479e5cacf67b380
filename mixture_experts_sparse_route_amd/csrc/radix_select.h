// Block-wide selection helpers shared by the affinity drop and expert-choice
// routing: the want-th largest of a set of distinct 64-bit keys, and the
// exclusive rank of a flag in thread order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// A threshold thr such that exactly `want` of the n distinct keys s[0 .. n)
// are >= thr, 1 <= want <= n.  Most-significant-digit radix select: up to 8
// passes, each histogramming the next 8 bits of the keys that share the
// prefix found so far and keeping the bin that holds the want-th largest
// key; it stops early once every key of that bin is wanted (thr is then the
// prefix with its lower bits zero).  Every thread of the NT-thread block
// calls it.  hist: 256 ints of LDS; sel: 2 ints of LDS.
template <int NT>
__device__ uint64_t radix_select_desc(const uint64_t* __restrict__ s, int n, int want, int* hist, int* sel) {
  uint64_t prefix = 0, pmask = 0;
  for (int shift = 56; shift >= 0; shift -= 8) {
    for (int b = threadIdx.x; b < 256; b += NT) hist[b] = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += NT) {
      const uint64_t k = s[i];
      if ((k & pmask) == prefix) atomicAdd(&hist[(k >> shift) & 255], 1);
    }
    __syncthreads();
    if (threadIdx.x < 64) {
      // lane l holds bins 4l .. 4l+3; suffix sums over the lanes above it
      const int l = threadIdx.x;
      const int c0 = hist[4 * l], c1 = hist[4 * l + 1], c2 = hist[4 * l + 2], c3 = hist[4 * l + 3];
      const int local = c0 + c1 + c2 + c3;
      int suf = local;
      for (int off = 1; off < 64; off <<= 1) {
        const int v = __shfl_down(suf, off, 64);
        if (l + off < 64) suf += v;
      }
      const int above = suf - local;  // keys in bins above 4l+3
      if (above < want && want <= suf) {
        int acc = above, b;
        if (acc + c3 >= want) {
          b = 4 * l + 3;
        } else {
          acc += c3;
          if (acc + c2 >= want) {
            b = 4 * l + 2;
          } else {
            acc += c2;
            if (acc + c1 >= want) {
              b = 4 * l + 1;
            } else {
              acc += c1;
              b = 4 * l;
            }
          }
        }
        sel[0] = b;
        sel[1] = want - acc;
      }
    }
    __syncthreads();
    prefix |= (uint64_t)sel[0] << shift;
    pmask |= 0xFFull << shift;
    want = sel[1];
    // every key of the chosen bin is wanted: the keys >= prefix (lower bits
    // zero) are exactly the wanted ones, whatever their lower bits hold
    const bool whole_bin = want == hist[sel[0]];
    __syncthreads();
    if (whole_bin) break;
  }
  return prefix;
}

// Exclusive rank of `flag` among the block's NT threads in thread order; the
// block's count goes to *total.  wtot: NT/64 ints of LDS.  Ends with a
// barrier, so wtot may be reused by the next call.
template <int NT>
__device__ int block_rank(bool flag, int* wtot, int* total) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const uint64_t bal = __ballot(flag);
  if (lane == 0) wtot[wave] = __popcll(bal);
  __syncthreads();
  int before = 0, all = 0;
  for (int q = 0; q < NT / 64; ++q) {
    if (q < wave) before += wtot[q];
    all += wtot[q];
  }
  const uint64_t lt = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  *total = all;
  __syncthreads();
  return before + __popcll(bal & lt);
}

}  // namespace moe
