// Grouped expert GEMMs on bf16 MFMA: launcher of GEMM1 (gate_up, with the
// SiLU*gate epilogue); the kernel is in gemm_bf16.h.
#include "gemm_bf16.h"

namespace moe {

hipError_t gemm_bf16_gate_up(const FfnPlan& pl, const AOperand& A, const int4* tab, const int32_t* count,
                             const int32_t* offsets, int64_t grid, const void* W1, const void* W3, const float* s1,
                             const float* s3, void* h, int64_t h_blk, int64_t F, int64_t d, hipStream_t s) {
  GemmArgs a{(const uint16_t*)A.ptr, W1, W3, s1, s3, h, tab, count, (int)F, (int)d};
  if ((A.gather && A.gather_div < 1) || (A.blk_rows && A.kbw != 32 && A.kbw != 64) || (A.blk_rows && d % A.kbw))
    return hipErrorInvalidValue;
  set_layout(a, A.blk_rows, h_blk, A.blk_rows ? A.kbw : BKS);
  set_weight_layout(a, pl.packed_up, pl.nt_up, pl.w8 ? 1 : 2);
  a.w_nt_rows = pl.nt_rows_up;
  a.offsets = offsets;
  a.gather = A.gather;
  a.gather_div = A.gather_div;
  if (d / (pl.k64_up ? 2 * BKS : BKS) < pl.ns_up - 1) return hipErrorInvalidValue;
  a.xcd_chunk = pl.wg_per_cu > 0 ? 0 : pl.xcd_chunk_up;
  const unsigned g = (unsigned)launch_grid(pl, grid, a.xcd_chunk);
// A row-major (x itself, or a caller's xp), k-blocked (the layer's own
// dispatch output, or x k-blocked), or x (k-blocked or row-major) with the
// rows gathered through the routing: separate instantiations, so the row
// stride of a k-blocked A is a compile-time constant
#define MOE_LAUNCH(B, W, N)                                                   \
  if (pl.bm == B && pl.bnb_up == W && pl.ns_up == N) {                        \
    if (A.gather && A.kbw == 64)                                              \
      gemm_bf16_kernel<B, W, N, true, WKV, AM_GATHER64><<<g, 256, 0, s>>>(a); \
    else if (A.gather && A.blk_rows)                                          \
      gemm_bf16_kernel<B, W, N, true, WKV, AM_GATHER><<<g, 256, 0, s>>>(a);   \
    else if (A.gather)                                                        \
      gemm_bf16_kernel<B, W, N, true, WKV, AM_GATHER_ROW><<<g, 256, 0, s>>>(a); \
    else if (A.blk_rows && A.kbw == 64)                                       \
      gemm_bf16_kernel<B, W, N, true, WKV, AM_KB64><<<g, 256, 0, s>>>(a);     \
    else if (A.blk_rows)                                                      \
      gemm_bf16_kernel<B, W, N, true, WKV, AM_KB><<<g, 256, 0, s>>>(a);       \
    else                                                                      \
      gemm_bf16_kernel<B, W, N, true, WKV, AM_ROW><<<g, 256, 0, s>>>(a);      \
    return hipGetLastError();                                                 \
  }
  MOE_DISPATCH_KIND(pl.k64_up, MOE_LAUNCH)
#undef MOE_LAUNCH
  return hipErrorInvalidValue;
}

#undef MOE_DISPATCH_KIND

}  // namespace moe
