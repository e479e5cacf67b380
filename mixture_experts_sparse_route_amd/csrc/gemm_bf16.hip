// Grouped expert GEMMs on bf16 MFMA: launcher of GEMM2 (down) and the
// compiled-configuration query; the kernel is in gemm_bf16.h.
#include "gemm_bf16.h"

namespace moe {

bool gemm_bf16_has_config(bool w8, bool k64, int bm, int bnb, int ns) {
#define MOE_HAS(B, W, N) \
  if (bm == B && bnb == W && ns == N) return true;
  if (w8 && k64) {
    MOE_GEMM8K64_CONFIGS(MOE_HAS)
  } else if (k64) {
    MOE_GEMM16K64_CONFIGS(MOE_HAS)
  } else if (w8) {
    MOE_GEMM8_CONFIGS(MOE_HAS)
  } else {
    MOE_GEMM_CONFIGS(MOE_HAS)
  }
#undef MOE_HAS
  return false;
}

hipError_t gemm_bf16_down(const FfnPlan& pl, const void* h, int64_t h_blk, const int4* tab, const int32_t* count,
                          const int32_t* offsets, int64_t grid, const void* W2, const float* s2, float* yp,
                          const CombineFuse* fuse, int64_t F, int64_t d, hipStream_t s) {
  GemmArgs a{(const uint16_t*)h, W2, nullptr, s2, nullptr, yp, tab, count, (int)d, (int)F};
  set_layout(a, h_blk, 0);
  set_weight_layout(a, pl.packed_down, pl.nt_down, pl.w8 ? 1 : 2);
  a.w_nt_rows = pl.nt_rows_down;
  a.offsets = offsets;
  if (fuse) a.fuse = *fuse;
  if (F / (pl.k64_down ? 2 * BKS : BKS) < pl.ns_down - 1) return hipErrorInvalidValue;
  a.xcd_chunk = pl.wg_per_cu > 0 ? 0 : pl.xcd_chunk_down;
  const unsigned g = (unsigned)launch_grid(pl, grid, a.xcd_chunk);
#define MOE_LAUNCH(B, W, N)                                     \
  if (pl.bm_down == B && pl.bnb_down == W && pl.ns_down == N) { \
    gemm_bf16_kernel<B, W, N, false, WKV, AM_KB><<<g, 256, 0, s>>>(a); \
    return hipGetLastError();                                   \
  }
  MOE_DISPATCH_KIND(pl.k64_down, MOE_LAUNCH)
#undef MOE_LAUNCH
  return hipErrorInvalidValue;
}

#undef MOE_DISPATCH_KIND

}  // namespace moe
