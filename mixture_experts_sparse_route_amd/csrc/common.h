// Device helpers shared by the gfx950 kernels of the MoE layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;

// bf16 bits -> fp32 (exact)
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bf16 bits, round to nearest even: one v_cvt_pk_bf16_f32 on gfx950
// (checked on the GPU against integer round-to-nearest-even on 4M finite
// values, half of them exact ties)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  const __bf16 b = (__bf16)f;
  uint16_t u;
  __builtin_memcpy(&u, &b, 2);
  return u;
}

template <typename T>
__device__ __forceinline__ float load_act(const T* p, int64_t i);
template <>
__device__ __forceinline__ float load_act<float>(const float* p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float load_act<uint16_t>(const uint16_t* p, int64_t i) { return bf16_to_f32(p[i]); }

template <typename T>
__device__ __forceinline__ void store_act(T* p, int64_t i, float v);
template <>
__device__ __forceinline__ void store_act<float>(float* p, int64_t i, float v) { p[i] = v; }
template <>
__device__ __forceinline__ void store_act<uint16_t>(uint16_t* p, int64_t i, float v) { p[i] = f32_to_bf16(v); }

// SiLU(a) = a * sigmoid(a); the reciprocal is the hardware one (1 ulp)
__device__ __forceinline__ float silu(float a) { return a * __builtin_amdgcn_rcpf(1.0f + __expf(-a)); }

// MI355X has 8 XCDs; the dispatcher hands workgroup b to XCD (b mod 8).
constexpr int kXcds = 8;

// Maps hardware workgroup id b to a logical tile id so that each XCD works on
// one contiguous range of `total` tiles (neighbouring tiles share operands in
// that XCD's L2).  Returns -1 for workgroups past the end.
__device__ __forceinline__ int64_t xcd_tile(int64_t b, int64_t total) {
  const int64_t per = (total + kXcds - 1) / kXcds;
  const int64_t local = b / kXcds, xcd = b % kXcds;
  if (local >= per) return -1;
  const int64_t t = xcd * per + local;
  return t < total ? t : -1;
}

}  // namespace moe
