// moe_forward_noalloc: the layer forward for callers that cannot allocate
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// allocation).  Its scratch is a file-scope device array; see moe.h.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "api_internal.h"
#include "moe.h"

namespace moe {
namespace {

// Every GPU the library runs on holds its own copy of this array, from the
// module's load on that GPU until the process ends.  In host code the name
// `scratch` is only a host-side stand-in, never device memory: the array's
// address on each device is looked up once, with that device current, and
// only that address is handed to kernels.
static __device__ __align__(256) char scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices];  // device address of `scratch` per device, once looked up

// The device address of `scratch` on device `dev`, which must be current.
moe_status scratch_of(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return fail_detail(MOE_ERR_UNSUPPORTED, "device id out of range");
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      char buf[256];
      snprintf(buf, sizeof buf, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
      return fail_detail(MOE_ERR_HIP, buf);
    }
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return MOE_OK;
}

}  // namespace
}  // namespace moe

extern "C" moe_status moe_forward_noalloc(const moe_config* cfg, const void* x, const float* Wg,
                                          const float* logit_bias, const float* sel_bias, const void* W1,
                                          const void* W3, const void* W2, const void* Ws1, const void* Ws3,
                                          const void* Ws2, const moe_scales* scales, void* y, const moe_routing* r,
                                          moe_stream_t stream) {
  using namespace moe;
  // the config and the scratch it needs, on the host before any HIP call
  size_t need = 0;
  moe_status st = moe_workspace_size(cfg, &need);
  if (st != MOE_OK) return st;
  char buf[256];
  if (need > MOE_NOALLOC_SCRATCH_BYTES) {
    snprintf(buf, sizeof buf,
             "moe_forward_noalloc: this layer needs %zu bytes of scratch, more than the built-in %zu; call "
             "moe_forward with a workspace", need, (size_t)MOE_NOALLOC_SCRATCH_BYTES);
    return fail_detail(MOE_ERR_WORKSPACE, buf);
  }
  int cur = -1, sdev = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e == hipSuccess) e = hipStreamGetDevice((hipStream_t)stream, &sdev);
  if (e != hipSuccess) {
    snprintf(buf, sizeof buf, "moe_forward_noalloc: %s", hipGetErrorString(e));
    return fail_detail(MOE_ERR_HIP, buf);
  }
  if (sdev != cur) {
    snprintf(buf, sizeof buf, "moe_forward_noalloc: the stream belongs to device %d, not the current device %d",
             sdev, cur);
    return fail_detail(MOE_ERR_INVALID_ARG, buf);
  }
  void* ws = nullptr;
  if ((st = scratch_of(cur, &ws)) != MOE_OK) return st;
  return forward_in_scratch(cfg, x, Wg, logit_bias, sel_bias, W1, W3, W2, Ws1, Ws3, Ws2, scales, y, r, ws,
                            MOE_NOALLOC_SCRATCH_BYTES, (hipStream_t)stream);
}
