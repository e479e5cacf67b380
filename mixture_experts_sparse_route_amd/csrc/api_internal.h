// Pieces of the C-ABI layer (api.cpp) used by the entry point that allocates
// nothing (noalloc.hip).
#pragma once

#include <hip/hip_runtime.h>

#include "moe.h"

namespace moe {

// moe_forward in a caller-given scratch buffer, allocating nothing: the
// shared expert runs in order on hs (no side stream) and the timing facility
// is off for the call.  A layer whose workspace exceeds ws_bytes returns
// MOE_ERR_WORKSPACE before any HIP call.
moe_status forward_in_scratch(const moe_config* cfg, const void* x, const float* Wg, const float* logit_bias,
                              const float* sel_bias, const void* W1, const void* W3, const void* W2,
                              const void* Ws1, const void* Ws3, const void* Ws2, const moe_scales* scales, void* y,
                              const moe_routing* r, void* ws, size_t ws_bytes, hipStream_t hs);

// Returns s and makes msg the calling thread's moe_last_error() detail.
moe_status fail_detail(moe_status s, const char* msg);

}  // namespace moe
