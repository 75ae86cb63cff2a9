// Host-side helpers shared by the C-ABI entry points.
#pragma once

#include <hip/hip_runtime.h>

#include "../../include/moe_token_block.h"

#define MTB_EXPORT extern "C" __attribute__((visibility("default")))

namespace mtb {

// Size arguments at or above this are refused before any arithmetic on them,
// so that the validation's own products and sums cannot overflow int64_t.
constexpr int64_t kSizeLimit = (int64_t)1 << 31;

// Status of the launches just issued on this thread: EP_ERR_HIP (and the HIP
// error cleared) if any failed.
inline int32_t launch_status() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? EP_OK : EP_ERR_HIP;
}

}  // namespace mtb
