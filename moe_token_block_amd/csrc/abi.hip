// Version, status strings and small size helpers of the C ABI.
#include "common.h"
#include "launch.h"

MTB_EXPORT int32_t ep_abi_version(void) { return EP_ABI_VERSION; }

MTB_EXPORT const char* ep_status_string(int32_t status) {
  switch (status) {
    case EP_OK: return "ok";
    case EP_ERR_NULL: return "a required pointer is NULL";
    case EP_ERR_SHAPE: return "a size is negative, zero where it must not be, or not a multiple the format needs";
    case EP_ERR_ALIGN: return "alignment is not a positive multiple of 16";
    case EP_ERR_CAPACITY: return "r_cap is below the routing capacity";
    case EP_ERR_DTYPE: return "unknown index dtype or rounding mode";
    case EP_ERR_HIP: return "a kernel launch failed";
    case EP_ERR_WORKSPACE: return "workspace missing or too small";
    case EP_ERR_RANGE: return "a size exceeds the 32-bit indexing the kernels use";
    case EP_ERR_SCRATCH: return "sizes need more than the static scratch of the allocation-free entry point";
    default: return "unknown status";
  }
}

MTB_EXPORT int64_t ep_nvfp4_packed_row_bytes(int64_t hidden) {
  if (hidden <= 0 || hidden % 64 != 0) return EP_ERR_SHAPE;
  if (hidden >= mtb::kSizeLimit) return EP_ERR_RANGE;
  return 9 * hidden / 16 + 4;
}

MTB_EXPORT uint32_t ep_rht_sign_mask(void) { return mtb::kRhtSignMask; }
