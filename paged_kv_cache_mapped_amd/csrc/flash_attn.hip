// placeholder: prefill / extend kernels
#include "common.h"
#include "internal.h"
namespace pkv {
hipError_t launch_prefill(const void*, const void*, const void*, const int32_t*, int32_t, int32_t,
                          int32_t, int32_t, float, int32_t, void*, float*, hipStream_t) {
  return hipErrorNotSupported;
}
ExtendPlan plan_extend(const kv_cache_t&, int32_t, int32_t, int32_t) { return ExtendPlan{16, 0, 1}; }
size_t extend_workspace_bytes(const ExtendPlan&, int32_t, int32_t, int32_t) { return 0; }
hipError_t launch_extend(const kv_cache_t&, const ExtendPlan&, const void*, const void*, const void*,
                         const int32_t*, const int32_t*, const int32_t*, int32_t, int32_t, int32_t,
                         int32_t, int32_t, float, void*, float*, void*, hipStream_t) {
  return hipErrorNotSupported;
}
}  // namespace pkv
