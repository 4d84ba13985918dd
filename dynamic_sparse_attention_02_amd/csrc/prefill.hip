// Causal block-sparse prefill (placeholder until the kernels land).
#include "sa_internal.h"

namespace sa {

size_t prefill_select_workspace_bytes(const Shape&, int32_t) { return 0; }

hipError_t launch_prefill_select(const Shape&, const sa_pages&, int32_t, const void*, const void*,
                                 const void*, sa_dtype, float, int32_t, int32_t, int32_t*,
                                 int32_t*, int32_t, void*, hipStream_t) {
  return hipErrorNotSupported;
}

hipError_t launch_sparse_prefill(const Shape&, const sa_pages&, int32_t, const void*, const void*,
                                 const void*, const int32_t*, const int32_t*, int32_t, int32_t,
                                 float, void*, sa_dtype, float*, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace sa
