// Backward pass (placeholder until the kernels land).
#include <hip/hip_runtime.h>
#include "libra.h"
#include "plan_layout.h"

extern "C" libra_status libra_attn_bwd_workspace(const void *plan, size_t *bytes) {
  libra_plan_info h;
  if (!bytes || libra::plan_header(plan, &h) != LIBRA_OK) return LIBRA_EINVAL;
  *bytes = 0;
  return LIBRA_OK;
}

extern "C" libra_status libra_attn_bwd(const void *, const void *, const void *, const void *,
                                       const void *, const void *, const void *, const float *,
                                       const int32_t *, void *, void *, void *, float, void *, size_t,
                                       libra_cu_record *, void *) {
  return LIBRA_EUNSUPPORTED;
}
