// Placeholder until the MFMA kernels land: the fast path is switched off in
// fast_shape(), so these are never reached.
#include "plan.h"
namespace mla {
mla_status fast_fwd(const Plan&, const void*, const void*, const void*, const void*, const void*,
                    const int32_t*, float*, float*, char*, hipStream_t) {
  return fail(MLA_ERR_UNSUPPORTED, "fast path not built");
}
mla_status fast_bwd(const Plan&, const void*, const void*, const void*, const void*, const void*,
                    const void*, const int32_t*, const float*, const float*, float*, float*,
                    float*, float*, float*, char*, hipStream_t) {
  return fail(MLA_ERR_UNSUPPORTED, "fast path not built");
}
}  // namespace mla
