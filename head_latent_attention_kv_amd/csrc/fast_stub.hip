// Placeholder until the MFMA backward lands: kFastBwdBuilt keeps the
// backward on the plain path, so this is never reached.
#include "plan.h"
namespace mla {
mla_status fast_bwd(const Plan&, const void*, const void*, const void*, const void*, const void*,
                    const void*, const int32_t*, const float*, const float*, float*, float*,
                    float*, float*, float*, char*, hipStream_t) {
  return fail(MLA_ERR_UNSUPPORTED, "fast path not built");
}
}  // namespace mla
