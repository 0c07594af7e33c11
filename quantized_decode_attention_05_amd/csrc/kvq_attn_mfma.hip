// MFMA decode attention for the hot cache formats (placeholder: no format is
// routed here yet).
#include "kvq_internal.h"
#include "kvq_launch.h"

namespace kvq {

bool mfma_supported(const Plan& p) {
  (void)p;
  return false;
}

hipError_t launch_attention_mfma(const Plan& p, const AttnPlan& ap, const void* arena, const void* q,
                                 float sm_scale, void* ws, hipStream_t s) {
  (void)p; (void)ap; (void)arena; (void)q; (void)sm_scale; (void)ws; (void)s;
  return hipErrorInvalidValue;
}

}  // namespace kvq
