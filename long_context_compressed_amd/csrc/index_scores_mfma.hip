// Matrix-core (MFMA) lightning-indexer scores for bf16 operands on gfx950.
// (Filled in by the MFMA kernel; until a shape is covered here the scalar kernel runs.)
#include "csa_device.h"
#include "csa_launch.h"

namespace csa {

hipError_t launch_index_scores_mfma(const Shape& sh, const void* qI, const float* qI_scale,
                                    const float* w, const void* kI, const float* kI_scale,
                                    float* scores, int64_t ld, hipStream_t s, bool* handled) {
  (void)sh; (void)qI; (void)qI_scale; (void)w; (void)kI; (void)kI_scale; (void)scores;
  (void)ld; (void)s;
  *handled = false;
  return hipSuccess;
}

}  // namespace csa
