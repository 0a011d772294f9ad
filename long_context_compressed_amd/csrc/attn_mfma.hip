// Matrix-core (MFMA) sparse attention for bf16, H = 64 heads, D = 512 on gfx950.
// (Filled in by the MFMA kernels; until a shape is covered here the scalar kernels run.)
#include "csa_device.h"
#include "csa_launch.h"

namespace csa {

hipError_t launch_attn_fwd_mfma(const Shape& sh, const AttnIO& io, hipStream_t s, bool* handled) {
  (void)sh; (void)io; (void)s;
  *handled = false;
  return hipSuccess;
}

hipError_t launch_attn_bwd_mfma(const Shape& sh, const AttnIO& io, hipStream_t s, bool* handled) {
  (void)sh; (void)io; (void)s;
  *handled = false;
  return hipSuccess;
}

}  // namespace csa
