// Instantiates the general (VGPR-staged) matrix-core GEMM kernel for the
// 128x128 output tile, masked form only: it serves float32 operands (rounded
// while staged) and operands whose pitch needs 64-bit addressing; every other
// 128x128 call runs on the direct-to-LDS ring kernel.
#include "gemm_mfma_impl.h"

namespace dgt {

hipError_t launch_mfma_128(int dtype, bool ta, bool tb, bool masked, const GemmArgs& a,
                         hipStream_t s) {
  return launch_mfma_cfg<Cfg128, FORMS_MASKED>(dtype, ta, tb, masked, a, s);
}

}  // namespace dgt
