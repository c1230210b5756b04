// Instantiates the matrix-core GEMM kernels for the 32x32 output tile with K
// split over four wave groups (grids with few output tiles).
#include "gemm_mfma_impl.h"

namespace dgt {

hipError_t launch_mfma_32k4(int dtype, bool ta, bool tb, bool masked, const GemmArgs& a,
                            hipStream_t s) {
  return launch_mfma_cfg<Cfg32k4>(dtype, ta, tb, masked, a, s);
}

}  // namespace dgt
