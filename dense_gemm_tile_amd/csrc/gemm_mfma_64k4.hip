// Instantiates the matrix-core GEMM kernels for the 64x64 output tile with K
// split over four groups of 2x2 waves (one round of 64x64 tiles with a long
// K: each group walks a quarter of the tile's slices). Whole tiles only: at
// 1024 threads a wave has 128 registers, which the masked loaders exceed.
#include "gemm_mfma_impl.h"

namespace dgt {

hipError_t launch_mfma_64k4(int dtype, bool ta, bool tb, bool masked, const GemmArgs& a,
                            hipStream_t s) {
  return launch_mfma_cfg<Cfg64k4, FORMS_WHOLE>(dtype, ta, tb, masked, a, s);
}

}  // namespace dgt
