// Instantiates the matrix-core GEMM kernels for the 32x32 output tile with K
// split over eight wave groups (few output tiles and a long K: each wave
// then walks an eighth of K, which shortens the chain of dependent slice
// loads that bounds such grids).
#include "gemm_mfma_impl.h"

namespace dgt {

hipError_t launch_mfma_32k8(int dtype, bool ta, bool tb, bool masked, const GemmArgs& a,
                            hipStream_t s) {
  return launch_mfma_cfg<Cfg32k8>(dtype, ta, tb, masked, a, s);
}

}  // namespace dgt
