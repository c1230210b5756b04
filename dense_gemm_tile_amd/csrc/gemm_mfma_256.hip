// Instantiates the matrix-core GEMM kernels for the 256x256 output tile.
#include "gemm_mfma_impl.h"

namespace dgt {

hipError_t launch_mfma_256(int dtype, bool ta, bool tb, bool masked, const GemmArgs& a,
                         hipStream_t s) {
  return launch_mfma_cfg<Cfg256>(dtype, ta, tb, masked, a, s);
}

}  // namespace dgt
