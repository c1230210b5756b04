// Instantiates the matrix-core GEMM kernels for the 64x64 output tile.
#include "gemm_mfma_impl.h"

namespace dgt {

hipError_t launch_mfma_64(int dtype, bool ta, bool tb, bool masked, const GemmArgs& a,
                         hipStream_t s) {
  return launch_mfma_cfg<Cfg64>(dtype, ta, tb, masked, a, s);
}

}  // namespace dgt
