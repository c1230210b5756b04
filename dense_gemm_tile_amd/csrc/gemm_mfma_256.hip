// Instantiates the matrix-core GEMM kernels for the 256x256 output tile. Whole
// tiles with both operands K-contiguous (A not transposed, B transposed) take
// the two-group direct-to-LDS kernel; every other case takes the general
// kernel.
#include "gemm_mfma_pingpong.h"

namespace dgt {

hipError_t launch_mfma_256(int dtype, bool ta, bool tb, bool masked, const GemmArgs& a,
                           hipStream_t s) {
  if (!ta && tb && !masked) {
    const dim3 grid(a.tiles_m * a.tiles_n), block(PingPongCfg::THREADS);
#define DGT_PP(TAG)                                                                          \
  do {                                                                                       \
    if (a.epi == EPI_BETA0) gemm_mfma_pingpong_kernel<TAG, EPI_BETA0><<<grid, block, 0, s>>>(a); \
    else if (a.epi == EPI_ACC_PLUS_C)                                                        \
      gemm_mfma_pingpong_kernel<TAG, EPI_ACC_PLUS_C><<<grid, block, 0, s>>>(a);              \
    else gemm_mfma_pingpong_kernel<TAG, EPI_GENERAL><<<grid, block, 0, s>>>(a);              \
  } while (0)
    if (dtype == 0) DGT_PP(TagF16);
    else DGT_PP(TagBF16);
#undef DGT_PP
    return hipGetLastError();
  }
  return launch_mfma_cfg<Cfg256>(dtype, ta, tb, masked, a, s);
}

}  // namespace dgt
