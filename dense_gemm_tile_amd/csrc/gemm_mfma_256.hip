// Instantiates the matrix-core GEMM kernels for the 256x256 output tile. Whole
// tiles take the two-group direct-to-LDS kernel, in any of the four operand
// layouts; tiles that need masking (or 64-bit addressing, or narrow staging)
// take the general kernel.
#include "gemm_mfma_pingpong.h"

namespace dgt {

namespace {

template <class TAG, bool AMN, bool BMN>
void launch_pingpong(const GemmArgs& a, hipStream_t s) {
  const dim3 grid(a.tiles_m * a.tiles_n), block(PingPongCfg::THREADS);
  if (a.epi == EPI_BETA0) gemm_mfma_pingpong_kernel<TAG, EPI_BETA0, AMN, BMN><<<grid, block, 0, s>>>(a);
  else if (a.epi == EPI_ACC_PLUS_C)
    gemm_mfma_pingpong_kernel<TAG, EPI_ACC_PLUS_C, AMN, BMN><<<grid, block, 0, s>>>(a);
  else gemm_mfma_pingpong_kernel<TAG, EPI_GENERAL, AMN, BMN><<<grid, block, 0, s>>>(a);
}

template <class TAG>
void launch_pingpong_layout(bool ta, bool tb, const GemmArgs& a, hipStream_t s) {
  // A is M-contiguous when stored transposed; B is N-contiguous when not.
  if (!ta && tb) launch_pingpong<TAG, false, false>(a, s);
  else if (!ta && !tb) launch_pingpong<TAG, false, true>(a, s);
  else if (ta && tb) launch_pingpong<TAG, true, false>(a, s);
  else launch_pingpong<TAG, true, true>(a, s);
}

}  // namespace

hipError_t launch_mfma_256(int dtype, bool ta, bool tb, bool masked, const GemmArgs& a,
                           hipStream_t s) {
  if (!masked) {
    if (dtype == 0) launch_pingpong_layout<TagF16>(ta, tb, a, s);
    else launch_pingpong_layout<TagBF16>(ta, tb, a, s);
    return hipGetLastError();
  }
  return launch_mfma_cfg<Cfg256>(dtype, ta, tb, masked, a, s);
}

}  // namespace dgt
