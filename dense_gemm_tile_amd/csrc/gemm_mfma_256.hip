// Instantiates the matrix-core GEMM kernel for whole 256x256 output tiles: the
// two-group direct-to-LDS kernel, in any of the four operand layouts. Tiles of
// that size that would need masking, 64-bit addressing or narrow staging are
// planned on the 128x128 general kernel instead (see choose_tile), so no
// general kernel is compiled at this size: with 256 accumulators per lane it
// could not keep its staging registers without spilling.
#include "gemm_mfma_pingpong.h"

namespace dgt {

namespace {

template <class TAG, bool AMN, bool BMN>
hipError_t launch_pingpong(const GemmArgs& a, hipStream_t s) {
  const dim3 grid(a.tiles_m * a.tiles_n), block(PingPongCfg::THREADS);
  if (a.epi == EPI_BETA0)
    return launch_kernel(gemm_mfma_pingpong_kernel<TAG, EPI_BETA0, AMN, BMN>, grid, block, s, a);
  if (a.epi == EPI_ACC_PLUS_C)
    return launch_kernel(gemm_mfma_pingpong_kernel<TAG, EPI_ACC_PLUS_C, AMN, BMN>, grid, block, s,
                         a);
  return launch_kernel(gemm_mfma_pingpong_kernel<TAG, EPI_GENERAL, AMN, BMN>, grid, block, s, a);
}

template <class TAG>
hipError_t launch_pingpong_layout(bool ta, bool tb, const GemmArgs& a, hipStream_t s) {
  // A is M-contiguous when stored transposed; B is N-contiguous when not.
  if (!ta && tb) return launch_pingpong<TAG, false, false>(a, s);
  if (!ta && !tb) return launch_pingpong<TAG, false, true>(a, s);
  if (ta && tb) return launch_pingpong<TAG, true, false>(a, s);
  return launch_pingpong<TAG, true, true>(a, s);
}

}  // namespace

hipError_t launch_mfma_256(int dtype, bool ta, bool tb, bool masked, const GemmArgs& a,
                           hipStream_t s) {
  if (masked) return hipErrorInvalidValue;  // the host never plans a masked 256x256 launch
  if (dtype == 0) return launch_pingpong_layout<TagF16>(ta, tb, a, s);
  return launch_pingpong_layout<TagBF16>(ta, tb, a, s);
}

}  // namespace dgt
