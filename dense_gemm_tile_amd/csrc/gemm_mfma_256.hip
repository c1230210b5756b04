// Instantiates the matrix-core GEMM kernel for 256x256 output tiles: the
// two-group direct-to-LDS kernel, in any of the four operand layouts, for
// whole tiles or with edge tiles (16-byte pieces whose contiguous dimension
// ends on a multiple of 8 elements). Tiles of that size that would need
// 64-bit addressing or narrow staging are planned on the 128x128 kernels
// instead, so no general kernel is compiled at this size: with 256
// accumulators per lane it could not keep its staging registers without
// spilling.
#include "gemm_mfma_pingpong.h"

namespace dgt {

namespace {

// Whole tiles: at most one workgroup per CU (one fits, by its LDS), each
// walking its tiles in turn; edge tiles: one workgroup per tile.
constexpr int kPingPongGrid = 256;

template <class TAG, bool AMN, bool BMN, bool MASK>
hipError_t launch_pingpong(const GemmArgs& a, hipStream_t s) {
  const int ntiles = a.tiles_m * a.tiles_n;
  const dim3 grid(MASK || ntiles < kPingPongGrid ? ntiles : kPingPongGrid),
      block(PingPongCfg::THREADS);
  if (a.epi == EPI_BETA0)
    return launch_kernel(gemm_mfma_pingpong_kernel<TAG, EPI_BETA0, AMN, BMN, MASK>, grid, block,
                         s, a);
  if (a.epi == EPI_ACC_PLUS_C)
    return launch_kernel(gemm_mfma_pingpong_kernel<TAG, EPI_ACC_PLUS_C, AMN, BMN, MASK>, grid,
                         block, s, a);
  return launch_kernel(gemm_mfma_pingpong_kernel<TAG, EPI_GENERAL, AMN, BMN, MASK>, grid, block,
                       s, a);
}

template <class TAG, bool MASK>
hipError_t launch_pingpong_layout(bool ta, bool tb, const GemmArgs& a, hipStream_t s) {
  // A is M-contiguous when stored transposed; B is N-contiguous when not.
  if (!ta && tb) return launch_pingpong<TAG, false, false, MASK>(a, s);
  if (!ta && !tb) return launch_pingpong<TAG, false, true, MASK>(a, s);
  if (ta && tb) return launch_pingpong<TAG, true, false, MASK>(a, s);
  return launch_pingpong<TAG, true, true, MASK>(a, s);
}

}  // namespace

hipError_t launch_mfma_256(int dtype, bool ta, bool tb, bool masked, const GemmArgs& a,
                           hipStream_t s) {
  if (masked) {
    if (dtype == 0) return launch_pingpong_layout<TagF16, true>(ta, tb, a, s);
    return launch_pingpong_layout<TagBF16, true>(ta, tb, a, s);
  }
  if (dtype == 0) return launch_pingpong_layout<TagF16, false>(ta, tb, a, s);
  return launch_pingpong_layout<TagBF16, false>(ta, tb, a, s);
}

}  // namespace dgt
