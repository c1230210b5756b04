// Tile-configuration table and launcher dispatch for the matrix-core path.
#include "gemm_mfma_impl.h"

namespace dgt {

namespace {
template <class C>
constexpr MfmaTileInfo info(const char* name) {
  return MfmaTileInfo{name, C::BM, C::BN, C::BK, C::WM, C::WN, C::At::M, C::At::N, C::At::K, C::KG};
}
const MfmaTileInfo kTiles[NUM_MFMA_TILES] = {
    info<Cfg256>("t256x256x64"),
    info<Cfg128>("t128x128x64"),
    info<Cfg64>("t64x64x64"),
    info<Cfg16>("t16x16x64"),
    info<Cfg32k4>("t32x32x64k4"),
    info<Cfg32k8>("t32x32x64k8"),
    info<Cfg64k4>("t64x64x64k4"),
};
}  // namespace

const MfmaTileInfo& mfma_tile_info(int tile) { return kTiles[tile]; }

hipError_t launch_mfma(int tile, int dtype, bool ta, bool tb, bool masked, const GemmArgs& a,
                       hipStream_t s) {
  switch (tile) {
    case TILE_256x256: return launch_mfma_256(dtype, ta, tb, masked, a, s);
    case TILE_128x128: return launch_mfma_128(dtype, ta, tb, masked, a, s);
    case TILE_64x64: return launch_mfma_64(dtype, ta, tb, masked, a, s);
    case TILE_16x16: return launch_mfma_16(dtype, ta, tb, masked, a, s);
    case TILE_32x32K4: return launch_mfma_32k4(dtype, ta, tb, masked, a, s);
    case TILE_32x32K8: return launch_mfma_32k8(dtype, ta, tb, masked, a, s);
    case TILE_64x64K4: return launch_mfma_64k4(dtype, ta, tb, masked, a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dgt
