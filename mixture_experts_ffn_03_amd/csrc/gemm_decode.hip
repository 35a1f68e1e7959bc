// 32-row tiles (decode-sized expert groups, and the router GEMM).
#include "gemm_kernels.h"

namespace moe {

static_assert(pack16_tile<DecodeFcTile>() && pack16_tile<DecodeDownTile>(),
              "decode tiles and prepared weight layout agree");
static_assert(DecodeFcTile::BM == DecodeDTile::BM && DecodeDownTile::BM == DecodeDTile::BM &&
                  (DecodeFcTile::BN / 2) % DecodeDownTile::BK == 0,
              "one token-tile height; a down-GEMM k-step lies inside one h tile");

int decode16_bn1() { return DecodeFcTile::BN; }
int decode16_bn2() { return DecodeDownTile::BN; }

hipError_t launch_decode(bool mxfp4, int epi, const GemmArgs &a, int64_t max_m_tiles,
                         hipStream_t s)
{
    if (mxfp4) return launch_epi<DecodeMXTile>(epi, a, max_m_tiles, s);
    if (epi == kEpiDown) return launch_dma<DecodeDownTile, kEpiDown>(a, max_m_tiles, s);
    if (epi == kEpiPlain) return launch_dma<DecodeDTile, kEpiPlain>(a, max_m_tiles, s);
    if (epi == kEpiGated) return launch_dma<DecodeFcTile, kEpiGated>(a, max_m_tiles, s);
    return launch_dma<DecodeFcTile, kEpiAct>(a, max_m_tiles, s);
}

}  // namespace moe
