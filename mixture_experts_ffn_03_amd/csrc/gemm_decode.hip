// 32-row tiles (decode-sized expert groups, and the router GEMM).
#include "gemm_kernels.h"

namespace moe {

hipError_t launch_decode(bool mxfp4, int epi, const GemmArgs &a, int64_t max_m_tiles,
                         hipStream_t s)
{
    if (mxfp4) return launch_epi<DecodeMXTile>(epi, a, max_m_tiles, s);
    if (epi == kEpiDown) return launch_dma<DecodeDownTile, kEpiDown>(a, max_m_tiles, s);
    return launch_epi<DecodeDTile>(epi, a, max_m_tiles, s);
}

}  // namespace moe
