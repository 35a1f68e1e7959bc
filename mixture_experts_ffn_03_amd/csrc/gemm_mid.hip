// 128-row tiles (16-bit and MXFP4 weights).
#include "gemm_kernels.h"

namespace moe {

hipError_t launch_mid(bool mxfp4, int epi, const GemmArgs &a, int64_t max_m_tiles, hipStream_t s)
{
    return mxfp4 ? launch_epi<MidMXTile>(epi, a, max_m_tiles, s)
                 : launch_epi<MidDTile>(epi, a, max_m_tiles, s);
}

}  // namespace moe
