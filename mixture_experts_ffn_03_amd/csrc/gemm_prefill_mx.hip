// 256-row tiles with MXFP4 weights.
#include "gemm_kernels.h"

namespace moe {

hipError_t launch_prefill_mx(int epi, const GemmArgs &a, int64_t max_m_tiles, hipStream_t s)
{
    return launch_epi<PrefillMXTile>(epi, a, max_m_tiles, s);
}

}  // namespace moe
