// 256-row tiles with 16-bit weights (GEMM 1 and, streaming the fp16 weight
// copy, the down GEMM on the 4-wave hand-laid loop; otherwise the 8-wave tile).
#include "gemm_kernels.h"

namespace moe {

hipError_t launch_prefill16(int epi, const GemmArgs &a, int64_t max_m_tiles, hipStream_t s)
{
    if (epi == kEpiGated) return launch_dma<PrefillFcTile, kEpiGated>(a, max_m_tiles, s);
    if (epi == kEpiAct) return launch_dma<PrefillFcTile, kEpiAct>(a, max_m_tiles, s);
    // with fp16 down weights (no per-tile conversion) the 4-wave loop is
    // the faster one for the down GEMM too (1.16 -> 1.03 ms on the
    // Mixtral shape); converting in registers, the 8-wave tile is
    if (epi == kEpiDown && a.w_f16) return launch_dma<PrefillFcTile, kEpiDown>(a, max_m_tiles, s);
    return launch_epi<PrefillDTile>(epi, a, max_m_tiles, s);
}

}  // namespace moe
