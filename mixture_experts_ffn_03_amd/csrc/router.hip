// Router logits from the layer's own router ("MoeSpec" `wr`, `router_bias`:
// logits = x . Wr + Br, Wr indexed as a [d, E] matrix).  The product runs on
// the grouped-GEMM kernel as one group of T rows against the transposed
// router [E, H] (made once at prepare, so that its rows are K-contiguous like
// every expert stack); these are the two small helpers around it.
#include "moe_kernels.h"

namespace moe {
namespace {

// dst[c][r] = src[r][c] for a rows x cols matrix of 2- or 4-byte elements,
// through a 32x32 LDS tile (coalesced reads and writes).
template <typename T>
__global__ __launch_bounds__(256) void transpose_kernel(const T *src, T *dst, int rows, int cols)
{
    __shared__ T tile[32][33];
    const int c0 = blockIdx.x * 32, r0 = blockIdx.y * 32;
    const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;   // 32 x 8
    for (int i = ty; i < 32; i += 8) {
        const int r = r0 + i, c = c0 + tx;
        if (r < rows && c < cols) tile[i][tx] = src[(int64_t)r * cols + c];
    }
    __syncthreads();
    for (int i = ty; i < 32; i += 8) {
        const int c = c0 + i, r = r0 + tx;
        if (r < rows && c < cols) dst[(int64_t)c * rows + r] = tile[tx][i];
    }
}

__global__ void single_group_kernel(int32_t *counts, int32_t *offsets, int32_t *tile_cum,
                                    int32_t *full_cum, int T, int bm)
{
    if (threadIdx.x == 0) {
        counts[0] = T;
        offsets[0] = 0;
        offsets[1] = T;
        tile_cum[0] = 0;
        tile_cum[1] = (T + bm - 1) / bm;
        full_cum[0] = 0;
        full_cum[1] = T >= bm ? (T + bm - 1) / bm : 0;
    }
}

}  // namespace

hipError_t launch_transpose(const void *src, void *dst, int rows, int cols, int elem_bytes,
                            hipStream_t s)
{
    const dim3 grid((unsigned)((cols + 31) / 32), (unsigned)((rows + 31) / 32));
    if (elem_bytes == 2)
        transpose_kernel<uint16_t><<<grid, 256, 0, s>>>((const uint16_t *)src, (uint16_t *)dst,
                                                        rows, cols);
    else
        transpose_kernel<uint32_t><<<grid, 256, 0, s>>>((const uint32_t *)src, (uint32_t *)dst,
                                                        rows, cols);
    return hipGetLastError();
}

hipError_t launch_single_group(int32_t *counts, int32_t *offsets, int32_t *tile_cum,
                               int32_t *full_cum, int T, int bm, hipStream_t s)
{
    single_group_kernel<<<1, 64, 0, s>>>(counts, offsets, tile_cum, full_cum, T, bm);
    return hipGetLastError();
}

}  // namespace moe
