// Expert-contiguous permutation of the (token, slot) pairs, so that each
// expert's GEMM runs on its own rows (the "per-expert kernels" of the clika
// "ClikaRT::nn::QMoEWoQ" page).  Rows of expert e are its (t, j) pairs in
// increasing token order; a token never holds one expert twice.
//
// Three launches, all integer work and fully deterministic (no value
// atomics; the only atomics are bitwise ORs, whose result is order-free):
//   1. block histogram: each block of 256 tokens marks, per expert, which of
//      its tokens chose that expert (a 256-bit mask per expert in LDS) and
//      writes the per-block counts;
//   2. scan (one block): per-expert totals, exclusive scan over experts
//      (offsets), per-block bases, and the cumulative M-tile counts the
//      grouped GEMMs schedule from;
//   3. scatter: each block rebuilds its masks; a pair's row is its block
//      base plus the number of lower tokens in its block with the same expert
//      (popcount of the mask below it).
#include "moe_kernels.h"

namespace moe {
namespace {

constexpr int kWords = kPermTokens / 32;   // mask words per expert

__device__ inline void build_masks(const PermuteArgs &a, uint32_t *masks, int t0)
{
    for (int i = threadIdx.x; i < a.E * kWords; i += blockDim.x) masks[i] = 0u;
    __syncthreads();
    const int t = t0 + (int)threadIdx.x;
    if (t < a.T) {
        for (int j = 0; j < a.K; ++j) {
            const int e = min(max(a.ids[(int64_t)t * a.K + j], 0), a.E - 1);  // memory safety
            atomicOr(&masks[e * kWords + (threadIdx.x >> 5)], 1u << (threadIdx.x & 31));
        }
    }
    __syncthreads();
}

__global__ __launch_bounds__(kPermTokens) void hist_kernel(PermuteArgs a)
{
    extern __shared__ uint32_t masks[];
    build_masks(a, masks, blockIdx.x * kPermTokens);
    for (int e = threadIdx.x; e < a.E; e += blockDim.x) {
        int c = 0;
#pragma unroll
        for (int w = 0; w < kWords; ++w) c += __popc(masks[e * kWords + w]);
        a.block_counts[(int64_t)blockIdx.x * a.E + e] = c;
    }
}

// Block-wide exclusive scan of one int per thread (blockDim.x == 1024).
__device__ inline int block_exclusive_scan(int v, int *buf, int *total)
{
    const int tid = threadIdx.x;
    buf[tid] = v;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
        int add = tid >= off ? buf[tid - off] : 0;
        __syncthreads();
        buf[tid] += add;
        __syncthreads();
    }
    const int incl = buf[tid];
    *total = buf[1023];
    __syncthreads();
    return incl - v;
}

__global__ __launch_bounds__(1024) void scan_kernel(PermuteArgs a)
{
    __shared__ int buf[1024];
    const int e = threadIdx.x;
    const int NB = (a.T + kPermTokens - 1) / kPermTokens;
    int run = 0;
    if (e < a.E) {
        for (int b = 0; b < NB; ++b) {
            const int64_t i = (int64_t)b * a.E + e;
            const int c = a.block_counts[i];
            a.block_base[i] = run;
            run += c;
        }
    }
    int total;
    const int off = block_exclusive_scan(e < a.E ? run : 0, buf, &total);
    const int mt1 = e < a.E ? (run + a.bm1 - 1) / a.bm1 : 0;
    const int mt2 = e < a.E ? (run + a.bm2 - 1) / a.bm2 : 0;
    // M-tiles of the full class: every tile of an expert with at least bm
    // rows (the GEMMs spread its rows evenly over them); an expert with
    // fewer rows has one partial tile
    const int ft1 = run >= a.bm1 ? mt1 : 0;
    const int ft2 = run >= a.bm2 ? mt2 : 0;
    int tot1, tot2, ftot1, ftot2;
    const int cum1 = block_exclusive_scan(mt1, buf, &tot1);
    const int cum2 = block_exclusive_scan(mt2, buf, &tot2);
    const int fcum1 = block_exclusive_scan(ft1, buf, &ftot1);
    const int fcum2 = block_exclusive_scan(ft2, buf, &ftot2);
    if (e < a.E) {
        a.counts[e] = run;
        a.offsets[e] = off;
        a.tile_cum1[e] = cum1;
        a.tile_cum2[e] = cum2;
        a.full_cum1[e] = fcum1;
        a.full_cum2[e] = fcum2;
        for (int b = 0; b < NB; ++b) a.block_base[(int64_t)b * a.E + e] += off;
    }
    if (e == 0) {
        a.offsets[a.E] = total;
        a.tile_cum1[a.E] = tot1;
        a.tile_cum2[a.E] = tot2;
        a.full_cum1[a.E] = ftot1;
        a.full_cum2[a.E] = ftot2;
    }
}

__global__ __launch_bounds__(kPermTokens) void scatter_kernel(PermuteArgs a)
{
    extern __shared__ uint32_t masks[];
    const int t0 = blockIdx.x * kPermTokens;
    build_masks(a, masks, t0);
    const int t = t0 + (int)threadIdx.x;
    if (t >= a.T) return;
    const int w = threadIdx.x >> 5;
    const uint32_t below = (1u << (threadIdx.x & 31)) - 1u;
    for (int j = 0; j < a.K; ++j) {
        const int e = min(max(a.ids[(int64_t)t * a.K + j], 0), a.E - 1);
        int rank = __popc(masks[e * kWords + w] & below);
        for (int q = 0; q < w; ++q) rank += __popc(masks[e * kWords + q]);
        const int row = a.block_base[(int64_t)blockIdx.x * a.E + e] + rank;
        a.row_token[row] = t;
        a.slot_row[(int64_t)t * a.K + j] = row;
        // weigh-inputs routing: the row's weight travels with it to GEMM 1
        if (a.row_weight) a.row_weight[row] = a.weights[(int64_t)t * a.K + j];
    }
}

}  // namespace

hipError_t launch_permute(const PermuteArgs &a, hipStream_t s)
{
    const int NB = (a.T + kPermTokens - 1) / kPermTokens;
    const size_t lds = (size_t)a.E * kWords * sizeof(uint32_t);
    hist_kernel<<<NB, kPermTokens, lds, s>>>(a);
    scan_kernel<<<1, 1024, 0, s>>>(a);
    scatter_kernel<<<NB, kPermTokens, lds, s>>>(a);
    return hipGetLastError();
}

}  // namespace moe
