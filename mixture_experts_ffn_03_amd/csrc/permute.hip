// Expert-contiguous permutation of the (token, slot) pairs, so that each
// expert's GEMM runs on its own rows (the "per-expert kernels" of the clika
// "ClikaRT::nn::QMoEWoQ" page).  Rows of expert e are its (t, j) pairs in
// increasing token order; a token never holds one expert twice.
//
// Three launches (one when T <= kPermTokens, below), all integer work and
// fully deterministic (no value atomics; the only atomics are bitwise ORs,
// whose result is order-free):
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

// Per-expert masks of the tokens [t0, t0 + kPermTokens); threads past
// kPermTokens (a 1024-thread block) only help clear them.
__device__ inline void build_masks(const PermuteArgs &a, uint32_t *masks, int t0)
{
    for (int i = threadIdx.x; i < a.E * kWords; i += blockDim.x) masks[i] = 0u;
    __syncthreads();
    const int t = t0 + (int)threadIdx.x;
    if (threadIdx.x < kPermTokens && t < a.T) {
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

// Block-wide exclusive scans of N ints per thread at once (blockDim.x ==
// 1024): shuffle scans inside each wave, then the 16 wave totals through
// LDS; two barriers for all N scans.  buf holds 16 * N ints.
template <int N>
__device__ inline void block_exclusive_scan(int (&v)[N], int *buf, int (&total)[N])
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int incl[N];
#pragma unroll
    for (int i = 0; i < N; ++i) incl[i] = v[i];
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int u = __shfl_up(incl[i], off, 64);
            if (lane >= off) incl[i] += u;
        }
    }
    if (lane == 63) {
#pragma unroll
        for (int i = 0; i < N; ++i) buf[wave * N + i] = incl[i];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < N; ++i) {
        int before = 0, all = 0;
        for (int w = 0; w < 16; ++w) {
            const int x = buf[w * N + i];
            before += w < wave ? x : 0;
            all += x;
        }
        total[i] = all;
        v[i] = before + incl[i] - v[i];          // exclusive prefix
    }
    __syncthreads();
}

// Thread e < E holds its expert's row count: writes counts, offsets and the
// cumulative M-tile counts of both GEMMs; returns expert e's first row.
__device__ inline int scan_experts(const PermuteArgs &a, int run, int *buf)
{
    const int e = threadIdx.x;
    if (e >= a.E) run = 0;
    // M-tiles of both GEMMs, and those of the full class: every tile of an
    // expert with at least bm rows (the GEMMs spread its rows evenly over
    // them); an expert with fewer rows has one partial tile
    const int mt1 = (run + a.bm1 - 1) / a.bm1, mt2 = (run + a.bm2 - 1) / a.bm2;
    int v[5] = {run, mt1, mt2, run >= a.bm1 ? mt1 : 0, run >= a.bm2 ? mt2 : 0};
    int tot[5];
    block_exclusive_scan(v, buf, tot);
    if (e < a.E) {
        a.counts[e] = run;
        a.offsets[e] = v[0];
        a.tile_cum1[e] = v[1];
        a.tile_cum2[e] = v[2];
        a.full_cum1[e] = v[3];
        a.full_cum2[e] = v[4];
    }
    if (e == 0) {
        a.offsets[a.E] = tot[0];
        a.tile_cum1[a.E] = tot[1];
        a.tile_cum2[a.E] = tot[2];
        a.full_cum1[a.E] = tot[3];
        a.full_cum2[a.E] = tot[4];
    }
    return v[0];
}

__global__ __launch_bounds__(1024) void scan_kernel(PermuteArgs a)
{
    __shared__ int buf[16 * 5];
    const int e = threadIdx.x;
    const int NB = (a.T + kPermTokens - 1) / kPermTokens;
    // block_base gets expert e's rows before each block, within the expert
    // (the scatter adds the expert's offset); the counts are read 16 blocks
    // at a time, so their loads overlap instead of one round trip per block
    int run = 0;
    if (e < a.E) {
        for (int b0 = 0; b0 < NB; b0 += 16) {
            int c[16];
#pragma unroll
            for (int i = 0; i < 16; ++i)
                c[i] = b0 + i < NB ? a.block_counts[(int64_t)(b0 + i) * a.E + e] : 0;
#pragma unroll
            for (int i = 0; i < 16; ++i)
                if (b0 + i < NB) {
                    a.block_base[(int64_t)(b0 + i) * a.E + e] = run;
                    run += c[i];
                }
        }
    }
    scan_experts(a, run, buf);
}

// Rows of the pairs of tokens [t0, t0 + kPermTokens) from the block's masks;
// base(e) is the block's first row of expert e.
template <class Base>
__device__ inline void scatter_block(const PermuteArgs &a, const uint32_t *masks, int t0,
                                     Base base)
{
    const int t = t0 + (int)threadIdx.x;
    if (threadIdx.x >= kPermTokens || t >= a.T) return;
    const int w = threadIdx.x >> 5;
    const uint32_t below = (1u << (threadIdx.x & 31)) - 1u;
    for (int j = 0; j < a.K; ++j) {
        const int e = min(max(a.ids[(int64_t)t * a.K + j], 0), a.E - 1);
        int rank = __popc(masks[e * kWords + w] & below);
        for (int q = 0; q < w; ++q) rank += __popc(masks[e * kWords + q]);
        const int row = base(e) + rank;
        a.row_token[row] = t;
        a.slot_row[(int64_t)t * a.K + j] = row;
        // weigh-inputs routing: the row's weight travels with it to GEMM 1
        if (a.row_weight) a.row_weight[row] = a.weights[(int64_t)t * a.K + j];
    }
}

__global__ __launch_bounds__(kPermTokens) void scatter_kernel(PermuteArgs a)
{
    extern __shared__ uint32_t masks[];
    const int t0 = blockIdx.x * kPermTokens;
    build_masks(a, masks, t0);
    scatter_block(a, masks, t0, [&](int e) {
        return a.offsets[e] + a.block_base[(int64_t)blockIdx.x * a.E + e];
    });
}

// T <= kPermTokens (decode sizes): one token block, so masks, scan and
// scatter run in one 1024-thread workgroup; one launch instead of three
// (each a few microseconds of fixed cost next to a decode step's GEMMs).
__global__ __launch_bounds__(1024) void permute_small_kernel(PermuteArgs a)
{
    extern __shared__ uint32_t masks[];          // E * kWords, then E offsets
    __shared__ int buf[16 * 5];
    int *s_off = (int *)(masks + a.E * kWords);
    build_masks(a, masks, 0);
    int run = 0;
    if ((int)threadIdx.x < a.E) {
#pragma unroll
        for (int w = 0; w < kWords; ++w) run += __popc(masks[threadIdx.x * kWords + w]);
    }
    const int off = scan_experts(a, run, buf);
    if ((int)threadIdx.x < a.E) s_off[threadIdx.x] = off;
    __syncthreads();
    scatter_block(a, masks, 0, [&](int e) { return s_off[e]; });
}

}  // namespace

hipError_t launch_permute(const PermuteArgs &a, hipStream_t s)
{
    const int NB = (a.T + kPermTokens - 1) / kPermTokens;
    const size_t lds = (size_t)a.E * kWords * sizeof(uint32_t);
    if (NB <= 1) {
        permute_small_kernel<<<1, 1024, lds + (size_t)a.E * sizeof(int), s>>>(a);
        return hipGetLastError();
    }
    hist_kernel<<<NB, kPermTokens, lds, s>>>(a);
    scan_kernel<<<1, 1024, 0, s>>>(a);
    scatter_kernel<<<NB, kPermTokens, lds, s>>>(a);
    return hipGetLastError();
}

}  // namespace moe
