// Device helpers shared by the grouped-GEMM kernels: tile scheduling and the
// gated activation.
#pragma once

#include "moe_kernels.h"

namespace moe {

// One work tile of a grouped GEMM: expert e, rows [row0, row0 + nrows) of the
// permutation, output features [n0, n0 + tile width).
struct TileWork {
    int e, row0, nrows, n0;
    int mg;      // global M-tile index (tile_cum[e] + token tile)
    int nt;      // feature tile index
};

// Map this workgroup to a tile, or return false when it has none.
//
// Tiles are numbered expert-major, then feature tile, then token tile, so
// the token tiles that share one expert's weight panel are consecutive.
// Hardware dispatches workgroup b to XCD b % 8; consecutive tile numbers are
// gathered onto one XCD (its L2 then serves the shared weight panel and the
// shared activation rows), with the XCD loads differing by at most one tile.
// The count of tiles is data dependent and read from tile_cum (staged in
// LDS); surplus workgroups of the worst-case grid return at once.
__device__ inline bool find_tile(const GemmArgs &g, int *s_cum, int bm, int n_width,
                                 TileWork *w)
{
    for (int i = threadIdx.x; i <= g.E; i += blockDim.x) s_cum[i] = g.tile_cum[i];
    __syncthreads();
    const int total = s_cum[g.E] * g.nN;
    const int bid = blockIdx.x;
    const int q = total >> 3, rem = total & 7, xcd = bid & 7, slot = bid >> 3;
    if (slot >= q + (xcd < rem ? 1 : 0)) return false;
    const int v = xcd * q + min(xcd, rem) + slot;
    // expert e with s_cum[e]*nN <= v < s_cum[e+1]*nN (it has >= 1 tile)
    int lo = 0, hi = g.E;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_cum[mid] * g.nN <= v) lo = mid;
        else hi = mid;
    }
    const int e = lo;
    const int mt = s_cum[e + 1] - s_cum[e];
    const int local = v - s_cum[e] * g.nN;
    const int nt = local / mt, mtile = local - nt * mt;
    w->e = e;
    w->row0 = g.offsets[e] + mtile * bm;
    w->nrows = min(bm, g.counts[e] - mtile * bm);
    w->n0 = nt * n_width;
    w->mg = s_cum[e] + mtile;
    w->nt = nt;
    return true;
}

// Gated activation in fp32.  act 0: SiLU-gated, h = g*sigmoid(g)*u.
// act 1: clamped SwiGLU, g' = min(g, L), u' = clamp(u, -L, L) when L > 0,
// h = g'*sigmoid(alpha*g')*(u' + beta).
__device__ inline float gated_act(int act, float g, float u, float alpha,
                                  float beta, float limit)
{
    if (act == 0) return g * (1.0f / (1.0f + __expf(-g))) * u;
    if (limit > 0.0f) {
        g = fminf(g, limit);
        u = fminf(fmaxf(u, -limit), limit);
    }
    return g * (1.0f / (1.0f + __expf(-alpha * g))) * (u + beta);
}

// Activation of a non-gated expert's fc1 output (act 2 relu, 3 gelu in the
// erf form or, gelu_mode 1, the tanh form, 4 silu, 5 identity).
__device__ inline float single_act(int act, int gelu_mode, float v)
{
    switch (act) {
    case 2: return fmaxf(v, 0.0f);
    case 3:
        if (gelu_mode == 1)
            return 0.5f * v * (1.0f + tanhf(0.7978845608f * (v + 0.044715f * v * v * v)));
        return 0.5f * v * (1.0f + erff(v * 0.70710678118654752f));
    case 4: return v * (1.0f / (1.0f + __expf(-v)));
    default: return v;
    }
}

__device__ inline float bf16_bits_to_float(uint16_t b)
{
    return __uint_as_float((uint32_t)b << 16);
}

}  // namespace moe
