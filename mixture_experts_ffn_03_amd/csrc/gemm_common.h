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
    int ks;      // reduction split (0 .. ksplit-1)
};

// Map this workgroup to a tile, or return false when it has none.
//
// An expert with n >= bm rows has ceil(n / bm) M-tiles and its rows are
// spread evenly over them (tile t holds rows [t n / m, (t+1) n / m)): its
// tiles then take the same time, so those that share a weight panel run
// side by side and the XCD's L2 serves the repeats of each k-slice, and no
// short remainder tile streams the whole panel again for a few rows (with
// bm-row tiles plus a remainder, tiles of 1..32 rows took 0.6 of a full
// tile's time, and 10% of the GEMM).  These tiles form the full class; an
// expert with fewer than bm rows has one partial tile, which skips its
// empty row blocks and finishes early: interleaved with full tiles it would
// let its CU run ahead and scatter the sharers apart in time (measured:
// about twice the memory traffic).  So every full tile comes first, the
// partial ones last.
// Within each class tiles are numbered expert-major, then feature tile, then
// token tile, so the token tiles that share one expert's weight panel are
// consecutive.  Hardware dispatches workgroup b to XCD b % 8; each class is
// cut into 8 contiguous chunks, one per XCD (its L2 then serves the shared
// panels and rows), and workgroup slot b / 8 walks its XCD's full chunk and
// then its partial chunk.  The count of tiles is data dependent: the
// prefix sums, and the experts' row counts and offsets, are read with scalar
// loads (the values are the same for every workgroup of the launch, so after
// the first workgroup on a CU they come from the scalar cache instead of a
// vector round trip to L2 at every tile start), and surplus workgroups of
// the worst-case grid return at once.  s_cum is not used.
//
// Scalar loads of launch-constant ints, each statement waiting for its own
// loads (no result register is left in flight).
__device__ __forceinline__ int sload(const int *p)
{
    int v;
    asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(p) : "memory");
    return v;
}
__device__ __forceinline__ void sload2(const int *p, const int *q, int &a, int &b)
{
    asm volatile("s_load_dword %0, %2, 0x0\n\ts_load_dword %1, %3, 0x0\n\ts_waitcnt lgkmcnt(0)"
                 : "=&s"(a), "=&s"(b) : "s"(p), "s"(q) : "memory");
}

__device__ inline bool find_tile(const GemmArgs &g, int *s_cum, int n_width, TileWork *w)
{
    (void)s_cum;
    const int E = g.E;
    // a split reduction multiplies the feature tiles: tile column
    // s * nN + nt is split s of feature tile nt
    const int nN = g.nN * g.ksplit;
    int full_e, cum_e;
    sload2(g.full_cum + E, g.tile_cum + E, full_e, cum_e);
    const int F = full_e * nN;                    // full tiles
    const int P = cum_e * nN - F;                 // partial tiles (one per expert and N tile)
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int qF = F >> 3, rF = F & 7, qP = P >> 3, rP = P & 7;
    const int cntF = qF + (xcd < rF ? 1 : 0);
    const int cntP = qP + (xcd < rP ? 1 : 0);
    int e, nt, mtile;
    if (slot < cntF) {
        const int v = xcd * qF + min(xcd, rF) + slot;
        // expert e with full_cum[e]*nN <= v < full_cum[e+1]*nN
        int lo = 0, hi = E;
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (sload(g.full_cum + mid) * nN <= v) lo = mid;
            else hi = mid;
        }
        e = lo;
        int f0, f1;
        sload2(g.full_cum + e, g.full_cum + e + 1, f0, f1);
        const int mt = f1 - f0;
        const int local = v - f0 * nN;
        nt = local / mt;
        mtile = local - nt * mt;
    } else if (slot < cntF + cntP) {
        const int v = xcd * qP + min(xcd, rP) + (slot - cntF);
        // partial tiles before expert e: (tile_cum[e] - full_cum[e]) * nN
        int lo = 0, hi = E;
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            int c, f;
            sload2(g.tile_cum + mid, g.full_cum + mid, c, f);
            if ((c - f) * nN <= v) lo = mid;
            else hi = mid;
        }
        e = lo;
        int c0, f0;
        sload2(g.tile_cum + e, g.full_cum + e, c0, f0);
        nt = v - (c0 - f0) * nN;
        mtile = 0;                                // the expert's only tile
    } else {
        return false;
    }
    int c0, c1, cnt, off;
    sload2(g.tile_cum + e, g.tile_cum + e + 1, c0, c1);
    sload2(g.counts + e, g.offsets + e, cnt, off);
    // rows of M-tile mtile of the expert's ntl tiles
    const int ntl = c1 - c0;
    const int r0 = (int)((int64_t)mtile * cnt / ntl);
    const int r1 = (int)((int64_t)(mtile + 1) * cnt / ntl);
    w->e = e;
    w->row0 = off + r0;
    w->nrows = r1 - r0;
    w->mg = c0 + mtile;
    w->ks = nt / g.nN;
    nt -= w->ks * g.nN;
    w->n0 = nt * n_width;
    w->nt = nt;
    return true;
}

// sigmoid(v) = 1 / (1 + e^-v) with the hardware exponential and reciprocal
// (each within ~1 ulp of f32; h is stored in 16 bits, 2^-11 at best), instead
// of an IEEE division sequence per value.  v -> -inf gives rcp(inf) = 0.
__device__ inline float sigmoid_fast(float v)
{
    return __builtin_amdgcn_rcpf(1.0f + __expf(-v));
}

// GELU for the 16-bit GEMM-1 epilogue, where h is stored in 16 bits, in
// branch-free forms (inlined per accumulator, the library erff / tanhf made
// the fully unrolled epilogue spill thousands of registers).
// Erf form: x * Phi(x), with Phi taken from erfc(z), z = |x| / sqrt(2), by
// the rational approximation of Abramowitz & Stegun, formula 7.1.26
// (|error| <= 1.5e-7): erfc(z) ~ t (a1 + t (a2 + t (a3 + t (a4 + t a5)))) e^(-z^2),
// t = 1 / (1 + p z).  For x < 0, Phi(x) = erfc(z) / 2 directly, with no
// cancellation; for x >= 0, Phi(x) = 1 - erfc(z) / 2.
__device__ inline float gelu_erf_fast(float x)
{
    const float z = fabsf(x) * 0.70710678118654752f;
    const float t = __builtin_amdgcn_rcpf(1.0f + 0.3275911f * z);
    const float p = t * (0.254829592f +
                         t * (-0.284496736f + t * (1.421413741f + t * (-1.453152027f + t * 1.061405429f))));
    const float ec = p * __expf(-z * z);
    return x >= 0.0f ? x * (1.0f - 0.5f * ec) : 0.5f * x * ec;
}

// Tanh form: 0.5 x (1 + tanh(u)) = x * sigmoid(2u), u = sqrt(2/pi) (x + 0.044715 x^3).
__device__ inline float gelu_tanh_fast(float x)
{
    return x * sigmoid_fast(1.5957691216057308f * (x + 0.044715f * x * x * x));
}

// Gated activation in fp32.  act 0: SiLU-gated, h = g*sigmoid(g)*u.
// act 1: clamped SwiGLU, g' = min(g, L), u' = clamp(u, -L, L) when L > 0,
// h = g'*sigmoid(alpha*g')*(u' + beta).
__device__ inline float gated_act(int act, float g, float u, float alpha,
                                  float beta, float limit)
{
    if (act == 0) return g * sigmoid_fast(g) * u;
    if (limit > 0.0f) {
        g = fminf(g, limit);
        u = fminf(fmaxf(u, -limit), limit);
    }
    return g * sigmoid_fast(alpha * g) * (u + beta);
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
    case 4: return v * sigmoid_fast(v);
    default: return v;
    }
}

__device__ inline float bf16_bits_to_float(uint16_t b)
{
    return __uint_as_float((uint32_t)b << 16);
}

}  // namespace moe
