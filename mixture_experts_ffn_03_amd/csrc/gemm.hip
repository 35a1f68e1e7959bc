// Grouped expert GEMMs on gfx950 bf16 MFMA (v_mfma_f32_32x32x16_bf16).
//
// Each workgroup computes one tile of Y^T = W_e * A^T for one expert e:
// BN weight rows (output features) by BM permutation rows (tokens), fp32
// accumulation, reduction in BK-wide steps through double-buffered LDS.
// The weight panel is the MFMA "A" operand and the token panel the "B"
// operand, so each lane ends with four consecutive output features of one
// token -- 8-byte bf16 / 16-byte f32 stores in the epilogue.
//
// Two epilogues:
//  gated  (gate||up GEMM, ONNX "MoE" fc1/fc3): the BN weight rows of a tile
//         are BN/2 gate rows and the BN/2 up rows of the same features; a
//         wave holds the gate and up accumulators of the same features in
//         the same lanes, adds the biases, applies the gated activation and
//         stores h in bf16 (the MFMA operand of the next GEMM).
//  down   (ONNX "MoE" fc2): adds the down bias and stores y in f32; the
//         combine rounds once, after the weighted sum.
//
// The A operand of the gated GEMM is gathered straight from x through the
// permutation (row_token), so the permuted activations are never written.
//
// MXFP4 weights ("ClikaRT::nn::QMoEWoQ": decode one block at a time inside
// the GEMM dot, never a dense copy): each 16-byte code chunk is one 32-element
// block; it is decoded with its e8m0 scale to bf16 by the gfx950 scaled
// conversion (exact: e2m1 times a power of two fits bf16) on its way into
// LDS, and the MFMA stays bf16 x bf16 (weight-only; the activation is not
// quantised).
#include "gemm_common.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int BN_, int BM_, int BK_, int WN_, int WM_>
struct Tile {
    static constexpr int BN = BN_, BM = BM_, BK = BK_, WN = WN_, WM = WM_;
    static constexpr int NT = 64 * WN * WM;          // threads
    static constexpr int TN = BN / WN, TM = BM / WM; // wave tile
    static constexpr int FN = TN / 32, FM = TM / 32; // 32x32 MFMA blocks per wave
    static constexpr int LDK = BK + 8;               // padded LDS row (elements)
    static constexpr int CPR = BK / 8;               // 16-byte bf16 chunks per row
    static constexpr int QPR = BK / 32;              // 16-byte MXFP4 chunks per row
    static constexpr int A_CH = BM * CPR / NT;
    static constexpr int B_CH_BF16 = BN * CPR / NT;
    static constexpr int B_CH_MX = BN * QPR / NT;
    static constexpr int STAGE = (BM + BN) * LDK;    // elements per LDS stage
    static_assert(A_CH * NT == BM * CPR, "A tile chunks");
    static_assert(B_CH_BF16 * NT == BN * CPR, "B tile chunks");
    static_assert(B_CH_MX * NT == BN * QPR, "MXFP4 tile chunks");
    static_assert(FN >= 2 && FN % 2 == 0, "gate/up pairs per wave");
    static_assert(2 * STAGE * 2 + (kMaxExperts + 1) * 4 <= 160 * 1024, "LDS");
};

using PrefillTile = Tile<256, 256, 64, 4, 2>;   // 512 threads, wave 64x128
using DecodeTile = Tile<256, 32, 128, 4, 1>;    // 256 threads, wave 64x32

__device__ inline float bias_at(const void *b, int64_t i)
{
    return bf16_bits_to_float(((const uint16_t *)b)[i]);
}

// e8m0 byte -> the fp32 multiplier 2^(X-127) (X = 0 is 2^-127, 255 is NaN).
__device__ inline float e8m0_scale(uint32_t x)
{
    if (x == 0u) return __uint_as_float(0x00400000u);
    if (x == 255u) return __uint_as_float(0x7fc00000u);
    return __uint_as_float(x << 23);
}

template <class TL, bool MX, bool GATED>
__global__ __launch_bounds__(TL::NT) void gemm_kernel(GemmArgs g)
{
    constexpr int B_CH = MX ? TL::B_CH_MX : TL::B_CH_BF16;
    constexpr int NW = GATED ? TL::BN / 2 : TL::BN;   // output features per tile
    __shared__ __attribute__((aligned(16))) __bf16 lds[2 * TL::STAGE];
    __shared__ int s_cum[kMaxExperts + 1];

    TileWork tw;
    if (!find_tile(g, s_cum, TL::BM, NW, &tw)) return;
    const int tid = threadIdx.x;
    const int Kd = g.Kd;

    // ---- A (token) rows: gathered through the permutation when row_token is set
    const int a_kc = (tid % TL::CPR) * 8;
    const __bf16 *a_ptr[TL::A_CH];
    int a_lr[TL::A_CH];
#pragma unroll
    for (int i = 0; i < TL::A_CH; ++i) {
        const int lr = tid / TL::CPR + i * (TL::NT / TL::CPR);
        const int r = tw.row0 + min(lr, tw.nrows - 1);
        const int src = g.row_token ? g.row_token[r] : r;
        a_lr[i] = lr;
        a_ptr[i] = (const __bf16 *)g.a + (int64_t)src * Kd + a_kc;
    }

    // ---- B (weight) rows
    constexpr int BPR = MX ? TL::QPR : TL::CPR;       // chunks per row
    const int b_kc = tid % BPR;
    const uint8_t *b_ptr[B_CH];
    const uint8_t *s_ptr[B_CH];
    int b_lr[B_CH];
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
        const int lr = tid / BPR + i * (TL::NT / BPR);
        const bool up = GATED && lr >= TL::BN / 2;
        const int c = min(tw.n0 + (up ? lr - TL::BN / 2 : lr), g.Nout - 1);
        const int64_t row = (int64_t)tw.e * g.w.e_rows + (int64_t)c * g.w.row_mul +
                            (up ? g.w.off_up : g.w.off_gate);
        const void *base = up ? g.w.w_up : g.w.w_gate;
        b_lr[i] = lr;
        if (MX) {
            b_ptr[i] = (const uint8_t *)base + row * (Kd / 2) + b_kc * 16;
            s_ptr[i] = (up ? g.w.s_up : g.w.s_gate) + row * (Kd / 32) + b_kc;
        } else {
            b_ptr[i] = (const uint8_t *)base + (row * Kd + b_kc * 8) * 2;
            s_ptr[i] = nullptr;
        }
    }

    u32x4 ra[TL::A_CH], rb[B_CH];
    uint32_t rs[B_CH];
    const u32x4 zero4 = {0u, 0u, 0u, 0u};

    auto gload = [&](int kt) {
        const int k0 = kt * TL::BK;
#pragma unroll
        for (int i = 0; i < TL::A_CH; ++i)
            ra[i] = (k0 + a_kc < Kd) ? *(const u32x4 *)(a_ptr[i] + k0) : zero4;
#pragma unroll
        for (int i = 0; i < B_CH; ++i) {
            if (MX) {
                const bool ok = k0 + b_kc * 32 < Kd;
                rb[i] = ok ? *(const u32x4 *)(b_ptr[i] + k0 / 2) : zero4;
                rs[i] = ok ? (uint32_t)s_ptr[i][k0 / 32] : 127u;
            } else {
                rb[i] = (k0 + b_kc * 8 < Kd) ? *(const u32x4 *)(b_ptr[i] + 2 * k0) : zero4;
            }
        }
    };

    auto lstore = [&](int st) {
        __bf16 *la = lds + st * TL::STAGE;
        __bf16 *lb = la + TL::BM * TL::LDK;
#pragma unroll
        for (int i = 0; i < TL::A_CH; ++i)
            *(u32x4 *)(la + a_lr[i] * TL::LDK + a_kc) = ra[i];
#pragma unroll
        for (int i = 0; i < B_CH; ++i) {
            if (MX) {
                const float sc = e8m0_scale(rs[i]);
                __bf16 *dst = lb + b_lr[i] * TL::LDK + b_kc * 32;
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const uint32_t word = rb[i][w];
                    bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, sc, 0);
                    bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, sc, 1);
                    bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, sc, 2);
                    bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, sc, 3);
                    bf16x8 o = {p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
                    *(bf16x8 *)(dst + w * 8) = o;
                }
            } else {
                *(u32x4 *)(lb + b_lr[i] * TL::LDK + b_kc * 8) = rb[i];
            }
        }
    };

    const int lane = tid & 63, wave = tid >> 6;
    const int wn = wave % TL::WN, wm = wave / TL::WN;
    const int lrow = lane & 31, lk = (lane >> 5) * 8;

    // LDS row of weight block f of this wave
    auto brow = [&](int f) {
        if (GATED)
            return (f < TL::FN / 2) ? wn * (TL::TN / 2) + f * 32
                                    : TL::BN / 2 + wn * (TL::TN / 2) + (f - TL::FN / 2) * 32;
        return wn * TL::TN + f * 32;
    };

    f32x16 acc[TL::FN][TL::FM];
#pragma unroll
    for (int f = 0; f < TL::FN; ++f)
#pragma unroll
        for (int m = 0; m < TL::FM; ++m)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[f][m][r] = 0.0f;

    const int nk = (Kd + TL::BK - 1) / TL::BK;
    gload(0);
    lstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) gload(kt + 1);
        const __bf16 *la = lds + cur * TL::STAGE;
        const __bf16 *lb = la + TL::BM * TL::LDK;
#pragma unroll
        for (int ks = 0; ks < TL::BK / 16; ++ks) {
            bf16x8 bf[TL::FN], af[TL::FM];
#pragma unroll
            for (int f = 0; f < TL::FN; ++f)
                bf[f] = *(const bf16x8 *)(lb + (brow(f) + lrow) * TL::LDK + ks * 16 + lk);
#pragma unroll
            for (int m = 0; m < TL::FM; ++m)
                af[m] = *(const bf16x8 *)(la + (wm * TL::TM + m * 32 + lrow) * TL::LDK +
                                          ks * 16 + lk);
#pragma unroll
            for (int f = 0; f < TL::FN; ++f)
#pragma unroll
                for (int m = 0; m < TL::FM; ++m)
                    acc[f][m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf[f], af[m],
                                                                        acc[f][m], 0, 0, 0);
        }
        if (kt + 1 < nk) lstore(cur ^ 1);
        __syncthreads();
    }

    // ---- epilogue: lane holds features 8*i4 + 4*(lane/32) + j of token lane%32
    const int fq = (lane >> 5) * 4;
    if (GATED) {
        __bf16 *h = (__bf16 *)g.out;
        const int64_t eb = (int64_t)tw.e * g.w.e_rows;
#pragma unroll
        for (int fp = 0; fp < TL::FN / 2; ++fp)
#pragma unroll
            for (int m = 0; m < TL::FM; ++m) {
                const int tl = wm * TL::TM + m * 32 + lrow;
                if (tl >= tw.nrows) continue;
                __bf16 *hrow = h + (int64_t)(tw.row0 + tl) * g.Nout;
#pragma unroll
                for (int i4 = 0; i4 < 4; ++i4) {
                    const int c = tw.n0 + wn * (TL::TN / 2) + fp * 32 + i4 * 8 + fq;
                    if (c >= g.Nout) continue;
                    bf16x4 o;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        float gv = acc[fp][m][i4 * 4 + j];
                        float uv = acc[fp + TL::FN / 2][m][i4 * 4 + j];
                        if (g.w.b_gate)
                            gv += bias_at(g.w.b_gate,
                                          eb + (int64_t)(c + j) * g.w.row_mul + g.w.off_gate);
                        if (g.w.b_up)
                            uv += bias_at(g.w.b_up,
                                          eb + (int64_t)(c + j) * g.w.row_mul + g.w.off_up);
                        o[j] = (__bf16)gated_act(g.act, gv, uv, g.alpha, g.beta, g.limit);
                    }
                    *(bf16x4 *)(hrow + c) = o;
                }
            }
    } else {
        float *y = (float *)g.out;
        const int64_t eb = (int64_t)tw.e * g.w.e_rows;
#pragma unroll
        for (int f = 0; f < TL::FN; ++f)
#pragma unroll
            for (int m = 0; m < TL::FM; ++m) {
                const int tl = wm * TL::TM + m * 32 + lrow;
                if (tl >= tw.nrows) continue;
                float *yrow = y + (int64_t)(tw.row0 + tl) * g.Nout;
#pragma unroll
                for (int i4 = 0; i4 < 4; ++i4) {
                    const int c = tw.n0 + wn * TL::TN + f * 32 + i4 * 8 + fq;
                    if (c >= g.Nout) continue;
                    f32x4 o;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        float v = acc[f][m][i4 * 4 + j];
                        if (g.w.b_gate) v += bias_at(g.w.b_gate, eb + c + j);
                        o[j] = v;
                    }
                    *(f32x4 *)(yrow + c) = o;
                }
            }
    }
}

template <class TL, bool MX, bool GATED>
hipError_t launch(const GemmArgs &a, int64_t max_m_tiles, hipStream_t s)
{
    const int64_t grid = max_m_tiles * a.nN + 8;
    gemm_kernel<TL, MX, GATED><<<dim3((unsigned)grid), dim3(TL::NT), 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace

int gemm_bm(GemmKind kind)
{
    return kind == GemmKind::kPrefill ? PrefillTile::BM : DecodeTile::BM;
}

int gemm_bn(GemmKind kind, bool gated)
{
    const int bn = kind == GemmKind::kPrefill ? PrefillTile::BN : DecodeTile::BN;
    return gated ? bn / 2 : bn;
}

hipError_t launch_gemm_bf16(GemmKind kind, bool gated, bool mxfp4, const GemmArgs &a,
                            int64_t max_m_tiles, hipStream_t s)
{
    if (kind == GemmKind::kPrefill) {
        if (mxfp4)
            return gated ? launch<PrefillTile, true, true>(a, max_m_tiles, s)
                         : launch<PrefillTile, true, false>(a, max_m_tiles, s);
        return gated ? launch<PrefillTile, false, true>(a, max_m_tiles, s)
                     : launch<PrefillTile, false, false>(a, max_m_tiles, s);
    }
    if (mxfp4)
        return gated ? launch<DecodeTile, true, true>(a, max_m_tiles, s)
                     : launch<DecodeTile, true, false>(a, max_m_tiles, s);
    return gated ? launch<DecodeTile, false, true>(a, max_m_tiles, s)
                 : launch<DecodeTile, false, false>(a, max_m_tiles, s);
}

}  // namespace moe
