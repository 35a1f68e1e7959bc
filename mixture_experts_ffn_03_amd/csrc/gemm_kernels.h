// Grouped expert GEMMs on gfx950 MFMA (v_mfma_f32_32x32x16_{bf16,f16}).
//
// Each workgroup computes one tile of Y^T = W_e * A^T for one expert e:
// BN weight rows (output features) by BM permutation rows (tokens), fp32
// accumulation, reduction in 64-wide k-steps through LDS stages filled by
// direct global->LDS loads.  The weight panel is the MFMA "A" operand and the
// token panel the "B" operand, so each lane ends with four consecutive output
// features of one token -- 8-byte 16-bit / 16-byte f32 stores in the epilogue.
//
// Epilogues (EpiMode):
//  gated  (gate||up GEMM, ONNX "MoE" fc1/fc3): the BN weight rows of a tile
//         are BN/2 gate rows and the BN/2 up rows of the same features; a
//         wave holds the gate and up accumulators of the same features in
//         the same lanes, adds the biases and applies the gated activation.
//         h is stored in fp16 (11-bit significand, 8x finer than bf16) when
//         the whole tile fits fp16's range and the down weights lie in it,
//         else in bf16; one format byte per tile records the choice.
//  act    (fc1 of a non-gated expert): the activation of every feature,
//         stored like the gated h.
//  down   (ONNX "MoE" fc2): when every h tile of its rows is fp16 (the
//         normal case), a workgroup runs the f16 MFMA on the prepared fp16
//         copy of the down weights, or, without one, converts the bf16 (or
//         MXFP4) weights to fp16 after their LDS read (exact in fp16's
//         normal range); otherwise it rounds the fp16 h fragments to bf16
//         and runs the bf16 MFMA (on the fp16 copy rounded back to bf16 when
//         the layer has one, so it never reads the caller's stack).  Adds
//         the down bias and stores y (or, with a split reduction, each
//         split's partial sums) per 64-feature chunk of a row: fp16 when the
//         chunk fits fp16's range (half the bytes the combine reads back),
//         else f32, with one format byte per chunk.  The combine rounds to
//         the output dtype once, after the weighted sum.
//  plain  (the router GEMM): x times the transposed router weights, f32 out.
//
// The token operand of the gated GEMM is gathered straight from x through the
// permutation (row_token), so the permuted activations are never written.
//
// MXFP4 weights (the clika "ClikaRT::nn::QMoEWoQ" class description: the
// experts are quantised, the activation is not, and the dequantisation
// happens per block inside the product with no dense weight tensor in
// memory): the packed codes and e8m0 scales
// travel to LDS at 4.25 bits per weight; after the LDS read each lane turns
// its 8 codes of a sub-step into 8 16-bit values with the gfx950 scaled
// conversion (exact: e2m1 times a power of two fits bf16, and fp16 for the
// scale range the prepare-time check admits), and the MFMA stays 16-bit x
// 16-bit (the activation is not quantised).
//
// Kernel templates and tile shapes, included by the translation units that
// instantiate them (one per tile family, compiled in parallel) and by the
// dispatcher in gemm.hip.
#pragma once

#include "gemm_common.h"

#include <type_traits>

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ inline float bias_at(const void *b, int64_t i)
{
    return bf16_bits_to_float(((const uint16_t *)b)[i]);
}

// stands in for an absent bias (read at index 0)
__device__ const uint16_t g_zero_bias[1] = {0};

// e8m0 byte -> the fp32 multiplier 2^(X-127) (X = 0 is 2^-127, 255 is NaN).
// Selects, not branches: in the k-loop a branch here put a wait for the
// byte's LDS read, and the divergent-exec bookkeeping, between two MFMAs.
__device__ inline float e8m0_scale(uint32_t x)
{
    const uint32_t bits = x == 0u ? 0x00400000u : (x == 255u ? 0x7fc00000u : x << 23);
    return __uint_as_float(bits);
}

// Two bf16 (low, high half of w) -> two fp16, rounded to nearest even like
// the prepared fp16 copy (so both down paths compute on the same values):
// exact in fp16's normal range, whose top the prepare-time range check
// guarantees; a value below 2^-14 keeps the fewer bits of an fp16 subnormal
// (absolute error at most 2^-25).
__device__ inline uint32_t bf16x2_to_f16x2(uint32_t w)
{
    const f16x2 p = {(_Float16)__uint_as_float(w << 16), (_Float16)__uint_as_float(w & 0xffff0000u)};
    return __builtin_bit_cast(uint32_t, p);
}

// Two fp16 -> two bf16, round to nearest even.
__device__ inline uint32_t f16x2_to_bf16x2(uint32_t w)
{
    const f16x2 h = __builtin_bit_cast(f16x2, w);
    const bf16x2 b = {(__bf16)(float)h[0], (__bf16)(float)h[1]};
    return __builtin_bit_cast(uint32_t, b);
}

// Eight MXFP4 elements (one code word, element 2i in the low nibble of byte
// i) times the e8m0 multiplier sc -> eight 16-bit values (bf16 or fp16).
template <bool F16>
__device__ inline u32x4 decode_mxfp4_8(uint32_t word, float sc)
{
    u32x4 o;
    if (F16) {
        o[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, sc, 0));
        o[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, sc, 1));
        o[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, sc, 2));
        o[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, sc, 3));
    } else {
        o[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, sc, 0));
        o[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, sc, 1));
        o[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, sc, 2));
        o[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, sc, 3));
    }
    return o;
}

template <bool F16>
__device__ inline f32x16 mfma(const u32x4 &a, const u32x4 &b, const f32x16 &c)
{
    if (F16)
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Epilogue: lane holds output features 8*i4 + 4*(lane/32) + j (j = 0..3) of
// token lane % 32 of each 32x32 block.
//  gated / act: (weigh-inputs: times the row's routing weight) + fc1 bias,
//      activation, then h stored in fp16 when the tile's max |h| fits fp16
//      and the down weights lie in fp16's range, else bf16 (format byte per
//      tile);
//  down / plain: + bias, f32 store.
template <class TL, int EPI>
__device__ __forceinline__ void epilogue(const GemmArgs &g, const TileWork &tw,
                                         f32x16 (&acc)[TL::FN][TL::FM], float *s_red,
                                         uint8_t *lds)
{
    constexpr int NWAVES = TL::NT / 64;
    constexpr bool GATED = EPI == kEpiGated;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wn = wave % TL::WN, wm = wave / TL::WN;
    const int lrow = lane & 31;
    const int fq = (lane >> 5) * 4;
    // accumulator (f, m) element i; the 4-wave tile's accumulators live in
    // AGPRs and are moved out one by one where they are used (otherwise the
    // compiler copies all 256 to VGPRs after the k-loop, and spills)
    auto accv = [&](int f, int m, int i) {
        float a = acc[f][m][i];
        if constexpr (TL::WPE == 1) asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(a) : "a"(a));
        return a;
    };
    if constexpr (EPI == kEpiAct) {
        // fc1 of a non-gated expert: h = act(rs * acc + b), rs the row's
        // weight under weigh-inputs routing.  Pass 1 takes the tile's max |h|
        // without keeping h; pass 2 recomputes h at the store (keeping every
        // activated accumulator live across the block max spilled thousands
        // of registers).  The activation is uniform: one unrolled body each.
        const int64_t eb = (int64_t)tw.e * g.w.e_rows;
        const int cw = tw.n0 + wn * TL::TN;           // first feature of this wave
        float rs[TL::FM];
        bool tok_ok[TL::FM];
#pragma unroll
        for (int m = 0; m < TL::FM; ++m) {
            const int tl = wm * TL::TM + m * 32 + lrow;
            tok_ok[m] = tl < tw.nrows;
            rs[m] = (g.row_w && tok_ok[m]) ? g.row_w[tw.row0 + tl] : 1.0f;
        }
        // bias of each held feature (a column past Nout reads the last
        // one's): read once into registers on the 4-wave tile, whose
        // accumulators sit in AGPRs; at each use (an L1 hit) on the others,
        // where registers are the scarcer
        const uint16_t *bp = (const uint16_t *)g.w.b_gate;
        auto bias_of = [&](int f, int i) {
            const int c = min(cw + f * 32 + (i / 4) * 8 + fq + i % 4, g.Nout - 1);
            return bp ? bf16_bits_to_float(bp[eb + (int64_t)c * g.w.row_mul + g.w.off_gate]) : 0.0f;
        };
        float bv[TL::FN][16];
        if constexpr (TL::WPE == 1) {
#pragma unroll
            for (int f = 0; f < TL::FN; ++f)
#pragma unroll
                for (int i = 0; i < 16; ++i) bv[f][i] = bias_of(f, i);
        }
        constexpr int PITCH = TL::BN * 2 + 16;
        constexpr bool STAGED = 256 + TL::BM * PITCH <= TL::LDS_BYTES;
        uint16_t *h = (uint16_t *)g.out;
        auto finish = [&](auto act) {
            auto hval = [&](int f, int m, int i) {
                float b;
                if constexpr (TL::WPE == 1) b = bv[f][i];
                else b = bias_of(f, i);
                return act(accv(f, m, i) * rs[m] + b);
            };
            float hm = 0.0f;
#pragma unroll
            for (int f = 0; f < TL::FN; ++f)
#pragma unroll
                for (int m = 0; m < TL::FM; ++m)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const bool ok = tok_ok[m] && cw + f * 32 + (i / 4) * 8 + fq + i % 4 < g.Nout;
                        const float v = hval(f, m, i);
                        hm = fmaxf(hm, ok ? fabsf(v) : 0.0f);
                    }
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) hm = fmaxf(hm, __shfl_xor(hm, off, 64));
            if (lane == 0) s_red[wave] = hm;
            __syncthreads();
            float bmax = s_red[0];
#pragma unroll
            for (int w = 1; w < NWAVES; ++w) bmax = fmaxf(bmax, s_red[w]);
            const bool f16 = g.f16_ok && bmax <= 65504.0f;
            if (tid == 0) g.hfmt[(int64_t)tw.mg * g.h_tiles + tw.nt] = f16 ? kHF16 : kHBF16;
            // pass 2: 4 features of a token per lane, through LDS when the
            // tile fits (whole 16-byte row chunks out), else straight to h
            auto put = [&](int f, int m, int i4, uint16_t *dst) {
                const int r0 = i4 * 4;
                if (f16) {
                    f16x4 o = {(_Float16)hval(f, m, r0), (_Float16)hval(f, m, r0 + 1),
                               (_Float16)hval(f, m, r0 + 2), (_Float16)hval(f, m, r0 + 3)};
                    *(f16x4 *)dst = o;
                } else {
                    bf16x4 o = {(__bf16)hval(f, m, r0), (__bf16)hval(f, m, r0 + 1),
                                (__bf16)hval(f, m, r0 + 2), (__bf16)hval(f, m, r0 + 3)};
                    *(bf16x4 *)dst = o;
                }
            };
            if constexpr (STAGED) {
                uint8_t *hs = lds + 256;
                __syncthreads();                 // every wave has read s_red
#pragma unroll
                for (int f = 0; f < TL::FN; ++f)
#pragma unroll
                    for (int m = 0; m < TL::FM; ++m) {
                        const int tl = wm * TL::TM + m * 32 + lrow;
#pragma unroll
                        for (int i4 = 0; i4 < 4; ++i4) {
                            const int cl = wn * TL::TN + f * 32 + i4 * 8 + fq;
                            put(f, m, i4, (uint16_t *)(hs + tl * PITCH + cl * 2));
                        }
                    }
                __syncthreads();
                constexpr int CPRH = TL::BN / 8;
                for (int q = tid; q < TL::BM * CPRH; q += TL::NT) {
                    const int r = q / CPRH, ch = q % CPRH;
                    const int c = tw.n0 + ch * 8;
                    if (r < tw.nrows && c < g.Nout)
                        *(u32x4 *)(h + (int64_t)(tw.row0 + r) * g.Nout + c) =
                            *(const u32x4 *)(hs + r * PITCH + ch * 16);
                }
            } else {
#pragma unroll
                for (int f = 0; f < TL::FN; ++f)
#pragma unroll
                    for (int m = 0; m < TL::FM; ++m) {
                        if (!tok_ok[m]) continue;
                        const int tl = wm * TL::TM + m * 32 + lrow;
                        uint16_t *hrow = h + (int64_t)(tw.row0 + tl) * g.Nout;
#pragma unroll
                        for (int i4 = 0; i4 < 4; ++i4) {
                            const int c = cw + f * 32 + i4 * 8 + fq;
                            if (c < g.Nout) put(f, m, i4, hrow + c);
                        }
                    }
            }
        };
        switch (g.act) {
        case 2: finish([](float x) { return fmaxf(x, 0.0f); }); break;
        case 3:
            if (g.gelu_mode == 1) finish([](float x) { return gelu_tanh_fast(x); });
            else finish([](float x) { return gelu_erf_fast(x); });
            break;
        case 4: finish([](float x) { return x * sigmoid_fast(x); }); break;
        default: finish([](float x) { return x; });
        }
    } else if constexpr (EPI == kEpiGated) {
        // features of the h tile held per wave: gate/up pairs
        constexpr int FH = GATED ? TL::FN / 2 : TL::FN;
        constexpr int WH = GATED ? TL::TN / 2 : TL::TN;
        // pass 1: activation into the (gate) accumulators, tile max |h|.
        // The activation is uniform, so each one gets its own unrolled loop:
        // tested per value (with the bias tests) it cost as much as the rest
        // of the epilogue together.  Biases are read once per feature; an
        // absent one reads a zero, and a column past Nout reads the last
        // feature's (its value is never stored or counted in the max).  The
        // gated loops also come in a no-bias form (the bias reads cost 2% of
        // a Mixtral-shaped gate||up GEMM).
        const int64_t eb = (int64_t)tw.e * g.w.e_rows;
        float rs[TL::FM];
        bool tok_ok[TL::FM];
#pragma unroll
        for (int m = 0; m < TL::FM; ++m) {
            const int tl = wm * TL::TM + m * 32 + lrow;
            tok_ok[m] = tl < tw.nrows;
            rs[m] = (g.row_w && tok_ok[m]) ? g.row_w[tw.row0 + tl] : 1.0f;
        }
        const uint16_t *bgp = g.w.b_gate ? (const uint16_t *)g.w.b_gate : g_zero_bias;
        const uint16_t *bup = (GATED && g.w.b_up) ? (const uint16_t *)g.w.b_up : g_zero_bias;
        const int64_t bgs = g.w.b_gate ? 1 : 0, bus = (GATED && g.w.b_up) ? 1 : 0;
        // FAST: no row weights and every feature of this wave below Nout
        // (the common case): no scaling and no per-value column test.  The max is kept per 32-row block and the
        // rows past the tile's tokens (whose LDS rows were never loaded) are
        // dropped once per block.  In a one-wave-per-SIMD tile every VALU
        // instruction here costs the matrix pipe four idle cycles.
        auto pass1 = [&](auto bias_tag, auto fast_tag, auto act) {
            constexpr bool BIAS = decltype(bias_tag)::value;
            constexpr bool FAST = decltype(fast_tag)::value;
            float hmb[TL::FM];
#pragma unroll
            for (int m = 0; m < TL::FM; ++m) hmb[m] = 0.0f;
#pragma unroll
            for (int fp = 0; fp < FH; ++fp)
#pragma unroll
                for (int i4 = 0; i4 < 4; ++i4) {
                    const int c = tw.n0 + wn * WH + fp * 32 + i4 * 8 + fq;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const bool c_ok = FAST || c + j < g.Nout;
                        float bg = 0.0f, bu = 0.0f;
                        if constexpr (BIAS) {
                            const int64_t f = eb + (int64_t)min(c + j, g.Nout - 1) * g.w.row_mul;
                            bg = bf16_bits_to_float(bgp[(f + g.w.off_gate) * bgs]);
                            if constexpr (GATED) bu = bf16_bits_to_float(bup[(f + g.w.off_up) * bus]);
                        }
#pragma unroll
                        for (int m = 0; m < TL::FM; ++m) {
                            float gv = acc[fp][m][i4 * 4 + j];
                            if constexpr (!FAST) gv *= rs[m];
                            if constexpr (BIAS) gv += bg;
                            float uv = 0.0f;
                            if constexpr (GATED) {
                                uv = acc[fp + TL::FN / 2][m][i4 * 4 + j];
                                if constexpr (!FAST) uv *= rs[m];
                                if constexpr (BIAS) uv += bu;
                            }
                            const float h = act(gv, uv);
                            acc[fp][m][i4 * 4 + j] = h;
                            hmb[m] = fmaxf(hmb[m], c_ok ? fabsf(h) : 0.0f);
                        }
                    }
                }
            float hm = 0.0f;
#pragma unroll
            for (int m = 0; m < TL::FM; ++m) hm = fmaxf(hm, tok_ok[m] ? hmb[m] : 0.0f);
            return hm;
        };
        const bool bias = bgs != 0 || bus != 0;
        const bool fast = !g.row_w && tw.n0 + (wn + 1) * WH <= g.Nout;
        auto run = [&](auto act) {
            if (fast) {
                return bias ? pass1(std::true_type{}, std::true_type{}, act)
                            : pass1(std::false_type{}, std::true_type{}, act);
            }
            return bias ? pass1(std::true_type{}, std::false_type{}, act)
                        : pass1(std::false_type{}, std::false_type{}, act);
        };
        float hmax;
        if constexpr (GATED) {
            if (g.act == 0) {
                hmax = run([](float x, float u) { return x * sigmoid_fast(x) * u; });
            } else {
                const float al = g.alpha, be = g.beta, L = g.limit;
                if (L > 0.0f)
                    hmax = run([=](float x, float u) {
                        x = fminf(x, L);
                        u = fminf(fmaxf(u, -L), L);
                        return x * sigmoid_fast(al * x) * (u + be);
                    });
                else
                    hmax = run([=](float x, float u) { return x * sigmoid_fast(al * x) * (u + be); });
            }
        }
        // block max -> storage format of this h tile
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) hmax = fmaxf(hmax, __shfl_xor(hmax, off, 64));
        if (lane == 0) s_red[wave] = hmax;
        __syncthreads();
        float bmax = s_red[0];
#pragma unroll
        for (int w = 1; w < NWAVES; ++w) bmax = fmaxf(bmax, s_red[w]);
        const bool f16 = g.f16_ok && bmax <= 65504.0f;
        if (tid == 0) g.hfmt[(int64_t)tw.mg * g.h_tiles + tw.nt] = f16 ? kHF16 : kHBF16;
        // pass 2: store h.  When the whole h tile fits in LDS (beside the
        // reduction scratch), each lane parks its 4 features of a token there
        // (row pitch padded by 16 bytes: the 32 tokens of a 64-lane write
        // fall on every bank at most twice), then the workgroup writes whole
        // 16-byte chunks, a wave covering full row segments -- instead of
        // 8-byte pieces scattered over 32 rows per store instruction.
        constexpr int HW = GATED ? TL::BN / 2 : TL::BN;     // h features per tile
        constexpr int PITCH = HW * 2 + 16;
        constexpr bool STAGED = 256 + TL::BM * PITCH <= TL::LDS_BYTES;
        uint16_t *h = (uint16_t *)g.out;
        if constexpr (STAGED) {
            uint8_t *hs = lds + 256;
            __syncthreads();                 // every wave has read s_red
            // one loop per storage format (the format test per value put a
            // branch around every LDS write)
            auto park = [&](auto f16_tag) {
                constexpr bool H16 = decltype(f16_tag)::value;
#pragma unroll
                for (int fp = 0; fp < FH; ++fp)
#pragma unroll
                    for (int m = 0; m < TL::FM; ++m) {
                        const int tl = wm * TL::TM + m * 32 + lrow;
#pragma unroll
                        for (int i4 = 0; i4 < 4; ++i4) {
                            const int cl = wn * WH + fp * 32 + i4 * 8 + fq;   // feature in tile
                            const f32x16 &a = acc[fp][m];
                            const int r0 = i4 * 4;
                            uint8_t *dst = hs + tl * PITCH + cl * 2;
                            if constexpr (H16) {
                                f16x4 o = {(_Float16)a[r0], (_Float16)a[r0 + 1],
                                           (_Float16)a[r0 + 2], (_Float16)a[r0 + 3]};
                                *(f16x4 *)dst = o;
                            } else {
                                bf16x4 o = {(__bf16)a[r0], (__bf16)a[r0 + 1], (__bf16)a[r0 + 2],
                                            (__bf16)a[r0 + 3]};
                                *(bf16x4 *)dst = o;
                            }
                        }
                    }
            };
            if (f16) park(std::true_type{});
            else park(std::false_type{});
            __syncthreads();
            // every chunk's LDS read goes out before the first store
            constexpr int CPRH = HW / 8;                     // 16-byte chunks per h row
            constexpr int NQ = (TL::BM * CPRH + TL::NT - 1) / TL::NT;
            u32x4 hv[NQ];
#pragma unroll
            for (int i = 0; i < NQ; ++i) {
                const int q = tid + i * TL::NT;
                if (q < TL::BM * CPRH)
                    hv[i] = *(const u32x4 *)(hs + (q / CPRH) * PITCH + (q % CPRH) * 16);
            }
#pragma unroll
            for (int i = 0; i < NQ; ++i) {
                const int q = tid + i * TL::NT;
                const int r = q / CPRH, ch = q % CPRH;
                const int c = tw.n0 + ch * 8;
                if (q < TL::BM * CPRH && r < tw.nrows && c < g.Nout)
                    *(u32x4 *)(h + (int64_t)(tw.row0 + r) * g.Nout + c) = hv[i];
            }
        } else {
#pragma unroll
            for (int fp = 0; fp < FH; ++fp)
#pragma unroll
                for (int m = 0; m < TL::FM; ++m) {
                    const int tl = wm * TL::TM + m * 32 + lrow;
                    if (tl >= tw.nrows) continue;
                    uint16_t *hrow = h + (int64_t)(tw.row0 + tl) * g.Nout;
#pragma unroll
                    for (int i4 = 0; i4 < 4; ++i4) {
                        const int c = tw.n0 + wn * WH + fp * 32 + i4 * 8 + fq;
                        if (c >= g.Nout) continue;
                        const f32x16 &a = acc[fp][m];
                        const int r0 = i4 * 4;
                        if (f16) {
                            f16x4 o = {(_Float16)a[r0], (_Float16)a[r0 + 1], (_Float16)a[r0 + 2],
                                       (_Float16)a[r0 + 3]};
                            *(f16x4 *)(hrow + c) = o;
                        } else {
                            bf16x4 o = {(__bf16)a[r0], (__bf16)a[r0 + 1], (__bf16)a[r0 + 2],
                                        (__bf16)a[r0 + 3]};
                            *(bf16x4 *)(hrow + c) = o;
                        }
                    }
                }
        }
    } else {
        // split s of a split reduction writes its partial sums to its own
        // buffer; the bias goes in once, with split 0
        float *y = (float *)g.out + (int64_t)tw.ks * g.split_stride;
        const void *bias = tw.ks == 0 ? g.w.b_gate : nullptr;
        const int64_t eb = (int64_t)tw.e * g.w.e_rows;
        if constexpr (EPI == kEpiDown) {
            // a wave's features of one row form one chunk, held by lanes l
            // and l ^ 32: with yfmt, fp16 when its max |y| fits (every chunk is
            // written, so the formats need no clearing); else (f32 layers) f32.  The bias, if any, is read once.  (One
            // store path for both: two made the 4-wave tile spill.)
            static_assert(TL::TN == kYWidth, "one y chunk per wave and row");
            const int q0 = tw.n0 + wn * TL::TN;
            // FULL: the wave's whole chunk lies below Nout (no column tests)
            auto chunks = [&](auto with_bias, auto full_tag) {
                constexpr bool B = decltype(with_bias)::value;
                constexpr bool FULL = decltype(full_tag)::value;
                float bv[TL::FN][16];
                if constexpr (B) {
#pragma unroll
                    for (int f = 0; f < TL::FN; ++f)
#pragma unroll
                        for (int i = 0; i < 16; ++i) {
                            const int c = q0 + f * 32 + (i / 4) * 8 + fq + i % 4;
                            bv[f][i] = c < g.Nout ? bias_at(bias, eb + c) : 0.f;
                        }
                }
                auto yval = [&](int f, int m, int i) {
                    float a = acc[f][m][i];
                    // the 4-wave tile's accumulators live in AGPRs: move each
                    // where it is used (the compiler otherwise copies all
                    // 256 to VGPRs after the k-loop, and spills)
                    if constexpr (TL::WPE == 1)
                        asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(a) : "a"(a));
                    if constexpr (B) return a + bv[f][i];
                    else return a;
                };
                if (q0 >= g.Nout) return;
                // one pass per row block: its chunk max, then its stores
#pragma unroll
                for (int m = 0; m < TL::FM; ++m) {
                    float v[TL::FN][16];
                    float mx = 0.f;
#pragma unroll
                    for (int f = 0; f < TL::FN; ++f)
#pragma unroll
                        for (int i = 0; i < 16; ++i) {
                            v[f][i] = yval(f, m, i);
                            if (FULL || q0 + f * 32 + (i / 4) * 8 + fq < g.Nout)
                                mx = fmaxf(mx, fabsf(v[f][i]));
                        }
                    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
                    const int tl = wm * TL::TM + m * 32 + lrow;
                    if (tl >= tw.nrows) continue;
                    const int64_t row = tw.row0 + tl;
                    const bool h16 = g.yfmt && mx <= 65504.f;
                    if (g.yfmt && fq == 0)
                        g.yfmt[tw.ks * g.yfmt_split_stride + row * g.yfmt_stride + q0 / kYWidth] =
                            h16 ? kYF16 : kYF32;
                    float *yq = y + row * g.Nout + q0;
#pragma unroll
                    for (int f = 0; f < TL::FN; ++f)
#pragma unroll
                        for (int i4 = 0; i4 < 4; ++i4) {
                            const int cc = f * 32 + i4 * 8 + fq, r0 = i4 * 4;
                            if (!FULL && q0 + cc >= g.Nout) continue;
                            if (h16) {
                                f16x4 o = {(_Float16)v[f][r0], (_Float16)v[f][r0 + 1],
                                           (_Float16)v[f][r0 + 2], (_Float16)v[f][r0 + 3]};
                                *(f16x4 *)((_Float16 *)yq + cc) = o;
                            } else {
                                f32x4 o = {v[f][r0], v[f][r0 + 1], v[f][r0 + 2], v[f][r0 + 3]};
                                *(f32x4 *)(yq + cc) = o;
                            }
                        }
                }
            };
            const bool full = q0 + kYWidth <= g.Nout;
            if (full) {
                if (bias) chunks(std::true_type{}, std::true_type{});
                else chunks(std::false_type{}, std::true_type{});
            } else {
                if (bias) chunks(std::true_type{}, std::false_type{});
                else chunks(std::false_type{}, std::false_type{});
            }
            return;
        }
        // plain (router logits [T, Nout], Nout = E of any size): a lane's 4
        // features c .. c+3 go out as one 16-byte store when Nout is a
        // multiple of 4 (every row then starts 16-byte aligned and a quad
        // that starts inside the row ends inside it), else one by one up to
        // Nout (a quad past the row's end would write into the next row, or
        // past the buffer)
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
                        if (bias && c + j < g.Nout) v += bias_at(bias, eb + c + j);
                        o[j] = v;
                    }
                    if ((g.Nout & 3) == 0) {
                        *(f32x4 *)(yrow + c) = o;
                    } else {
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            if (c + j < g.Nout) yrow[c + j] = o[j];
                    }
                }
            }
    }
}

// ---------------------------------------------------------------------------
// Pipelined kernel: gfx950 direct global->LDS loads.
//
// Each k-step's token and weight panels are fetched by global_load_lds_dwordx4
// (16 bytes per lane straight into LDS, no staging registers) into one of
// SA (tokens) / SB (weights) LDS stages; the next token step and SB-1 weight
// steps are in flight while one is computed.  One barrier per k-step,
// preceded by a wait for this thread's own loads of the step about to be read.
//
// 16-bit LDS rows are BK*2 bytes; the 16-byte chunk c of row r sits at
// physical chunk c ^ sw(r).  gfx950 serves a 16-byte-per-lane LDS read 16
// lanes at a time across 64 four-byte banks (measured: this swizzle has no
// bank conflicts, one built for 8 lanes / 32 banks had a conflict on half the
// LDS cycles), so the 16 lanes that read one chunk column of 16 consecutive
// rows must land in 16 different 16-byte bank groups.  Each load instruction
// of a wave fills one contiguous KiB of LDS; the swizzle is applied by
// choosing which global chunk each lane fetches.
//
// MXFP4 weight stages hold the packed layout unchanged: per 32-row block one
// KiB of codes (32 bytes a row, halves swapped on bit 3 of the row: the 16
// lanes of a read hit 64 distinct banks) and 64 bytes of scales.  A k-step
// of 64 is consumed in a permuted k order that both operands share: MFMA
// sub-step s, lane half h covers k = 32h + 8s .. 32h + 8s + 7 (instead of
// 16s + 8h ..).  A lane's weight codes for the whole k-step are then one
// 16-byte LDS read and lie in one scale block (h).
//
// Operand conversion happens after the LDS read, in registers: fp16 down GEMM
// steps convert the bf16 weight fragments to fp16 (exact in fp16's normal
// range, whose top is checked at prepare) or decode MXFP4 to fp16; bf16 down
// GEMM steps round fp16-stored h fragments to bf16 (and, on a layer with the
// prepared fp16 copy, that copy's fragments back to bf16).  Token chunks past the reduction length are read from a
// zero buffer; packed MXFP4 weights are zero past it already.

template <int BN_, int BM_, int BK_, int WN_, int WM_, int SA_, int SB_, bool MX_, int WPE_ = 2>
struct DTile {
    static constexpr int BN = BN_, BM = BM_, BK = BK_, WN = WN_, WM = WM_;
    // waves per SIMD the registers are budgeted for: 2 (256 each), or 1 (512:
    // the 128 x 128 accumulators of a 4-wave 256 x 256 tile)
    static constexpr int WPE = WPE_;
    static constexpr int SA = SA_, SB = SB_;            // LDS stages of A and of B
    static constexpr bool MX = MX_;                     // MXFP4 weights (packed)
    static constexpr int NT = 64 * WN * WM;
    static constexpr int NWAVES = WN * WM;
    static constexpr int TN = BN / WN, TM = BM / WM;
    static constexpr int FN = TN / 32, FM = TM / 32;
    static constexpr int CPR = BK / 8;                  // 16-byte chunks per token row
    static constexpr int ROWB = BK * 2;                 // bytes per token row
    static constexpr int NA = BM * CPR / NT;            // token loads per thread per step
    // weights: 16-bit rows like the tokens, or MXFP4 KiB code blocks plus one
    // scale load (RBW row-blocks of 64 bytes per wave)
    static constexpr int RB = BN / 32;                  // 32-row weight blocks
    static constexpr int RBW = RB / NWAVES;             // scale pieces per wave (MXFP4)
    static constexpr int NBC = MX ? RB / NWAVES : BN * CPR / NT;   // weight-row loads
    static constexpr int NB = MX ? NBC + 1 : NBC;       // weight loads per thread per step
    static constexpr int CODE_BYTES = BN * BK / 2;      // MXFP4 codes of a stage
    static constexpr int A_BYTES = BM * ROWB;
    static constexpr int B_BYTES = MX ? CODE_BYTES + RB * 64 : BN * ROWB;
    static constexpr int B_BASE = SA * A_BYTES;         // B stages follow the A stages
    static constexpr int LDS_BYTES = SA * A_BYTES + SB * B_BYTES;
    static_assert(NA * NT == BM * CPR, "whole token loads per thread");
    static_assert(MX ? (RBW * NWAVES == RB && RBW >= 1 && BK == 64)
                     : (NBC * NT == BN * CPR), "whole weight loads per thread");
    static_assert(NA >= 1 && NBC >= 1, "every thread loads A and B");
    static_assert(FN >= 2 && FN % 2 == 0, "gate/up pairs per wave");
    // tokens one step ahead (SA = 2), or (the compiler-scheduled loop's deep
    // mode) as many token stages as weight stages
    static constexpr bool DEEP = SA == SB && SA > 2;
    static_assert((SA == 2 || DEEP) && SB >= SA && SB <= 4, "A one or SB-1 steps ahead, B up to three");
    static_assert(2 * NB <= 63, "vmcnt range");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS");
    static_assert(B_BYTES % 1024 == 0 || MX, "KiB-aligned stages");
    static_assert(LDS_BYTES >= 4 * (kMaxExperts + 1) * 4 && LDS_BYTES >= NWAVES * 4,
                  "scheduling tables and epilogue scratch overlay the stages");
    // swizzle of token row r: rows r and r + 16/CPR start in the same bank group
    __device__ static inline int sw(int r) { return (r / (16 / CPR)) % CPR; }
    static_assert(CPR == 4 || CPR == 8 || CPR == 16, "row of 64, 128 or 256 bytes");
};

// A 16-bit tile reads weight stages from the prepared copy's blocks
// (kPack16Rows rows of 64-wide k-steps, Pack16Args): its rows are a whole
// block or an equal share of one, at 64-element k-steps of 128-byte rows.
template <class TL>
constexpr bool pack16_tile()
{
    return !TL::MX && TL::BK == 64 && TL::CPR == 8 && kPack16Rows % TL::BN == 0 &&
           (TL::BN / 2) % 16 == 0;
}

// 512 threads, wave 64x128; k-steps of 64 (128-byte rows: a 64-byte row
// piece halves the L2->LDS rate); A (token rows, L2/MALL resident) two
// stages, B (weights, first touch from HBM) three: 2 x 32 + 3 x 32 KiB.
using PrefillDTile = DTile<256, 256, 64, 4, 2, 2, 3, false>;
// The same tile and stages for the gate||up (and fc1) GEMM on 256 threads:
// one wave per SIMD, each 64 features x all 256 token rows (accumulators in
// AGPRs), its MFMAs interleaved by hand with the reads and loads (kloop_il
// below).  Every wave spans the tile's rows, so a tile of n rows keeps all
// four SIMDs at ceil(n / 32) row blocks (a 2 x 2 layout of 128 x 128 waves
// reads less LDS per MFMA but leaves the SIMDs of the lower half idle or
// short on a partial tile).
using PrefillFcTile = DTile<256, 256, 64, 4, 1, 2, 3, false, 1>;
// Its loop body for a tile of at most 128 rows (the 256-row schedule gives
// one to each expert with that few): token stages of half the size leave room
// for a fourth weight stage in the same 160 KiB, and such a tile, with half
// the MFMA work per k-step, waits on its weight stream.
using ShortFcTile = DTile<256, 128, 64, 4, 1, 2, 4, false, 1>;
static_assert(ShortFcTile::NT == PrefillFcTile::NT && ShortFcTile::WPE == PrefillFcTile::WPE &&
                  ShortFcTile::LDS_BYTES <= PrefillFcTile::LDS_BYTES,
              "the short body runs in the 256-row tile's workgroup and LDS");
// 256 threads, wave 64x32; weights stream from HBM: four B stages, and four
// token stages (4 KiB each, the loop's deep mode) so that two weight stages
// stay in flight through each barrier and three between barriers.
using DecodeDTile = DTile<256, 32, 64, 4, 1, 4, 4, false>;
// The down GEMM at decode sizes has short reductions (I / 64 k-steps): two
// B stages (72 KiB) let two workgroups share a CU, one streaming while the
// other starts up (measured 0.081 -> 0.071 ms on the Qwen3-shaped step; the
// gate||up GEMM, 32 k-steps per tile, keeps four stages).
using DecodeDownTile = DTile<256, 32, 64, 4, 1, 2, 2, false>;
// GEMM 1 at decode sizes: 128 weight rows (64 gate/up feature pairs), two
// waves, four token and four weight stages of 16 KiB in 80 KiB, so that two
// workgroups share a CU: one tile's start (its tile lookup, token rows and
// first weight stages, a few microseconds) overlaps the other's stream.
using DecodeFcTile = DTile<128, 32, 64, 2, 1, 4, 4, false>;
// MXFP4 weights: a weight stage is 8.5 KiB, so four of them fit beside the
// token stages (2 x 32 + 4 x 8.5 KiB; decode 2 x 4 + 4 x 8.5 KiB).
using PrefillMXTile = DTile<256, 256, 64, 4, 2, 2, 4, true>;
using DecodeMXTile = DTile<256, 32, 64, 4, 1, 2, 4, true>;
// Mid tiles, 256 x 128 rows, for experts of a few hundred rows (a 256-row
// tile would run a mostly empty second tile per expert).  16-bit: 512
// threads, wave 64x64, 2 x 16 + 3 x 32 KiB.  MXFP4: 256 threads, wave
// 64x128, 2 x 16 + 4 x 8.5 KiB, so two workgroups share a CU.
using MidDTile = DTile<256, 128, 64, 4, 2, 2, 3, false>;
using MidMXTile = DTile<256, 128, 64, 4, 1, 2, 4, true>;

// 16 bytes per lane from global memory straight into LDS: lane l writes
// LDS bytes [m0 + 16 l, m0 + 16 l + 16).  Issued as inline asm so that the
// compiler inserts no waits of its own for it: every wait on these loads is
// the explicit vmcnt in wait_loads_barrier.
__device__ __forceinline__ void dma16(const void *src, uint32_t lds_byte)
{
    asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(lds_byte) : "memory");
}

// The same with the non-temporal cache policy: for weights that one tile
// reads once (decode-sized tiles, one token tile per expert).  A read probe
// on MI355X: 5.1-5.5 TB/s for these loads without it, 5.4-5.9 with it.
__device__ __forceinline__ void dma16_nt(const void *src, uint32_t lds_byte)
{
    asm volatile("global_load_lds_dwordx4 %0, off nt" ::"v"(src), "{m0}"(lds_byte) : "memory");
}

// weight loads of tile TL: non-temporal for the decode-sized (32-row) tiles
// of the expert GEMMs (not the router GEMM, whose token tiles all read the
// same weights)
template <class TL, int EPI>
__device__ __forceinline__ void dma16_w(const void *src, uint32_t lds_byte)
{
    if constexpr (TL::BM == 32 && EPI != kEpiPlain) dma16_nt(src, lds_byte);
    else dma16(src, lds_byte);
}

// The same load in the scalar-base form: the address is a uniform 64-bit
// base in SGPRs plus this lane's 32-bit offset, so a k-step moves only the
// base (one scalar add for all of a thread's loads) and the loads need no
// per-lane 64-bit address arithmetic.
__device__ __forceinline__ void dma16s(uint32_t voff, const void *sbase, uint32_t lds_byte)
{
    asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "{m0}"(lds_byte) : "memory");
}

// The same with the non-temporal cache policy, for the weights of the
// gate||up short body.  A tile of at most 128 rows is almost always the only
// tile of a small expert, so no other tile reads its weight panel (DeepSeek-
// V3-shaped gate||up 4.38 -> 4.32 ms; in the down GEMM it measured no gain).
__device__ __forceinline__ void dma16s_nt(uint32_t voff, const void *sbase, uint32_t lds_byte)
{
    asm volatile("global_load_lds_dwordx4 %0, %1 nt" ::"v"(voff), "s"(sbase), "{m0}"(lds_byte) : "memory");
}

__device__ __forceinline__ uint32_t lds_offset(const void *p)
{
    return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void *)p;
}

// Wait until at most N of this thread's DMA loads are outstanding and all of
// its LDS reads have returned, then synchronise the workgroup.
template <int N>
__device__ __forceinline__ void wait_loads_barrier()
{
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// 16 zero bytes in global memory: the source of every DMA chunk past the
// reduction length, so a ragged last k-step needs no masking.
__device__ const u32x4 g_zero16 = {0u, 0u, 0u, 0u};

// RAGGED: the reduction length is not a multiple of BK (the last k-step's
// token chunks past it read zeros); otherwise no k-step needs a bounds test.
// WH (the down GEMM): the weights are the prepared copy in fp16 (g.wpk with
// g.wpk_f16): with F16 streamed as they are, without F16 (a bf16 down GEMM,
// some h tile of its rows stored in bf16) each fragment rounded back to bf16
// after its LDS read (exact: the copy came from bf16 values), so a layer with
// the copy never reads the caller's down stack.  Without WH, F16 converts
// bf16 weight fragments to fp16 in registers.  The weights come from the
// prepared stage-layout copy whenever g.wpk is set, else from the caller's
// rows.
template <class TL, int EPI, bool F16, bool RAGGED, bool WH = false>
__device__ __forceinline__ void dma_body(const GemmArgs &g, const TileWork &tw, uint8_t *lds,
                                         float *s_red)
{
    constexpr bool GATED = EPI == kEpiGated;
    constexpr bool HIN = EPI == kEpiDown;    // A operand is h with per-tile formats
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int Kd = g.Kd;

    // ---- token rows of the per-load chunks (their global sources are set
    // once the rows' token ids are known, below)
    const uint8_t *a_src[TL::NA];
    int a_k[TL::NA];                   // first k of the chunk this load fetches
    bool a_ok[TL::NA];                 // the chunk's row holds a token
    int a_r[TL::NA];                   // its permutation row (clamped into the tile)
#pragma unroll
    for (int i = 0; i < TL::NA; ++i) {
        const int q = (i * TL::NWAVES + wave) * 64 + lane;   // LDS chunk index
        const int row = q / TL::CPR, p = q % TL::CPR;
        const int c = p ^ TL::sw(row);
        a_r[i] = tw.row0 + min(row, tw.nrows - 1);
        a_k[i] = c * 8;
        a_ok[i] = row < tw.nrows;
    }
    // ---- weight sources.  16-bit: row base + swizzled chunk.  MXFP4: this
    // lane's 16 bytes of the KiB code block of tile row-block t (load i), and
    // of the 64-byte scale piece of row-block RBW * wave + lane / 4.
    // blocks per expert and k-step in the prepared 16-bit copy
    const int pk_nblk = (g.Nout + (GATED ? kPack16Rows / 2 : kPack16Rows) - 1) /
                        (GATED ? kPack16Rows / 2 : kPack16Rows);
    const uint8_t *b_src[TL::NBC];
    int b_k[TL::NBC];
    const uint8_t *s_src = nullptr;
    const uint8_t *b_blk = nullptr;      // the tile's block of the prepared copy
    uint32_t b_off[TL::NBC] = {};         // this load's byte offset in a block
    if constexpr (TL::MX) {
        // logical row-block (packed layout) of tile row-block t
        const int nrb_tot = (GATED ? 2 : 1) * g.nrb_half;
        auto lrb = [&](int t) {
            const bool up = GATED && t >= TL::RB / 2;
            const int tt = up ? t - TL::RB / 2 : t;
            return (up ? g.nrb_half : 0) + min(tw.n0 / 32 + tt, g.nrb_half - 1);
        };
#pragma unroll
        for (int i = 0; i < TL::NBC; ++i) {
            const int t = i * TL::NWAVES + wave;
            b_k[i] = 0;
            b_src[i] = g.pk + ((int64_t)tw.e * nrb_tot + lrb(t)) * g.nks * 1024 + lane * 16;
        }
        const int t = wave * TL::RBW + min(lane / 4, TL::RBW - 1);
        s_src = g.pks + ((int64_t)tw.e * nrb_tot + lrb(t)) * g.nks * 64 + (lane % 4) * 16;
    } else if (g.wpk) {
        // the prepared stage-layout copy of kPack16Rows-row blocks: this
        // load's 16 bytes of the tile's block of k-step 0 (LDS chunk q of the
        // stage, the bank swizzle baked in); a k-step moves on by the
        // expert's nblk blocks.  A tile of fewer rows reads its share of a
        // block -- for the gated GEMM its gate rows and its up rows -- whose
        // rows start a multiple of 16 rows in, so they carry the same swizzle
        // as in the tile's own stage.
        constexpr int SUB = kPack16Rows / TL::BN;               // tiles per block
        const int bi = tw.nt / SUB, h = tw.nt % SUB;
        const uint8_t *blk = g.wpk + ((int64_t)tw.e * g.nks * pk_nblk + bi) * kPack16Stage;
        b_blk = blk;
#pragma unroll
        for (int i = 0; i < TL::NBC; ++i) {
            const int q = (i * TL::NWAVES + wave) * 64 + lane;
            const int r = q / TL::CPR;
            const int pr = GATED ? (r < TL::BN / 2 ? h * (TL::BN / 2) + r
                                                   : kPack16Rows / 2 + h * (TL::BN / 2) +
                                                         (r - TL::BN / 2))
                                 : h * TL::BN + r;
            b_k[i] = 0;
            b_off[i] = (uint32_t)((pr * TL::CPR + q % TL::CPR) * 16);
            b_src[i] = blk + b_off[i];
        }
    } else {
#pragma unroll
        for (int i = 0; i < TL::NBC; ++i) {
            const int q = (i * TL::NWAVES + wave) * 64 + lane;
            const int row = q / TL::CPR, p = q % TL::CPR;
            const int c = p ^ TL::sw(row);
            const bool up = GATED && row >= TL::BN / 2;
            const int f = min(tw.n0 + (up ? row - TL::BN / 2 : row), g.Nout - 1);
            const int64_t wrow = (int64_t)tw.e * g.w.e_rows + (int64_t)f * g.w.row_mul +
                                 (up ? g.w.off_up : g.w.off_gate);
            const void *base = up ? g.w.w_up : g.w.w_gate;
            b_k[i] = c * 8;
            b_src[i] = (const uint8_t *)base + (wrow * Kd + c * 8) * 2;
        }
    }
    // bytes between a weight load's sources of consecutive k-steps, and
    // whether a ragged last k-step selects zeros (the prepared copy is zero
    // past the reduction length already)
    const uint32_t b_step = (!TL::MX && g.wpk) ? (uint32_t)(pk_nblk * kPack16Stage) : 2u * TL::BK;
    const bool b_ragged = RAGGED && !(!TL::MX && g.wpk);
    const uint8_t *zero = (const uint8_t *)&g_zero16;

    // LDS byte offset of this wave's first KiB of a stage, and of its scale
    // pieces (wave-uniform)
    const uint32_t wave_lds = __builtin_amdgcn_readfirstlane(lds_offset(lds) + wave * 1024);
    const uint32_t wave_sc = __builtin_amdgcn_readfirstlane(
        lds_offset(lds) + TL::B_BASE + TL::CODE_BYTES + wave * TL::RBW * 64);
    // k-steps [kbeg, kend) of the reduction: all of them, or this tile's
    // split; kt below counts from kbeg (LDS stages by kt, addresses by kx(kt))
    const int nk_all = (Kd + TL::BK - 1) / TL::BK;
    const int kbeg = tw.ks * nk_all / g.ksplit;
    const int nk = (tw.ks + 1) * nk_all / g.ksplit - kbeg;
    const int nfull = RAGGED ? Kd / TL::BK : nk_all;   // k-steps with no chunk past Kd
    auto kx = [&](int kt) { return kt + kbeg; };
    auto issue_a_one = [&](int kt, int i) {
        const uint32_t st = wave_lds + (kt % TL::SA) * TL::A_BYTES;
        const int k0 = kx(kt) * TL::BK;
        const bool full = kx(kt) < nfull;
        // rows past the tile's tokens are not fetched (their LDS rows only
        // feed output columns the epilogue drops).  Only token loads are
        // ever skipped, so every wait below, which counts the weight loads
        // issued after a step's token loads, still covers what it must.
        if (a_ok[i])
            dma16((!RAGGED || full || k0 + a_k[i] < Kd) ? a_src[i] + 2 * k0 : zero,
                  st + i * TL::NWAVES * 1024);
    };
    // weight load i of step kt (MXFP4: i == NBC is the scale load)
    auto issue_b_one = [&](int kt, int i) {
        if constexpr (TL::MX) {
            if (i < TL::NBC) {
                dma16_w<TL, EPI>(b_src[i] + (int64_t)kx(kt) * 1024,
                      wave_lds + TL::B_BASE + (kt % TL::SB) * TL::B_BYTES + i * TL::NWAVES * 1024);
            } else if (lane < 4 * TL::RBW) {
                dma16_w<TL, EPI>(s_src + (int64_t)kx(kt) * 64, wave_sc + (kt % TL::SB) * TL::B_BYTES);
            }
        } else {
            const uint32_t st = wave_lds + TL::B_BASE + (kt % TL::SB) * TL::B_BYTES;
            const int k0 = kx(kt) * TL::BK;
            const bool full = kx(kt) < nfull;
            dma16_w<TL, EPI>((!b_ragged || full || k0 + b_k[i] < Kd) ? b_src[i] + (int64_t)kx(kt) * b_step
                                                          : zero,
                  st + i * TL::NWAVES * 1024);
        }
    };
    // the token rows' global sources (row_token: the gathered token of each row)
#pragma unroll
    for (int i = 0; i < TL::NA; ++i) {
        const int src = g.row_token ? g.row_token[a_r[i]] : a_r[i];
        a_src[i] = (const uint8_t *)g.a + ((int64_t)src * Kd + a_k[i]) * 2;
    }

    // Branch-free forms for the interleaved loop.  A token row past the
    // tile fetches the 16 zero bytes at every step (its step is 0 bytes); a
    // step past the last one fetches the last step again (L2 hits) into its
    // free stage; so every k-step issues the same loads, the address is one
    // multiply-add, and the waits need no cases.
    const uint8_t *a_base[TL::NA];
    uint32_t a_step[TL::NA];
#pragma unroll
    for (int i = 0; i < TL::NA; ++i) {
        a_base[i] = a_ok[i] ? a_src[i] : zero;
        a_step[i] = a_ok[i] ? 2 * TL::BK : 0;
    }
    // The 4-wave 16-bit tile with a whole number of k-steps: token chunk i of
    // a k-step is a + k-step offset (uniform, in SGPRs) + a fixed 32-bit lane
    // offset (the launcher checks that A lies within 4 GiB).  A row past the
    // tile's tokens reads its clamped row's data (finite values in rows whose
    // outputs are dropped) instead of the zero chunk.
    constexpr bool A_SBASE = !TL::MX && TL::WPE == 1 && !RAGGED;
    uint32_t a_voff[TL::NA];
#pragma unroll
    for (int i = 0; i < TL::NA; ++i)
        a_voff[i] = (uint32_t)(a_src[i] - (const uint8_t *)g.a);
    auto issue_a_nb = [&](int kt, int i) {
        const uint32_t st = wave_lds + (kt % TL::SA) * TL::A_BYTES;
        const uint32_t kc = (uint32_t)(kbeg + min(kt, nk - 1));
        if constexpr (A_SBASE) {
            dma16s(a_voff[i], (const uint8_t *)g.a + (uint64_t)kc * (2 * TL::BK),
                   st + i * TL::NWAVES * 1024);
            return;
        }
        const uint8_t *p = a_base[i] + (uint64_t)kc * a_step[i];
        if (RAGGED) p = ((int)kc * TL::BK + a_k[i] < Kd) ? p : zero;
        dma16(p, st + i * TL::NWAVES * 1024);
    };
    auto issue_b_nb = [&](int kt, int i) {
        const uint32_t kc = (uint32_t)(kbeg + min(kt, nk - 1));
        if constexpr (TL::MX) {
            // packed codes are zero past K; load NBC is the scale piece
            if (i < TL::NBC) {
                dma16_w<TL, EPI>(b_src[i] + (int64_t)kc * 1024,
                      wave_lds + TL::B_BASE + (kt % TL::SB) * TL::B_BYTES + i * TL::NWAVES * 1024);
            } else if (lane < 4 * TL::RBW) {
                dma16_w<TL, EPI>(s_src + (int64_t)kc * 64, wave_sc + (kt % TL::SB) * TL::B_BYTES);
            }
        } else {
            // the 16-bit interleaved loop streams the prepared copy only (the
            // launchers send a layer without one to the 8-wave tile): a
            // uniform block base per k-step and fixed lane offsets, and no
            // ragged select (the copy is zero past the reduction length)
            const uint32_t st = wave_lds + TL::B_BASE + (kt % TL::SB) * TL::B_BYTES;
            if constexpr (std::is_same<TL, ShortFcTile>::value && EPI != kEpiDown)
                dma16s_nt(b_off[i], b_blk + (uint64_t)kc * b_step, st + i * TL::NWAVES * 1024);
            else
                dma16s(b_off[i], b_blk + (uint64_t)kc * b_step, st + i * TL::NWAVES * 1024);
        }
    };
    auto issue_a = [&](int kt) {
#pragma unroll
        for (int i = 0; i < TL::NA; ++i) issue_a_one(kt, i);
    };
    auto issue_b = [&](int kt) {
#pragma unroll
        for (int i = 0; i < TL::NB; ++i) issue_b_one(kt, i);
    };

    // ---- fragment addressing (row r of a 32-row block = lane % 32)
    const int wn = wave % TL::WN, wm = wave / TL::WN;
    const int lrow = lane & 31, lhalf = lane >> 5;
    const int lsw = TL::sw(lrow);
    auto brow = [&](int f) {
        if (GATED)
            return (f < TL::FN / 2) ? wn * (TL::TN / 2) + f * 32
                                    : TL::BN / 2 + wn * (TL::TN / 2) + (f - TL::FN / 2) * 32;
        return wn * TL::TN + f * 32;
    };
    // MXFP4: this lane's code chunk within a row-block's KiB, and scale byte
    const int mx_code = lrow * 32 + 16 * (lhalf ^ ((lrow >> 3) & 1));
    const int mx_scale = lhalf * 32 + lrow;

    // h formats of these rows (bf16 down GEMM only; read from global memory,
    // whose waits only ever lengthen the explicit ones)
    const uint8_t *hf = HIN ? g.hfmt + (int64_t)tw.mg * g.h_tiles : nullptr;

    f32x16 acc[TL::FN][TL::FM];
#pragma unroll
    for (int f = 0; f < TL::FN; ++f)
#pragma unroll
        for (int m = 0; m < TL::FM; ++m)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[f][m][r] = 0.0f;

    constexpr int NKS = TL::BK / 16;     // MFMA sub-steps per k-step
    static_assert(NKS % 2 == 0, "fragment ping-pong over an even number of sub-steps");

    // MV: 32-row token blocks of this wave that hold rows (the others skip
    // their LDS reads and MFMAs; an expert's last tile is usually short)
    auto kloop = [&](auto mv_tag) {
        constexpr int MV = decltype(mv_tag)::value;
        u32x4 bf[2][TL::FN], af[2][TL::FM > 0 ? TL::FM : 1];
        u32x4 cq[TL::MX ? TL::FN : 1];     // MXFP4 codes of the current k-step
        float scf[TL::MX ? TL::FN : 1];    // and their scale multipliers
        // read the fragments of sub-step ks of k-step kt into buffer b
        auto read = [&](int kt, int ks, int b) {
            const uint8_t *sa = lds + (kt % TL::SA) * TL::A_BYTES;
            const uint8_t *sb = lds + TL::B_BASE + (kt % TL::SB) * TL::B_BYTES;
            if constexpr (TL::MX) {
                if (ks == 0) {
#pragma unroll
                    for (int f = 0; f < TL::FN; ++f) {
                        const int t = brow(f) / 32;
                        cq[f] = *(const u32x4 *)(sb + t * 1024 + mx_code);
                        scf[f] = e8m0_scale(sb[TL::CODE_BYTES + t * 64 + mx_scale]);
                    }
                }
#pragma unroll
                for (int f = 0; f < TL::FN; ++f) bf[b][f] = decode_mxfp4_8<F16>(cq[f][ks], scf[f]);
            } else {
                const int coff = ((ks * 2 + lhalf) ^ lsw) * 16;
#pragma unroll
                for (int f = 0; f < TL::FN; ++f) {
                    bf[b][f] = *(const u32x4 *)(sb + (brow(f) + lrow) * TL::ROWB + coff);
                    if (F16 && !WH) {
#pragma unroll
                        for (int w = 0; w < 4; ++w) bf[b][f][w] = bf16x2_to_f16x2(bf[b][f][w]);
                    } else if (!F16 && WH) {
#pragma unroll
                        for (int w = 0; w < 4; ++w) bf[b][f][w] = f16x2_to_bf16x2(bf[b][f][w]);
                    }
                }
            }
            // token chunk of this sub-step (MXFP4: the permuted k order)
            const int acoff = ((TL::MX ? 4 * lhalf + ks : ks * 2 + lhalf) ^ lsw) * 16;
            // bf16 down GEMM: an fp16-stored h step is rounded to bf16
            const bool a_f16 = HIN && !F16 && hf[(kx(kt) * TL::BK) / g.h_width] == kHF16;
#pragma unroll
            for (int m = 0; m < MV; ++m) {
                af[b][m] = *(const u32x4 *)(sa + (wm * TL::TM + m * 32 + lrow) * TL::ROWB + acoff);
                if (a_f16) {
#pragma unroll
                    for (int w = 0; w < 4; ++w) af[b][m][w] = f16x2_to_bf16x2(af[b][m][w]);
                }
            }
        };
        auto mma = [&](int b) {
#pragma unroll
            for (int f = 0; f < TL::FN; ++f)
#pragma unroll
                for (int m = 0; m < MV; ++m)
                    acc[f][m] = mfma<F16>(bf[b][f], af[b][m], acc[f][m]);
        };
        // Barrier of step j: A(j) and B(j) are in LDS and every wave has
        // finished reading step j-1, whose stages A(j+1) and B(j+SB-1) then
        // refill.  Issue order: prologue B(0), A(0), B(1), ..., B(SB-2);
        // after barrier j the group A(j+1), B(j+SB-1).  Loads complete in
        // issue order, so A(j) and B(j) (issued before A(j)) are done once at
        // most the loads issued after A(j) are pending: B(j+SB-2) for j >= 1,
        // B(1..SB-2) for j = 0.
        // Deep mode (SA = SB = S): the group after barrier j is A(j+S-1),
        // B(j+S-1), prologue B(0), A(0), B(1), A(1), ..., B(S-2), A(S-2), so S-2 whole
        // stages stay in flight through each barrier (with two token stages
        // a barrier needs B(j+1) as well, which leaves one; a weight stream
        // from HBM then stalls on latency).  Token loads of rows past the
        // tile are skipped, so every wait counts weight loads only: at most
        // c*NB pending, c the steps issued after the one needed, means that
        // one is done (each later group holds NB weight loads).
        auto issue_group = [&](int j) {
            if constexpr (TL::DEEP) {
                if (j + TL::SB - 1 < nk) {
                    issue_a(j + TL::SB - 1);
                    issue_b(j + TL::SB - 1);
                }
            } else {
                if (j + 1 < nk) issue_a(j + 1);
                if (j + TL::SB - 1 < nk) issue_b(j + TL::SB - 1);
            }
        };
        // wait until at most c steps' weight loads are pending, then barrier
        auto wait_pending_steps = [&](int c) {
            if (c >= 2) wait_loads_barrier<2 * TL::NB>();
            else if (c == 1) wait_loads_barrier<TL::NB>();
            else wait_loads_barrier<0>();
        };
        // the same group, load by load, spread over the sub-steps of step j
        // (a burst of DMA issues stalls the wave before its MFMAs); the
        // order of issue, which the waits rely on, is unchanged
        auto issue_group_part = [&](int j, int part) {
            constexpr int L = TL::NA + TL::NB;
            const int ja = TL::DEEP ? j + TL::SB - 1 : j + 1;
#pragma unroll
            for (int q = 0; q < L; ++q) {
                if (q < part * L / NKS || q >= (part + 1) * L / NKS) continue;
                if (q < TL::NA) {
                    if (ja < nk) issue_a_one(ja, q);
                } else {
                    if (j + TL::SB - 1 < nk) issue_b_one(j + TL::SB - 1, q - TL::NA);
                }
            }
        };
        static_assert(TL::SB - 2 <= 2, "prologue wait cases");
        if constexpr (TL::DEEP) {
            issue_b(0);
            issue_a(0);
#pragma unroll
            for (int s = 1; s < TL::SB - 1; ++s)
                if (s < nk) {
                    issue_b(s);
                    issue_a(s);
                }
            wait_pending_steps(min(TL::SB - 2, nk - 1));   // steps issued after step 0
        } else {
            issue_b(0);
            issue_a(0);
#pragma unroll
            for (int s = 1; s < TL::SB - 1; ++s)
                if (s < nk) issue_b(s);
            wait_pending_steps(min(TL::SB - 2, nk - 1));   // B steps issued after A(0)
        }
        issue_group(0);
        auto step_barrier = [&](int j) {
            if constexpr (TL::DEEP) {
                // steps j+1 .. j+S-2 issued after step j (those below nk)
                wait_pending_steps(min(TL::SB - 2, nk - 1 - j));
            } else {
                // (with SB = 2, B(j) follows A(j) in its group: wait for all)
                if (TL::SB >= 3 && j + TL::SB - 2 < nk) wait_loads_barrier<TL::NB>();
                else wait_loads_barrier<0>();
            }
        };
        read(0, 0, 0);
        for (int kt = 0; kt < nk; ++kt) {
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const int cur = ks & 1;
                if (kt > 0) issue_group_part(kt, ks);   // group 0 went out whole
                if (ks + 1 < NKS) {
                    read(kt, ks + 1, cur ^ 1);
                } else if (kt + 1 < nk) {
                    // the MFMAs of the previous sub-step keep the matrix
                    // pipe busy through the barrier
                    step_barrier(kt + 1);
                    read(kt + 1, 0, cur ^ 1);
                }
                mma(cur);
            }
        }
    };
    // The hand-laid k-loop (the 4-wave 16-bit tile, where one wave per SIMD
    // must keep the matrix pipe fed by itself, and the MXFP4 tiles, whose
    // decode work then sits between the MFMAs; each sched_barrier fences the
    // compiler's scheduler).  Every MFMA is followed by one item: a fragment
    // read of the next sub-step, then a DMA load of a step's group (its A
    // loads, then its B loads).  16-bit tiles put the step barrier at the end
    // of sub-step 2 (below).  MXFP4 tiles issue the group of k-step kt --
    // A(kt+1), B(kt+SB-1) -- over sub-steps 0 .. NKS-2; their last sub-step
    // issues half of its MFMAs, then the step barrier (its own fragments
    // were read in the sub-step before), then the next step's code fetches,
    // token reads and decodes between its remaining MFMAs.
    auto kloop_il = [&](auto mv_tag) {
        constexpr int MV = decltype(mv_tag)::value;
        u32x4 bf[2][TL::FN], af[2][TL::FM > 0 ? TL::FM : 1];
        u32x4 cq[TL::MX ? TL::FN : 1];     // MXFP4 codes of the current k-step
        float scf[TL::MX ? TL::FN : 1];    // and their scale multipliers
        auto fence = [] { __builtin_amdgcn_sched_barrier(0); };
        // fragment r of sub-step (kt, ks) into buffer b: weights r < FN,
        // then tokens FN + m.  MXFP4: the k-step's codes and scale are read
        // with sub-step 0, every sub-step decodes its 8 values per lane.
        auto read_one = [&](int kt, int ks, int b, int r) {
            const uint8_t *sa = lds + (kt % TL::SA) * TL::A_BYTES;
            const uint8_t *sb = lds + TL::B_BASE + (kt % TL::SB) * TL::B_BYTES;
            const int coff = ((ks * 2 + lhalf) ^ lsw) * 16;
            if (r < TL::FN) {
                if constexpr (TL::MX) {
                    if (ks == 0) {
                        const int t = brow(r) / 32;
                        cq[r] = *(const u32x4 *)(sb + t * 1024 + mx_code);
                        scf[r] = e8m0_scale(sb[TL::CODE_BYTES + t * 64 + mx_scale]);
                    }
                    bf[b][r] = decode_mxfp4_8<F16>(cq[r][ks], scf[r]);
                } else {
                    bf[b][r] = *(const u32x4 *)(sb + (brow(r) + lrow) * TL::ROWB + coff);
                    if (F16 && !WH) {
#pragma unroll
                        for (int w = 0; w < 4; ++w) bf[b][r][w] = bf16x2_to_f16x2(bf[b][r][w]);
                    } else if (!F16 && WH) {
#pragma unroll
                        for (int w = 0; w < 4; ++w) bf[b][r][w] = f16x2_to_bf16x2(bf[b][r][w]);
                    }
                }
            } else {
                const int m = r - TL::FN;
                const int acoff = ((TL::MX ? 4 * lhalf + ks : ks * 2 + lhalf) ^ lsw) * 16;
                af[b][m] = *(const u32x4 *)(sa + (wm * TL::TM + m * 32 + lrow) * TL::ROWB + acoff);
                if (HIN && !F16 && hf[(kx(kt) * TL::BK) / g.h_width] == kHF16) {
#pragma unroll
                    for (int w = 0; w < 4; ++w) af[b][m][w] = f16x2_to_bf16x2(af[b][m][w]);
                }
            }
        };
        // MXFP4, next k-step: its code words and raw scale bytes are fetched
        // right after the step barrier (all of them before any is used), and
        // sub-step 0's fragments decoded only after the token reads, so the
        // LDS round trip overlaps MFMAs instead of sitting between two
        uint32_t sbyte[TL::MX ? TL::FN : 1];
        auto mx_fetch = [&](int kt, int r) {
            const uint8_t *sb = lds + TL::B_BASE + (kt % TL::SB) * TL::B_BYTES;
            const int t = brow(r) / 32;
            cq[r] = *(const u32x4 *)(sb + t * 1024 + mx_code);
            sbyte[r] = sb[TL::CODE_BYTES + t * 64 + mx_scale];
        };
        auto mx_decode0 = [&](int b, int r) {
            scf[r] = e8m0_scale(sbyte[r]);
            bf[b][r] = decode_mxfp4_8<F16>(cq[r][0], scf[r]);
        };
        constexpr int NR = TL::FN + MV;                // reads per sub-step
        constexpr int L = TL::NA + TL::NB;             // loads per k-step
        constexpr int Q = TL::FN * MV;                 // MFMAs per sub-step
        // load q of step j's group
        auto load_one = [&](int j, int q) {
            if (q < TL::NA) issue_a_nb(j + 1, q);
            else issue_b_nb(j + TL::SB - 1, q - TL::NA);
        };
        auto mfma_q = [&](int cur, int q) {
            const int f = q / (MV > 0 ? MV : 1), m = q % (MV > 0 ? MV : 1);
            acc[f][m] = mfma<F16>(bf[cur][f], af[cur][m], acc[f][m]);
        };
        // prologue: B(0), A(0), B(1 .. SB-2); A(0) and B(0) landed
#pragma unroll
        for (int i = 0; i < TL::NB; ++i) issue_b_nb(0, i);
#pragma unroll
        for (int i = 0; i < TL::NA; ++i) issue_a_nb(0, i);
#pragma unroll
        for (int s = 1; s < TL::SB - 1; ++s)
#pragma unroll
            for (int i = 0; i < TL::NB; ++i) issue_b_nb(s, i);
        wait_loads_barrier<(TL::SB - 2) * TL::NB>();
#pragma unroll
        for (int r = 0; r < NR; ++r) read_one(0, 0, 0, r);
        fence();
        if constexpr (!TL::MX) {
            // 16-bit weights.  The step barrier of k-step kt+1 closes sub-step
            // 2 of k-step kt: by then every fragment of stage kt has been read
            // (sub-step 3's in sub-step 2), so all 16 MFMAs of sub-step 3 can
            // carry the reads of k-step kt+1's sub-step 0, and the group of
            // loads that refills stage kt's slots -- A(kt+2), B(kt+SB) --
            // starts right there: loads [0, P0) of group g in sub-step 3 of
            // k-step g-1 (after the prologue for g = 0), [P0, P1) in sub-step
            // 0 and [P1, L) in sub-step 1 of k-step g.  At the barrier of
            // k-step kt+1 only the B loads of group kt are younger than
            // A(kt+1), so a wait for at most NB pending loads covers A(kt+1)
            // and B(kt+1).  (With the barrier inside sub-step 3, the next
            // step's reads had only the MFMAs after it to hide behind.)
            static_assert(NKS == 4, "four MFMA sub-steps per k-step");
            constexpr int P0 = L * 3 / 8, P1 = P0 + (L - P0 + 1) / 2;
#pragma unroll
            for (int q = 0; q < P0; ++q) {
                load_one(0, q);
                fence();
            }
            for (int kt = 0; kt < nk; ++kt) {
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
                    const int cur = ks & 1;
                    const int lo = ks == 0 ? P0 : ks == 1 ? P1 : 0;
                    const int hi = ks == 0 ? P1 : ks == 1 ? L : ks == 3 ? P0 : 0;
                    const int g = ks == 3 ? kt + 1 : kt;
                    const int rk = ks == 3 ? kt + 1 : kt, rs = ks == 3 ? 0 : ks + 1;
                    constexpr int NI = NR + (P1 - P0 > P0 ? P1 - P0 : P0);
#pragma unroll
                    for (int i = 0; i < (Q > NI ? Q : NI); ++i) {
                        if (i < Q) mfma_q(cur, i);
                        // (past the last step the reads take a stale stage
                        // into the idle buffer: in bounds and never used)
                        if (i < NR) read_one(rk, rs, cur ^ 1, i);
                        else if (i - NR < hi - lo) load_one(g, lo + i - NR);
                        fence();
                    }
                    if (ks == NKS - 2 && kt + 1 < nk) {
                        wait_loads_barrier<TL::NB>();
                        fence();
                    }
                }
            }
            return;
        }
        for (int kt = 0; kt < nk; ++kt) {
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const int cur = ks & 1;
                const int l0 = ks * L / (NKS - 1), l1 = (ks + 1) * L / (NKS - 1);
                if (ks + 1 < NKS) {
                    constexpr int NI = NR + (L + NKS - 2) / (NKS - 1);
#pragma unroll
                    for (int i = 0; i < (Q > NI ? Q : NI); ++i) {
                        if (i < Q) mfma_q(cur, i);
                        if (i < NR) read_one(kt, ks + 1, cur ^ 1, i);
                        else if (i - NR < l1 - l0) load_one(kt, l0 + i - NR);
                        fence();
                    }
                } else {
                    // half of the sub-step's MFMAs go out before the step
                    // barrier (they cover part of its wait: the down GEMM
                    // on the Mixtral shape 0.99 -> 0.96 ms against one)
                    constexpr int PRE = Q > 1 ? Q / 2 : Q;
#pragma unroll
                    for (int i = 0; i < PRE; ++i) {
                        mfma_q(cur, i);
                        fence();
                    }
                    // A(kt+1) and B(kt+1) landed: only B(kt+SB-1) may be pending
                    if (kt + 1 < nk) wait_loads_barrier<TL::SB >= 3 ? TL::NB : 0>();
                    fence();
                    // MXFP4 items: FN code/scale fetches, MV token reads, FN
                    // decodes; two items per MFMA.  (Past the last step the
                    // reads take a stale stage into the idle buffer: in bounds
                    // and never used.)
                    constexpr int NI = 2 * TL::FN + MV;
                    constexpr int NM = Q - PRE;
                    constexpr int IPM = NM > 0 ? (NI + NM - 1) / NM : NI;
#pragma unroll
                    for (int i = 0; i < (NM > NI ? NM : NI); ++i) {
                        if (i < NM) mfma_q(cur, PRE + i);
#pragma unroll
                        for (int u = 0; u < IPM; ++u) {
                            const int it = i * IPM + u;
                            if (it < TL::FN) mx_fetch(kt + 1, it);
                            else if (it < TL::FN + MV) read_one(kt + 1, 0, cur ^ 1, it);
                            else if (it < NI) mx_decode0(cur ^ 1, it - TL::FN - MV);
                        }
                        fence();
                    }
                }
            }
        }
    };
    // every wave runs the same loads and barriers; only its MFMA work differs
    const int mv = min(max((tw.nrows - wm * TL::TM + 31) / 32, 0), TL::FM);
    if constexpr (TL::WPE == 1 || TL::MX) {
        static_assert(TL::SB >= 3 && NKS >= 2 && !TL::DEEP, "interleaved loop");
        // every count of 32-row blocks up to FM has its own loop
        static_assert(TL::FM <= 8, "block counts");
        switch (mv) {
        case 1: kloop_il(std::integral_constant<int, 1>{}); break;
        case 2: kloop_il(std::integral_constant<int, (TL::FM >= 2 ? 2 : 1)>{}); break;
        case 3: kloop_il(std::integral_constant<int, (TL::FM >= 3 ? 3 : 1)>{}); break;
        case 4: kloop_il(std::integral_constant<int, (TL::FM >= 4 ? 4 : 1)>{}); break;
        case 5: kloop_il(std::integral_constant<int, (TL::FM >= 5 ? 5 : 1)>{}); break;
        case 6: kloop_il(std::integral_constant<int, (TL::FM >= 6 ? 6 : 1)>{}); break;
        case 7: kloop_il(std::integral_constant<int, (TL::FM >= 7 ? 7 : 1)>{}); break;
        case 8: kloop_il(std::integral_constant<int, (TL::FM >= 8 ? 8 : 1)>{}); break;
        default: kloop_il(std::integral_constant<int, 0>{});
        }
        // the repeated loads past the last step land before LDS is reused
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        epilogue<TL, EPI>(g, tw, acc, s_red, lds);
        return;
    }
    if (mv == TL::FM) kloop(std::integral_constant<int, TL::FM>{});
    else if (TL::FM > 1 && mv == 1) kloop(std::integral_constant<int, 1>{});
    else if (TL::FM > 2 && mv == 2) kloop(std::integral_constant<int, (TL::FM > 2 ? 2 : 1)>{});
    else if (TL::FM > 3 && mv == 3) kloop(std::integral_constant<int, (TL::FM > 3 ? 3 : 1)>{});
    else kloop(std::integral_constant<int, 0>{});
    // all waves are done reading LDS before the epilogue reuses it as scratch
    __syncthreads();
    epilogue<TL, EPI>(g, tw, acc, s_red, lds);
}

// Registers for TL::WPE waves per SIMD: with 2 (256 VGPRs each) the 4-wave
// MXFP4 mid tile runs two workgroups per CU; the 4-wave fc tile takes 512.
template <class TL, int EPI>
__global__ __launch_bounds__(TL::NT, TL::WPE) void gemm_dma_kernel(GemmArgs g)
{
    constexpr int NW = EPI == kEpiGated ? TL::BN / 2 : TL::BN;
    // one LDS allocation: the scheduling table, then the stages, then the
    // epilogue scratch use it in turn
    __shared__ __attribute__((aligned(1024))) uint8_t lds[TL::LDS_BYTES];
    int *s_cum = (int *)lds;
    float *s_red = (float *)lds;

    TileWork tw;
    if (!find_tile(g, s_cum, NW, &tw)) return;
    const bool ragged = g.Kd % TL::BK != 0;
    if constexpr (EPI == kEpiDown) {
        // down GEMM: fp16 operands iff every h tile of these rows is fp16
        const uint8_t *hf = g.hfmt + (int64_t)tw.mg * g.h_tiles;
        int all16 = g.f16_ok;
        for (int i = threadIdx.x; i < g.h_tiles; i += TL::NT) all16 &= hf[i] == kHF16;
        // block AND through an LDS word (the library's own reduction would
        // need LDS beyond the stages)
        volatile int *flag = (volatile int *)lds;
        __syncthreads();                     // every s_cum read is done
        if (threadIdx.x == 0) *flag = 1;
        __syncthreads();
        if (!all16) *flag = 0;
        __syncthreads();
        const bool f16 = *flag != 0;
        __syncthreads();                     // before the loads overwrite it
        if (f16 && !TL::MX && g.wpk_f16) {
            if constexpr (std::is_same<TL, PrefillFcTile>::value) {
                if (tw.nrows <= ShortFcTile::BM && !ragged) {
                    dma_body<ShortFcTile, EPI, true, false, true>(g, tw, lds, s_red);
                    return;
                }
            }
            if (ragged) dma_body<TL, EPI, true, true, !TL::MX>(g, tw, lds, s_red);
            else dma_body<TL, EPI, true, false, !TL::MX>(g, tw, lds, s_red);
        } else if (TL::WPE != 1 && f16) {
            // (the one-wave-per-SIMD tile runs only with the prepared fp16 copy)
            if constexpr (TL::WPE != 1) {
                if (ragged) dma_body<TL, EPI, true, true>(g, tw, lds, s_red);
                else dma_body<TL, EPI, true, false>(g, tw, lds, s_red);
            }
        } else if (!TL::MX && g.wpk_f16) {
            // bf16 down GEMM of a layer with the fp16 copy: weights from the copy
            if (ragged) dma_body<TL, EPI, false, true, true>(g, tw, lds, s_red);
            else dma_body<TL, EPI, false, false, true>(g, tw, lds, s_red);
        } else {
            if (ragged) dma_body<TL, EPI, false, true>(g, tw, lds, s_red);
            else dma_body<TL, EPI, false, false>(g, tw, lds, s_red);
        }
    } else {
        __syncthreads();                     // every s_cum read is done
        if constexpr (std::is_same<TL, PrefillFcTile>::value && EPI == kEpiGated) {
            if (tw.nrows <= ShortFcTile::BM && !ragged) {
                dma_body<ShortFcTile, EPI, false, false>(g, tw, lds, s_red);
                return;
            }
        }
        if (ragged) dma_body<TL, EPI, false, true>(g, tw, lds, s_red);
        else dma_body<TL, EPI, false, false>(g, tw, lds, s_red);
    }
}

template <class TL, int EPI>
hipError_t launch_dma(const GemmArgs &a, int64_t max_m_tiles, hipStream_t s)
{
    const int64_t grid = max_m_tiles * a.nN * a.ksplit + 8;
    gemm_dma_kernel<TL, EPI><<<dim3((unsigned)grid), dim3(TL::NT), 0, s>>>(a);
    return hipGetLastError();
}

// every epilogue mode of one tile shape
template <class TL>
hipError_t launch_epi(int epi, const GemmArgs &a, int64_t max_m_tiles, hipStream_t s)
{
    switch (epi) {
    case kEpiGated: return launch_dma<TL, kEpiGated>(a, max_m_tiles, s);
    case kEpiAct: return launch_dma<TL, kEpiAct>(a, max_m_tiles, s);
    case kEpiPlain:
        // the router GEMM runs on the 16-bit 32-row tiles only
        if constexpr (!TL::MX && TL::BM == 32) return launch_dma<TL, kEpiPlain>(a, max_m_tiles, s);
        else return hipErrorInvalidValue;
    default: return launch_dma<TL, kEpiDown>(a, max_m_tiles, s);
    }
}

}  // namespace

// Launchers of the tile families, one translation unit each.
hipError_t launch_prefill16(int epi, const GemmArgs &a, int64_t max_m_tiles, hipStream_t s);
hipError_t launch_prefill_mx(int epi, const GemmArgs &a, int64_t max_m_tiles, hipStream_t s);
hipError_t launch_mid(bool mxfp4, int epi, const GemmArgs &a, int64_t max_m_tiles, hipStream_t s);
hipError_t launch_decode(bool mxfp4, int epi, const GemmArgs &a, int64_t max_m_tiles,
                         hipStream_t s);

}  // namespace moe
