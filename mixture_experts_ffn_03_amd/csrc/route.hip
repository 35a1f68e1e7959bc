// Router top-K: one 64-lane wavefront per token.
//
// Semantics (logicaffeine "MoeSpec" fields `score`, `selection_bias`,
// `groups`, `renormalize`, `scale`, method `sum_can_clamp`; "Moe" fields
// `norm_top_k`, `weights_scale`, `groups`; graiphic ONNX "MoE" attribute `k`):
//   score   softmax over every logit, or each logit's own sigmoid;
//   key     score + selection bias (selection only);
//   groups  E split into n_group equal contiguous groups, each scored by the
//           sum of its two best keys; experts outside the topk_group best
//           groups are ineligible;
//   top-K   the K largest eligible keys in rank order, equal keys toward the
//           lower expert index (lower group index for groups);
//   weight  the kept scores, renormalised by max(sum, 2^-14) when asked,
//           then times the routed scale.
// Scores, keys, group sums and weights are computed in fp64 so that the
// discrete choices agree with an fp64 reference except at fp64 near-ties;
// the weights are stored as f32.
//
// Lane layout: lane l holds experts l, l+64, l+128, ... (coalesced logit
// loads).  Argmax and max run as all-reductions over the wavefront: within
// each 16-lane row by DPP lane moves (quad swaps, then the half-row and row
// mirrors: each step pairs lanes that hold disjoint groups), across rows by
// two shuffles.  The result is the best element of a total order, so the
// pairing order cannot change it.
// Every argmax runs over a set that still holds a candidate (validated
// options guarantee >= K eligible experts), and a NaN key counts as -inf, so
// every stored id is a real expert index.
#include "moe_kernels.h"

#include <math.h>

namespace moe {
namespace {

struct KeyIdx {
    double key;
    int idx;
};

// (key, idx) is better than (k2, i2) when its key is larger or, on equal
// keys, its index is lower.  Missing entries carry key = -inf, idx = INT_MAX.
__device__ inline bool better(double k1, int i1, double k2, int i2)
{
    return k1 > k2 || (k1 == k2 && i1 < i2);
}

// value of lane (lane's partner under DPP control CTRL) within its 16-lane row
template <int CTRL>
__device__ inline int dpp(int v)
{
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xf, 0xf, false);
}

template <int CTRL>
__device__ inline double dpp(double v)
{
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)dpp<CTRL>((int)(uint32_t)b);
    const uint32_t hi = (uint32_t)dpp<CTRL>((int)(uint32_t)(b >> 32));
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// DPP controls: quad permutations [1,0,3,2] and [2,3,0,1], half-row mirror
// (lane i <-> 7 - i within 8), row mirror (i <-> 15 - i within 16)
constexpr int kQuadXor1 = 0xb1, kQuadXor2 = 0x4e, kHalfMirror = 0x141, kMirror = 0x140;

template <int CTRL>
__device__ inline void argmax_step_dpp(KeyIdx &v)
{
    const double ok = dpp<CTRL>(v.key);
    const int oi = dpp<CTRL>(v.idx);
    if (better(ok, oi, v.key, v.idx)) {
        v.key = ok;
        v.idx = oi;
    }
}

__device__ inline KeyIdx wave_argmax(KeyIdx v)
{
    argmax_step_dpp<kQuadXor1>(v);
    argmax_step_dpp<kQuadXor2>(v);
    argmax_step_dpp<kHalfMirror>(v);
    argmax_step_dpp<kMirror>(v);
#pragma unroll
    for (int off = 16; off <= 32; off <<= 1) {
        double ok = __shfl_xor(v.key, off, 64);
        int oi = __shfl_xor(v.idx, off, 64);
        if (better(ok, oi, v.key, v.idx)) {
            v.key = ok;
            v.idx = oi;
        }
    }
    return v;
}

__device__ inline double wave_max(double v)
{
    v = fmax(v, dpp<kQuadXor1>(v));
    v = fmax(v, dpp<kQuadXor2>(v));
    v = fmax(v, dpp<kHalfMirror>(v));
    v = fmax(v, dpp<kMirror>(v));
    v = fmax(v, __shfl_xor(v, 16, 64));
    return fmax(v, __shfl_xor(v, 32, 64));
}

// The two best (key, idx) of a lane's set, best first; missing entries are
// (-inf, kNone).
struct Top2 {
    double k1, k2;
    int i1, i2;
};

// union of two disjoint sets' best two
__device__ inline Top2 merge_top2(Top2 a, Top2 b)
{
    // first: the better of the two firsts; second: the better of the other
    // list's first and the winning list's second
    const bool bw = better(b.k1, b.i1, a.k1, a.i1);
    const double f_k = bw ? b.k1 : a.k1, o_k = bw ? a.k1 : b.k1, s_k = bw ? b.k2 : a.k2;
    const int f_i = bw ? b.i1 : a.i1, o_i = bw ? a.i1 : b.i1, s_i = bw ? b.i2 : a.i2;
    const bool ow = better(o_k, o_i, s_k, s_i);
    return Top2{f_k, ow ? o_k : s_k, f_i, ow ? o_i : s_i};
}

template <int CTRL>
__device__ inline Top2 top2_step_dpp(Top2 v)
{
    return merge_top2(v, Top2{dpp<CTRL>(v.k1), dpp<CTRL>(v.k2), dpp<CTRL>(v.i1), dpp<CTRL>(v.i2)});
}

__device__ inline Top2 top2_step_shfl(Top2 v, int off)
{
    return merge_top2(v, Top2{__shfl_xor(v.k1, off, 64), __shfl_xor(v.k2, off, 64),
                              __shfl_xor(v.i1, off, 64), __shfl_xor(v.i2, off, 64)});
}

// lane `src` (the same for every lane)'s value, through a scalar register
__device__ inline double lane_value(double v, int src)
{
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, src);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), src);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

__device__ inline double wave_sum(double v)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        v += __shfl_xor(v, off, 64);
    return v;
}

constexpr int kNone = 0x7fffffff;

// bf16 bits -> f32 (exact)
__device__ inline float bf16_to_float(uint16_t b)
{
    return __uint_as_float((uint32_t)b << 16);
}

template <int EPL>
__global__ __launch_bounds__(256) void route_kernel(RouteArgs a)
{
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= a.T) return;   // whole wavefront leaves together
    const int E = a.E;
    const float *lg = a.logits + (int64_t)t * E;

    double score[EPL], key[EPL];
    bool live[EPL];   // a real expert, eligible and not yet taken
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = lane + 64 * i;
        live[i] = e < E;
        score[i] = live[i] ? (double)lg[e] : -INFINITY;
    }

    // scores
    if (a.scoring == 0) {
        double m = -INFINITY;
#pragma unroll
        for (int i = 0; i < EPL; ++i) m = fmax(m, score[i]);
        m = wave_max(m);
        double s = 0.0;
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            score[i] = live[i] ? exp(score[i] - m) : 0.0;
            s += score[i];
        }
        s = wave_sum(s);
#pragma unroll
        for (int i = 0; i < EPL; ++i) score[i] = score[i] / s;
    } else {
#pragma unroll
        for (int i = 0; i < EPL; ++i)
            score[i] = live[i] ? 1.0 / (1.0 + exp(-score[i])) : 0.0;
    }

    // selection keys
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = lane + 64 * i;
        key[i] = live[i] ? (a.sel_bias ? score[i] + (double)a.sel_bias[e] : score[i])
                         : -INFINITY;
        if (key[i] != key[i]) key[i] = -INFINITY;   // NaN input: never preferred
    }

    // group limit
    if (a.n_group > 0) {
        const int gs = E / a.n_group;
        double my_gscore = -INFINITY;   // lane g holds the score of group g
        if ((gs & (gs - 1)) == 0 && gs <= 64) {
            // groups of 2^n <= 64 experts are aligned lane segments of one
            // slot: a top-2 all-reduction within segments (DPP moves up to 16
            // lanes, then shuffles) gives every group's two best keys at once
            double gsum_slot[EPL];
#pragma unroll
            for (int i = 0; i < EPL; ++i) {
                const int e = lane + 64 * i;
                Top2 v{live[i] ? key[i] : -INFINITY, -INFINITY, live[i] ? e : kNone, kNone};
                if (gs >= 2) v = top2_step_dpp<kQuadXor1>(v);
                if (gs >= 4) v = top2_step_dpp<kQuadXor2>(v);
                if (gs >= 8) v = top2_step_dpp<kHalfMirror>(v);
                if (gs >= 16) v = top2_step_dpp<kMirror>(v);
                if (gs >= 32) v = top2_step_shfl(v, 16);
                if (gs >= 64) v = top2_step_shfl(v, 32);
                double gsum = v.k1;
                if (gs >= 2) {
                    gsum = v.k1 + v.k2;
                    if (gsum != gsum) gsum = -INFINITY;
                }
                gsum_slot[i] = gsum;
            }
            // group g's first expert g * gs sits in slot g * gs / 64
            const int src = (lane * gs) & 63, src_slot = (lane * gs) >> 6;
#pragma unroll
            for (int i = 0; i < EPL; ++i) {
                const double v = __shfl(gsum_slot[i], src, 64);
                if (lane < a.n_group && src_slot == i) my_gscore = v;
            }
        } else
        for (int g = 0; g < a.n_group; ++g) {
            KeyIdx b1{-INFINITY, kNone};
#pragma unroll
            for (int i = 0; i < EPL; ++i) {
                const int e = lane + 64 * i;
                if (live[i] && e / gs == g && better(key[i], e, b1.key, b1.idx))
                    b1 = KeyIdx{key[i], e};
            }
            b1 = wave_argmax(b1);
            double gsum = b1.key;
            if (gs >= 2) {
                KeyIdx b2{-INFINITY, kNone};
#pragma unroll
                for (int i = 0; i < EPL; ++i) {
                    const int e = lane + 64 * i;
                    if (live[i] && e / gs == g && e != b1.idx &&
                        better(key[i], e, b2.key, b2.idx))
                        b2 = KeyIdx{key[i], e};
                }
                b2 = wave_argmax(b2);
                gsum = b1.key + b2.key;
                if (gsum != gsum) gsum = -INFINITY;
            }
            if (lane == g) my_gscore = gsum;
        }
        uint64_t kept = 0;
        for (int r = 0; r < a.topk_group; ++r) {
            KeyIdx c{lane < a.n_group && !((kept >> lane) & 1) ? my_gscore : -INFINITY,
                     lane < a.n_group && !((kept >> lane) & 1) ? lane : kNone};
            c = wave_argmax(c);
            kept |= 1ull << c.idx;
        }
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            const int e = lane + 64 * i;
            if (live[i] && !((kept >> (e / gs)) & 1)) live[i] = false;
        }
    }

    // top-K; lane j keeps slot j
    int my_id = 0;
    double my_w = 0.0;
    for (int j = 0; j < a.K; ++j) {
        KeyIdx c{-INFINITY, kNone};
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            const int e = lane + 64 * i;
            if (live[i] && better(key[i], e, c.key, c.idx)) c = KeyIdx{key[i], e};
        }
        c = wave_argmax(c);
        const int owner = c.idx & 63, slot = c.idx >> 6;
        double sc = 0.0;
#pragma unroll
        for (int i = 0; i < EPL; ++i)
            if (i == slot) sc = score[i];
        sc = lane_value(sc, __builtin_amdgcn_readfirstlane(owner));
        if (lane == owner) {
#pragma unroll
            for (int i = 0; i < EPL; ++i)
                if (i == slot) live[i] = false;
        }
        if (lane == j) {
            my_id = c.idx;
            my_w = sc;
        }
    }

    // weights: renormalise (sum in slot order, clamped at 2^-14), then scale
    if (a.renormalize) {
        double s = 0.0;
        for (int j = 0; j < a.K; ++j) s += lane_value(my_w, j);
        const double d = s > 0x1p-14 ? s : 0x1p-14;
        my_w = my_w / d;
    }
    my_w = my_w * (double)a.scale;
    if (lane < a.K) {
        a.ids[(int64_t)t * a.K + lane] = my_id;
        a.weights[(int64_t)t * a.K + lane] = (float)my_w;
    }

    // shared-expert gate of token t (logicaffeine "Moe" `shared_gate`):
    // sigmoid(x[t] . g), the dot product over the hidden features, lane l
    // taking features l, l + 64, ... (coalesced), summed in fp64
    if (a.sgate) {
        double d = 0.0;
        if (a.x_bf16) {
            const uint16_t *xr = (const uint16_t *)a.x + (int64_t)t * a.H;
            const uint16_t *gr = (const uint16_t *)a.sgate;
            for (int c = lane; c < a.H; c += 64)
                d += (double)bf16_to_float(xr[c]) * (double)bf16_to_float(gr[c]);
        } else {
            const float *xr = (const float *)a.x + (int64_t)t * a.H;
            const float *gr = (const float *)a.sgate;
            for (int c = lane; c < a.H; c += 64) d += (double)xr[c] * (double)gr[c];
        }
        d = wave_sum(d);
        if (lane == 0) a.sgate_out[t] = (float)(1.0 / (1.0 + exp(-d)));
    }
}

}  // namespace

hipError_t launch_route(const RouteArgs &a, hipStream_t s)
{
    const dim3 grid((a.T + 3) / 4), block(256);
    const int epl = (a.E + 63) / 64;
    if (epl <= 1)
        route_kernel<1><<<grid, block, 0, s>>>(a);
    else if (epl <= 2)
        route_kernel<2><<<grid, block, 0, s>>>(a);
    else if (epl <= 4)
        route_kernel<4><<<grid, block, 0, s>>>(a);
    else if (epl <= 8)
        route_kernel<8><<<grid, block, 0, s>>>(a);
    else
        route_kernel<16><<<grid, block, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace moe
