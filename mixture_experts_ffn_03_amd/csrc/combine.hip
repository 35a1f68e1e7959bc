// Router-weighted combine (clika "MoE": the expert outputs combine under the
// router weights; "ClikaRT::nn::QMoEWoQ::forward": an optional shared-expert
// output folds into the same epilogue).  With weigh-inputs routing
// ("MoeSpec" `weigh_inputs`) the weights were applied to the experts' inputs
// and every kept output joins the sum with weight one.
//
// out[t, :] = sum_{j=0..K-1} w[t, j] * y[slot_row[t, j], :]  (+ s[t] shared[t, :])
// with s[t] = sigmoid(x[t] . g) when the layer's shared-expert gate is bound
// (logicaffeine "Moe" `shared_gate`; computed by the route kernel), else 1.
// accumulated in f32 in slot order j = 0, 1, ..., rounded once to the output
// dtype (round to nearest even for bf16).  No atomics: each output element
// is produced by one thread, so results are bitwise reproducible.  A chunk
// of y the down GEMM stored in fp16 (its format byte says so) is read as
// fp16 and widened exactly.  y is read once, with non-temporal loads
// (DeepSeek-V3-shaped step: 0.203 -> 0.186 ms).
#include "moe_kernels.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// Each thread produces 8 consecutive features of one token (one 16-byte bf16
// store).  The (slot, split) pieces of y it sums are taken 8 at a time
// (8 / splits slots per group): the slots' rows and weights first, then, with
// chunk formats, each piece's format byte together with its 16-byte fp16 load
// (both depend only on the row), so a group costs two dependent memory round
// trips; an f32 piece is loaded once its format is known.  S = splits is a
// template parameter so that every piece index is a compile-time constant.
template <int S>
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a)
{
    const int H8 = a.H / 8;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (int64_t)a.T * H8) return;
    const int t = (int)(idx / H8), c = (int)(idx % H8) * 8;
    const int q = c / kYWidth, q0 = q * kYWidth;
    const int32_t *srow = a.slot_row + (int64_t)t * a.K;
    const float *wrow = a.weights + (int64_t)t * a.K;
    constexpr int G = 8 / S;                 // slots per group
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int j0 = 0; j0 < a.K; j0 += G) {
        const int n = a.K - j0 < G ? a.K - j0 : G;
        // branch-free loads: slots past the group's end repeat its last one
        // (and are not summed)
        int row[G];
        float w[G];
#pragma unroll
        for (int jj = 0; jj < G; ++jj) {
            const int j = j0 + (jj < n ? jj : n - 1);
            row[jj] = srow[j];
            w[jj] = wrow[j];
        }
        // piece p = (slot p / S, split p % S)
        uint8_t fmt[G * S];
        f16x8 h[G * S];
        if (a.yfmt) {
#pragma unroll
            for (int p = 0; p < G * S; ++p) {
                const int jj = p / S, sp = p % S;
                const float *yr = a.y + sp * a.split_stride + (int64_t)row[jj] * a.H;
                fmt[p] = a.yfmt[sp * a.yfmt_split_stride + (int64_t)row[jj] * a.yfmt_stride + q];
                h[p] = __builtin_nontemporal_load((const f16x8 *)((const _Float16 *)(yr + q0) + (c - q0)));
            }
        }
#pragma unroll
        for (int jj = 0; jj < G; ++jj) {
            if (jj >= n) break;
            // the partial sums of a split down GEMM, added in split order,
            // each chunk in its own format
            float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int sp = 0; sp < S; ++sp) {
                const int p = jj * S + sp;
                if (a.yfmt && fmt[p] == kYF16) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) v[e] += (float)h[p][e];
                } else {
                    const float *yr = a.y + sp * a.split_stride + (int64_t)row[jj] * a.H + c;
                    const f32x4 lo = __builtin_nontemporal_load((const f32x4 *)yr), hi = __builtin_nontemporal_load((const f32x4 *)(yr + 4));
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        v[e] += lo[e];
                        v[e + 4] += hi[e];
                    }
                }
            }
            const float wj = a.unit_weights ? 1.0f : w[jj];
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] += wj * v[e];
        }
    }
    const int64_t o = (int64_t)t * a.H + c;
    if (a.out_bf16) {
        if (a.shared) {
            const bf16x8 sh = *(const bf16x8 *)((const __bf16 *)a.shared + o);
            const float sc = a.shared_scale ? a.shared_scale[t] : 1.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] += sc * (float)sh[e];
        }
        bf16x8 r;
#pragma unroll
        for (int e = 0; e < 8; ++e) r[e] = (__bf16)acc[e];
        *(bf16x8 *)((__bf16 *)a.out + o) = r;
    } else {
        float *out = (float *)a.out + o;
        if (a.shared) {
            const float *sh = (const float *)a.shared + o;
            const float sc = a.shared_scale ? a.shared_scale[t] : 1.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] += sc * sh[e];
        }
        *(f32x4 *)out = f32x4{acc[0], acc[1], acc[2], acc[3]};
        *(f32x4 *)(out + 4) = f32x4{acc[4], acc[5], acc[6], acc[7]};
    }
}

}  // namespace

hipError_t launch_combine(const CombineArgs &a, hipStream_t s)
{
    // one thread per 8 features of a token (H is a multiple of 8)
    const int64_t n = (int64_t)a.T * (a.H / 8);
    const int64_t blocks = (n + 255) / 256;
    switch (a.splits) {
    case 1: combine_kernel<1><<<dim3((unsigned)blocks), dim3(256), 0, s>>>(a); break;
    case 2: combine_kernel<2><<<dim3((unsigned)blocks), dim3(256), 0, s>>>(a); break;
    case 3: combine_kernel<3><<<dim3((unsigned)blocks), dim3(256), 0, s>>>(a); break;
    case 4: combine_kernel<4><<<dim3((unsigned)blocks), dim3(256), 0, s>>>(a); break;
    default: return hipErrorInvalidValue;    // the down GEMM splits at most 4 ways
    }
    return hipGetLastError();
}

}  // namespace moe
