// Router-weighted combine (clika "MoE": the expert outputs combine under the
// router weights; "ClikaRT::nn::QMoEWoQ::forward": an optional shared-expert
// output folds into the same epilogue).  With weigh-inputs routing
// ("MoeSpec" `weigh_inputs`) the weights were applied to the experts' inputs
// and every kept output joins the sum with weight one.
//
// out[t, :] = sum_{j=0..K-1} w[t, j] * y[slot_row[t, j], :]  (+ shared[t, :])
// accumulated in f32 in slot order j = 0, 1, ..., rounded once to the output
// dtype (round to nearest even for bf16).  No atomics: each output element
// is produced by one thread, so results are bitwise reproducible.
#include "moe_kernels.h"

namespace moe {
namespace {

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a)
{
    const int H4 = a.H / 4;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (int64_t)a.T * H4) return;
    const int t = (int)(idx / H4), c = (int)(idx % H4) * 4;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < a.K; ++j) {
        const float w = a.unit_weights ? 1.0f : a.weights[(int64_t)t * a.K + j];
        const int row = a.slot_row[(int64_t)t * a.K + j];
        // the partial sums of a split down GEMM, added in split order
        f32x4 v = *(const f32x4 *)(a.y + (int64_t)row * a.H + c);
        for (int s = 1; s < a.splits; ++s)
            v += *(const f32x4 *)(a.y + s * a.split_stride + (int64_t)row * a.H + c);
        acc += w * v;
    }
    const int64_t o = (int64_t)t * a.H + c;
    if (a.out_bf16) {
        if (a.shared) {
            const bf16x4 s = *(const bf16x4 *)((const __bf16 *)a.shared + o);
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[j] += (float)s[j];
        }
        bf16x4 r;
#pragma unroll
        for (int j = 0; j < 4; ++j) r[j] = (__bf16)acc[j];
        *(bf16x4 *)((__bf16 *)a.out + o) = r;
    } else {
        if (a.shared) acc += *(const f32x4 *)((const float *)a.shared + o);
        *(f32x4 *)((float *)a.out + o) = acc;
    }
}

}  // namespace

hipError_t launch_combine(const CombineArgs &a, hipStream_t s)
{
    const int64_t n = (int64_t)a.T * (a.H / 4);
    const int64_t blocks = (n + 255) / 256;
    combine_kernel<<<dim3((unsigned)blocks), dim3(256), 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace moe
