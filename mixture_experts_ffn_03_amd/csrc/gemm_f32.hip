// Grouped expert GEMMs for f32 layers (x, weights, h and y all f32), on the
// vector ALUs with LDS-staged tiles.  Same scheduling and epilogue modes as
// the 16-bit MFMA kernels: gated computes BNF gate and BNF up features of BM
// tokens and applies the gated activation; act applies a non-gated
// activation to BNF fc1 features; down and plain add the bias.  Used for the
// f32 layer, whose tolerance (1e-4 of the output RMS) rules out bf16
// operands.  With weigh-inputs routing (row_w) the fc1 output of a row is
// scaled by its routing weight before the bias, which equals running the
// expert on the scaled input.
#include "gemm_common.h"

namespace moe {
namespace {

constexpr int BM = 32;      // tokens per tile
constexpr int BNF = 32;     // output features per tile
constexpr int BK = 32;
constexpr int NT = 256;     // thread (tl = tid % 32, features 4*(tid/32) .. +3)

template <int EPI>
__global__ __launch_bounds__(NT) void gemm_f32_kernel(GemmArgs g)
{
    constexpr bool GATED = EPI == kEpiGated;
    constexpr int NB = GATED ? 2 * BNF : BNF;   // weight rows per tile
    __shared__ float As[BM][BK + 1];
    __shared__ float Bs[NB][BK + 1];
    __shared__ int s_cum[4 * (kMaxExperts + 1)];
    TileWork tw;
    if (!find_tile(g, s_cum, BNF, &tw)) return;
    const int tid = threadIdx.x, Kd = g.Kd;
    const float *A = (const float *)g.a;
    const int64_t eb = (int64_t)tw.e * g.w.e_rows;

    float ag[4] = {0, 0, 0, 0}, au[4] = {0, 0, 0, 0};
    const int tl = tid % 32, fg = tid / 32;
    for (int k0 = 0; k0 < Kd; k0 += BK) {
        for (int i = tid; i < BM * BK; i += NT) {
            const int r = i / BK, k = i % BK;
            const int row = tw.row0 + min(r, tw.nrows - 1);
            const int src = g.row_token ? g.row_token[row] : row;
            As[r][k] = (k0 + k < Kd) ? A[(int64_t)src * Kd + k0 + k] : 0.0f;
        }
        for (int i = tid; i < NB * BK; i += NT) {
            const int r = i / BK, k = i % BK;
            const bool up = GATED && r >= BNF;
            const int c = min(tw.n0 + (up ? r - BNF : r), g.Nout - 1);
            const int64_t row = eb + (int64_t)c * g.w.row_mul + (up ? g.w.off_up : g.w.off_gate);
            const float *W = (const float *)(up ? g.w.w_up : g.w.w_gate);
            Bs[r][k] = (k0 + k < Kd) ? W[row * Kd + k0 + k] : 0.0f;
        }
        __syncthreads();
        for (int k = 0; k < BK; ++k) {
            const float a = As[tl][k];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                ag[j] += Bs[fg * 4 + j][k] * a;
                if (GATED) au[j] += Bs[BNF + fg * 4 + j][k] * a;
            }
        }
        __syncthreads();
    }
    if (tl >= tw.nrows) return;
    float *out = (float *)g.out + (int64_t)(tw.row0 + tl) * g.Nout;
    const float rs = ((EPI == kEpiGated || EPI == kEpiAct) && g.row_w) ? g.row_w[tw.row0 + tl]
                                                                        : 1.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int c = tw.n0 + fg * 4 + j;
        if (c >= g.Nout) continue;
        float gv = ag[j] * rs;
        if (g.w.b_gate)
            gv += ((const float *)g.w.b_gate)[eb + (int64_t)c * g.w.row_mul + g.w.off_gate];
        if (GATED) {
            float uv = au[j] * rs;
            if (g.w.b_up)
                uv += ((const float *)g.w.b_up)[eb + (int64_t)c * g.w.row_mul + g.w.off_up];
            out[c] = gated_act(g.act, gv, uv, g.alpha, g.beta, g.limit);
        } else if (EPI == kEpiAct) {
            out[c] = single_act(g.act, g.gelu_mode, gv);
        } else {
            out[c] = gv;
        }
    }
}

}  // namespace

int gemm_f32_bm() { return BM; }
int gemm_f32_bn(bool) { return BNF; }

hipError_t launch_gemm_f32(int epi, const GemmArgs &a, int64_t max_m_tiles, hipStream_t s)
{
    const int64_t grid = max_m_tiles * a.nN * a.ksplit + 8;
    const dim3 gd((unsigned)grid), bd(NT);
    switch (epi) {
    case kEpiGated: gemm_f32_kernel<kEpiGated><<<gd, bd, 0, s>>>(a); break;
    case kEpiAct: gemm_f32_kernel<kEpiAct><<<gd, bd, 0, s>>>(a); break;
    default: gemm_f32_kernel<kEpiDown><<<gd, bd, 0, s>>>(a); break;   // down and plain
    }
    return hipGetLastError();
}

}  // namespace moe
