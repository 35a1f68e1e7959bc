// Grouped expert GEMMs on gfx950 MFMA: the variant dispatcher and the
// prepare-time kernels (16-bit stage-layout copy, range scan, MXFP4 repack).  The GEMM
// kernels themselves are in gemm_kernels.h, instantiated per tile family in
// gemm_prefill.hip, gemm_prefill_mx.hip, gemm_mid.hip and gemm_decode.hip.
#include "gemm_kernels.h"

namespace moe {
namespace {

// ---- prepare-time copy of a 16-bit stack in the stage layout (Pack16Args).
// Thread i writes 16-byte chunk i of the copy.
__global__ __launch_bounds__(256) void pack16_kernel(Pack16Args a)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t total = (int64_t)a.E * a.nN * a.nks * (kPack16Stage / 16);
    if (i >= total) return;
    const int q = (int)(i % (kPack16Stage / 16));
    const int64_t blk = i / (kPack16Stage / 16);         // (e, ks, nt)
    const int nt = (int)(blk % a.nN);
    const int64_t eks = blk / a.nN;
    const int ks = (int)(eks % a.nks), e = (int)(eks / a.nks);
    const int row = q / 8, c = (q % 8) ^ ((row / 2) % 8);
    const bool up = a.gated && row >= kPack16Rows / 2;
    const int width = a.gated ? kPack16Rows / 2 : kPack16Rows;
    const int f = nt * width + (up ? row - kPack16Rows / 2 : row);
    const int k0 = ks * 64 + c * 8;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (f < a.Nout && k0 < a.K) {
        const int64_t wrow = (int64_t)e * a.w.e_rows + (int64_t)f * a.w.row_mul +
                             (up ? a.w.off_up : a.w.off_gate);
        const uint16_t *src = (const uint16_t *)(up ? a.w.w_up : a.w.w_gate) + wrow * a.K + k0;
        v = *(const u32x4 *)src;
        if (a.to_f16) {
#pragma unroll
            for (int j = 0; j < 4; ++j) v[j] = bf16x2_to_f16x2(v[j]);
        }
    }
    *(u32x4 *)(a.dst + i * 16) = v;
}

// ---- prepare-time range scan of a down-weight stack
__global__ __launch_bounds__(256) void weight_range_kernel(const uint32_t *w, const uint8_t *sc,
                                                           int64_t n_words, int64_t n_scales,
                                                           uint32_t *out)
{
    uint32_t mx = 0, smin = 255, smax = 0;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_words; i += stride) {
        const uint32_t v = w[i];
        mx = max(mx, max(v & 0x7fffu, (v >> 16) & 0x7fffu));
    }
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_scales; i += stride) {
        const uint32_t b = sc[i];
        smin = min(smin, b);
        smax = max(smax, b);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        mx = max(mx, (uint32_t)__shfl_xor((int)mx, off, 64));
        smin = min(smin, (uint32_t)__shfl_xor((int)smin, off, 64));
        smax = max(smax, (uint32_t)__shfl_xor((int)smax, off, 64));
    }
    if ((threadIdx.x & 63) == 0) {
        atomicMax(&out[0], mx);
        atomicMin(&out[1], smin);
        atomicMax(&out[2], smax);
    }
}

// ---- prepare-time repack of an MXFP4 stack (layout: PackArgs).  Thread i
// writes packed code chunk i (16 bytes) and packed scale byte i.
__global__ __launch_bounds__(256) void mx_pack_kernel(PackArgs a)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int rbh = a.Nh / 32;                       // row-blocks per operand
    const int64_t nrb = (int64_t)a.ops * rbh;
    const int64_t total = (int64_t)a.E * nrb * a.nks * 64;
    if (i >= total) return;
    const int kq = a.K / 2, ksc = a.K / 32;          // code / scale bytes per row
    {
        // code chunk: (e, lb, ks, r, p)
        const int p = (int)(i & 1), r = (int)((i >> 1) & 31);
        const int64_t blk = i >> 6;                  // (e, lb, ks)
        const int ks = (int)(blk % a.nks);
        const int64_t elb = blk / a.nks;
        const int lb = (int)(elb % nrb), e = (int)(elb / nrb);
        const int op = lb / rbh, f = (lb % rbh) * 32 + r;
        const int c = p ^ ((r >> 3) & 1);           // logical half stored here
        const int64_t row = (int64_t)e * a.e_rows + (int64_t)f * a.row_mul + a.off[op];
        const int kb = ks * 32 + 16 * c;             // first code byte
        uint8_t v[16];
        const uint8_t *src = a.codes[op] + row * kq + kb;
#pragma unroll
        for (int j = 0; j < 16; ++j) v[j] = kb + j < kq ? src[j] : 0;
        uint8_t *dst = a.pk + i * 16;
#pragma unroll
        for (int j = 0; j < 16; ++j) dst[j] = v[j];
    }
    {
        // scale byte: (e, lb, ks, h, r)
        const int r = (int)(i & 31), h = (int)((i >> 5) & 1);
        const int64_t blk = i >> 6;
        const int ks = (int)(blk % a.nks);
        const int64_t elb = blk / a.nks;
        const int lb = (int)(elb % nrb), e = (int)(elb / nrb);
        const int op = lb / rbh, f = (lb % rbh) * 32 + r;
        const int64_t row = (int64_t)e * a.e_rows + (int64_t)f * a.row_mul + a.off[op];
        const int sbk = ks * 2 + h;
        a.pks[i] = sbk < ksc ? a.scales[op][row * ksc + sbk] : (uint8_t)127;
    }
}

}  // namespace

// The MXFP4 and 16-bit kernels of one variant share their tile shape, which
// the host uses for scheduling and the h formats.
static_assert(PrefillMXTile::BM == PrefillDTile::BM && PrefillMXTile::BN == PrefillDTile::BN, "");
static_assert(DecodeMXTile::BM == DecodeDTile::BM && DecodeMXTile::BN == DecodeDTile::BN, "");
static_assert(MidMXTile::BM == MidDTile::BM && MidMXTile::BN == MidDTile::BN, "");
// Every 16-bit tile streams weight stages of the prepared copy's layout
// (pack16_tile in gemm_kernels.h); the decode tiles assert it beside their
// definitions.
static_assert(pack16_tile<PrefillDTile>() && pack16_tile<PrefillFcTile>() &&
                  pack16_tile<ShortFcTile>() && pack16_tile<DecodeDTile>() &&
                  pack16_tile<MidDTile>(),
              "tile and prepared weight layout agree");
static_assert((PrefillDTile::BN / 2) % PrefillDTile::BK == 0 &&
              (DecodeDTile::BN / 2) % DecodeDTile::BK == 0 &&
              (MidDTile::BN / 2) % MidDTile::BK == 0,
              "a down-GEMM k-step lies inside one h tile");

int gemm_bm(GemmKind kind)
{
    return kind == GemmKind::kPrefill ? PrefillDTile::BM
           : kind == GemmKind::kMid   ? MidDTile::BM
                                      : DecodeDTile::BM;
}

int gemm1_bn(GemmKind kind, bool mxfp4, bool gated)
{
    const int bn = kind == GemmKind::kPrefill ? PrefillDTile::BN
                   : kind == GemmKind::kMid   ? MidDTile::BN
                   : mxfp4                    ? DecodeMXTile::BN
                                              : decode16_bn1();
    return gated ? bn / 2 : bn;
}

int gemm2_bn(GemmKind kind, bool mxfp4)
{
    return kind == GemmKind::kPrefill ? PrefillDTile::BN
           : kind == GemmKind::kMid   ? MidDTile::BN
           : mxfp4                    ? DecodeMXTile::BN
                                      : decode16_bn2();
}

int router_bn()
{
    return DecodeDTile::BN;
}

hipError_t launch_gemm_bf16(GemmKind kind, int epi, bool mxfp4, const GemmArgs &a,
                            int64_t max_m_tiles, hipStream_t s)
{
    if (mxfp4 && epi == kEpiPlain) return hipErrorInvalidValue;   // router weights are 16-bit
    switch (kind) {
    case GemmKind::kPrefill:
        return mxfp4 ? launch_prefill_mx(epi, a, max_m_tiles, s)
                     : launch_prefill16(epi, a, max_m_tiles, s);
    case GemmKind::kMid: return launch_mid(mxfp4, epi, a, max_m_tiles, s);
    default: return launch_decode(mxfp4, epi, a, max_m_tiles, s);
    }
}

hipError_t launch_mx_pack(const PackArgs &a, hipStream_t s)
{
    const int64_t nrb = (int64_t)a.ops * (a.Nh / 32);
    const int64_t chunks = (int64_t)a.E * nrb * a.nks * 64;     // 16-byte code chunks
    const int64_t sbytes = (int64_t)a.E * nrb * a.nks * 64;     // scale bytes
    const int64_t n = chunks > sbytes ? chunks : sbytes;
    const int64_t blocks = (n + 255) / 256;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    mx_pack_kernel<<<dim3((unsigned)blocks), dim3(256), 0, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_pack16(const Pack16Args &a, hipStream_t s)
{
    const int64_t chunks = (int64_t)a.E * a.nN * a.nks * (kPack16Stage / 16);
    const int64_t blocks = (chunks + 255) / 256;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    pack16_kernel<<<dim3((unsigned)blocks), dim3(256), 0, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_weight_range(const void *w, const uint8_t *scales, int64_t n_words,
                               int64_t n_scales, uint32_t *out, hipStream_t s)
{
    weight_range_kernel<<<1024, 256, 0, s>>>((const uint32_t *)w, scales, n_words, n_scales,
                                             out);
    return hipGetLastError();
}

}  // namespace moe
