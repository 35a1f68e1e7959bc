// Internal launch interface between the C-ABI host code (api.cpp) and the
// HIP kernels.  Not installed; the public boundary is include/moe_mi355x.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Upper limits the kernels are written for (checked by the host before launch).
constexpr int kMaxExperts = 1024;   // routing keeps E/64 experts per lane
constexpr int kMaxTopK = 64;        // one lane per kept slot
constexpr int kMaxGroups = 64;      // one lane per group score
constexpr int kPermTokens = 256;    // tokens per permutation block
constexpr int kMaxHTiles = 1024;    // h tiles per row (I <= 1024 * 128)

struct RouteArgs {
    const float *logits;     // [T, E]
    const float *sel_bias;   // [E] or null
    int32_t *ids;            // [T, K]
    float *weights;          // [T, K]
    int T, E, K;
    int scoring;             // 0 softmax, 1 sigmoid
    int renormalize;
    int n_group, topk_group;
    float scale;             // routed scaling factor
    // shared-expert gate (logicaffeine "Moe" `shared_gate`), or sgate null:
    // sgate_out[t] = sigmoid(x[t] . g), x [T, H] and g [H] in x's dtype
    const void *x;
    const void *sgate;
    float *sgate_out;
    int H;
    int x_bf16;
};

struct PermuteArgs {
    const int32_t *ids;      // [T, K]
    int T, E, K;
    int32_t *block_counts;   // [NB, E]   NB = ceil(T / kPermTokens)
    int32_t *block_base;     // [NB, E] rows of expert e in blocks before b
    int32_t *counts;         // [E]
    int32_t *offsets;        // [E + 1]
    int32_t *row_token;      // [T*K]
    int32_t *slot_row;       // [T*K]
    int32_t *tile_cum1;      // [E + 1] cumulative M-tiles of GEMM 1
    int32_t *tile_cum2;      // [E + 1] cumulative M-tiles of GEMM 2
    int32_t *full_cum1;      // [E + 1] cumulative M-tiles of experts with >= bm rows, GEMM 1
    int32_t *full_cum2;      // [E + 1] same for GEMM 2
    int bm1, bm2;            // token-tile heights of the two GEMMs
    const float *weights;    // [T, K] routing weights, read when row_weight is set
    float *row_weight;       // [T*K] weight of each row (weigh-inputs), or null
};

// Weight-operand description of one grouped GEMM.  Feature row c of expert e
// lives at row (e * e_rows + c * row_mul + off) of the stack whose base is
// w_gate (gate / only operand) or w_up (up operand of the gated GEMM).
struct WeightRows {
    const void *w_gate;          // element base (bf16 / f32) or MXFP4 codes
    const void *w_up;
    const uint8_t *s_gate;       // MXFP4 scales (same row mapping), else null
    const uint8_t *s_up;
    int64_t e_rows;              // rows per expert slab
    int row_mul;                 // 2 for interleaved gate||up, else 1
    int off_gate, off_up;        // row offsets of the gate / up operands
    const void *b_gate;          // bias (x dtype), indexed like the rows; or null
    const void *b_up;
};

// Storage format of one h tile (GEMM-1 output tile, read by the down GEMM).
enum : uint8_t { kHF16 = 0, kHBF16 = 1 };

// Storage format of one chunk of y: kYWidth consecutive features of one row.
// An fp16 chunk (every value within fp16's range) occupies the first half of
// the chunk's f32 space; the combine reads each chunk in its own format.
enum : uint8_t { kYF32 = 0, kYF16 = 1 };
constexpr int kYWidth = 64;

// Epilogue (and operand) mode of a grouped GEMM launch.
//  kEpiDown   down GEMM: A = h (16-bit, per-tile formats), y = acc + bias, f32 or
//             fp16 per 64-feature chunk (yfmt)
//  kEpiGated  gate||up GEMM: gate/up row pairs, gated activation, 16-bit h
//  kEpiAct    fc1 GEMM of a non-gated expert: activation of each row, 16-bit h
//  kEpiPlain  A = x, y = acc + bias, f32 (the router GEMM, one group)
enum EpiMode : int { kEpiDown = 0, kEpiGated = 1, kEpiAct = 2, kEpiPlain = 3 };

struct GemmArgs {
    const void *a;               // activations: x [T, Kd] or h [T*K, Kd]
    const int32_t *row_token;    // if set, A row r reads a[row_token[r]]
    WeightRows w;
    const int32_t *counts;       // [E]
    const int32_t *offsets;      // [E + 1]
    const int32_t *tile_cum;     // [E + 1] cumulative M-tiles at this BM
    const int32_t *full_cum;     // [E + 1] cumulative M-tiles of experts with >= BM rows
    int E;
    int Kd;                      // reduction length
    int Nout;                    // output features: I (gated) or H (down)
    int nN;                      // feature tiles
    int ksplit;                  // reduction splits (>= 1): split s reduces k-steps
                                 // [s*nk/ksplit, (s+1)*nk/ksplit) into out + s*split_stride
    int64_t split_stride;        // elements between the splits' outputs (f32 space)
    void *out;                   // h 16-bit [T*K, I], or y [T*K, H] in f32 space (see yfmt)
    int act;                     // moe_activation code (0..5)
    int gelu_mode;               // 0 erf, 1 tanh
    float alpha, beta, limit;
    const float *row_w;          // weigh-inputs: row r's weight scales its fc1
                                 // output before the bias; null otherwise
    // h storage formats, one byte per (GEMM-1 M-tile, GEMM-1 feature tile):
    // written by the gated GEMM, read per reduction step by the down GEMM.
    uint8_t *hfmt;
    // The prepared copy of the 16-bit weight stack in the stage layout the GEMM
    // loads (see Pack16Args), or null: the kernel then reads w_gate / w_up
    // row by row.  Tile (e, nt)'s k-step ks is one contiguous kPack16Stage-byte
    // block at wpk + ((e * nks + ks) * nN + nt) * kPack16Stage.
    const uint8_t *wpk;
    int wpk_f16;                 // the prepared copy holds fp16 (the down GEMM's
                                 // copy when the range scan allows), else bf16
    // down GEMM, or null (y in f32): per-chunk storage format of y (of each
    // split's partial sums), one byte per (split s, row r, kYWidth-feature
    // chunk q) at yfmt[s * yfmt_split_stride + r * yfmt_stride + q]
    uint8_t *yfmt;
    int64_t yfmt_stride, yfmt_split_stride;
    int h_tiles;                 // GEMM-1 feature tiles (row stride of hfmt)
    int h_width;                 // h columns per GEMM-1 feature tile
    int f16_ok;                  // the down weights lie in fp16's range
    // MXFP4 weights, packed once at prepare (see PackArgs): codes and scales
    // of logical row-block lb, k-step ks at pk + (lb-major) KiB blocks
    const uint8_t *pk;           // [E][nrb][nks][32 rows][32 bytes]
    const uint8_t *pks;          // [E][nrb][nks][2 scale blocks][32 rows]
    int nks;                     // k-steps of 64 (the reduction length, rounded
                                 // up): MXFP4 and prepared 16-bit copies
    int nrb_half;                // row-blocks of one operand (Nout / 32)
    int a_off32;                 // every byte of the A operand lies within 4 GiB
                                 // of a (the 4-wave 16-bit tile addresses its
                                 // token rows as a + 32-bit lane offsets)
};

// Prepare-time repack of an MXFP4 weight stack into the layout the GEMM
// streams.  Logical rows: operand 0 (gate, or the only operand) then operand
// 1 (up), Nh rows each; logical row f of operand o lives at stack row
// e * e_rows + f * row_mul + off[o].  For row-block lb (32 rows) and k-step ks
// (64 elements) the packed codes are one KiB: row r's 32 code bytes at
// r * 32, its two 16-byte halves swapped when bit 3 of r is set (the LDS
// bank swizzle, applied here so the GEMM copies whole KiB blocks); the packed
// scales are 64 bytes: [scale block 0..1][row 0..31].  Past the reduction
// length codes are 0 (+0.0) and scale bytes 127 (1.0).
struct PackArgs {
    const uint8_t *codes[2];     // [.., K/2] per stack row
    const uint8_t *scales[2];    // [.., K/32] per stack row
    int64_t e_rows;
    int row_mul;
    int off[2];
    int ops;                     // 2 (gate, up) or 1
    int Nh;                      // rows per operand
    int K;                       // reduction length (multiple of 32)
    int nks;                     // ceil(K / 64)
    int E;
    uint8_t *pk;
    uint8_t *pks;
};
hipError_t launch_mx_pack(const PackArgs &a, hipStream_t s);
// bytes of the packed codes / scales of an MXFP4 stack
inline int64_t mx_pack_bytes(int ops, int64_t Nh, int64_t K, int64_t E)
{
    return E * (ops * Nh / 32) * ((K + 63) / 64) * 1024;
}
inline int64_t mx_pack_scale_bytes(int ops, int64_t Nh, int64_t K, int64_t E)
{
    return E * (ops * Nh / 32) * ((K + 63) / 64) * 64;
}

// Prepare-time copy of a 16-bit weight stack in the layout the grouped GEMMs
// stream: per expert e, per 64-wide k-step ks, per tile of kPack16Rows weight
// rows (nt), one block of kPack16Stage bytes that is the image of an LDS
// weight stage -- 16-byte chunk q of the block holds row q / 8 of the tile,
// columns 8 c .. 8 c + 7 of the k-step with c = (q % 8) ^ ((q / 8 / 2) % 8)
// (the bank swizzle the GEMMs read with, applied once here).  Tile rows of
// the gated GEMM are the tile's kPack16Rows / 2 gate features followed by
// the same up features; other GEMMs take kPack16Rows consecutive features.
// Rows past Nout and columns past K are zero.  A k-step of a tile is then
// one contiguous read (a row-by-row read of 128 bytes per row streams
// weights from HBM at 4.5 TB/s on MI355X, a contiguous one at 6.1), and the
// tiles of one expert, which run side by side, read adjacent blocks at each
// k-step: their reads sweep one window of memory together, as a grid-stride
// read does (7.1 TB/s), instead of each streaming its own slab (5.4-6.3).
constexpr int kPack16Rows = 256;
constexpr int kPack16Stage = kPack16Rows * 128;
struct Pack16Args {
    WeightRows w;                // source rows (w_gate / w_up, row mapping)
    int gated;                   // tile rows are gate / up pairs of features
    int Nout;                    // features (gate/up pairs when gated)
    int K;                       // reduction length (multiple of 8)
    int E, nN, nks;              // experts, tiles per expert, k-steps
    int to_f16;                  // convert bf16 to fp16 (round to nearest even)
    uint8_t *dst;
};
hipError_t launch_pack16(const Pack16Args &a, hipStream_t s);
inline int64_t pack16_bytes(int64_t E, int64_t nN, int64_t K)
{
    return E * nN * ((K + 63) / 64) * kPack16Stage;
}

// Range of a down-weight stack, for the choice of the fp16 down GEMM:
// out[0] = max over elements of the bf16 magnitude bits (0x7f80 = inf),
// out[1] = min MXFP4 scale byte, out[2] = max MXFP4 scale byte.
hipError_t launch_weight_range(const void *w, const uint8_t *scales, int64_t n_words,
                               int64_t n_scales, uint32_t *out, hipStream_t s);

struct CombineArgs {
    const float *y;              // [T*K, H] (row order of the permutation)
    const float *weights;        // [T, K]
    const int32_t *slot_row;     // [T, K]
    const void *shared;          // [T, H] x dtype or null
    const float *shared_scale;   // [T] scale of token t's shared output, or null (1)
    void *out;                   // [T, H] x dtype
    int T, H, K;
    int out_bf16;                // 1: bf16 x/out, 0: f32
    int unit_weights;            // weigh-inputs: every kept output weighs 1
    int splits;                  // y holds this many partial sums (split reduction),
    int64_t split_stride;        // split_stride elements apart, summed in order
    const uint8_t *yfmt;         // y chunk formats (GemmArgs yfmt), or null
    int64_t yfmt_stride, yfmt_split_stride;
};

// Dense f32 grouped GEMM (the fp32 layer): same contract as GemmArgs with
// f32 operands.
hipError_t launch_route(const RouteArgs &a, hipStream_t s);
hipError_t launch_permute(const PermuteArgs &a, hipStream_t s);
hipError_t launch_combine(const CombineArgs &a, hipStream_t s);

// Grouped-GEMM variants, by epilogue mode (EpiMode).  With mxfp4 the weights
// are read from the packed copy (GemmArgs pk / pks).
enum class GemmKind { kPrefill = 0, kDecode = 1, kMid = 2 };
int gemm_bm(GemmKind kind);          // token-tile height of a variant
// output features per tile: GEMM 1 (gate||up or fc1; gate/up pairs when
// gated), GEMM 2 (down), and the router GEMM
int gemm1_bn(GemmKind kind, bool mxfp4, bool gated);
int gemm2_bn(GemmKind kind, bool mxfp4);
int router_bn();
// the decode variant's 16-bit tiles (defined beside them, in gemm_decode.hip)
int decode16_bn1();                  // weight rows of a GEMM-1 tile
int decode16_bn2();
hipError_t launch_gemm_bf16(GemmKind kind, int epi, bool mxfp4,
                            const GemmArgs &a, int64_t max_m_tiles, hipStream_t s);
int gemm_f32_bm();
int gemm_f32_bn(bool gated);
hipError_t launch_gemm_f32(int epi, const GemmArgs &a, int64_t max_m_tiles,
                           hipStream_t s);

// One group of T rows (the router GEMM): counts = {T}, offsets = {0, T},
// tile_cum = {0, ceil(T / bm)}, full_cum = {0, T >= bm ? ceil(T / bm) : 0}.
hipError_t launch_single_group(int32_t *counts, int32_t *offsets, int32_t *tile_cum,
                               int32_t *full_cum, int T, int bm, hipStream_t s);
// Wr [H, E] -> its transpose [E, H] (elem_bytes 2 or 4).
hipError_t launch_transpose(const void *src, void *dst, int rows, int cols, int elem_bytes,
                            hipStream_t s);

}  // namespace moe
