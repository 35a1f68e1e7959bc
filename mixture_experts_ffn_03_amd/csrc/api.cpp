// C-ABI host runtime of the MI355X MoE FFN forward: argument validation,
// workspace carving, kernel selection and launches on the caller's stream.
// Lifecycle and error semantics follow the clika "ClikaRT::nn::QMoEWoQ" page
// (make, set_weights, initialize, forward, to) and the Python "MoE" page
// (constructor, set_weights slot names, forward signature).
#include "../../include/moe_mi355x.h"
#include "api_internal.h"
#include "moe_kernels.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>

using namespace moe;

struct moe_layer {
    int64_t E, H, I, K;
    moe_dtype wdtype;
    int has_gu_bias, has_d_bias;
    moe_options opts;
    moe_weights w;
    bool bound;
    // Prepared state (QMoEWoQ "pack once, thread-safe"): whether the down
    // weights lie in fp16's range, which enables the fp16 down GEMM, and
    // for MXFP4 weights the library-owned packed copy the GEMMs stream
    // (allocated at the first prepare, sized by the geometry alone, refilled
    // by every later prepare, freed by moe_destroy).
    mutable std::mutex mu;
    mutable bool prepared;
    mutable int down_f16_ok;
    mutable uint8_t *mx_pack = nullptr;
    mutable int64_t mx_off[4] = {0, 0, 0, 0};   // codes 1, scales 1, codes 2, scales 2
    // the bound router transposed to [E, H] (rows K-contiguous, like the
    // expert stacks) for the router GEMM; made at prepare, freed by destroy
    mutable void *wr_t = nullptr;
    // options.pack_weights: the 16-bit expert stacks in the stage layout the
    // GEMMs stream (Pack16Args): gate||up (or fc1) at pk16 + pk16_off[0], down
    // at pk16 + pk16_off[1] (in fp16 when pk16_down_f16).  Allocated at the
    // first prepare that needs it, refilled by later ones; pk16_ready says
    // whether the current binding's copy is in it.
    mutable uint8_t *pk16 = nullptr;
    mutable int64_t pk16_off[2] = {0, 0};
    mutable bool pk16_ready = false;
    mutable bool pk16_down_f16 = false;
};

namespace {

thread_local std::string g_err;

moe_status fail(moe_status s, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return s;
}

bool present(const moe_tensor &t)
{
    return t.data != nullptr && t.ndim > 0;
}

const char *dtype_name(int d)
{
    switch (d) {
    case MOE_DTYPE_F32: return "f32";
    case MOE_DTYPE_BF16: return "bf16";
    case MOE_DTYPE_MXFP4: return "mxfp4";
    case MOE_DTYPE_I32: return "i32";
    default: return "?";
    }
}

// Check dtype and exact shape of a bound tensor.
moe_status check_tensor(const char *name, const moe_tensor &t, int dtype,
                        std::initializer_list<int64_t> shape)
{
    if (t.dtype != dtype)
        return fail(MOE_ERR_SHAPE_MISMATCH, "%s: dtype %s, expected %s", name,
                    dtype_name(t.dtype), dtype_name(dtype));
    if (t.ndim != (int)shape.size())
        return fail(MOE_ERR_SHAPE_MISMATCH, "%s: %d dims, expected %d", name, t.ndim,
                    (int)shape.size());
    int i = 0;
    for (int64_t d : shape) {
        if (t.shape[i] != d)
            return fail(MOE_ERR_SHAPE_MISMATCH, "%s: dim %d is %lld, expected %lld", name, i,
                        (long long)t.shape[i], (long long)d);
        ++i;
    }
    if (dtype == MOE_DTYPE_MXFP4 && t.scales == nullptr)
        return fail(MOE_ERR_SHAPE_MISMATCH, "%s: MXFP4 stack without scales", name);
    return MOE_OK;
}

int act_dtype(const moe_layer *l)
{
    return l->wdtype == MOE_DTYPE_F32 ? MOE_DTYPE_F32 : MOE_DTYPE_BF16;
}

// Gated activations read a gate and an up projection (ONNX MoE fusion_size
// 2 when fused); the others one fc1 projection [E, I, H].
bool gated(const moe_layer *l)
{
    return l->opts.activation == MOE_ACT_SILU_GATED ||
           l->opts.activation == MOE_ACT_SWIGLU_CLAMPED;
}

bool fused(const moe_layer *l)
{
    return gated(l) && l->opts.swiglu_fusion != MOE_FUSION_NONE;
}

// gate and up in two stacks (gated, swiglu_fusion NONE)
bool two_stacks(const moe_layer *l)
{
    return gated(l) && l->opts.swiglu_fusion == MOE_FUSION_NONE;
}

bool has_router(const moe_layer *l)
{
    return present(l->w.router_weight);
}

moe_status check_bound(const moe_layer *l)
{
    if (!l->bound) return fail(MOE_ERR_UNBOUND, "weights not bound (call moe_set_weights)");
    if (!present(l->w.gate_up_experts) || !present(l->w.down_experts))
        return fail(MOE_ERR_UNBOUND, "gate_up_experts / down_experts slot unbound");
    if (two_stacks(l) && !present(l->w.gate_experts))
        return fail(MOE_ERR_UNBOUND, "gate_experts slot unbound (swiglu_fusion = NONE)");
    if (l->has_gu_bias) {
        if (!present(l->w.gate_up_bias))
            return fail(MOE_ERR_UNBOUND, "declared gate_up_bias slot unbound");
        if (two_stacks(l) && !present(l->w.gate_bias))
            return fail(MOE_ERR_UNBOUND, "declared gate_bias slot unbound");
    }
    if (l->has_d_bias && !present(l->w.down_bias))
        return fail(MOE_ERR_UNBOUND, "declared down_bias slot unbound");
    return MOE_OK;
}

// Row mapping of the GEMM-1 weight operands (gate||up, or the fc1 stack of
// a non-gated activation) and their biases.
WeightRows gemm1_rows(const moe_layer *l)
{
    WeightRows w1{};
    if (!gated(l)) {
        // one fc1 stack [E, I, H] and its bias [E, I]
        w1.w_gate = w1.w_up = l->w.gate_up_experts.data;
        w1.s_gate = w1.s_up = l->w.gate_up_experts.scales;
        w1.e_rows = l->I;
        w1.row_mul = 1;
        w1.off_gate = w1.off_up = 0;
        if (present(l->w.gate_up_bias)) w1.b_gate = l->w.gate_up_bias.data;
    } else if (fused(l)) {
        w1.w_gate = w1.w_up = l->w.gate_up_experts.data;
        w1.s_gate = w1.s_up = l->w.gate_up_experts.scales;
        w1.e_rows = 2 * l->I;
        if (l->opts.swiglu_fusion == MOE_FUSION_INTERLEAVED) {
            w1.row_mul = 2;
            w1.off_gate = 0;
            w1.off_up = 1;
        } else {
            w1.row_mul = 1;
            w1.off_gate = 0;
            w1.off_up = (int)l->I;
        }
        if (present(l->w.gate_up_bias)) w1.b_gate = w1.b_up = l->w.gate_up_bias.data;
    } else {
        w1.w_gate = l->w.gate_experts.data;
        w1.s_gate = l->w.gate_experts.scales;
        w1.w_up = l->w.gate_up_experts.data;
        w1.s_up = l->w.gate_up_experts.scales;
        w1.e_rows = l->I;
        w1.row_mul = 1;
        w1.off_gate = w1.off_up = 0;
        if (present(l->w.gate_bias)) w1.b_gate = l->w.gate_bias.data;
        if (present(l->w.gate_up_bias)) w1.b_up = l->w.gate_up_bias.data;
    }
    return w1;
}

WeightRows down_rows(const moe_layer *l)
{
    WeightRows w2{};
    w2.w_gate = w2.w_up = l->w.down_experts.data;
    w2.s_gate = w2.s_up = l->w.down_experts.scales;
    w2.e_rows = l->H;
    w2.row_mul = 1;
    if (present(l->w.down_bias)) w2.b_gate = l->w.down_bias.data;
    return w2;
}

// Feature tiles of the two 16-bit GEMMs (every 16-bit tile family is
// kPack16Rows weight rows wide: gate/up pairs of half that many features).
int64_t gemm1_tiles(const moe_layer *l)
{
    const int64_t w = gated(l) ? kPack16Rows / 2 : kPack16Rows;
    return (l->I + w - 1) / w;
}

int64_t gemm2_tiles(const moe_layer *l)
{
    return (l->H + kPack16Rows - 1) / kPack16Rows;
}

size_t align256(size_t v)
{
    return (v + 255) & ~(size_t)255;
}

// Workspace carving.  Every region starts on a 256-byte boundary.
struct Workspace {
    size_t ids, weights, block_counts, block_base, counts, offsets, tile_cum1, tile_cum2,
        full_cum1, full_cum2,
        row_token, slot_row, row_weight, logits, sgate, router_grp, hfmt, h, y, yfmt, total;
};

int64_t max_m_tiles_of(const moe_layer *l, int64_t T, int bm)
{
    const int64_t TK = T * l->K;
    return (TK + bm - 1) / bm + (l->E < TK ? l->E : TK);
}


// Kernel variant: f32 layers use the f32 kernels; otherwise by the average
// rows per expert: small-M (decode, 32-row) tiles below 96, mid (128-row)
// tiles for MXFP4 weights below 512, else the large-M (256-row) tiles.
enum class Path { kF32, kPrefill, kDecode, kMid };

Path choose_path(const moe_layer *l, int64_t T)
{
    if (l->wdtype == MOE_DTYPE_F32) return Path::kF32;
    if (l->opts.gemm_variant == 1) return Path::kPrefill;
    if (l->opts.gemm_variant == 2) return Path::kDecode;
    if (l->opts.gemm_variant == 3) return Path::kMid;
    const double rows_per_expert = (double)(T * l->K) / (double)l->E;
    if (rows_per_expert < 96.0) return Path::kDecode;
    // MXFP4 weight stages are small, so 128-row tiles cost little in loads
    // and avoid a mostly empty second tile per expert
    if (l->wdtype == MOE_DTYPE_MXFP4 && rows_per_expert < 512.0) return Path::kMid;
    return Path::kPrefill;
}

GemmKind kind_of(Path p)
{
    return p == Path::kPrefill ? GemmKind::kPrefill
           : p == Path::kMid   ? GemmKind::kMid
                               : GemmKind::kDecode;
}

int path_bm(Path p)
{
    if (p == Path::kF32) return gemm_f32_bm();
    return gemm_bm(kind_of(p));
}

// Output features per tile of GEMM 1 (gate/up pairs when gated) and of the
// down GEMM on a path.
int path_bn1(const moe_layer *l, Path p)
{
    if (p == Path::kF32) return gemm_f32_bn(gated(l));
    return gemm1_bn(kind_of(p), l->wdtype == MOE_DTYPE_MXFP4, gated(l));
}

int path_bn2(const moe_layer *l, Path p)
{
    if (p == Path::kF32) return gemm_f32_bn(false);
    return gemm2_bn(kind_of(p), l->wdtype == MOE_DTYPE_MXFP4);
}

// Reduction splits of the down GEMM: its tile count (token tiles x feature
// tiles) can be a few rounds of the device's CUs, leaving the last round
// mostly idle; splitting its long reduction (I) multiplies the tiles.  The
// partial sums go to separate f32 buffers that the combine adds in order,
// so the result stays deterministic.  Worst-case tile count, so the choice
// depends on (T, geometry) only and the workspace can be sized from it.
int down_splits(const moe_layer *l, int64_t T, Path path)
{
    if (path == Path::kF32) return 1;
    static int cus = 0;
    if (!cus) {
        int dev = 0, n = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
            n > 0)
            cus = n;
        else {
            (void)hipGetLastError();
            cus = 256;
        }
    }
    const int bm = path_bm(path), bn = path_bn2(l, path);
    const int64_t tiles = max_m_tiles_of(l, T, bm) * ((l->H + bn - 1) / bn);
    if (tiles == 0 || tiles >= 3 * (int64_t)cus) return 1;
    const int64_t ksteps = (l->I + 63) / 64;
    int s = (int)((4 * (int64_t)cus + tiles - 1) / tiles);
    if (s > 4) s = 4;
    while (s > 1 && ksteps / s < 16) --s;      // at least 16 k-steps per split
    return s;
}

Workspace layout(const moe_layer *l, int64_t T)
{
    Workspace w{};
    const int64_t TK = T * l->K;
    const int64_t NB = (T + kPermTokens - 1) / kPermTokens;
    const size_t hbytes = l->wdtype == MOE_DTYPE_F32 ? 4 : 2;
    size_t o = 0;
    auto take = [&](size_t bytes) {
        size_t at = o;
        o = align256(o + bytes);
        return at;
    };
    w.ids = take(TK * 4);
    w.weights = take(TK * 4);
    w.block_counts = take(NB * l->E * 4);
    w.block_base = take(NB * l->E * 4);
    w.counts = take(l->E * 4);
    w.offsets = take((l->E + 1) * 4);
    w.tile_cum1 = take((l->E + 1) * 4);
    w.tile_cum2 = take((l->E + 1) * 4);
    w.full_cum1 = take((l->E + 1) * 4);
    w.full_cum2 = take((l->E + 1) * 4);
    w.row_token = take(TK * 4);
    w.slot_row = take(TK * 4);
    w.row_weight = take(TK * 4);          // weigh-inputs: routing weight per row
    w.logits = take(T * l->E * 4);        // router logits when the layer's router runs
    w.sgate = take(T * 4);                // shared-expert gate per token
    w.router_grp = take(8 * 4);   // router GEMM: counts, offsets, tile_cum, full_cum
    // one h-format byte per (GEMM-1 M-tile, GEMM-1 feature tile), worst case
    // over the kernel variants
    size_t nfmt = 0;
    for (GemmKind k : {GemmKind::kPrefill, GemmKind::kDecode, GemmKind::kMid}) {
        const int bn = gemm1_bn(k, l->wdtype == MOE_DTYPE_MXFP4, gated(l));
        const int64_t ntile = (l->I + bn - 1) / bn;
        const size_t n = (size_t)(max_m_tiles_of(l, T, gemm_bm(k)) * ntile);
        if (n > nfmt) nfmt = n;
    }
    w.hfmt = take(nfmt);
    w.h = take(TK * l->I * hbytes);
    // y: one [T*K, H] f32 buffer per split of the down GEMM
    w.y = take(TK * l->H * 4 * down_splits(l, T, choose_path(l, T)));
    // one y-format byte per (split, row, feature chunk) when y may be stored in fp16
    w.yfmt = take(TK * ((l->H + kYWidth - 1) / kYWidth) * down_splits(l, T, choose_path(l, T)));
    w.total = o;
    return w;
}

moe_status hip_check(hipError_t e, const char *what)
{
    if (e != hipSuccess)
        return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return MOE_OK;
}

int64_t tokens_of(const moe_tensor &t, int64_t last, bool *okp)
{
    *okp = false;
    if (t.ndim < 2 || t.ndim > 3 || t.shape[t.ndim - 1] != last) return 0;
    int64_t T = 1;
    for (int i = 0; i < t.ndim - 1; ++i) {
        if (t.shape[i] < 0) return 0;
        T *= t.shape[i];
    }
    *okp = true;
    return T;
}

// Routing + permutation into the workspace.
moe_status run_route(const moe_layer *l, const float *logits, int64_t T, char *ws,
                     const Workspace &W, Path path, hipStream_t s, void *const *events,
                     const moe_tensor *x_gate = nullptr)
{
    RouteArgs ra{};
    if (x_gate) {
        // the shared-expert gate of every token, from x and g
        ra.x = x_gate->data;
        ra.x_bf16 = x_gate->dtype == MOE_DTYPE_BF16;
        ra.sgate = l->w.shared_gate.data;
        ra.sgate_out = (float *)(ws + W.sgate);
        ra.H = (int)l->H;
    }
    ra.logits = logits;
    ra.sel_bias = present(l->w.e_score_correction_bias)
                      ? (const float *)l->w.e_score_correction_bias.data
                      : nullptr;
    ra.ids = (int32_t *)(ws + W.ids);
    ra.weights = (float *)(ws + W.weights);
    ra.T = (int)T;
    ra.E = (int)l->E;
    ra.K = (int)l->K;
    ra.scoring = l->opts.scoring;
    ra.renormalize = l->opts.renormalize;
    ra.n_group = l->opts.n_group;
    ra.topk_group = l->opts.topk_group;
    ra.scale = l->opts.routed_scaling_factor;
    moe_status st = hip_check(launch_route(ra, s), "route launch");
    if (st) return st;
    if (events && events[1] &&
        (st = hip_check(hipEventRecord((hipEvent_t)events[1], s), "event record")))
        return st;

    PermuteArgs pa{};
    pa.ids = ra.ids;
    pa.T = (int)T;
    pa.E = (int)l->E;
    pa.K = (int)l->K;
    pa.block_counts = (int32_t *)(ws + W.block_counts);
    pa.block_base = (int32_t *)(ws + W.block_base);
    pa.counts = (int32_t *)(ws + W.counts);
    pa.offsets = (int32_t *)(ws + W.offsets);
    pa.row_token = (int32_t *)(ws + W.row_token);
    pa.slot_row = (int32_t *)(ws + W.slot_row);
    pa.tile_cum1 = (int32_t *)(ws + W.tile_cum1);
    pa.tile_cum2 = (int32_t *)(ws + W.tile_cum2);
    pa.full_cum1 = (int32_t *)(ws + W.full_cum1);
    pa.full_cum2 = (int32_t *)(ws + W.full_cum2);
    pa.bm1 = path_bm(path);
    pa.bm2 = path_bm(path);
    pa.weights = ra.weights;
    pa.row_weight = l->opts.weigh_inputs ? (float *)(ws + W.row_weight) : nullptr;
    if ((st = hip_check(launch_permute(pa, s), "permute launch"))) return st;
    if (events && events[2] &&
        (st = hip_check(hipEventRecord((hipEvent_t)events[2], s), "event record")))
        return st;
    return MOE_OK;
}

// Router logits [T, E] f32 = x . Wr + Br ("MoeSpec" wr, router_bias): the
// grouped GEMM as one group of T rows against the transposed router.
moe_status run_router(const moe_layer *l, const void *x, int64_t T, float *logits, char *ws,
                      const Workspace &W, Path path, hipStream_t s)
{
    GemmArgs g{};
    int32_t *grp = (int32_t *)(ws + W.router_grp);
    g.a = x;
    g.row_token = nullptr;
    g.counts = grp;
    g.offsets = grp + 1;
    g.tile_cum = grp + 3;
    g.full_cum = grp + 5;
    g.E = 1;
    g.Kd = (int)l->H;
    g.Nout = (int)l->E;
    // one group of T rows and few (E) features: the 32-row tiles give T / 32
    // workgroups where 256-row tiles would leave most CUs idle
    const Path rp = path == Path::kF32 ? Path::kF32 : Path::kDecode;
    const int bm = path_bm(rp), bn = rp == Path::kF32 ? gemm_f32_bn(false) : router_bn();
    g.nN = (int)((l->E + bn - 1) / bn);
    g.ksplit = 1;
    g.out = logits;
    g.w.w_gate = g.w.w_up = l->wr_t;
    g.w.e_rows = l->E;
    g.w.row_mul = 1;
    if (present(l->w.router_bias)) g.w.b_gate = l->w.router_bias.data;
    moe_status st = hip_check(launch_single_group(grp, grp + 1, grp + 3, grp + 5, (int)T, bm, s),
                              "router setup launch");
    if (st) return st;
    const int64_t m_tiles = (T + bm - 1) / bm;
    if (rp == Path::kF32)
        return hip_check(launch_gemm_f32(kEpiPlain, g, m_tiles, s), "router launch");
    return hip_check(launch_gemm_bf16(kind_of(rp), kEpiPlain, false, g, m_tiles, s),
                     "router launch");
}

moe_status copy_routing(const moe_layer *l, int64_t T, const char *ws, const Workspace &W,
                        moe_routing_out *r, hipStream_t s)
{
    if (!r) return MOE_OK;
    const int64_t TK = T * l->K;
    struct {
        void *dst;
        size_t src;
        size_t bytes;
    } cp[] = {
        {r->topk_ids, W.ids, (size_t)TK * 4},
        {r->topk_weights, W.weights, (size_t)TK * 4},
        {r->expert_counts, W.counts, (size_t)l->E * 4},
        {r->expert_offsets, W.offsets, (size_t)(l->E + 1) * 4},
        {r->row_token, W.row_token, (size_t)TK * 4},
        {r->slot_row, W.slot_row, (size_t)TK * 4},
    };
    for (auto &c : cp) {
        if (!c.dst || c.bytes == 0) continue;
        moe_status st = hip_check(
            hipMemcpyAsync(c.dst, ws + c.src, c.bytes, hipMemcpyDeviceToDevice, s),
            "routing copy");
        if (st) return st;
    }
    return MOE_OK;
}

moe_status check_workspace(const moe_layer *l, int64_t T, void *ws, size_t bytes,
                           Workspace *W)
{
    *W = layout(l, T);
    if (!ws) return fail(MOE_ERR_WORKSPACE, "workspace is NULL");
    if (((uintptr_t)ws & 255) != 0)
        return fail(MOE_ERR_WORKSPACE, "workspace not 256-byte aligned");
    if (bytes < W->total)
        return fail(MOE_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", bytes, W->total);
    return MOE_OK;
}

// Prepare once per binding: scan the down-weight range on `s` and decide
// whether the down GEMM may run in fp16 (bf16 magnitudes <= 65280, or MXFP4
// scale bytes in [104, 140]: every value then converts to fp16 exactly in
// its normal range, and one below 2^-14 keeps the fewer bits of an fp16
// subnormal, an absolute error of at most 2^-25).  Synchronises `s` once.
// Pack an MXFP4 layer's gate||up (GEMM 1, two operands) and down (GEMM 2)
// stacks into l->mx_pack.
moe_status pack_mxfp4(const moe_layer *l, hipStream_t s)
{
    const int64_t E = l->E, H = l->H, I = l->I;
    const int ops1 = gated(l) ? 2 : 1;
    const int64_t sz[4] = {mx_pack_bytes(ops1, I, H, E), mx_pack_scale_bytes(ops1, I, H, E),
                           mx_pack_bytes(1, H, I, E), mx_pack_scale_bytes(1, H, I, E)};
    if (!l->mx_pack) {
        int64_t total = 0;
        for (int i = 0; i < 4; ++i) {
            l->mx_off[i] = total;
            total += (sz[i] + 255) / 256 * 256;
        }
        void *p = nullptr;
        moe_status st = hip_check(hipMalloc(&p, (size_t)total), "MXFP4 pack alloc");
        if (st) return st;
        l->mx_pack = (uint8_t *)p;
    }
    PackArgs a{};
    a.E = (int)E;
    a.ops = ops1;
    a.Nh = (int)I;
    a.K = (int)H;
    a.nks = (int)((H + 63) / 64);
    if (!gated(l)) {
        // one fc1 stack [E, I, H]
        a.codes[0] = a.codes[1] = (const uint8_t *)l->w.gate_up_experts.data;
        a.scales[0] = a.scales[1] = l->w.gate_up_experts.scales;
        a.e_rows = I;
        a.row_mul = 1;
        a.off[0] = a.off[1] = 0;
    } else if (fused(l)) {
        a.codes[0] = a.codes[1] = (const uint8_t *)l->w.gate_up_experts.data;
        a.scales[0] = a.scales[1] = l->w.gate_up_experts.scales;
        a.e_rows = 2 * I;
        const bool il = l->opts.swiglu_fusion == MOE_FUSION_INTERLEAVED;
        a.row_mul = il ? 2 : 1;
        a.off[0] = 0;
        a.off[1] = il ? 1 : (int)I;
    } else {
        a.codes[0] = (const uint8_t *)l->w.gate_experts.data;
        a.scales[0] = l->w.gate_experts.scales;
        a.codes[1] = (const uint8_t *)l->w.gate_up_experts.data;
        a.scales[1] = l->w.gate_up_experts.scales;
        a.e_rows = I;
        a.row_mul = 1;
        a.off[0] = a.off[1] = 0;
    }
    a.pk = l->mx_pack + l->mx_off[0];
    a.pks = l->mx_pack + l->mx_off[1];
    moe_status st = hip_check(launch_mx_pack(a, s), "MXFP4 pack (gate/up)");
    if (st) return st;
    PackArgs d{};
    d.E = (int)E;
    d.ops = 1;
    d.Nh = (int)H;
    d.K = (int)I;
    d.nks = (int)((I + 63) / 64);
    d.codes[0] = d.codes[1] = (const uint8_t *)l->w.down_experts.data;
    d.scales[0] = d.scales[1] = l->w.down_experts.scales;
    d.e_rows = H;
    d.row_mul = 1;
    d.pk = l->mx_pack + l->mx_off[2];
    d.pks = l->mx_pack + l->mx_off[3];
    return hip_check(launch_mx_pack(d, s), "MXFP4 pack (down)");
}

moe_status prepare_locked(const moe_layer *l, hipStream_t s)
{
    std::lock_guard<std::mutex> lock(l->mu);
    if (l->prepared) return MOE_OK;
    int ok = 0;
    if (l->wdtype == MOE_DTYPE_MXFP4) {
        moe_status st = pack_mxfp4(l, s);
        if (st) return st;
    }
    if (has_router(l)) {
        const int eb = act_dtype(l) == MOE_DTYPE_F32 ? 4 : 2;
        if (!l->wr_t) {
            moe_status st = hip_check(hipMalloc(&l->wr_t, (size_t)(l->E * l->H * eb)),
                                      "router alloc");
            if (st) return st;
        }
        moe_status st = hip_check(launch_transpose(l->w.router_weight.data, l->wr_t, (int)l->H,
                                                   (int)l->E, eb, s),
                                  "router transpose");
        if (st) return st;
    }
    if (l->wdtype != MOE_DTYPE_F32) {
        uint32_t *d = nullptr;
        moe_status st = hip_check(hipMalloc((void **)&d, 16), "prepare alloc");
        if (st) return st;
        const uint32_t init[4] = {0u, 255u, 0u, 0u};
        const bool mx = l->wdtype == MOE_DTYPE_MXFP4;
        const int64_t elems = l->E * l->H * l->I;
        uint32_t r[4] = {0, 0, 0, 0};
        hipError_t e = hipMemcpyAsync(d, init, sizeof init, hipMemcpyHostToDevice, s);
        if (e == hipSuccess)
            e = launch_weight_range(l->w.down_experts.data, l->w.down_experts.scales,
                                    mx ? 0 : elems / 2, mx ? elems / 32 : 0, d, s);
        if (e == hipSuccess) e = hipMemcpyAsync(r, d, sizeof r, hipMemcpyDeviceToHost, s);
        if (e == hipSuccess) e = hipStreamSynchronize(s);
        (void)hipFree(d);
        if ((st = hip_check(e, "prepare weight scan"))) return st;
        ok = mx ? (r[1] >= 104u && r[2] <= 140u) : (r[0] <= 0x477fu);
    }
    l->pk16_ready = false;
    l->pk16_down_f16 = false;
    if (l->wdtype == MOE_DTYPE_BF16 && l->opts.pack_weights) {
        const int64_t n1 = gemm1_tiles(l), n2 = gemm2_tiles(l);
        const int64_t sz1 = pack16_bytes(l->E, n1, l->H), sz2 = pack16_bytes(l->E, n2, l->I);
        if (!l->pk16) {
            void *p = nullptr;
            if (hipMalloc(&p, (size_t)(sz1 + sz2)) != hipSuccess) {
                (void)hipGetLastError();   // no room: the GEMMs read the caller's rows
                p = nullptr;
            }
            l->pk16 = (uint8_t *)p;
            l->pk16_off[0] = 0;
            l->pk16_off[1] = sz1;
        }
        if (l->pk16) {
            Pack16Args a{};
            a.w = gemm1_rows(l);
            a.gated = gated(l) ? 1 : 0;
            a.Nout = (int)l->I;
            a.K = (int)l->H;
            a.E = (int)l->E;
            a.nN = (int)n1;
            a.nks = (int)((l->H + 63) / 64);
            a.dst = l->pk16 + l->pk16_off[0];
            moe_status st = hip_check(launch_pack16(a, s), "gate/up weight copy");
            if (st) return st;
            Pack16Args d{};
            d.w = down_rows(l);
            d.gated = 0;
            d.Nout = (int)l->H;
            d.K = (int)l->I;
            d.E = (int)l->E;
            d.nN = (int)n2;
            d.nks = (int)((l->I + 63) / 64);
            d.to_f16 = (ok && l->opts.down_fp16_copy) ? 1 : 0;
            d.dst = l->pk16 + l->pk16_off[1];
            if ((st = hip_check(launch_pack16(d, s), "down weight copy"))) return st;
            // complete before prepare returns, like the rest of it (a forward
            // on another stream may follow, and the caller may then release
            // its stacks)
            if ((st = hip_check(hipStreamSynchronize(s), "prepare sync"))) return st;
            l->pk16_ready = true;
            l->pk16_down_f16 = d.to_f16 != 0;
        }
    }
    if (l->wdtype == MOE_DTYPE_F32 && has_router(l)) {
        // (the 16-bit path synchronised in its weight scan)
        moe_status st = hip_check(hipStreamSynchronize(s), "prepare sync");
        if (st) return st;
    }
    l->down_f16_ok = ok;
    l->prepared = true;
    return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_options_default(moe_options *o)
{
    if (!o) return fail(MOE_ERR_INVALID_ARGUMENT, "options is NULL");
    std::memset(o, 0, sizeof *o);
    o->scoring = MOE_SCORING_SOFTMAX;
    o->renormalize = 0;
    o->n_group = 0;
    o->topk_group = 0;
    o->routed_scaling_factor = 1.0f;
    o->activation = MOE_ACT_SILU_GATED;
    o->swiglu_fusion = MOE_FUSION_SPLIT;
    o->swiglu_alpha = 1.0f;
    o->swiglu_beta = 0.0f;
    o->swiglu_limit = 0.0f;
    o->gemm_variant = 0;
    o->down_fp16_copy = 1;
    o->pack_weights = 1;
    return MOE_OK;
}

moe_status moe_create(int64_t E, int64_t H, int64_t I, int64_t K, moe_dtype wdtype,
                      int has_gu_bias, int has_d_bias, const moe_options *opts,
                      moe_layer **out)
{
    if (!out) return fail(MOE_ERR_INVALID_ARGUMENT, "out_layer is NULL");
    *out = nullptr;
    moe_options o;
    if (opts) o = *opts;
    else moe_options_default(&o);
    if (E < 1 || E > kMaxExperts)
        return fail(MOE_ERR_INVALID_ARGUMENT, "num_experts %lld outside 1..%d", (long long)E,
                    kMaxExperts);
    if (K < 1 || K > E || K > kMaxTopK)
        return fail(MOE_ERR_INVALID_ARGUMENT, "top_k %lld outside 1..min(E, %d)", (long long)K,
                    kMaxTopK);
    if (H < 1 || I < 1 || H > (1 << 20) || I > kMaxHTiles * 128)
        return fail(MOE_ERR_INVALID_ARGUMENT, "hidden size above 2^20 or intermediate size "
                    "above %d", kMaxHTiles * 128);
    if (wdtype != MOE_DTYPE_F32 && wdtype != MOE_DTYPE_BF16 && wdtype != MOE_DTYPE_MXFP4)
        return fail(MOE_ERR_INVALID_ARGUMENT, "weight dtype must be F32, BF16 or MXFP4");
    if (wdtype == MOE_DTYPE_MXFP4 && (H % 32 || I % 32))
        return fail(MOE_ERR_INVALID_ARGUMENT, "MXFP4 needs H and I multiples of 32");
    if (H % 8 || I % 8)
        return fail(MOE_ERR_INVALID_ARGUMENT, "H and I must be multiples of 8");
    if (o.scoring != MOE_SCORING_SOFTMAX && o.scoring != MOE_SCORING_SIGMOID)
        return fail(MOE_ERR_INVALID_ARGUMENT, "unknown scoring %d", o.scoring);
    if (o.n_group < 0)
        return fail(MOE_ERR_INVALID_ARGUMENT, "n_group < 0");
    if (o.n_group > 0) {
        if (o.n_group > kMaxGroups || E % o.n_group)
            return fail(MOE_ERR_INVALID_ARGUMENT, "n_group must divide E and be <= %d",
                        kMaxGroups);
        if (o.topk_group < 1 || o.topk_group > o.n_group)
            return fail(MOE_ERR_INVALID_ARGUMENT, "topk_group outside 1..n_group");
        if (K > (int64_t)o.topk_group * (E / o.n_group))
            return fail(MOE_ERR_INVALID_ARGUMENT,
                        "top_k exceeds the experts of topk_group groups");
    }
    if (o.activation < MOE_ACT_SILU_GATED || o.activation > MOE_ACT_IDENTITY)
        return fail(MOE_ERR_INVALID_ARGUMENT, "unknown activation %d", o.activation);
    if (o.gelu_mode != MOE_GELU_ERF && o.gelu_mode != MOE_GELU_TANH)
        return fail(MOE_ERR_INVALID_ARGUMENT, "unknown gelu_mode %d", o.gelu_mode);
    if (o.weigh_inputs != 0 && o.weigh_inputs != 1)
        return fail(MOE_ERR_INVALID_ARGUMENT, "weigh_inputs must be 0 or 1");
    if (o.down_fp16_copy != 0 && o.down_fp16_copy != 1)
        return fail(MOE_ERR_INVALID_ARGUMENT, "down_fp16_copy must be 0 or 1");
    if (o.pack_weights != 0 && o.pack_weights != 1)
        return fail(MOE_ERR_INVALID_ARGUMENT, "pack_weights must be 0 or 1");
    if (o.swiglu_fusion < MOE_FUSION_NONE || o.swiglu_fusion > MOE_FUSION_SPLIT)
        return fail(MOE_ERR_INVALID_ARGUMENT, "unknown swiglu_fusion %d", o.swiglu_fusion);
    if (o.gemm_variant < 0 || o.gemm_variant > 3)
        return fail(MOE_ERR_INVALID_ARGUMENT, "unknown gemm_variant %d", o.gemm_variant);
    if (!(o.routed_scaling_factor == o.routed_scaling_factor))
        return fail(MOE_ERR_INVALID_ARGUMENT, "routed_scaling_factor is NaN");
    moe_layer *l = new (std::nothrow) moe_layer();
    if (!l) return fail(MOE_ERR_INVALID_ARGUMENT, "out of host memory");
    l->E = E;
    l->H = H;
    l->I = I;
    l->K = K;
    l->wdtype = wdtype;
    l->has_gu_bias = has_gu_bias ? 1 : 0;
    l->has_d_bias = has_d_bias ? 1 : 0;
    l->opts = o;
    l->bound = false;
    l->prepared = false;
    l->down_f16_ok = 0;
    *out = l;
    return MOE_OK;
}

moe_status moe_set_weights(moe_layer *l, const moe_weights *w)
{
    if (!l || !w) return fail(MOE_ERR_INVALID_ARGUMENT, "layer or weights is NULL");
    const int64_t E = l->E, H = l->H, I = l->I;
    const int wd = l->wdtype, ad = act_dtype(l);
    const bool fz = fused(l), two = two_stacks(l);
    moe_status st;
    if (!present(w->gate_up_experts) || !present(w->down_experts))
        return fail(MOE_ERR_SHAPE_MISMATCH, "gate_up_experts and down_experts are required");
    if ((st = check_tensor("gate_up_experts", w->gate_up_experts, wd, {E, fz ? 2 * I : I, H})))
        return st;
    if ((st = check_tensor("down_experts", w->down_experts, wd, {E, H, I}))) return st;
    if (!two && present(w->gate_experts))
        return fail(MOE_ERR_SHAPE_MISMATCH, fz ? "gate_experts given for a fused gate||up layout"
                                               : "gate_experts given for a non-gated activation");
    if (two) {
        if (!present(w->gate_experts))
            return fail(MOE_ERR_SHAPE_MISMATCH,
                        "gate_experts is required when swiglu_fusion = NONE");
        if ((st = check_tensor("gate_experts", w->gate_experts, wd, {E, I, H}))) return st;
    }
    if (present(w->gate_up_bias)) {
        if (!l->has_gu_bias)
            return fail(MOE_ERR_NOT_DECLARED, "gate_up_bias given but not declared");
        if ((st = check_tensor("gate_up_bias", w->gate_up_bias, ad, {E, fz ? 2 * I : I})))
            return st;
    }
    if (present(w->gate_bias)) {
        if (!l->has_gu_bias)
            return fail(MOE_ERR_NOT_DECLARED, "gate_bias given but not declared");
        if (!two)
            return fail(MOE_ERR_SHAPE_MISMATCH,
                        "gate_bias given without a separate gate stack");
        if ((st = check_tensor("gate_bias", w->gate_bias, ad, {E, I}))) return st;
    }
    if (present(w->down_bias)) {
        if (!l->has_d_bias)
            return fail(MOE_ERR_NOT_DECLARED, "down_bias given but not declared");
        if ((st = check_tensor("down_bias", w->down_bias, ad, {E, H}))) return st;
    }
    if (present(w->e_score_correction_bias) &&
        (st = check_tensor("e_score_correction_bias", w->e_score_correction_bias,
                           MOE_DTYPE_F32, {E})))
        return st;
    // the layer's own router ("MoeSpec" wr [H, E], router_bias [E]); binds
    // whatever was declared, like the selection bias
    if (present(w->router_weight) &&
        (st = check_tensor("router_weight", w->router_weight, ad, {H, E})))
        return st;
    if (present(w->router_bias)) {
        if (!present(w->router_weight))
            return fail(MOE_ERR_SHAPE_MISMATCH, "router_bias given without router_weight");
        if ((st = check_tensor("router_bias", w->router_bias, ad, {E}))) return st;
    }
    // the shared-expert gate g [H] (logicaffeine "Moe" `shared_gate`)
    if (present(w->shared_gate) &&
        (st = check_tensor("shared_gate", w->shared_gate, ad, {H})))
        return st;
    std::lock_guard<std::mutex> lock(l->mu);
    l->w = *w;
    l->bound = true;
    l->prepared = false;   // re-binding drops the prepared state
    return MOE_OK;
}

moe_status moe_prepare(moe_layer *l, void *stream)
{
    if (!l) return fail(MOE_ERR_INVALID_ARGUMENT, "layer is NULL");
    moe_status st = check_bound(l);
    if (st) return st;
    return prepare_locked(l, (hipStream_t)stream);
}

moe_status moe_workspace_size(const moe_layer *l, int64_t T, size_t *bytes)
{
    if (!l || !bytes) return fail(MOE_ERR_INVALID_ARGUMENT, "layer or bytes is NULL");
    if (T < 0 || T > (1 << 24)) return fail(MOE_ERR_INVALID_ARGUMENT, "T out of range");
    *bytes = layout(l, T).total;
    return MOE_OK;
}

moe_status moe_route(const moe_layer *l, const moe_tensor *logits, moe_routing_out *r,
                     void *ws, size_t ws_bytes, void *stream)
{
    if (!l || !logits || !r) return fail(MOE_ERR_INVALID_ARGUMENT, "NULL argument");
    bool okT;
    const int64_t T = tokens_of(*logits, l->E, &okT);
    if (!okT || logits->dtype != MOE_DTYPE_F32)
        return fail(MOE_ERR_SHAPE_MISMATCH, "router_logits must be f32 [T, E]");
    if (T > (1 << 24)) return fail(MOE_ERR_INVALID_ARGUMENT, "T out of range");
    if (T == 0) return MOE_OK;
    if (!logits->data) return fail(MOE_ERR_INVALID_ARGUMENT, "router_logits data is NULL");
    Workspace W;
    moe_status st = check_workspace(l, T, ws, ws_bytes, &W);
    if (st) return st;
    hipStream_t s = (hipStream_t)stream;
    const Path path = choose_path(l, T);
    if ((st = run_route(l, (const float *)logits->data, T, (char *)ws, W, path, s, nullptr)))
        return st;
    return copy_routing(l, T, (const char *)ws, W, r, s);
}

moe_status moe_forward(const moe_layer *l, const moe_tensor *x, const moe_tensor *logits,
                       const moe_tensor *shared, moe_tensor *out, void *ws, size_t ws_bytes,
                       moe_routing_out *routing, void *stream)
{
    return moe_forward_timed(l, x, logits, shared, out, ws, ws_bytes, routing, stream, nullptr);
}

moe_status moe_forward_timed(const moe_layer *l, const moe_tensor *x, const moe_tensor *logits,
                             const moe_tensor *shared, moe_tensor *out, void *ws,
                             size_t ws_bytes, moe_routing_out *routing, void *stream,
                             void *const *events)
{
    return moe::forward_impl(l, x, logits, shared, out, ws, ws_bytes, routing, stream, events,
                             true);
}

}  // extern "C"

// The forward's body.  may_prepare = false (the allocation-free entry):
// a layer whose binding is not prepared yet is an error instead of a
// prepare, which allocates.
moe_status moe::forward_impl(const moe_layer *l, const moe_tensor *x, const moe_tensor *logits,
                             const moe_tensor *shared, moe_tensor *out, void *ws,
                             size_t ws_bytes, moe_routing_out *routing, void *stream,
                             void *const *events, bool may_prepare)
{
    if (!l || !x || !out) return fail(MOE_ERR_INVALID_ARGUMENT, "NULL argument");
    moe_status st = check_bound(l);
    if (st) return st;
    if (!may_prepare) {
        std::lock_guard<std::mutex> lock(l->mu);
        if (!l->prepared)
            return fail(MOE_ERR_INVALID_ARGUMENT,
                        "the layer is not prepared (call moe_prepare before an allocation-free "
                        "forward: preparing allocates)");
    }
    // no logits: the layer's bound router computes them
    // (absent means NULL or ndim 0: an empty [0, E] tensor may have no data)
    const bool own_router = !logits || logits->ndim == 0;
    if (own_router && !has_router(l))
        return fail(MOE_ERR_UNBOUND, "router_logits not given and no router_weight bound");
    const int ad = act_dtype(l);
    if (x->dtype != MOE_DTYPE_F32 && x->dtype != MOE_DTYPE_BF16)
        return fail(MOE_ERR_SHAPE_MISMATCH, "x dtype must be f32 or bf16");
    if (x->dtype != ad)
        return fail(MOE_ERR_UNSUPPORTED, "x dtype %s with %s weights (needs %s)",
                    dtype_name(x->dtype), dtype_name(l->wdtype), dtype_name(ad));
    bool okT;
    const int64_t T = tokens_of(*x, l->H, &okT);
    if (!okT) return fail(MOE_ERR_SHAPE_MISMATCH, "x must be [T, H] or [B, S, H]");
    if (!own_router) {
        bool okL;
        const int64_t TL = tokens_of(*logits, l->E, &okL);
        if (!okL || TL != T || logits->dtype != MOE_DTYPE_F32)
            return fail(MOE_ERR_SHAPE_MISMATCH,
                        "router_logits must be f32 [T, E] with T = %lld", (long long)T);
    }
    auto same_as_x = [&](const moe_tensor &t) {
        if (t.dtype != x->dtype || t.ndim != x->ndim) return false;
        for (int i = 0; i < x->ndim; ++i)
            if (t.shape[i] != x->shape[i]) return false;
        return true;
    };
    if (!same_as_x(*out)) return fail(MOE_ERR_SHAPE_MISMATCH, "out must match x's shape and dtype");
    const bool has_shared = shared && present(*shared);
    if (has_shared && !same_as_x(*shared))
        return fail(MOE_ERR_SHAPE_MISMATCH, "shared_output must match x's shape and dtype");
    if (T > (1 << 24)) return fail(MOE_ERR_INVALID_ARGUMENT, "T out of range");
    if (T == 0) return MOE_OK;
    if (!x->data || !out->data || (!own_router && !logits->data))
        return fail(MOE_ERR_INVALID_ARGUMENT, "x, router_logits or out data is NULL");
    Workspace W;
    if ((st = check_workspace(l, T, ws, ws_bytes, &W))) return st;

    hipStream_t s = (hipStream_t)stream;
    if ((st = prepare_locked(l, s))) return st;
    char *wsb = (char *)ws;
    auto mark = [&](int i) -> moe_status {
        if (events && events[i])
            return hip_check(hipEventRecord((hipEvent_t)events[i], s), "event record");
        return MOE_OK;
    };
    const Path path = choose_path(l, T);
    if ((st = mark(0))) return st;
    const float *lg = own_router ? (const float *)(wsb + W.logits) : (const float *)logits->data;
    if (own_router && (st = run_router(l, x->data, T, (float *)(wsb + W.logits), wsb, W, path, s)))
        return st;
    const bool sgate = has_shared && present(l->w.shared_gate);
    if ((st = run_route(l, lg, T, wsb, W, path, s, events, sgate ? x : nullptr))) return st;

    const int bm = path_bm(path);
    const int64_t max_m_tiles = max_m_tiles_of(l, T, bm);
    const bool mx = l->wdtype == MOE_DTYPE_MXFP4;

    // GEMM 1: gate||up with the fused activation -> h
    GemmArgs g1{};
    g1.a = x->data;
    g1.a_off32 = T * l->H * (x->dtype == MOE_DTYPE_F32 ? 4 : 2) <= (int64_t(1) << 32) ? 1 : 0;
    g1.row_token = (const int32_t *)(wsb + W.row_token);
    g1.counts = (const int32_t *)(wsb + W.counts);
    g1.offsets = (const int32_t *)(wsb + W.offsets);
    g1.tile_cum = (const int32_t *)(wsb + W.tile_cum1);
    g1.full_cum = (const int32_t *)(wsb + W.full_cum1);
    g1.E = (int)l->E;
    g1.Kd = (int)l->H;
    g1.Nout = (int)l->I;
    const bool gt = gated(l);
    const int epi1 = gt ? kEpiGated : kEpiAct;
    const int bn1 = path_bn1(l, path);
    g1.nN = (int)((l->I + bn1 - 1) / bn1);
    g1.ksplit = 1;
    g1.out = wsb + W.h;
    g1.act = l->opts.activation;
    g1.gelu_mode = l->opts.gelu_mode;
    g1.row_w = l->opts.weigh_inputs ? (const float *)(wsb + W.row_weight) : nullptr;
    g1.alpha = l->opts.swiglu_alpha;
    g1.beta = l->opts.swiglu_beta;
    g1.limit = l->opts.swiglu_limit;
    g1.hfmt = (uint8_t *)(wsb + W.hfmt);
    g1.h_tiles = g1.nN;
    g1.h_width = bn1;
    g1.f16_ok = l->down_f16_ok;
    g1.w = gemm1_rows(l);

    // GEMM 2: down + bias -> y (f32 space; in-range chunks stored in fp16 when yfmt is set)
    GemmArgs g2{};
    g2.a = wsb + W.h;
    g2.a_off32 = T * l->K * l->I * 2 <= (int64_t(1) << 32) ? 1 : 0;
    g2.row_token = nullptr;
    g2.counts = g1.counts;
    g2.offsets = g1.offsets;
    g2.tile_cum = (const int32_t *)(wsb + W.tile_cum2);
    g2.full_cum = (const int32_t *)(wsb + W.full_cum2);
    g2.E = (int)l->E;
    g2.Kd = (int)l->I;
    g2.Nout = (int)l->H;
    const int bn2 = path_bn2(l, path);
    g2.nN = (int)((l->H + bn2 - 1) / bn2);
    g2.out = wsb + W.y;
    const int splits = down_splits(l, T, path);
    g2.ksplit = splits;
    g2.split_stride = T * l->K * l->H;
    g2.w = down_rows(l);
    g2.hfmt = g1.hfmt;
    if (l->pk16_ready && path != Path::kF32) {
        // both GEMMs stream the prepared stage-layout copies
        g1.wpk = l->pk16 + l->pk16_off[0];
        g1.nks = (int)((l->H + 63) / 64);
        g2.wpk = l->pk16 + l->pk16_off[1];
        g2.nks = (int)((l->I + 63) / 64);
        g2.wpk_f16 = l->pk16_down_f16 ? 1 : 0;
    }
    g2.h_tiles = g1.nN;
    g2.h_width = bn1;
    g2.f16_ok = g1.f16_ok;
    // a 16-bit layer stores in-range y chunks (or partial-sum chunks) in fp16:
    // they are summed into a bf16 output whose rounding is 8x coarser than fp16's
    if (path != Path::kF32 && x->dtype == MOE_DTYPE_BF16) {
        g2.yfmt = (uint8_t *)(wsb + W.yfmt);
        g2.yfmt_stride = (l->H + kYWidth - 1) / kYWidth;
        g2.yfmt_split_stride = T * l->K * g2.yfmt_stride;
    }
    if (mx) {
        g1.pk = l->mx_pack + l->mx_off[0];
        g1.pks = l->mx_pack + l->mx_off[1];
        g1.nks = (int)((l->H + 63) / 64);
        g1.nrb_half = (int)(l->I / 32);
        g2.pk = l->mx_pack + l->mx_off[2];
        g2.pks = l->mx_pack + l->mx_off[3];
        g2.nks = (int)((l->I + 63) / 64);
        g2.nrb_half = (int)(l->H / 32);
    }

    if (max_m_tiles * (g1.nN > g2.nN * splits ? g1.nN : g2.nN * splits) + 8 > 0x7fffffffLL)
        return fail(MOE_ERR_UNSUPPORTED, "problem too large for one launch");

    if (path == Path::kF32) {
        if ((st = hip_check(launch_gemm_f32(epi1, g1, max_m_tiles, s), "gemm1 launch"))) return st;
        if ((st = mark(3))) return st;
        if ((st = hip_check(launch_gemm_f32(kEpiDown, g2, max_m_tiles, s), "gemm2 launch")))
            return st;
    } else {
        const GemmKind kind = kind_of(path);
        if ((st = hip_check(launch_gemm_bf16(kind, epi1, mx, g1, max_m_tiles, s), "gemm1 launch")))
            return st;
        if ((st = mark(3))) return st;
        if ((st = hip_check(launch_gemm_bf16(kind, kEpiDown, mx, g2, max_m_tiles, s),
                            "gemm2 launch")))
            return st;
    }
    if ((st = mark(4))) return st;

    CombineArgs ca{};
    ca.y = (const float *)(wsb + W.y);
    ca.weights = (const float *)(wsb + W.weights);
    ca.slot_row = (const int32_t *)(wsb + W.slot_row);
    ca.shared = has_shared ? shared->data : nullptr;
    ca.shared_scale = sgate ? (const float *)(wsb + W.sgate) : nullptr;
    ca.out = (void *)out->data;
    ca.T = (int)T;
    ca.H = (int)l->H;
    ca.K = (int)l->K;
    ca.out_bf16 = x->dtype == MOE_DTYPE_BF16;
    ca.unit_weights = l->opts.weigh_inputs;
    ca.splits = splits;
    ca.split_stride = g2.split_stride;
    ca.yfmt = g2.yfmt;
    ca.yfmt_stride = g2.yfmt_stride;
    ca.yfmt_split_stride = g2.yfmt_split_stride;
    if ((st = hip_check(launch_combine(ca, s), "combine launch"))) return st;
    if ((st = mark(5))) return st;
    return copy_routing(l, T, wsb, W, routing, s);
}

moe_status moe::set_error(moe_status s, const char *msg)
{
    return fail(s, "%s", msg);
}

extern "C" {

moe_status moe_router_logits(const moe_layer *l, const moe_tensor *x, moe_tensor *logits,
                             void *ws, size_t ws_bytes, void *stream)
{
    if (!l || !x || !logits) return fail(MOE_ERR_INVALID_ARGUMENT, "NULL argument");
    moe_status st = check_bound(l);
    if (st) return st;
    if (!has_router(l)) return fail(MOE_ERR_UNBOUND, "router_weight slot unbound");
    if (x->dtype != act_dtype(l))
        return fail(MOE_ERR_UNSUPPORTED, "x dtype %s with %s weights", dtype_name(x->dtype),
                    dtype_name(l->wdtype));
    bool okT, okL;
    const int64_t T = tokens_of(*x, l->H, &okT);
    if (!okT) return fail(MOE_ERR_SHAPE_MISMATCH, "x must be [T, H] or [B, S, H]");
    const int64_t TL = tokens_of(*logits, l->E, &okL);
    if (!okL || TL != T || logits->dtype != MOE_DTYPE_F32)
        return fail(MOE_ERR_SHAPE_MISMATCH, "logits must be f32 [T, E] with T = %lld",
                    (long long)T);
    if (T > (1 << 24)) return fail(MOE_ERR_INVALID_ARGUMENT, "T out of range");
    if (T == 0) return MOE_OK;
    if (!x->data || !logits->data)
        return fail(MOE_ERR_INVALID_ARGUMENT, "x or logits data is NULL");
    Workspace W;
    if ((st = check_workspace(l, T, ws, ws_bytes, &W))) return st;
    hipStream_t s = (hipStream_t)stream;
    if ((st = prepare_locked(l, s))) return st;
    return run_router(l, x->data, T, (float *)logits->data, (char *)ws, W, choose_path(l, T), s);
}

moe_status moe_borrowed_slots(const moe_layer *l, uint32_t *mask)
{
    if (!l || !mask) return fail(MOE_ERR_INVALID_ARGUMENT, "layer or mask is NULL");
    std::lock_guard<std::mutex> lock(l->mu);
    if (!l->bound) return fail(MOE_ERR_UNBOUND, "weights not bound (call moe_set_weights)");
    const moe_tensor *slot[10] = {&l->w.gate_up_experts, &l->w.down_experts, &l->w.gate_experts,
                                  &l->w.gate_up_bias, &l->w.down_bias, &l->w.gate_bias,
                                  &l->w.e_score_correction_bias, &l->w.router_weight,
                                  &l->w.router_bias, &l->w.shared_gate};
    uint32_t m = 0;
    for (int i = 0; i < 10; ++i)
        if (present(*slot[i])) m |= 1u << i;
    if (l->prepared) {
        // the GEMMs stream the library's packed copy of every expert stack
        // (MXFP4, or 16-bit in the stage layout), and the transposed router
        if (l->wdtype == MOE_DTYPE_MXFP4)
            m &= ~(MOE_SLOT_GATE_UP_EXPERTS | MOE_SLOT_DOWN_EXPERTS | MOE_SLOT_GATE_EXPERTS);
        if (l->wdtype == MOE_DTYPE_BF16 && l->pk16_ready)
            m &= ~(MOE_SLOT_GATE_UP_EXPERTS | MOE_SLOT_DOWN_EXPERTS | MOE_SLOT_GATE_EXPERTS);
        if (l->wr_t) m &= ~MOE_SLOT_ROUTER_WEIGHT;
    }
    *mask = m;
    return MOE_OK;
}

moe_status moe_destroy(moe_layer *l)
{
    if (l && l->mx_pack) (void)hipFree(l->mx_pack);
    if (l && l->wr_t) (void)hipFree(l->wr_t);
    if (l && l->pk16) (void)hipFree(l->pk16);
    delete l;
    return MOE_OK;
}

const char *moe_last_error(void)
{
    return g_err.c_str();
}

const char *moe_status_string(moe_status s)
{
    switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARGUMENT: return "MOE_ERR_INVALID_ARGUMENT";
    case MOE_ERR_SHAPE_MISMATCH: return "MOE_ERR_SHAPE_MISMATCH";
    case MOE_ERR_NOT_DECLARED: return "MOE_ERR_NOT_DECLARED";
    case MOE_ERR_UNBOUND: return "MOE_ERR_UNBOUND";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
    }
    return "MOE_ERR_UNKNOWN";
}

}  // extern "C"
