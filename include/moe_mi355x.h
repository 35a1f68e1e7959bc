/* moe_mi355x.h -- C ABI of the MI355X (gfx950) mixture-of-experts FFN forward.
 *
 * The layer: router top-K over caller-supplied logits, expert-contiguous
 * permutation of the (token, slot) pairs, a grouped gate||up GEMM with the
 * gated activation fused into its epilogue, a grouped down GEMM, and a
 * deterministic router-weighted combine.  Expert weights are dense f32, dense
 * bf16, or MXFP4 (weight-only: e2m1 codes with e8m0 block scales, decoded
 * inside the GEMM; the activation stays bf16).
 *
 * The calls mirror the lifecycle on the clika "ClikaRT::nn::QMoEWoQ" page
 * (make -> set_weights -> optional initialize -> forward) and the Python
 * "MoE" page (constructor geometry and options, set_weights slot names,
 * forward(x, router_logits, shared_output)).  Option semantics follow the
 * logicaffeine "MoeSpec" fields and the graiphic ONNX "MoE" attributes.
 *
 * Conventions for every call:
 *  - Tensors are described by moe_tensor: a DEVICE pointer to row-major,
 *    contiguous data plus its logical dtype and shape.  The library never
 *    copies, frees or retains caller memory beyond what each call states.
 *  - Every function returns a moe_status; on failure nothing was launched and
 *    moe_last_error() holds a message for the calling thread.  No C++
 *    exception crosses this boundary.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Calls are
 *    stream-ordered and never synchronise the host.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARGUMENT = 1, /* null handle/pointer, bad option value          */
    MOE_ERR_SHAPE_MISMATCH = 2,   /* a tensor's dtype or shape differs from the
                                     declaration (QMoEWoQ set_weights / forward)    */
    MOE_ERR_NOT_DECLARED = 3,     /* a bias bound to a slot make() did not declare
                                     (QMoEWoQ set_weights)                          */
    MOE_ERR_UNBOUND = 4,          /* forward/prepare before set_weights
                                     (QMoEWoQ initialize, "still-fake slot")        */
    MOE_ERR_UNSUPPORTED = 5,      /* a valid request this build does not serve,
                                     e.g. a dtype cast of quantised experts
                                     (QMoEWoQ to_impl(DataType))                    */
    MOE_ERR_WORKSPACE = 6,        /* workspace missing, too small or misaligned     */
    MOE_ERR_HIP = 7               /* the HIP runtime reported an error              */
} moe_status;

typedef enum moe_dtype {
    MOE_DTYPE_F32 = 0,
    MOE_DTYPE_BF16 = 1,
    MOE_DTYPE_MXFP4 = 2,  /* weights only: codes uint8 [..., K/2] (element 2i in the
                             low nibble of byte i) + e8m0 scales uint8 [..., K/32]   */
    MOE_DTYPE_I32 = 3
} moe_dtype;

/* MoeSpec `score`: softmax over every logit, or each logit's own sigmoid. */
typedef enum moe_scoring { MOE_SCORING_SOFTMAX = 0, MOE_SCORING_SIGMOID = 1 } moe_scoring;

/* Expert activation (ONNX MoE `activation_type`; clika MoE option
 * `activation`).  Gated (two projections, gate and up):
 *   SILU_GATED      h = silu(g)*u
 *   SWIGLU_CLAMPED  h = g'*sigmoid(alpha*g')*(u'+beta), g' = min(g,L),
 *                   u' = clamp(u,-L,L), L = swiglu_limit (L <= 0: no clamp)
 *                   -- ONNX MoE activation_alpha/beta and swiglu_limit; clika
 *                   MoE options swiglu_alpha/beta/limit.
 * Non-gated (one fc1 projection v, ONNX MoE fusion_size 1):
 *   RELU max(v,0); GELU v*Phi(v) (gelu_mode: erf form or tanh form);
 *   SILU v*sigmoid(v); IDENTITY v. */
typedef enum moe_activation {
    MOE_ACT_SILU_GATED = 0,
    MOE_ACT_SWIGLU_CLAMPED = 1,
    MOE_ACT_RELU = 2,
    MOE_ACT_GELU = 3,
    MOE_ACT_SILU = 4,
    MOE_ACT_IDENTITY = 5
} moe_activation;

/* clika MoE option `gelu_mode`: Phi(v) = (1+erf(v/sqrt 2))/2, or the tanh
 * approximation (1+tanh(sqrt(2/pi)(v+0.044715 v^3)))/2. */
typedef enum moe_gelu_mode { MOE_GELU_ERF = 0, MOE_GELU_TANH = 1 } moe_gelu_mode;

/* ONNX MoE `swiglu_fusion`: 0 not fused (separate gate and up stacks),
 * 1 fused interleaved (row 2i gate, 2i+1 up), 2 fused not interleaved
 * (rows [0,I) gate, [I,2I) up).  Non-gated activations ignore it. */
typedef enum moe_swiglu_fusion {
    MOE_FUSION_NONE = 0,
    MOE_FUSION_INTERLEAVED = 1,
    MOE_FUSION_SPLIT = 2
} moe_swiglu_fusion;

/* Routing and activation options (QMoEWoQ MoeOptions; clika MoE **options). */
typedef struct moe_options {
    int32_t scoring;              /* moe_scoring; default SOFTMAX                   */
    int32_t renormalize;          /* MoeSpec `renormalize`; default 0 (ONNX
                                     normalize_routing_weights default False).
                                     The renormalising sum is clamped at 2^-14
                                     (MoeSpec `sum_can_clamp`).                    */
    int32_t n_group;              /* group limit (MoeSpec/Moe `groups`): 0 = off;
                                     else E % n_group == 0, n_group <= 64          */
    int32_t topk_group;           /* groups kept, 1..n_group                         */
    float routed_scaling_factor;  /* MoeSpec `scale`, applied after renormalisation;
                                     default 1                                      */
    int32_t activation;           /* moe_activation; default SILU_GATED              */
    int32_t swiglu_fusion;        /* moe_swiglu_fusion; default SPLIT                */
    float swiglu_alpha;           /* default 1                                       */
    float swiglu_beta;            /* default 0                                       */
    float swiglu_limit;           /* default 0 = no clamp                            */
    int32_t gemm_variant;         /* grouped-GEMM tiles: 0 auto (by rows per expert
                                     and weight type), 1 large-M (prefill, 256-row)
                                     tiles, 2 small-M (decode, 32-row) tiles, 3
                                     mid (128-row) tiles; f32 layers ignore it.
                                     Default 0                                     */
    int32_t gelu_mode;            /* moe_gelu_mode; default ERF                      */
    int32_t weigh_inputs;         /* MoeSpec `weigh_inputs` (clika MoE
                                     apply_router_weight_on_input, Llama 4): a kept
                                     expert's weight scales the input it reads and
                                     its output joins the sum unweighted.  0 or 1;
                                     default 0                                      */
    int32_t down_fp16_copy;       /* bf16 layers with pack_weights whose down
                                     weights lie in fp16's range (checked by
                                     moe_prepare; the fp16 down GEMM runs only
                                     then): 1 stores the prepared down copy in
                                     fp16 (round to nearest even, exact in fp16's
                                     normal range), so the fp16 down GEMM streams
                                     it as it is; 0 keeps it bf16 and converts
                                     each tile's weight fragments in registers.
                                     0 or 1; default 1                              */
    int32_t pack_weights;         /* bf16 layers: 1 makes moe_prepare copy the
                                     gate||up (or fc1) and down stacks into
                                     library-owned device memory (E*2I*H*2 +
                                     E*H*I*2 bytes, rounded up to whole 256-row,
                                     64-column tiles; freed by moe_destroy) in the
                                     layout the GEMMs stream: per 256-row tile and
                                     64-wide k-step one contiguous 32 KiB block
                                     (the GEMMs then read weights from HBM at
                                     ~6.1 TB/s instead of ~4.5 TB/s row by row).
                                     The forward then reads no caller expert
                                     stack, which the caller may release
                                     (moe_borrowed_slots): one resident copy.  If
                                     the allocation fails the layer streams the
                                     caller's stacks instead, without error.
                                     0 or 1; default 1                              */
} moe_options;

/* A device tensor view.  ndim == 0 (or data == NULL) marks an absent tensor.
 * For MXFP4 the logical shape counts elements ([E, N, K]); `data` holds the
 * packed codes and `scales` the e8m0 bytes. */
typedef struct moe_tensor {
    const void *data;
    const uint8_t *scales;        /* MXFP4 only; NULL otherwise                     */
    int32_t dtype;                /* moe_dtype                                       */
    int32_t ndim;
    int64_t shape[4];
} moe_tensor;

/* Weight slots, named as clika MoE.set_weights / QMoEWoQ::set_weights.
 *  gate_up_experts : gated, fused [E, 2I, H] (layout per swiglu_fusion);
 *                    gated, not fused: the UP rows [E, I, H];
 *                    non-gated activation: the fc1 rows [E, I, H]
 *  gate_experts    : gated, not fused only: the GATE rows [E, I, H]
 *  down_experts    : [E, H, I]
 *  gate_up_bias    : fused [E, 2I]; otherwise up / fc1 bias [E, I] (x dtype)
 *  gate_bias       : gated, not fused only: gate bias [E, I]      (x dtype)
 *  down_bias       : [E, H]                                       (x dtype)
 *  e_score_correction_bias : [E] f32 selection bias; binds even when no bias
 *                    was declared (clika MoE.set_weights).  It is added to the
 *                    score for SELECTION only; weights use the score alone
 *                    (MoeSpec `selection_bias`).
 *  router_weight   : optional router Wr [H, E] (x dtype; MoeSpec `wr`, whose
 *                    index arithmetic makes it [d, E]); when bound, a forward
 *                    without router_logits computes logits = x . Wr + Br.
 *                    Binds whatever was declared, like the selection bias.
 *  router_bias     : optional router bias Br [E] (x dtype; MoeSpec
 *                    `router_bias`, added to each logit before scoring); needs
 *                    router_weight.
 *  shared_gate     : optional shared-expert gate g [H] (x dtype; logicaffeine
 *                    "Moe" field `shared_gate`: the shared experts' output is
 *                    scaled by the logistic sigmoid of x . g).  When bound, a
 *                    forward given shared_output adds sigmoid(x[t] . g) *
 *                    shared_output[t] instead of shared_output[t] (x . g
 *                    accumulated in fp64); without shared_output it is not
 *                    read.  Binds whatever was declared. */
typedef struct moe_weights {
    moe_tensor gate_up_experts;
    moe_tensor down_experts;
    moe_tensor gate_experts;
    moe_tensor gate_up_bias;
    moe_tensor down_bias;
    moe_tensor gate_bias;
    moe_tensor e_score_correction_bias;
    moe_tensor router_weight;
    moe_tensor router_bias;
    moe_tensor shared_gate;
} moe_weights;

/* Optional copies of the routing state of a forward (all DEVICE pointers,
 * each may be NULL).  Sizes: topk_ids, topk_weights [T, K]; expert_counts [E];
 * expert_offsets [E+1]; row_token, slot_row [T*K].  Rows of the permutation
 * are grouped by expert, ascending token order within an expert:
 * row_token[r] is the token of row r and slot_row[t*K+j] the row of (t, j). */
typedef struct moe_routing_out {
    int32_t *topk_ids;
    float *topk_weights;
    int32_t *expert_counts;
    int32_t *expert_offsets;
    int32_t *row_token;
    int32_t *slot_row;
} moe_routing_out;

typedef struct moe_layer moe_layer;

/* Fill `opts` with the defaults listed in moe_options. */
moe_status moe_options_default(moe_options *opts);

/* Declare a layer (QMoEWoQ::make / clika MoE.__init__): geometry E, H, I,
 * top_k (1 <= top_k <= min(E, 64)), the expert weight dtype (F32, BF16 or
 * MXFP4), which bias slots exist, and the options (NULL = defaults).
 * Validation: E <= 1024; H <= 2^20; I <= 131072; with a group limit,
 * E % n_group == 0 and top_k <= topk_group * E / n_group; MXFP4 needs H and I
 * multiples of 32; dense weights need H and I multiples of 8.  The handle
 * allocates device memory only at prepare: the packed copy of MXFP4 weights
 * and the transposed router, both freed by moe_destroy.
 * Errors: INVALID_ARGUMENT. */
moe_status moe_create(int64_t num_experts, int64_t hidden_size,
                      int64_t intermediate_size, int64_t top_k,
                      moe_dtype weight_dtype, int has_gate_up_bias,
                      int has_down_bias, const moe_options *opts,
                      moe_layer **out_layer);

/* Bind the weight slots (QMoEWoQ::set_weights).  The library BORROWS the
 * device buffers: the caller keeps them alive and unchanged until the next
 * set_weights or moe_destroy.  Re-binding replaces the previous binding.
 * Errors: SHAPE_MISMATCH (dtype/geometry differs from the declaration, or a
 * required stack is missing), NOT_DECLARED (a gate/up/down bias given
 * without its declared slot). */
moe_status moe_set_weights(moe_layer *layer, const moe_weights *w);

/* Optional warm-up (QMoEWoQ::initialize, "pack once"): checks that every
 * declared slot is bound, scans the down weights for fp16's range (a 16-bit
 * down stack whose magnitudes stay within it converts exactly in fp16's
 * normal range; a value below 2^-14 keeps the fewer bits of an fp16
 * subnormal, an absolute error of at most 2^-25), packs MXFP4 stacks and
 * (pack_weights) 16-bit stacks into the layouts the GEMMs stream, and
 * transposes a bound router.  Runs once per binding (a forward runs it
 * if needed) and synchronises `stream`.  Errors: UNBOUND, HIP. */
moe_status moe_prepare(moe_layer *layer, void *stream);

/* Bits of moe_borrowed_slots, one per moe_weights member in field order. */
#define MOE_SLOT_GATE_UP_EXPERTS 0x001u
#define MOE_SLOT_DOWN_EXPERTS 0x002u
#define MOE_SLOT_GATE_EXPERTS 0x004u
#define MOE_SLOT_GATE_UP_BIAS 0x008u
#define MOE_SLOT_DOWN_BIAS 0x010u
#define MOE_SLOT_GATE_BIAS 0x020u
#define MOE_SLOT_E_SCORE_CORRECTION_BIAS 0x040u
#define MOE_SLOT_ROUTER_WEIGHT 0x080u
#define MOE_SLOT_ROUTER_BIAS 0x100u
#define MOE_SLOT_SHARED_GATE 0x200u

/* Which bound caller buffers a forward still reads (the clika
 * "ClikaRT::nn::QMoEWoQ" class description: once packed, the layer keeps one
 * resident copy of its weights).  Sets *mask to the MOE_SLOT_* bits of the
 * bound slots whose caller buffer moe_forward, moe_route and
 * moe_router_logits read.  Before the binding is prepared every bound slot is
 * borrowed.  After moe_prepare:
 *  - MXFP4 layers read only the library's packed copy of gate_up_experts,
 *    gate_experts and down_experts (codes and scales);
 *  - 16-bit layers whose prepare made the stage-layout copy (pack_weights
 *    = 1 and the allocation succeeded) read it instead of gate_up_experts,
 *    gate_experts and down_experts, including the bf16 fallback of the down
 *    GEMM for h tiles beyond fp16's range;
 *  - a bound router is read from its transposed copy, not router_weight.
 * A slot whose bit is clear may be released or overwritten by the caller
 * until the next moe_set_weights (which drops the prepared state and makes
 * every slot borrowed again).  Biases, the selection bias and f32 layers'
 * stacks stay borrowed.  Errors: INVALID_ARGUMENT, UNBOUND. */
moe_status moe_borrowed_slots(const moe_layer *layer, uint32_t *mask);

/* Device workspace bytes a forward (or moe_route) on T tokens needs.  The
 * caller allocates it (256-byte aligned) and may reuse it across calls that
 * do not overlap in time. */
moe_status moe_workspace_size(const moe_layer *layer, int64_t T, size_t *bytes);

/* One MoE step (QMoEWoQ::forward): x [T, H] (or [B, S, H]) and the
 * caller-computed router_logits [T, E] f32 -> out with x's shape and dtype.
 * router_logits may be NULL (or ndim 0) when router_weight is bound: the
 * logits are then x . Wr + Br, computed on the GPU (f32 accumulation).
 * x dtype: F32 for F32 weights, BF16 for BF16 or MXFP4 weights.  Optional
 * shared_output (the shared-expert branch, EXACTLY x's shape and dtype) is
 * added inside the combine, scaled per token by sigmoid(x[t] . g) when the
 * shared_gate slot is bound.  `routing` (nullable) receives copies of the
 * routing state.  T = 0 launches nothing.
 * Errors: INVALID_ARGUMENT, SHAPE_MISMATCH, UNBOUND, UNSUPPORTED, WORKSPACE,
 * HIP.  Concurrent calls on one layer are allowed with distinct workspaces.
 * Once the layer is prepared (moe_prepare, or one earlier forward), a call
 * enqueues kernel launches on `stream` only (plus device-to-device copies
 * when `routing` is given): no allocation, memset or host synchronisation,
 * so it may be captured into a HIP graph and replayed, with the captured
 * buffers' contents changed between replays. */
moe_status moe_forward(const moe_layer *layer, const moe_tensor *x,
                       const moe_tensor *router_logits,
                       const moe_tensor *shared_output, moe_tensor *out,
                       void *workspace, size_t workspace_bytes,
                       moe_routing_out *routing, void *stream);

/* moe_forward with stage timing, for profilers and benchmarks: `events`
 * holds MOE_STAGE_EVENTS hipEvent_t handles created by the caller; they are
 * recorded on `stream` before routing, after routing, after the permutation,
 * after the gate||up GEMM, after the down GEMM and after the combine.  Any
 * entry may be NULL.  Same errors as moe_forward. */
#define MOE_STAGE_EVENTS 6
moe_status moe_forward_timed(const moe_layer *layer, const moe_tensor *x,
                             const moe_tensor *router_logits,
                             const moe_tensor *shared_output, moe_tensor *out,
                             void *workspace, size_t workspace_bytes,
                             moe_routing_out *routing, void *stream,
                             void *const *events);

/* Bytes of the static per-GPU workspace of moe_forward_noalloc. */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

/* moe_forward with no workspace argument and no device allocation, for the
 * callers that cannot allocate: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  The workspace is a static array of
 * MOE_NOALLOC_SCRATCH_BYTES (32 MiB) that the library holds on every GPU it
 * runs on until the process ends (the current device's copy is used).
 * Arguments and results are those of moe_forward without the workspace.
 *  - The layer must be prepared (moe_prepare, or one moe_forward since the
 *    last moe_set_weights): preparing allocates, so an unprepared layer is an
 *    INVALID_ARGUMENT error here.
 *  - The call must fit: moe_workspace_size(T) <= MOE_NOALLOC_SCRATCH_BYTES,
 *    else WORKSPACE (e.g. T = 32 at H 2048, I 768, E 128, K 8 needs < 3 MiB).
 *  - Every call on one GPU shares that GPU's array, which keeps the last
 *    call's contents: calls that overlap in time on one GPU (two host threads,
 *    or two streams with no ordering between them) race and give undefined
 *    results.  Calls ordered on one stream are safe.
 * Errors: as moe_forward. */
moe_status moe_forward_noalloc(const moe_layer *layer, const moe_tensor *x,
                               const moe_tensor *router_logits,
                               const moe_tensor *shared_output, moe_tensor *out,
                               moe_routing_out *routing, void *stream);

/* Routing and permutation alone (the first two steps of moe_forward):
 * router_logits [T, E] f32 -> `routing` (non-NULL; any member may be NULL).
 * Needs moe_workspace_size(T) bytes of workspace. */
moe_status moe_route(const moe_layer *layer, const moe_tensor *router_logits,
                     moe_routing_out *routing, void *workspace,
                     size_t workspace_bytes, void *stream);

/* Router logits alone (MoeSpec `wr`, `router_bias`): x [T, H] -> logits
 * [T, E] f32 = x . Wr + Br with f32 accumulation.  Needs router_weight bound
 * and moe_workspace_size(T) bytes of workspace.
 * Errors: INVALID_ARGUMENT, SHAPE_MISMATCH, UNBOUND, UNSUPPORTED, WORKSPACE, HIP. */
moe_status moe_router_logits(const moe_layer *layer, const moe_tensor *x, moe_tensor *logits,
                             void *workspace, size_t workspace_bytes, void *stream);

/* Release the handle (~QMoEWoQ).  Never frees caller buffers.  NULL is a no-op. */
moe_status moe_destroy(moe_layer *layer);

/* Message of the calling thread's last failed call ("" if none). */
const char *moe_last_error(void);

/* Static name of a status code. */
const char *moe_status_string(moe_status s);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
