/* CPU oracle for the mixture-of-experts FFN forward -- TEST INFRASTRUCTURE.
 *
 * A plain, slow, fp64 implementation of what the layer computes, written from
 * the documentation pages (clika "MoE" and "ClikaRT::nn::QMoEWoQ",
 * logicaffeine "MoeSpec" and "Moe", graiphic ONNX "MoE").  Only the test
 * suite, the smoke check and the benchmark's CPU-baseline leg may load it.
 * It shares no code, header or table with the GPU library.
 *
 * Parity status per function (details beside each definition):
 *   routing (scores, selection bias, group limit, top-k, weights) -- pinned
 *   permutation                                                   -- pinned
 *   SiLU-gated expert FFN, combine, shared-output fold            -- pinned
 *   clamped SwiGLU (alpha, beta, limit)                           -- parity
 *       unpinned beyond its reduction to SiLU-gated at (1, 0, no clamp):
 *       the pages name the three parameters but print no formula.
 *   MXFP4 decode                                                  -- pinned to
 *       the OCP MX v1.0 e2m1 / e8m0 tables (public spec, not the pages).
 *   non-gated activations relu / gelu / silu / identity           -- pinned
 *       (closed forms, tabulated normal CDF, linear-FFN reduction); the tanh
 *       form of gelu is pinned only by its identities and its distance to
 *       the erf form (the pages name gelu_mode but print neither form).
 *   weigh-inputs routing                                          -- pinned
 *   router logits x . Wr + Br                                     -- pinned
 *   shared-expert gate sigmoid(x . g) on the shared-output fold    -- pinned
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_MXFP4 = 2 };                 /* storage kinds   */
enum { ORC_UNFUSED = 0, ORC_INTERLEAVED = 1, ORC_SPLIT = 2 };       /* swiglu_fusion   */
enum { ORC_SOFTMAX = 0, ORC_SIGMOID = 1 };                          /* scoring         */
enum { ORC_SILU_GATED = 0, ORC_SWIGLU_CLAMPED = 1,                 /* gated (fc1||fc3) */
       ORC_RELU = 2, ORC_GELU = 3, ORC_SILU = 4, ORC_IDENTITY = 5 }; /* one fc1 stack   */
enum { ORC_GELU_ERF = 0, ORC_GELU_TANH = 1 };                       /* gelu_mode       */

typedef struct {
    int64_t T, H, I, E, K;
    int32_t x_kind;          /* ORC_F32 or ORC_BF16: x, biases, shared_output */
    int32_t w_kind;          /* ORC_F32, ORC_BF16 or ORC_MXFP4                */
    int32_t layout;          /* ORC_UNFUSED / ORC_INTERLEAVED / ORC_SPLIT     */
    int32_t scoring;         /* ORC_SOFTMAX / ORC_SIGMOID                     */
    int32_t renormalize;
    int32_t n_group;         /* 0 = no group limit                           */
    int32_t topk_group;
    int32_t activation;      /* ORC_SILU_GATED ... ORC_IDENTITY               */
    double routed_scaling_factor;
    double alpha, beta, limit;
    int32_t gelu_mode;       /* ORC_GELU_ERF / ORC_GELU_TANH                  */
    int32_t weigh_inputs;    /* kept weight scales the expert's input; the
                                outputs then sum unweighted                   */
} orc_params;

typedef struct {
    const void *x;              /* [T,H] x_kind                                  */
    const float *logits;        /* [T,E]                                         */
    const void *w_gu;           /* fused [E,2I,H]; unfused: up rows [E,I,H]      */
    const uint8_t *w_gu_scales; /* MXFP4 only: [E,rows,H/32]                      */
    const void *w_gate;         /* unfused only: gate rows [E,I,H]               */
    const uint8_t *w_gate_scales;
    const void *w_down;         /* [E,H,I]                                       */
    const uint8_t *w_down_scales;
    const void *b_gu;           /* fused [E,2I]; unfused: up bias [E,I]; nullable */
    const void *b_gate;         /* unfused gate bias [E,I]; nullable             */
    const void *b_down;         /* [E,H]; nullable                               */
    const float *sel_bias;      /* [E] selection bias; nullable                  */
    const void *shared_output;  /* [T,H] x_kind; nullable                        */
    const void *router_w;       /* [H,E] x_kind; when set, logits = x.Wr (+Br)
                                   and `logits` is not read                      */
    const void *router_b;       /* [E] x_kind; nullable                          */
    const void *shared_gate;    /* [H] x_kind; nullable: with shared_output, the
                                   fold is scaled by sigmoid(x . g)             */
} orc_inputs;

/* Routing for every token: ids [T,K] in rank order, weights [T,K] (fp64),
 * optionally the fp64 scores [T,E] and selection keys [T,E] (-inf where a
 * group limit made the expert ineligible).  Returns 0, or -1 on bad options. */
int orc_route(const orc_params *p, const float *logits, const float *sel_bias,
              int32_t *ids, double *weights, double *scores, double *keys);

/* Expert-contiguous permutation of the (token, slot) pairs: counts [E],
 * offsets [E+1] (exclusive scan), row_token [T*K] (token of each row),
 * slot_row [T*K] (row of each (t, j) pair). */
void orc_permute(const orc_params *p, const int32_t *ids, int32_t *counts,
                 int32_t *offsets, int32_t *row_token, int32_t *slot_row);

/* Full forward on a subset of tokens (tokens == NULL: all T in order).
 * out [n,H] fp64; ids/weights [n,K] for those tokens; h [n,K,I] and y [n,K,H]
 * are optional per-slot stage dumps (activation output and down projection
 * plus bias).  Work is spread over n_threads POSIX threads.  Returns 0 or -1. */
int orc_forward(const orc_params *p, const orc_inputs *in, int64_t n,
                const int64_t *tokens, int n_threads, double *out,
                int32_t *ids, double *weights, double *h, double *y);

/* Router logits of every token, fp64 [T,E]: x . Wr + Br (needs router_w). */
int orc_router_logits(const orc_params *p, const orc_inputs *in, double *logits);

/* Helpers exposed for the pins. */
double orc_activation1(const orc_params *p, double v);
double orc_mxfp4_value(uint8_t code4, uint8_t scale_byte);
double orc_activation(const orc_params *p, double g, double u);
double orc_bf16_to_double(uint16_t bits);

#ifdef __cplusplus
}
#endif
#endif
