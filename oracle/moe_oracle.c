/* CPU oracle for the mixture-of-experts FFN forward -- TEST INFRASTRUCTURE.
 *
 * Plain fp64 reference of the layer described by the documentation pages
 * (clika "MoE" / "ClikaRT::nn::QMoEWoQ", logicaffeine "MoeSpec" / "Moe",
 * graiphic ONNX "MoE").  Only tests/, the smoke check and the benchmark's
 * CPU-baseline leg may load it; the GPU library never does, and the two share
 * no code.  Built with gcc -O2 -ffp-contract=off (no fast-math), so every sum
 * below is a sequence of separately rounded fp64 multiplies and adds in the
 * order written.
 *
 * Inputs stored as bf16, f32 or MXFP4 are widened exactly to fp64; all
 * arithmetic is fp64.  Tokens are independent and are processed one at a time.
 */
#include "moe_oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ storage */

double orc_bf16_to_double(uint16_t bits)
{
    /* bf16 is the top half of an IEEE binary32: widening is exact. */
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* MXFP4 element (OCP Microscaling Formats v1.0: FP4 E2M1 element, E8M0 shared
 * scale).  Element bits s|e1 e0|m: exponent field 0 is subnormal (value
 * m * 0.5), otherwise 2^(e-1) * (1 + m/2).  Scale byte X means 2^(X-127);
 * 0xFF is NaN.  The QMoEWoQ page (class description) requires this to stay a
 * weight-only decode: the activation stays floating point. */
double orc_mxfp4_value(uint8_t code4, uint8_t scale_byte)
{
    int s = (code4 >> 3) & 1, e = (code4 >> 1) & 3, m = code4 & 1;
    double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    if (scale_byte == 0xFF)
        return NAN;
    double v = ldexp(mag, (int)scale_byte - 127);
    return s ? -v : v;
}

static double elem(int kind, const void *base, int64_t idx)
{
    if (kind == ORC_F32)
        return (double)((const float *)base)[idx];
    return orc_bf16_to_double(((const uint16_t *)base)[idx]);
}

/* Dot product of weight row `row` of a [rows, Kd] stack with the fp64 vector v,
 * accumulated left to right in fp64. */
static double dot_row(int kind, const void *base, const uint8_t *scales,
                      int64_t row, int64_t Kd, const double *v)
{
    double acc = 0.0;
    if (kind == ORC_F32) {
        const float *w = (const float *)base + row * Kd;
        for (int64_t k = 0; k < Kd; ++k)
            acc += (double)w[k] * v[k];
    } else if (kind == ORC_BF16) {
        const uint16_t *w = (const uint16_t *)base + row * Kd;
        for (int64_t k = 0; k < Kd; ++k)
            acc += orc_bf16_to_double(w[k]) * v[k];
    } else {
        const uint8_t *c = (const uint8_t *)base + row * (Kd / 2);
        const uint8_t *sc = scales + row * (Kd / 32);
        for (int64_t k = 0; k < Kd; ++k) {
            uint8_t byte = c[k / 2];
            uint8_t code = (k & 1) ? (byte >> 4) : (byte & 15);
            acc += orc_mxfp4_value(code, sc[k / 32]) * v[k];
        }
    }
    return acc;
}

/* Bytes of one [rows, Kd] weight matrix of the given kind (codes only for MXFP4). */
static int64_t mat_elems_bytes(int kind, int64_t rows, int64_t Kd)
{
    if (kind == ORC_F32) return rows * Kd * 4;
    if (kind == ORC_BF16) return rows * Kd * 2;
    return rows * (Kd / 2);
}

/* ------------------------------------------------------------------ routing */

/* Validation of the routing options: K of E experts (MoeSpec, "choosing K of
 * E"); the group limit splits the experts into equal groups (Moe, `groups`)
 * and must leave at least K eligible experts. */
static int check_params(const orc_params *p)
{
    if (p->E < 1 || p->K < 1 || p->K > p->E || p->H < 1 || p->I < 1 || p->T < 0)
        return -1;
    if (p->n_group > 0) {
        if (p->n_group > 1024 || p->E % p->n_group != 0) return -1;
        if (p->topk_group < 1 || p->topk_group > p->n_group) return -1;
        if (p->K > (int64_t)p->topk_group * (p->E / p->n_group)) return -1;
    }
    if (p->w_kind == ORC_MXFP4 && (p->H % 32 != 0 || p->I % 32 != 0))
        return -1;
    if (p->activation < ORC_SILU_GATED || p->activation > ORC_IDENTITY) return -1;
    if (p->gelu_mode != ORC_GELU_ERF && p->gelu_mode != ORC_GELU_TANH) return -1;
    return 0;
}

/* Gated activations read a gate and an up projection; the others one fc1
 * projection (ONNX MoE: fusion_size 2 for fused swiglu, 1 otherwise). */
static int is_gated(const orc_params *p)
{
    return p->activation == ORC_SILU_GATED || p->activation == ORC_SWIGLU_CLAMPED;
}

/* Route one token.
 *  1. Score (MoeSpec `score`): softmax over every logit, or each logit's own
 *     sigmoid.
 *  2. Selection key (MoeSpec `selection_bias`): score plus B[e]; the weight
 *     later uses the score alone.
 *  3. Group limit (MoeSpec `groups`, Moe `groups`): experts split into
 *     n_group equal contiguous groups; a group is scored by the sum of its two
 *     best keys; only experts of the topk_group best groups stay eligible.
 *  4. Top-K (MoeSpec, "choosing K of E"; ONNX MoE `k`): the K largest keys
 *     among eligible experts, in rank order; equal keys go to the lower index.
 *  5. Weights: the kept experts' scores; renormalised to sum to one when asked
 *     (MoeSpec `renormalize`, Moe `norm_top_k`) with the renormalising sum
 *     clamped below at 2^-14 (MoeSpec `sum_can_clamp`); then every weight
 *     times the routed scale S, after the renormalisation (MoeSpec `scale`,
 *     S = 1 when absent).
 */
static void route_token(const orc_params *p, const float *l, const float *b,
                        int32_t *ids, double *w, double *score, double *key)
{
    const int64_t E = p->E, K = p->K;

    /* 1. scores */
    if (p->scoring == ORC_SOFTMAX) {
        double m = -INFINITY;
        for (int64_t e = 0; e < E; ++e)
            if ((double)l[e] > m) m = (double)l[e];
        double sum = 0.0;
        for (int64_t e = 0; e < E; ++e) {
            score[e] = exp((double)l[e] - m);
            sum += score[e];
        }
        for (int64_t e = 0; e < E; ++e)
            score[e] = score[e] / sum;
    } else {
        for (int64_t e = 0; e < E; ++e)
            score[e] = 1.0 / (1.0 + exp(-(double)l[e]));
    }

    /* 2. selection keys */
    for (int64_t e = 0; e < E; ++e)
        key[e] = b ? score[e] + (double)b[e] : score[e];

    /* 3. group limit */
    if (p->n_group > 0) {
        const int64_t G = p->n_group, gs = E / G;
        double gscore[1024];
        int keep[1024];
        for (int64_t g = 0; g < G; ++g) {
            /* sum of the best min(2, gs) keys of the group */
            double best1 = -INFINITY, best2 = -INFINITY;
            for (int64_t e = g * gs; e < (g + 1) * gs; ++e) {
                if (key[e] > best1) { best2 = best1; best1 = key[e]; }
                else if (key[e] > best2) { best2 = key[e]; }
            }
            gscore[g] = (gs >= 2) ? best1 + best2 : best1;
            keep[g] = 0;
        }
        for (int64_t r = 0; r < p->topk_group; ++r) {
            int64_t bestg = -1;
            for (int64_t g = 0; g < G; ++g)
                if (!keep[g] && (bestg < 0 || gscore[g] > gscore[bestg]))
                    bestg = g;
            keep[bestg] = 1;
        }
        for (int64_t e = 0; e < E; ++e)
            if (!keep[e / gs]) key[e] = -INFINITY;
    }

    /* 4. top-K by (key descending, index ascending) among eligible experts */
    for (int64_t j = 0; j < K; ++j) {
        int64_t best = -1;
        for (int64_t e = 0; e < E; ++e) {
            if (key[e] == -INFINITY) continue;       /* ineligible */
            int taken = 0;
            for (int64_t i = 0; i < j; ++i)
                if (ids[i] == e) { taken = 1; break; }
            if (taken) continue;
            if (best < 0 || key[e] > key[best]) best = e;
        }
        ids[j] = (int32_t)best;
    }

    /* 5. weights */
    for (int64_t j = 0; j < K; ++j)
        w[j] = score[ids[j]];
    if (p->renormalize) {
        double sum = 0.0;
        for (int64_t j = 0; j < K; ++j) sum += w[j];
        const double floor_ = ldexp(1.0, -14);
        double d = sum > floor_ ? sum : floor_;
        for (int64_t j = 0; j < K; ++j) w[j] = w[j] / d;
    }
    for (int64_t j = 0; j < K; ++j)
        w[j] = w[j] * p->routed_scaling_factor;
}

int orc_route(const orc_params *p, const float *logits, const float *sel_bias,
              int32_t *ids, double *weights, double *scores, double *keys)
{
    if (check_params(p)) return -1;
    const int64_t E = p->E, K = p->K;
    double *sc = (double *)malloc(sizeof(double) * E);
    double *ky = (double *)malloc(sizeof(double) * E);
    for (int64_t t = 0; t < p->T; ++t) {
        route_token(p, logits + t * E, sel_bias, ids + t * K, weights + t * K, sc, ky);
        if (scores) memcpy(scores + t * E, sc, sizeof(double) * E);
        if (keys) memcpy(keys + t * E, ky, sizeof(double) * E);
    }
    free(sc);
    free(ky);
    return 0;
}

/* -------------------------------------------------------------- permutation */

/* Rows grouped by expert so that each expert's kernel runs on its own tokens
 * (QMoEWoQ, "decode inside the per-expert kernels").  Within an expert the
 * rows follow increasing token index; a token never holds one expert twice. */
void orc_permute(const orc_params *p, const int32_t *ids, int32_t *counts,
                 int32_t *offsets, int32_t *row_token, int32_t *slot_row)
{
    const int64_t T = p->T, E = p->E, K = p->K;
    for (int64_t e = 0; e < E; ++e) counts[e] = 0;
    for (int64_t i = 0; i < T * K; ++i) counts[ids[i]] += 1;
    offsets[0] = 0;
    for (int64_t e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
    int32_t *fill = (int32_t *)calloc((size_t)E, sizeof(int32_t));
    for (int64_t t = 0; t < T; ++t)
        for (int64_t j = 0; j < K; ++j) {
            int32_t e = ids[t * K + j];
            int32_t row = offsets[e] + fill[e]++;
            row_token[row] = (int32_t)t;
            slot_row[t * K + j] = row;
        }
    free(fill);
}

/* ------------------------------------------------------------------- expert */

/* Gated activation (ONNX MoE `activation_type` silu/swiglu with
 * `activation_alpha`, `activation_beta`, `swiglu_limit`; clika MoE options
 * `swiglu_alpha/beta/limit`).
 *   SiLU-gated:    h = silu(g) * u,  silu(g) = g * sigmoid(g).
 *   clamped SwiGLU: with L = limit > 0, g <- min(g, L), u <- clamp(u, -L, L);
 *                  h = g * sigmoid(alpha * g) * (u + beta).  L <= 0: no clamp.
 * The pages name the parameters and their defaults (alpha 1, beta 0, limit 0
 * = no clamp) but print no formula; the clamped form is read as the published
 * gpt-oss activation, which at (1, 0, no clamp) is exactly SiLU-gated.
 * Parity unpinned for alpha != 1, beta != 0 or an active clamp. */
double orc_activation(const orc_params *p, double g, double u)
{
    if (p->activation == ORC_SILU_GATED)
        return g * (1.0 / (1.0 + exp(-g))) * u;
    double L = p->limit;
    if (L > 0.0) {
        if (g > L) g = L;
        if (u > L) u = L;
        if (u < -L) u = -L;
    }
    return g * (1.0 / (1.0 + exp(-p->alpha * g))) * (u + p->beta);
}

/* Activation of a non-gated expert (ONNX MoE `activation_type` relu, gelu,
 * silu, identity on the fc1 output; clika MoE option `gelu_mode`):
 *   relu(v) = max(v, 0);  silu(v) = v * sigmoid(v);  identity(v) = v;
 *   gelu(v) = v * Phi(v) with Phi the standard normal CDF,
 *             Phi(v) = (1 + erf(v / sqrt 2)) / 2            (gelu_mode erf),
 *   or its tanh approximation
 *             (1 + tanh(sqrt(2/pi) (v + 0.044715 v^3))) / 2  (gelu_mode tanh).
 * The pages name gelu_mode without printing either form; both are the
 * published GELU definitions. */
double orc_activation1(const orc_params *p, double v)
{
    switch (p->activation) {
    case ORC_RELU: return v > 0.0 ? v : 0.0;
    case ORC_SILU: return v * (1.0 / (1.0 + exp(-v)));
    case ORC_IDENTITY: return v;
    case ORC_GELU:
        if (p->gelu_mode == ORC_GELU_TANH) {
            const double c = sqrt(2.0 / acos(-1.0));
            return 0.5 * v * (1.0 + tanh(c * (v + 0.044715 * v * v * v)));
        }
        return 0.5 * v * (1.0 + erf(v / sqrt(2.0)));
    default: return NAN;
    }
}

/* Router logits (MoeSpec `wr`, `router_bias`: wr[(t-1)E + e] indexes a
 * [d, E] matrix; the bias is added to each logit before scoring):
 * l[e] = sum_c x[c] * Wr[c, e] + Br[e], in fp64. */
static void router_logits_token(const orc_params *p, const orc_inputs *in, const double *xv,
                                double *l)
{
    const int64_t H = p->H, E = p->E;
    for (int64_t e = 0; e < E; ++e) {
        double v = 0.0;
        for (int64_t c = 0; c < H; ++c)
            v += xv[c] * elem(p->x_kind, in->router_w, c * E + e);
        if (in->router_b) v += elem(p->x_kind, in->router_b, e);
        l[e] = v;
    }
}

int orc_router_logits(const orc_params *p, const orc_inputs *in, double *logits)
{
    if (check_params(p) || !in->router_w) return -1;
    const int64_t H = p->H, E = p->E;
    double *xv = (double *)malloc(sizeof(double) * H);
    for (int64_t t = 0; t < p->T; ++t) {
        for (int64_t c = 0; c < H; ++c)
            xv[c] = elem(p->x_kind, in->x, t * H + c);
        router_logits_token(p, in, xv, logits + t * E);
    }
    free(xv);
    return 0;
}

typedef struct {
    const orc_params *p;
    const orc_inputs *in;
    int64_t n;
    const int64_t *tokens;
    double *out;
    int32_t *ids;
    double *weights;
    double *h, *y;
    int tid, nthreads;
} job_t;

/* One token: route, run each kept expert's gated FFN, combine under the
 * router weights (clika MoE: "the outputs combine under the router weights";
 * MoeSpec: `out` is the tensor the weighted accumulation writes), and fold the
 * optional shared-expert output into the same sum (QMoEWoQ::forward). */
/*
 * With a bound router the token's logits are x . Wr + Br, rounded to f32 (the
 * precision in which they are stored and the discrete choices are taken).
 * Weigh-inputs routing (MoeSpec `weigh_inputs`, Llama 4; clika MoE option
 * apply_router_weight_on_input): expert j reads w_j * x and its output joins
 * the sum with weight one.
 */
static void token_forward(const orc_params *p, const orc_inputs *in, int64_t t,
                          double *out, int32_t *ids, double *w, double *hdump,
                          double *ydump, double *x0, double *hv, double *yv,
                          double *sc, double *ky, double *xv, float *lf, double *ld)
{
    const int64_t H = p->H, I = p->I, E = p->E, K = p->K;
    const int gated = is_gated(p);
    const int fused = gated && p->layout != ORC_UNFUSED;
    const int64_t gu_rows = fused ? 2 * I : I;

    for (int64_t c = 0; c < H; ++c)
        x0[c] = elem(p->x_kind, in->x, t * H + c);
    const float *lt = in->logits ? in->logits + t * E : NULL;
    if (in->router_w) {
        router_logits_token(p, in, x0, ld);
        for (int64_t e = 0; e < E; ++e) lf[e] = (float)ld[e];
        lt = lf;
    }
    route_token(p, lt, in->sel_bias, ids, w, sc, ky);

    for (int64_t c = 0; c < H; ++c)
        out[c] = 0.0;

    for (int64_t j = 0; j < K; ++j) {
        const int64_t e = ids[j];
        const double xs = p->weigh_inputs ? w[j] : 1.0;     /* input scale  */
        const double ws = p->weigh_inputs ? 1.0 : w[j];     /* output weight */
        for (int64_t c = 0; c < H; ++c)
            xv[c] = xs * x0[c];
        /* expert e's slabs */
        const char *gu = (const char *)in->w_gu + e * mat_elems_bytes(p->w_kind, gu_rows, H);
        const uint8_t *gus = in->w_gu_scales ? in->w_gu_scales + e * gu_rows * (H / 32) : NULL;
        const char *gt = in->w_gate ? (const char *)in->w_gate + e * mat_elems_bytes(p->w_kind, I, H) : NULL;
        const uint8_t *gts = in->w_gate_scales ? in->w_gate_scales + e * I * (H / 32) : NULL;
        const char *dn = (const char *)in->w_down + e * mat_elems_bytes(p->w_kind, H, I);
        const uint8_t *dns = in->w_down_scales ? in->w_down_scales + e * H * (I / 32) : NULL;

        for (int64_t o = 0; o < I && !gated; ++o) {
            /* non-gated: one fc1 row per feature ([E, I, H], bias [E, I]) */
            double v = dot_row(p->w_kind, gu, gus, o, H, xv);
            if (in->b_gu) v += elem(p->x_kind, in->b_gu, e * I + o);
            hv[o] = orc_activation1(p, v);
        }
        for (int64_t o = 0; o < I && gated; ++o) {
            /* gate/up rows per ONNX MoE `swiglu_fusion`: 2 = fused, not
             * interleaved (gate rows [0,I), up rows [I,2I)); 1 = fused,
             * interleaved (gate 2o, up 2o+1); 0 = not fused (gate stack and
             * up stack separate). */
            double g, u;
            if (p->layout == ORC_SPLIT) {
                g = dot_row(p->w_kind, gu, gus, o, H, xv);
                u = dot_row(p->w_kind, gu, gus, I + o, H, xv);
                if (in->b_gu) {
                    g += elem(p->x_kind, in->b_gu, e * 2 * I + o);
                    u += elem(p->x_kind, in->b_gu, e * 2 * I + I + o);
                }
            } else if (p->layout == ORC_INTERLEAVED) {
                g = dot_row(p->w_kind, gu, gus, 2 * o, H, xv);
                u = dot_row(p->w_kind, gu, gus, 2 * o + 1, H, xv);
                if (in->b_gu) {
                    g += elem(p->x_kind, in->b_gu, e * 2 * I + 2 * o);
                    u += elem(p->x_kind, in->b_gu, e * 2 * I + 2 * o + 1);
                }
            } else {
                g = dot_row(p->w_kind, gt, gts, o, H, xv);
                u = dot_row(p->w_kind, gu, gus, o, H, xv);
                if (in->b_gate) g += elem(p->x_kind, in->b_gate, e * I + o);
                if (in->b_gu) u += elem(p->x_kind, in->b_gu, e * I + o);
            }
            hv[o] = orc_activation(p, g, u);
        }
        /* down projection (ONNX MoE fc2 [E, H, I] plus bias [E, H]) */
        for (int64_t c = 0; c < H; ++c) {
            double v = dot_row(p->w_kind, dn, dns, c, I, hv);
            if (in->b_down) v += elem(p->x_kind, in->b_down, e * H + c);
            yv[c] = v;
        }
        for (int64_t c = 0; c < H; ++c)
            out[c] += ws * yv[c];
        if (hdump) memcpy(hdump + j * I, hv, sizeof(double) * I);
        if (ydump) memcpy(ydump + j * H, yv, sizeof(double) * H);
    }
    if (in->shared_output) {
        /* logicaffeine "Moe" field `shared_gate`: the shared experts' output
         * enters scaled by the logistic sigmoid of x . g (g a vector over the
         * hidden features; the unscaled x, not a weigh-inputs copy) */
        double sg = 1.0;
        if (in->shared_gate) {
            double d = 0.0;
            for (int64_t c = 0; c < H; ++c)
                d += x0[c] * elem(p->x_kind, in->shared_gate, c);
            sg = 1.0 / (1.0 + exp(-d));
        }
        for (int64_t c = 0; c < H; ++c)
            out[c] += sg * elem(p->x_kind, in->shared_output, t * H + c);
    }
}

static void *worker(void *arg)
{
    job_t *jb = (job_t *)arg;
    const orc_params *p = jb->p;
    const int64_t H = p->H, I = p->I, K = p->K, E = p->E;
    double *x0 = (double *)malloc(sizeof(double) * H);
    double *xv = (double *)malloc(sizeof(double) * H);
    double *hv = (double *)malloc(sizeof(double) * I);
    double *yv = (double *)malloc(sizeof(double) * H);
    double *sc = (double *)malloc(sizeof(double) * E);
    double *ky = (double *)malloc(sizeof(double) * E);
    double *ld = (double *)malloc(sizeof(double) * E);
    float *lf = (float *)malloc(sizeof(float) * E);
    for (int64_t i = jb->tid; i < jb->n; i += jb->nthreads) {
        int64_t t = jb->tokens ? jb->tokens[i] : i;
        token_forward(p, jb->in, t, jb->out + i * H, jb->ids + i * K,
                      jb->weights + i * K, jb->h ? jb->h + i * K * I : NULL,
                      jb->y ? jb->y + i * K * H : NULL, x0, hv, yv, sc, ky, xv, lf, ld);
    }
    free(x0); free(xv); free(hv); free(yv); free(sc); free(ky); free(ld); free(lf);
    return NULL;
}

int orc_forward(const orc_params *p, const orc_inputs *in, int64_t n,
                const int64_t *tokens, int n_threads, double *out,
                int32_t *ids, double *weights, double *h, double *y)
{
    if (check_params(p)) return -1;
    const int two_stacks = is_gated(p) && p->layout == ORC_UNFUSED;
    if (two_stacks && !in->w_gate) return -1;
    if (p->w_kind == ORC_MXFP4 && (!in->w_gu_scales || !in->w_down_scales ||
                                   (two_stacks && !in->w_gate_scales)))
        return -1;
    if (!in->logits && !in->router_w) return -1;
    if (tokens)
        for (int64_t i = 0; i < n; ++i)
            if (tokens[i] < 0 || tokens[i] >= p->T) return -1;
    if (n_threads < 1) n_threads = 1;
    if (n_threads > 256) n_threads = 256;
    pthread_t th[256];
    job_t jobs[256];
    for (int i = 0; i < n_threads; ++i) {
        jobs[i] = (job_t){p, in, n, tokens, out, ids, weights, h, y, i, n_threads};
        pthread_create(&th[i], NULL, worker, &jobs[i]);
    }
    for (int i = 0; i < n_threads; ++i)
        pthread_join(th[i], NULL);
    return 0;
}
