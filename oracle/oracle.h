/*
 * oracle.h - plain, slow, single-threaded C reference for the routed
 * mixture-of-experts block.  TEST INFRASTRUCTURE ONLY: the tests, the smoke
 * check and the benchmark's CPU-baseline leg use it; the GPU library never
 * includes, links or calls it, and it includes nothing from the GPU library.
 *
 * Sources (cited by page title and section):
 *  [UDS]  "Understanding Dwarf Star" (ldazrz.com): 2.3.2 K-quant formats (the
 *         Q4_K block layout), the
 *         Q2_K subsection (printed as 3.3.3), 2.3.4 IQ2_XXS, 2.4 the
 *         quantize-by-role table, 2.8.1-2.8.2 dequantize-on-the-fly grouped
 *         dot, 5.2.1 layer structure (norm + residual), 5.2.4 FFN, 5.3.2 MoE
 *         formula, 5.3.4 shared expert, 5.3.5 routing, 5.3.7 the MoE kernel
 *         steps, 5.6.2 RMSNorm per layer.
 *  [SPE]  "The sparsity that pays for everything else in DwarfStar": "Where the
 *         parameters actually are" (shape and parameter arithmetic), "Quantize
 *         by role, not by tensor", "Some experts run far more often than
 *         others" (selection counts and the hot list).
 *  [RDM]  antirez/ds4 README mirror: the --batched-session paragraph
 *         ("batching is exact").
 * Where the pages are silent the oracle takes the readings listed in the design doc
 * (block byte orders, tie order, fp64 logits, the bf16 mode's one cast point).
 *
 * Everything here is computed in double precision; in bf16 mode the input x
 * is given as bf16 values and nothing else is rounded.
 */
#ifndef ORACLE_H
#define ORACLE_H
#include <stdint.h>

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_Q2K = 2, ORC_Q8_0 = 3, ORC_CB2 = 4, ORC_Q4K = 5 };

typedef struct {
    int32_t n_embd;        /* D */
    int32_t n_expert;      /* E */
    int32_t n_expert_used; /* k */
    int32_t n_ff_exp;      /* F */
    int32_t n_ff_shared;   /* Fs, 0 = no shared expert */
    int32_t gate_fmt, up_fmt, down_fmt, shared_fmt;
    const float *router_w;    /* [E][D]: row e = expert e's weights */
    const float *router_bias; /* [E] or NULL, added to the logits */
    double route_scale;       /* multiplies the renormalized weights */
    const uint8_t *gate, *up; /* [E][F][D] blocks */
    const uint8_t *down;      /* [E][D][F] blocks */
    const uint8_t *sh_gate, *sh_up, *sh_down; /* [Fs][D], [Fs][D], [D][Fs] */
    const int8_t *codebook;   /* [256][8] for CB2 */
} orc_layer;

/* Bytes of an n-weight tensor in a block format (-1 if n does not fill whole blocks). */
int64_t orc_tensor_bytes(int fmt, int64_t n_weights);
/* Decode n weights of a flattened block tensor to fp32. 0 on success. */
int orc_dequant(int fmt, const uint8_t *src, int64_t n_weights, const int8_t *codebook, float *out);
/* Router logits l[t][e] = sum_k x[t][k] W[e][k] (+ bias[e]) in double, ascending k. */
int orc_logits(const orc_layer *L, const double *x, int32_t T, double *logits);
/* Top-k by (logit desc, index asc); weights = route_scale * softmax over the k chosen logits.
 * gap_out[t] (optional) = l_(k) - l_(k+1), the margin that decided the set. */
int orc_topk(const double *logits, int32_t T, int32_t E, int32_t k, double route_scale, int32_t *idx,
             float *w, double *gap_out);
/* Stable bucketing of the T*k (token, slot) pairs by expert. */
int orc_bucket(const int32_t *idx, int32_t T, int32_t k, int32_t E, int32_t *count, int32_t *offset,
               int32_t *perm, int32_t *pos, int32_t *active, int32_t *n_active);
/* The block: y[t] = shared(x_t) + sum over chosen e of w_e * FFN_e(x_t).
 * mode ORC_F32: x_f32 used; ORC_BF16: x_bf16 (bf16 bits) used; everything
 * after the input is computed the same way in both modes (x's cast to bf16
 * is the only cast point of the bf16 workload).
 * Rows listed in rows[0..n_rows) (NULL = all T) are computed; y is [T][D]
 * and only those rows are written.  idx/w (optional, [T][k]) receive the routing. */
int orc_moe_forward(const orc_layer *L, int mode, const float *x_f32, const uint16_t *x_bf16, int32_t T,
                    const int32_t *rows, int32_t n_rows, float *y, int32_t *idx, float *w);
/* Same result by the plain definition: every expert's FFN on every token,
 * multiplied by the masked gate (zero off the top-k) and summed over all E. */
int orc_moe_forward_dense(const orc_layer *L, int mode, const float *x_f32, const uint16_t *x_bf16,
                          int32_t T, float *y);
/* out[t][i] = gamma[i] * x[t][i] / sqrt(mean_i x[t][i]^2 + eps). */
int orc_rmsnorm(const float *x, const float *gamma, double eps, int32_t T, int32_t D, float *out);
/* One SwiGLU FFN on one token (weights [F][D], [F][D], [D][F]); y[D] in double. */
int orc_swiglu(int fmt_gu, int fmt_down, const uint8_t *gate, const uint8_t *up, const uint8_t *down,
               const int8_t *cb, int32_t D, int32_t F, int mode, const double *x, double *y);
/* Expert selection counts and the hot list ([SPE] "Some experts run far
 * more often than others": a run counts expert selections per {layer,
 * expert}, merges them into an existing profile, sorts and writes the list).
 * counts[layer*E + e] += the number of pairs (t, s) with topk_idx[t*k+s] == e;
 * entries outside [0, E) are not counted. */
void orc_count_selections(const int32_t *topk_idx, int32_t T, int32_t k, int32_t E, int32_t layer, int64_t *counts);
/* order[0..n) = 0..n-1 sorted by counts descending, ties by index ascending
 * (counts clamped to [0, 2^39)); returns how many counts are positive. */
int32_t orc_hotlist(const int64_t *counts, int32_t n, int32_t *order);

const char *orc_version(void);

#endif
