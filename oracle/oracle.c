/*
 * oracle.c - plain, slow, single-threaded reference of the routed
 * mixture-of-experts block.  TEST INFRASTRUCTURE ONLY (tests, smoke check,
 * CPU-baseline leg of the benchmark).  Shares no code with the GPU library.
 * Build: gcc -O2 -ffp-contract=off (no fast-math), see oracle/build.py.
 *
 * Each function names the passage it follows; "[UDS]" is the page
 * "Understanding Dwarf Star", "[SPE]" the page "The sparsity that pays for
 * everything else in DwarfStar", "[RDM]" the antirez/ds4 README mirror.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ---- scalar helpers ------------------------------------------------------ */

/* IEEE binary16 -> double, exactly ([UDS] 2.3.1: F16 is a 2-byte float). */
static double orc_half(const uint8_t *p) {
    unsigned h = (unsigned)p[0] | ((unsigned)p[1] << 8);
    int sign = (h >> 15) & 1, e = (h >> 10) & 31, m = h & 1023;
    double v;
    if (e == 0) v = ldexp((double)m, -24);
    else if (e == 31) v = m ? NAN : INFINITY;
    else v = ldexp((double)(1024 + m), e - 25);
    return sign ? -v : v;
}

/* bfloat16 bits -> double, exactly ([UDS] 2.3.1: BF16 keeps fp32's exponent). */
static double orc_bf16(uint16_t b) {
    uint32_t bits = (uint32_t)b << 16;
    float f;
    memcpy(&f, &bits, 4);
    return (double)f;
}

/* silu(z) = z * sigmoid(z), the gate activation of SwiGLU ([UDS] 5.2.4). */
static double orc_silu(double z) { return z / (1.0 + exp(-z)); }

/* ---- block formats ([UDS] 2.3.2-2.3.4; byte orders are this project's) -- */

static int orc_block_weights(int fmt) {
    return fmt == ORC_Q8_0 ? 32 : (fmt == ORC_Q2K || fmt == ORC_CB2 || fmt == ORC_Q4K) ? 256 : 0;
}
static int orc_block_bytes(int fmt) {
    return fmt == ORC_Q2K ? 84 : fmt == ORC_Q8_0 ? 34 : fmt == ORC_CB2 ? 66 : fmt == ORC_Q4K ? 144 : 0;
}

int64_t orc_tensor_bytes(int fmt, int64_t n) {
    int bw = orc_block_weights(fmt);
    if (bw == 0 || n < 0 || n % bw) return -1;
    return n / bw * orc_block_bytes(fmt);
}

/* Q2_K super-block ([UDS] Q2_K subsection): 256 weights in 16 groups of 16,
 * fp16 d and dmin, a 4-bit scale and a 4-bit min per group, 2-bit codes.
 * Weight value: d * scale_g * q - dmin * min_g. */
static void orc_block_q2k(const uint8_t *b, float *w) {
    double d = orc_half(b), dmin = orc_half(b + 2);
    for (int i = 0; i < 256; ++i) {
        int g = i / 16;
        int sc = b[4 + g] & 15, mn = b[4 + g] >> 4;
        int q = (b[20 + i / 4] >> (2 * (i % 4))) & 3;
        w[i] = (float)(d * sc * q - dmin * mn);
    }
}

/* Q4_K super-block ([UDS] 2.3.2, the Q4_K layout): 256 weights in 8 sub-blocks
 * of 32, fp16 d @0 and dmin @2, a 6-bit scale and a 6-bit min per sub-block
 * packed into the 12 bytes @4, 4-bit codes @16.  The pages leave the packing
 * order open: field f (scale of sub-block f for f < 8, min of sub-block f-8
 * after) takes bits 6f..6f+5 of the 12 bytes read as one little-endian
 * integer, and weight i's code takes bits 4*(i%2) of byte i/2.
 * Weight value: d * scale_j * q - dmin * min_j. */
static int orc_q4k_field(const uint8_t *p12, int f) {
    int v = 0;
    for (int b = 0; b < 6; ++b) {
        int bit = 6 * f + b;
        v |= ((p12[bit / 8] >> (bit % 8)) & 1) << b;
    }
    return v;
}
static void orc_block_q4k(const uint8_t *b, float *w) {
    double d = orc_half(b), dmin = orc_half(b + 2);
    for (int i = 0; i < 256; ++i) {
        int j = i / 32;
        int sc = orc_q4k_field(b + 4, j), mn = orc_q4k_field(b + 4, 8 + j);
        int q = (b[16 + i / 2] >> (4 * (i % 2))) & 15;
        w[i] = (float)(d * sc * q - dmin * mn);
    }
}

/* Q8_0 block ([UDS] 2.4 table: 8-bit shared expert; layout 32 int8 + fp16 scale). */
static void orc_block_q8_0(const uint8_t *b, float *w) {
    double d = orc_half(b);
    for (int i = 0; i < 32; ++i) w[i] = (float)(d * (double)(int8_t)b[2 + i]);
}

/* 2.0625-bpw codebook block ([UDS] 2.3.4: 66 bytes per 256 weights, codebook
 * lookup): fp16 scale, one 8-bit codebook row per 8 weights, one sign mask per
 * 8 weights.  Weight value: d * (+/-) codebook[idx][j]. */
static void orc_block_cb2(const uint8_t *b, const int8_t *cb, float *w) {
    double d = orc_half(b);
    for (int i = 0; i < 256; ++i) {
        int g = i / 8, j = i % 8;
        int c = cb[8 * b[2 + g] + j];
        if ((b[34 + g] >> j) & 1) c = -c;
        w[i] = (float)(d * (double)c);
    }
}

static void orc_block(int fmt, const uint8_t *b, const int8_t *cb, float *w) {
    if (fmt == ORC_Q2K) orc_block_q2k(b, w);
    else if (fmt == ORC_Q4K) orc_block_q4k(b, w);
    else if (fmt == ORC_Q8_0) orc_block_q8_0(b, w);
    else orc_block_cb2(b, cb, w);
}

/* Decode weights [first, first+n) of a flattened block tensor ([UDS] 2.8.2
 * steps 1-3: load a block, its scales, dequantize). */
static int orc_dequant_range(int fmt, const uint8_t *src, int64_t first, int64_t n, const int8_t *cb,
                             float *out) {
    int bw = orc_block_weights(fmt), bb = orc_block_bytes(fmt);
    if (bw == 0 || (fmt == ORC_CB2 && !cb)) return -1;
    float tmp[256];
    int64_t i = 0;
    while (i < n) {
        int64_t e = first + i, blk = e / bw, off = e % bw;
        orc_block(fmt, src + blk * bb, cb, tmp);
        int64_t take = bw - off < n - i ? bw - off : n - i;
        memcpy(out + i, tmp + off, (size_t)take * sizeof(float));
        i += take;
    }
    return 0;
}

int orc_dequant(int fmt, const uint8_t *src, int64_t n, const int8_t *cb, float *out) {
    if (orc_tensor_bytes(fmt, n) < 0) return -1;
    return orc_dequant_range(fmt, src, 0, n, cb, out);
}

/* ---- routing ([UDS] 5.3.2, 5.3.5, 5.3.7 step 1) ------------------------- */

/* router(x) starts from the logits x * W_router ([UDS] 5.3.2); W_router is
 * stored expert-major, row e = the D weights of expert e. */
int orc_logits(const orc_layer *L, const double *x, int32_t T, double *logits) {
    int32_t D = L->n_embd, E = L->n_expert;
    for (int32_t t = 0; t < T; ++t)
        for (int32_t e = 0; e < E; ++e) {
            double s = 0.0;
            for (int32_t k = 0; k < D; ++k) s += x[(int64_t)t * D + k] * (double)L->router_w[(int64_t)e * D + k];
            if (L->router_bias) s += (double)L->router_bias[e];
            logits[(int64_t)t * E + e] = s;
        }
    return 0;
}

/* The comparator's keys, one pointer per calling thread, so that several
 * threads may run the oracle at once on different rows. */
static _Thread_local const double *orc_sort_keys;
static int orc_cmp_desc(const void *a, const void *b) {
    int32_t i = *(const int32_t *)a, j = *(const int32_t *)b;
    double li = orc_sort_keys[i], lj = orc_sort_keys[j];
    if (li > lj) return -1;
    if (li < lj) return 1;
    return (i > j) - (i < j); /* equal logits: lower expert index first */
}

/* top-k of softmax(x W) = top-k of the logits (softmax is monotone); the k
 * chosen probabilities renormalized, i.e. a softmax over the chosen logits
 * ([UDS] 5.3.2 MoE(x) = sum over top-k of router(x)_i expert_i(x)). */
int orc_topk(const double *logits, int32_t T, int32_t E, int32_t k, double route_scale, int32_t *idx,
             float *w, double *gap_out) {
    if (k < 1 || k > E) return -1;
    int32_t *order = (int32_t *)malloc(sizeof(int32_t) * (size_t)E);
    if (!order) return -1;
    for (int32_t t = 0; t < T; ++t) {
        const double *l = logits + (int64_t)t * E;
        for (int32_t e = 0; e < E; ++e) order[e] = e;
        orc_sort_keys = l;
        qsort(order, (size_t)E, sizeof(int32_t), orc_cmp_desc);
        double mx = l[order[0]], den = 0.0;
        for (int32_t s = 0; s < k; ++s) den += exp(l[order[s]] - mx);
        for (int32_t s = 0; s < k; ++s) {
            idx[(int64_t)t * k + s] = order[s];
            w[(int64_t)t * k + s] = (float)(route_scale * exp(l[order[s]] - mx) / den);
        }
        if (gap_out) gap_out[t] = k < E ? l[order[k - 1]] - l[order[k]] : INFINITY;
    }
    free(order);
    return 0;
}

/* Group the (token, slot) pairs by expert so each chosen expert's rows are
 * contiguous ([UDS] 5.3.7: gather only the selected experts).  A counting sort
 * in ascending pair id, hence stable. */
int orc_bucket(const int32_t *idx, int32_t T, int32_t k, int32_t E, int32_t *count, int32_t *offset,
               int32_t *perm, int32_t *pos, int32_t *active, int32_t *n_active) {
    if (T < 0 || k < 1 || E < 1) return -1;
    int64_t P = (int64_t)T * k;
    for (int32_t e = 0; e < E; ++e) count[e] = 0;
    for (int64_t p = 0; p < P; ++p) {
        if (idx[p] < 0 || idx[p] >= E) return -1;
        count[idx[p]]++;
    }
    offset[0] = 0;
    for (int32_t e = 0; e < E; ++e) offset[e + 1] = offset[e] + count[e];
    int32_t *fill = (int32_t *)calloc((size_t)E, sizeof(int32_t));
    if (!fill) return -1;
    for (int64_t p = 0; p < P; ++p) {
        int32_t e = idx[p];
        int32_t at = offset[e] + fill[e]++;
        perm[at] = (int32_t)p;
        pos[p] = at;
    }
    free(fill);
    int32_t na = 0;
    for (int32_t e = 0; e < E; ++e)
        if (count[e] > 0) active[na++] = e;
    for (int32_t i = na; i < E; ++i) active[i] = -1;
    *n_active = na;
    return 0;
}

/* ---- expert FFN ([UDS] 5.2.4, 5.3.7 step 4; [SPE] gate, up, down) --------- */

/* y = W_down (silu(W_gate x) * (W_up x)); W_gate, W_up [F][D], W_down [D][F].
 * The mode only says how x was given: h is never rounded (the activations'
 * cast to bf16 is the only cast point of the bf16 workload). */
int orc_swiglu(int fmt_gu, int fmt_down, const uint8_t *gate, const uint8_t *up, const uint8_t *down,
               const int8_t *cb, int32_t D, int32_t F, int mode, const double *x, double *y) {
    (void)mode;
    float *row = (float *)malloc(sizeof(float) * (size_t)(D > F ? D : F));
    double *h = (double *)malloc(sizeof(double) * (size_t)F);
    if (!row || !h) { free(row); free(h); return -1; }
    for (int32_t f = 0; f < F; ++f) {
        double g = 0.0, u = 0.0;
        orc_dequant_range(fmt_gu, gate, (int64_t)f * D, D, cb, row);
        for (int32_t k = 0; k < D; ++k) g += (double)row[k] * x[k];
        orc_dequant_range(fmt_gu, up, (int64_t)f * D, D, cb, row);
        for (int32_t k = 0; k < D; ++k) u += (double)row[k] * x[k];
        h[f] = orc_silu(g) * u;
    }
    for (int32_t d = 0; d < D; ++d) {
        double s = 0.0;
        orc_dequant_range(fmt_down, down, (int64_t)d * F, F, cb, row);
        for (int32_t f = 0; f < F; ++f) s += (double)row[f] * h[f];
        y[d] = s;
    }
    free(row);
    free(h);
    return 0;
}

static int orc_check(const orc_layer *L) {
    if (!L || L->n_embd <= 0 || L->n_expert <= 0 || L->n_ff_exp <= 0 || L->n_expert_used < 1 ||
        L->n_expert_used > L->n_expert || L->n_ff_shared < 0 || !L->router_w || !L->gate || !L->up || !L->down)
        return -1;
    if (orc_tensor_bytes(L->gate_fmt, (int64_t)L->n_ff_exp * L->n_embd) < 0) return -1;
    if (orc_tensor_bytes(L->up_fmt, (int64_t)L->n_ff_exp * L->n_embd) < 0) return -1;
    if (orc_tensor_bytes(L->down_fmt, (int64_t)L->n_ff_exp * L->n_embd) < 0) return -1;
    if (L->gate_fmt != L->up_fmt) return -1;
    if (L->n_ff_shared > 0 &&
        (!L->sh_gate || !L->sh_up || !L->sh_down ||
         orc_tensor_bytes(L->shared_fmt, (int64_t)L->n_ff_shared * L->n_embd) < 0))
        return -1;
    if ((L->gate_fmt == ORC_CB2 || L->down_fmt == ORC_CB2 || L->shared_fmt == ORC_CB2) && !L->codebook) return -1;
    return 0;
}

static double *orc_input(int mode, const float *x_f32, const uint16_t *x_bf16, int32_t T, int32_t D) {
    double *x = (double *)malloc(sizeof(double) * (size_t)T * (size_t)D);
    if (!x) return NULL;
    for (int64_t i = 0; i < (int64_t)T * D; ++i) x[i] = mode == ORC_BF16 ? orc_bf16(x_bf16[i]) : (double)x_f32[i];
    return x;
}

static int orc_route_all(const orc_layer *L, const double *x, int32_t T, int32_t *idx, float *w) {
    double *lg = (double *)malloc(sizeof(double) * (size_t)T * (size_t)L->n_expert);
    if (!lg) return -1;
    orc_logits(L, x, T, lg);
    int rc = orc_topk(lg, T, L->n_expert, L->n_expert_used, L->route_scale, idx, w, NULL);
    free(lg);
    return rc;
}

/* expert e's slice of an expert-major tensor of n_rows x n_in weights */
static const uint8_t *orc_expert(const uint8_t *base, int fmt, int32_t e, int64_t n_w) {
    return base + (int64_t)e * orc_tensor_bytes(fmt, n_w);
}

static int orc_cmp_int(const void *a, const void *b) {
    int32_t i = *(const int32_t *)a, j = *(const int32_t *)b;
    return (i > j) - (i < j);
}

/* y_t = S(x_t) + sum_{e in top-k(t)} w_{t,e} FFN_e(x_t)
 * ([UDS] 5.3.2 formula; 5.3.4 the shared expert is always on and added;
 *  5.3.7 step 5 multiply by the router weight and accumulate).
 * The routed terms are added in ascending expert order so that this sum and
 * the dense definition below perform the same additions. */
int orc_moe_forward(const orc_layer *L, int mode, const float *x_f32, const uint16_t *x_bf16, int32_t T,
                    const int32_t *rows, int32_t n_rows, float *y, int32_t *idx_out, float *w_out) {
    if (orc_check(L) || T < 0 || (mode != ORC_F32 && mode != ORC_BF16) || L->n_expert_used > 64) return -1;
    if (T == 0) return 0;
    int32_t D = L->n_embd, F = L->n_ff_exp, k = L->n_expert_used;
    double *x = orc_input(mode, x_f32, x_bf16, T, D);
    int32_t *idx = (int32_t *)malloc(sizeof(int32_t) * (size_t)T * (size_t)k);
    float *w = (float *)malloc(sizeof(float) * (size_t)T * (size_t)k);
    double *acc = (double *)malloc(sizeof(double) * (size_t)D);
    double *tmp = (double *)malloc(sizeof(double) * (size_t)D);
    int rc = (!x || !idx || !w || !acc || !tmp) ? -1 : orc_route_all(L, x, T, idx, w);
    int64_t nw = (int64_t)F * D;
    int32_t nr = rows ? n_rows : T;
    for (int32_t r = 0; rc == 0 && r < nr; ++r) {
        int32_t t = rows ? rows[r] : r;
        if (t < 0 || t >= T) { rc = -1; break; }
        const double *xt = x + (int64_t)t * D;
        for (int32_t d = 0; d < D; ++d) acc[d] = 0.0;
        if (L->n_ff_shared > 0) {
            rc = orc_swiglu(L->shared_fmt, L->shared_fmt, L->sh_gate, L->sh_up, L->sh_down, L->codebook, D,
                            L->n_ff_shared, mode, xt, acc);
            if (rc) break;
        }
        /* slots taken in ascending expert id (ids are distinct within a token) */
        int32_t ids[64];
        for (int32_t s = 0; s < k; ++s) ids[s] = idx[(int64_t)t * k + s];
        qsort(ids, (size_t)k, sizeof(int32_t), orc_cmp_int);
        for (int32_t j = 0; j < k; ++j) {
            int32_t e = ids[j], s = 0;
            while (idx[(int64_t)t * k + s] != e) ++s;
            rc = orc_swiglu(L->gate_fmt, L->down_fmt, orc_expert(L->gate, L->gate_fmt, e, nw),
                            orc_expert(L->up, L->up_fmt, e, nw), orc_expert(L->down, L->down_fmt, e, nw),
                            L->codebook, D, F, mode, xt, tmp);
            if (rc) break;
            double g = (double)w[(int64_t)t * k + s];
            for (int32_t d = 0; d < D; ++d) acc[d] += g * tmp[d];
        }
        for (int32_t d = 0; d < D; ++d) y[(int64_t)t * D + d] = (float)acc[d];
    }
    if (rc == 0 && idx_out) memcpy(idx_out, idx, sizeof(int32_t) * (size_t)T * (size_t)k);
    if (rc == 0 && w_out) memcpy(w_out, w, sizeof(float) * (size_t)T * (size_t)k);
    free(x);
    free(idx);
    free(w);
    free(acc);
    free(tmp);
    return rc;
}

/* The plain definition: G_{t,e} = renormalized weight if e is in the top-k
 * of token t, else 0; y_t = S(x_t) + sum_{e=0}^{E-1} G_{t,e} FFN_e(x_t). */
int orc_moe_forward_dense(const orc_layer *L, int mode, const float *x_f32, const uint16_t *x_bf16,
                          int32_t T, float *y) {
    if (orc_check(L) || T < 0) return -1;
    if (T == 0) return 0;
    int32_t D = L->n_embd, F = L->n_ff_exp, E = L->n_expert, k = L->n_expert_used;
    double *x = orc_input(mode, x_f32, x_bf16, T, D);
    int32_t *idx = (int32_t *)malloc(sizeof(int32_t) * (size_t)T * (size_t)k);
    float *w = (float *)malloc(sizeof(float) * (size_t)T * (size_t)k);
    double *acc = (double *)malloc(sizeof(double) * (size_t)D);
    double *tmp = (double *)malloc(sizeof(double) * (size_t)D);
    int rc = (!x || !idx || !w || !acc || !tmp) ? -1 : orc_route_all(L, x, T, idx, w);
    int64_t nw = (int64_t)F * D;
    for (int32_t t = 0; rc == 0 && t < T; ++t) {
        const double *xt = x + (int64_t)t * D;
        for (int32_t d = 0; d < D; ++d) acc[d] = 0.0;
        if (L->n_ff_shared > 0)
            rc = orc_swiglu(L->shared_fmt, L->shared_fmt, L->sh_gate, L->sh_up, L->sh_down, L->codebook, D,
                            L->n_ff_shared, mode, xt, acc);
        for (int32_t e = 0; rc == 0 && e < E; ++e) {
            double G = 0.0;
            for (int32_t s = 0; s < k; ++s)
                if (idx[(int64_t)t * k + s] == e) G = (double)w[(int64_t)t * k + s];
            rc = orc_swiglu(L->gate_fmt, L->down_fmt, orc_expert(L->gate, L->gate_fmt, e, nw),
                            orc_expert(L->up, L->up_fmt, e, nw), orc_expert(L->down, L->down_fmt, e, nw),
                            L->codebook, D, F, mode, xt, tmp);
            if (G != 0.0)
                for (int32_t d = 0; d < D; ++d) acc[d] += G * tmp[d];
        }
        for (int32_t d = 0; d < D; ++d) y[(int64_t)t * D + d] = (float)acc[d];
    }
    free(x);
    free(idx);
    free(w);
    free(acc);
    free(tmp);
    return rc;
}

/* RMSNorm applied before each block ([UDS] 5.2.1 norm + residual; 5.6.2 step 1). */
int orc_rmsnorm(const float *x, const float *gamma, double eps, int32_t T, int32_t D, float *out) {
    if (T < 0 || D <= 0) return -1;
    for (int32_t t = 0; t < T; ++t) {
        const float *xt = x + (int64_t)t * D;
        double ss = 0.0;
        for (int32_t i = 0; i < D; ++i) ss += (double)xt[i] * (double)xt[i];
        double inv = 1.0 / sqrt(ss / D + eps);
        for (int32_t i = 0; i < D; ++i) out[(int64_t)t * D + i] = (float)((double)gamma[i] * (double)xt[i] * inv);
    }
    return 0;
}

/* Selections per {layer, expert} ([SPE] "Some experts run far more often than
 * others"), added into an existing profile. */
void orc_count_selections(const int32_t *topk_idx, int32_t T, int32_t k, int32_t E, int32_t layer, int64_t *counts) {
    for (int64_t p = 0; p < (int64_t)T * k; ++p) {
        const int32_t e = topk_idx[p];
        if (e >= 0 && e < E) counts[(int64_t)layer * E + e] += 1;
    }
}

static _Thread_local const int64_t *hot_counts;
static int64_t hot_key(int32_t i) {
    const int64_t c = hot_counts[i];
    return c < 0 ? 0 : (c >= ((int64_t)1 << 39) ? ((int64_t)1 << 39) - 1 : c);
}
static int hot_cmp(const void *a, const void *b) {
    const int32_t i = *(const int32_t *)a, j = *(const int32_t *)b;
    const int64_t ci = hot_key(i), cj = hot_key(j);
    if (ci != cj) return ci > cj ? -1 : 1;  /* more hits first */
    return i < j ? -1 : (i > j);             /* then lower {layer, expert} index */
}

/* The hot list: {layer, expert} entries sorted by hits ([SPE] "Some experts run
 * far more often than others"; ties by index, our reading). */
int32_t orc_hotlist(const int64_t *counts, int32_t n, int32_t *order) {
    int32_t hot = 0;
    for (int32_t i = 0; i < n; ++i) {
        order[i] = i;
        hot += counts[i] > 0;
    }
    hot_counts = counts;
    qsort(order, (size_t)n, sizeof(int32_t), hot_cmp);
    return hot;
}

const char *orc_version(void) { return "oracle-1"; }
