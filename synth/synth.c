/*
 * synth.c - seeded synthetic inputs for the routed mixture-of-experts block.
 *
 * This module draws the random numbers (activations, router matrix, RMSNorm
 * weights, the codebook) and *encodes* Gaussian expert weights into the four
 * block formats the layer stores.  It holds none of the block's arithmetic: no
 * decoding of a block back to values, no routing, no products.  Both the GPU
 * library's tests and the CPU oracle read the bytes written here.
 *
 * Random numbers: counter-based splitmix64 (Steele, Lea and Flood, "Fast
 * splittable pseudorandom number generators", OOPSLA 2014).  Value number c of
 * the stream with key K is mix(K + (c+1)*golden).  Every tensor has its own key
 * derived from (seed, layer, tag, expert), so the bytes do not depend on the
 * number of threads or on the order in which tensors are generated.
 * Normals: Box-Muller in double precision with the host libm.
 *
 * Block formats written (byte layouts are this project's own):
 *   Q2K  84 B / 256 w: d f16 @0, dmin f16 @2, sm[16] @4 (low nibble scale,
 *        high nibble min of group g = 16 consecutive weights), qs[64] @20
 *        (weight i in bits 2*(i&3) of byte i>>2).
 *   Q8_0 34 B / 32 w:  d f16 @0, int8 q[32] @2.
 *   CB2  66 B / 256 w: d f16 @0, idx[32] u8 @2 (one codebook row per 8
 *        weights), sgn[32] u8 @34 (bit j flips the sign of weight j of the 8).
 *   Q4K 144 B / 256 w: d f16 @0, dmin f16 @2, 12 bytes @4 of sixteen 6-bit
 *        fields (bits 6f..6f+5; f < 8 the scale of sub-block f of 32 weights,
 *        f >= 8 the min of sub-block f-8), codes @16 (weight i in bits
 *        4*(i&1) of byte i>>1).
 * Matrices are [n_out][n_in] row-major, flattened and cut into consecutive
 * blocks.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define SY_GOLDEN 0x9E3779B97F4A7C15ULL

static inline uint64_t sy_mix(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

static inline uint64_t sy_at(uint64_t key, uint64_t ctr) {
    return sy_mix(key + (ctr + 1u) * SY_GOLDEN);
}

uint64_t sy_key(uint64_t seed, uint32_t layer, uint32_t tag, uint32_t expert) {
    uint64_t k = sy_mix(seed * SY_GOLDEN + 0x5851F42D4C957F2DULL);
    k = sy_mix(k ^ (0x1000000000ULL + layer));
    k = sy_mix(k ^ (0x2000000000ULL + tag));
    k = sy_mix(k ^ (0x3000000000ULL + expert));
    return k;
}

static inline double sy_u01(uint64_t r) { return (double)(r >> 11) * 0x1.0p-53; }

/* Normal number i of stream key (pairs 2j, 2j+1 share one Box-Muller draw). */
static inline void sy_normal_pair(uint64_t key, uint64_t pair, double *z0, double *z1) {
    double u1 = ((double)(sy_at(key, 2 * pair) >> 11) + 1.0) * 0x1.0p-53; /* (0,1] */
    double u2 = sy_u01(sy_at(key, 2 * pair + 1));
    double r = sqrt(-2.0 * log(u1));
    double a = 6.283185307179586 * u2;
    *z0 = r * cos(a);
    *z1 = r * sin(a);
}

/* n values sigma*z (rounded to fp32), elements [first, first+n) of the stream. */
static void sy_normals(uint64_t key, int64_t first, int64_t n, double sigma, float *out) {
    int64_t i = 0;
    while (i < n) {
        int64_t e = first + i;
        double z0, z1;
        sy_normal_pair(key, (uint64_t)(e >> 1), &z0, &z1);
        if ((e & 1) == 0) {
            out[i++] = (float)(sigma * z0);
            if (i < n) out[i++] = (float)(sigma * z1);
        } else {
            out[i++] = (float)(sigma * z1);
        }
    }
}

/* float -> IEEE binary16 bits, round to nearest even (handles subnormals). */
static uint16_t sy_f16_bits(float f) {
    uint32_t x;
    memcpy(&x, &f, 4);
    uint32_t sign = (x >> 16) & 0x8000u;
    uint32_t ax = x & 0x7FFFFFFFu;
    if (ax >= 0x7F800000u) return (uint16_t)(sign | 0x7C00u | (ax > 0x7F800000u ? 0x200u : 0));
    if (ax >= 0x477FF000u) return (uint16_t)(sign | 0x7C00u); /* rounds to >= 65520: inf */
    if (ax < 0x38800000u) {                                    /* below 2^-14: subnormal */
        /* value = ax as float; subnormal unit 2^-24 */
        float af;
        memcpy(&af, &ax, 4);
        double scaled = (double)af * 16777216.0; /* exact */
        double fl = floor(scaled);
        double rem = scaled - fl;
        uint32_t m = (uint32_t)fl;
        if (rem > 0.5 || (rem == 0.5 && (m & 1u))) m++;
        return (uint16_t)(sign | m); /* m == 0x400 is the smallest normal, still right */
    }
    uint32_t e = (ax >> 23) - 112u; /* rebias 127 -> 15 */
    uint32_t mant = ax & 0x7FFFFFu;
    uint32_t h = (e << 10) | (mant >> 13);
    uint32_t rest = mant & 0x1FFFu;
    if (rest > 0x1000u || (rest == 0x1000u && (h & 1u))) h++;
    return (uint16_t)(sign | h);
}

/* IEEE binary16 bits -> float (exact). */
static float sy_f16_val(uint16_t h) {
    uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
    uint32_t e = (h >> 10) & 0x1Fu, m = h & 0x3FFu;
    float v;
    if (e == 0) {
        v = (float)m * 0x1.0p-24f;
    } else if (e == 31) {
        v = m ? NAN : INFINITY;
    } else {
        uint32_t bits = ((e + 112u) << 23) | (m << 13);
        memcpy(&v, &bits, 4);
    }
    uint32_t vb;
    memcpy(&vb, &v, 4);
    vb |= sign;
    memcpy(&v, &vb, 4);
    return v;
}

static inline float sy_rint_clamp(float v, float lo, float hi) {
    float r = rintf(v);
    return r < lo ? lo : (r > hi ? hi : r);
}

/* ---- encoders ---------------------------------------------------------- */

static void sy_encode_q2k(const float *v, uint8_t *blk) {
    float sr[16], mn[16], max_sr = 0.f, max_mn = 0.f;
    for (int g = 0; g < 16; ++g) {
        float lo = v[16 * g], hi = v[16 * g];
        for (int i = 1; i < 16; ++i) {
            float t = v[16 * g + i];
            lo = t < lo ? t : lo;
            hi = t > hi ? t : hi;
        }
        mn[g] = lo < 0.f ? -lo : 0.f;
        sr[g] = (hi + mn[g]) / 3.f;
        if (sr[g] > max_sr) max_sr = sr[g];
        if (mn[g] > max_mn) max_mn = mn[g];
    }
    uint16_t dh = sy_f16_bits(max_sr / 15.f), mh = sy_f16_bits(max_mn / 15.f);
    float d = sy_f16_val(dh), dmin = sy_f16_val(mh);
    memset(blk, 0, 84);
    memcpy(blk + 0, &dh, 2);
    memcpy(blk + 2, &mh, 2);
    for (int g = 0; g < 16; ++g) {
        float sc = d > 0.f ? sy_rint_clamp(sr[g] / d, 0.f, 15.f) : 0.f;
        float m = dmin > 0.f ? sy_rint_clamp(mn[g] / dmin, 0.f, 15.f) : 0.f;
        blk[4 + g] = (uint8_t)((unsigned)sc | ((unsigned)m << 4));
        float step = d * sc, off = dmin * m;
        for (int i = 0; i < 16; ++i) {
            int idx = 16 * g + i;
            float q = step > 0.f ? sy_rint_clamp((v[idx] + off) / step, 0.f, 3.f) : 0.f;
            blk[20 + (idx >> 2)] |= (uint8_t)((unsigned)q << (2 * (idx & 3)));
        }
    }
}

/* Q4K (144 B): per sub-block j of 32 weights a 6-bit scale and min; field f
 * of the 12 bytes @4 in bits 6f..6f+5 (scales f = 0..7, mins f = 8..15);
 * weight i's 4-bit code in bits 4*(i%2) of byte 16 + i/2. */
static void sy_put6(uint8_t *p12, int f, unsigned v) {
    for (int b = 0; b < 6; ++b) {
        int bit = 6 * f + b;
        if ((v >> b) & 1u) p12[bit / 8] |= (uint8_t)(1u << (bit % 8));
    }
}

static void sy_encode_q4k(const float *v, uint8_t *blk) {
    float sr[8], mn[8], max_sr = 0.f, max_mn = 0.f;
    for (int j = 0; j < 8; ++j) {
        float lo = v[32 * j], hi = v[32 * j];
        for (int i = 1; i < 32; ++i) {
            float t = v[32 * j + i];
            lo = t < lo ? t : lo;
            hi = t > hi ? t : hi;
        }
        mn[j] = lo < 0.f ? -lo : 0.f;
        sr[j] = (hi + mn[j]) / 15.f;
        if (sr[j] > max_sr) max_sr = sr[j];
        if (mn[j] > max_mn) max_mn = mn[j];
    }
    uint16_t dh = sy_f16_bits(max_sr / 63.f), mh = sy_f16_bits(max_mn / 63.f);
    float d = sy_f16_val(dh), dmin = sy_f16_val(mh);
    memset(blk, 0, 144);
    memcpy(blk + 0, &dh, 2);
    memcpy(blk + 2, &mh, 2);
    for (int j = 0; j < 8; ++j) {
        float sc = d > 0.f ? sy_rint_clamp(sr[j] / d, 0.f, 63.f) : 0.f;
        float m = dmin > 0.f ? sy_rint_clamp(mn[j] / dmin, 0.f, 63.f) : 0.f;
        sy_put6(blk + 4, j, (unsigned)sc);
        sy_put6(blk + 4, 8 + j, (unsigned)m);
        float step = d * sc, off = dmin * m;
        for (int i = 0; i < 32; ++i) {
            int idx = 32 * j + i;
            float q = step > 0.f ? sy_rint_clamp((v[idx] + off) / step, 0.f, 15.f) : 0.f;
            blk[16 + (idx >> 1)] |= (uint8_t)((unsigned)q << (4 * (idx & 1)));
        }
    }
}

static void sy_encode_q8_0(const float *v, uint8_t *blk) {
    float amax = 0.f;
    for (int i = 0; i < 32; ++i) {
        float a = fabsf(v[i]);
        if (a > amax) amax = a;
    }
    uint16_t dh = sy_f16_bits(amax / 127.f);
    float d = sy_f16_val(dh);
    memcpy(blk, &dh, 2);
    for (int i = 0; i < 32; ++i) {
        float q = d > 0.f ? sy_rint_clamp(v[i] / d, -127.f, 127.f) : 0.f;
        blk[2 + i] = (uint8_t)(int8_t)q;
    }
}

typedef struct {
    float babs[8][256]; /* |cb[c][j]| laid out j-major for the search loop */
    float norm[256];    /* sum_j |cb[c][j]|^2 */
    const int8_t *cb;
} sy_cb_index;

static void sy_cb_prepare(const int8_t *cb, sy_cb_index *ix) {
    ix->cb = cb;
    for (int c = 0; c < 256; ++c) {
        float s = 0.f;
        for (int j = 0; j < 8; ++j) {
            float a = (float)abs(cb[8 * c + j]);
            ix->babs[j][c] = a;
            s += a * a;
        }
        ix->norm[c] = s;
    }
}

/* Nearest codebook row in magnitude: argmin_c sum_j (a_j - |cb_cj|)^2, written
 * as norm_c - 2 a.|cb_c| (the a.a term is common); ties go to the lowest c. */
static void sy_encode_cb2(const float *v, uint8_t *blk, const sy_cb_index *ix) {
    float amax = 0.f;
    for (int i = 0; i < 256; ++i) {
        float a = fabsf(v[i]);
        if (a > amax) amax = a;
    }
    uint16_t dh = sy_f16_bits(amax / 8.f);
    float d = sy_f16_val(dh);
    memcpy(blk, &dh, 2);
    for (int g = 0; g < 32; ++g) {
        float score[256];
        float a[8];
        for (int j = 0; j < 8; ++j) a[j] = d > 0.f ? 2.f * (fabsf(v[8 * g + j]) / d) : 0.f;
        for (int c = 0; c < 256; ++c) score[c] = ix->norm[c];
        for (int j = 0; j < 8; ++j) {
            const float *bj = ix->babs[j];
            float aj = a[j];
            for (int c = 0; c < 256; ++c) score[c] -= aj * bj[c];
        }
        int best = 0;
        float bs = score[0];
        for (int c = 1; c < 256; ++c)
            if (score[c] < bs) { bs = score[c]; best = c; }
        uint8_t sg = 0;
        for (int j = 0; j < 8; ++j) {
            int neg_v = v[8 * g + j] < 0.f;
            int neg_c = ix->cb[8 * best + j] < 0;
            if (neg_v ^ neg_c) sg |= (uint8_t)(1u << j);
        }
        blk[2 + g] = (uint8_t)best;
        blk[34 + g] = sg;
    }
}

/* ---- parallel tensor generation ---------------------------------------- */

enum { SY_Q2K = 2, SY_Q8_0 = 3, SY_CB2 = 4, SY_Q4K = 5 };

static int sy_block_w(int fmt) { return fmt == SY_Q8_0 ? 32 : 256; }
static int sy_block_b(int fmt) { return fmt == SY_Q2K ? 84 : (fmt == SY_Q8_0 ? 34 : (fmt == SY_Q4K ? 144 : 66)); }

typedef struct {
    int fmt;
    uint64_t seed;
    uint32_t layer, tag;
    int64_t n_expert, blocks_per_expert;
    double sigma;
    const sy_cb_index *cbix;
    uint8_t *out;
    int64_t n_items, chunk;
    int64_t next; /* protected by mu */
    pthread_mutex_t mu;
} sy_job;

static void *sy_worker(void *arg) {
    sy_job *J = (sy_job *)arg;
    int bw = sy_block_w(J->fmt), bb = sy_block_b(J->fmt);
    float v[256];
    for (;;) {
        pthread_mutex_lock(&J->mu);
        int64_t it = J->next;
        J->next += J->chunk;
        pthread_mutex_unlock(&J->mu);
        if (it >= J->n_items) break;
        int64_t end = it + J->chunk < J->n_items ? it + J->chunk : J->n_items;
        for (int64_t g = it; g < end; ++g) {
            int64_t e = g / J->blocks_per_expert, b = g % J->blocks_per_expert;
            uint64_t key = sy_key(J->seed, J->layer, J->tag, (uint32_t)e);
            sy_normals(key, b * bw, bw, J->sigma, v);
            uint8_t *dst = J->out + g * bb;
            if (J->fmt == SY_Q2K) sy_encode_q2k(v, dst);
            else if (J->fmt == SY_Q4K) sy_encode_q4k(v, dst);
            else if (J->fmt == SY_Q8_0) sy_encode_q8_0(v, dst);
            else sy_encode_cb2(v, dst, J->cbix);
        }
    }
    return NULL;
}

/*
 * Generate n_expert matrices [n_rows][n_in] of N(0, sigma) weights and encode
 * them in format fmt, expert-major, into out.  Expert e uses the stream
 * sy_key(seed, layer, tag, e).  Returns the number of bytes written, or -1.
 */
int64_t sy_gen_expert_tensor(int fmt, uint64_t seed, uint32_t layer, uint32_t tag, int64_t n_expert,
                             int64_t n_rows, int64_t n_in, double sigma, const int8_t *codebook,
                             uint8_t *out, int nthreads) {
    if (fmt != SY_Q2K && fmt != SY_Q8_0 && fmt != SY_CB2 && fmt != SY_Q4K) return -1;
    int64_t bw = sy_block_w(fmt);
    if ((n_rows * n_in) % bw) return -1;
    sy_cb_index *cbix = NULL;
    if (fmt == SY_CB2) {
        if (!codebook) return -1;
        cbix = (sy_cb_index *)malloc(sizeof(sy_cb_index));
        sy_cb_prepare(codebook, cbix);
    }
    sy_job J;
    memset(&J, 0, sizeof J);
    J.fmt = fmt;
    J.seed = seed;
    J.layer = layer;
    J.tag = tag;
    J.n_expert = n_expert;
    J.blocks_per_expert = n_rows * n_in / bw;
    J.sigma = sigma;
    J.cbix = cbix;
    J.out = out;
    J.n_items = n_expert * J.blocks_per_expert;
    J.chunk = 512;
    J.next = 0;
    pthread_mutex_init(&J.mu, NULL);
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    pthread_t th[256];
    int started = 0;
    for (int t = 1; t < nthreads; ++t)
        if (pthread_create(&th[started], NULL, sy_worker, &J) == 0) started++;
    sy_worker(&J);
    for (int t = 0; t < started; ++t) pthread_join(th[t], NULL);
    pthread_mutex_destroy(&J.mu);
    free(cbix);
    return J.n_items * sy_block_b(fmt);
}

/* n fp32 values sigma*N(0,1), elements [first, first+n) of stream (seed,layer,tag,idx). */
void sy_gen_normal(uint64_t seed, uint32_t layer, uint32_t tag, uint32_t idx, int64_t first, int64_t n,
                   double sigma, float *out) {
    sy_normals(sy_key(seed, layer, tag, idx), first, n, sigma, out);
}

/* n doubles uniform in [0,1), elements [first, first+n) of stream (seed,layer,tag,idx). */
void sy_gen_uniform(uint64_t seed, uint32_t layer, uint32_t tag, uint32_t idx, int64_t first, int64_t n,
                    double *out) {
    uint64_t key = sy_key(seed, layer, tag, idx);
    for (int64_t i = 0; i < n; ++i) out[i] = sy_u01(sy_at(key, (uint64_t)(first + i)));
}

/* Codebook of 256 rows x 8 int8 entries, each uniform in {-8..8}. */
void sy_gen_codebook(uint64_t seed, uint32_t tag, int8_t *cb) {
    uint64_t key = sy_key(seed, 0, tag, 0);
    for (int i = 0; i < 256 * 8; ++i) cb[i] = (int8_t)((int)floor(sy_u01(sy_at(key, (uint64_t)i)) * 17.0) - 8);
}

/* fp32 -> fp16 / bf16 bit encoders exposed for building inputs (RNE). */
void sy_f32_to_f16(const float *in, int64_t n, uint16_t *out) {
    for (int64_t i = 0; i < n; ++i) out[i] = sy_f16_bits(in[i]);
}

void sy_f32_to_bf16(const float *in, int64_t n, uint16_t *out) {
    for (int64_t i = 0; i < n; ++i) {
        uint32_t x;
        memcpy(&x, &in[i], 4);
        if ((x & 0x7FFFFFFFu) > 0x7F800000u) { out[i] = (uint16_t)((x >> 16) | 0x40u); continue; }
        uint32_t lsb = (x >> 16) & 1u;
        out[i] = (uint16_t)((x + 0x7FFFu + lsb) >> 16);
    }
}

/* ---- code-sampled blocks ------------------------------------------------
 * For the 43-layer stack (79 GB of blocks) encoding Gaussian draws would cost
 * tens of CPU-minutes per run, so its blocks are drawn directly as codes:
 * every field uniform, with the block scale chosen so that the decoded weights
 * have a standard deviation close to sigma.
 *   Q2K : sc_g uniform in 8..15, m_g = sc_g, dmin = fp16(1.5 d): weights are
 *         d*sc_g*(q - 1.5) for uniform q, i.e. symmetric about zero.
 *   Q8_0: q uniform in -127..127.
 *   CB2 : idx and sign bits uniform.
 *   Q4K : sc_j uniform in 32..63, m_j = sc_j, dmin = fp16(7.5 d): weights are
 *         d*sc_j*(q - 7.5) for uniform q.
 * Block b of expert e uses stream sy_key(seed, layer, tag, e), values
 * [b*64, b*64+64). */
static void sy_sample_block(int fmt, uint64_t key, int64_t b, double sigma, const double cb_rms, uint8_t *blk) {
    uint64_t r[64];
    int need = fmt == SY_Q2K || fmt == SY_Q4K ? 25 : (fmt == SY_Q8_0 ? 33 : 9);
    for (int i = 0; i < need; ++i) r[i] = sy_at(key, (uint64_t)b * 64u + (uint64_t)i);
    double jit = 0.8 + 0.4 * sy_u01(r[0]);
    if (fmt == SY_Q2K) {
        uint16_t dh = sy_f16_bits((float)(sigma * jit / (11.5 * 1.118033988749895)));
        uint16_t mh = sy_f16_bits(1.5f * sy_f16_val(dh));
        memcpy(blk, &dh, 2);
        memcpy(blk + 2, &mh, 2);
        for (int g = 0; g < 16; ++g) {
            unsigned sc = 8u + (unsigned)((r[1 + g] >> 40) & 7u);
            blk[4 + g] = (uint8_t)(sc | (sc << 4));
        }
        for (int i = 0; i < 64; ++i) blk[20 + i] = (uint8_t)(r[17 + (i >> 3)] >> (8 * (i & 7)));
    } else if (fmt == SY_Q4K) {
        uint16_t dh = sy_f16_bits((float)(sigma * jit / (47.5 * 4.6097722286464435)));
        uint16_t mh = sy_f16_bits(7.5f * sy_f16_val(dh));
        memset(blk, 0, 144);
        memcpy(blk, &dh, 2);
        memcpy(blk + 2, &mh, 2);
        for (int j = 0; j < 8; ++j) {
            unsigned sc = 32u + (unsigned)((r[1 + j] >> 40) & 31u);
            sy_put6(blk + 4, j, sc);
            sy_put6(blk + 4, 8 + j, sc);
        }
        for (int i = 0; i < 128; ++i) blk[16 + i] = (uint8_t)(r[9 + (i >> 3)] >> (8 * (i & 7)));
    } else if (fmt == SY_Q8_0) {
        uint16_t dh = sy_f16_bits((float)(sigma * jit / 73.33333333333333));
        memcpy(blk, &dh, 2);
        for (int i = 0; i < 32; ++i) blk[2 + i] = (uint8_t)(int8_t)((int)((r[1 + i] >> 11) % 255u) - 127);
    } else {
        uint16_t dh = sy_f16_bits((float)(sigma * jit / cb_rms));
        memcpy(blk, &dh, 2);
        for (int i = 0; i < 64; ++i) blk[2 + i] = (uint8_t)(r[1 + (i >> 3)] >> (8 * (i & 7)));
    }
}

typedef struct {
    int fmt;
    uint64_t seed;
    uint32_t layer, tag;
    int64_t blocks_per_expert, n_items;
    double sigma, cb_rms;
    uint8_t *out;
    int64_t next;
    pthread_mutex_t mu;
} sy_sjob;

static void *sy_sworker(void *arg) {
    sy_sjob *J = (sy_sjob *)arg;
    int bb = sy_block_b(J->fmt);
    const int64_t chunk = 4096;
    for (;;) {
        pthread_mutex_lock(&J->mu);
        int64_t it = J->next;
        J->next += chunk;
        pthread_mutex_unlock(&J->mu);
        if (it >= J->n_items) break;
        int64_t end = it + chunk < J->n_items ? it + chunk : J->n_items;
        for (int64_t g = it; g < end; ++g) {
            int64_t e = g / J->blocks_per_expert, b = g % J->blocks_per_expert;
            sy_sample_block(J->fmt, sy_key(J->seed, J->layer, J->tag, (uint32_t)e), b, J->sigma, J->cb_rms,
                            J->out + g * bb);
        }
    }
    return NULL;
}

int64_t sy_sample_expert_tensor(int fmt, uint64_t seed, uint32_t layer, uint32_t tag, int64_t n_expert,
                                int64_t n_rows, int64_t n_in, double sigma, const int8_t *codebook,
                                uint8_t *out, int nthreads) {
    if (fmt != SY_Q2K && fmt != SY_Q8_0 && fmt != SY_CB2 && fmt != SY_Q4K) return -1;
    int64_t bw = sy_block_w(fmt);
    if ((n_rows * n_in) % bw) return -1;
    double cb_rms = 1.0;
    if (fmt == SY_CB2) {
        if (!codebook) return -1;
        double s = 0.0;
        for (int i = 0; i < 2048; ++i) s += (double)codebook[i] * codebook[i];
        cb_rms = sqrt(s / 2048.0);
        if (cb_rms <= 0.0) cb_rms = 1.0;
    }
    sy_sjob J;
    memset(&J, 0, sizeof J);
    J.fmt = fmt;
    J.seed = seed;
    J.layer = layer;
    J.tag = tag;
    J.blocks_per_expert = n_rows * n_in / bw;
    J.n_items = n_expert * J.blocks_per_expert;
    J.sigma = sigma;
    J.cb_rms = cb_rms;
    J.out = out;
    pthread_mutex_init(&J.mu, NULL);
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    pthread_t th[256];
    int started = 0;
    for (int t = 1; t < nthreads; ++t)
        if (pthread_create(&th[started], NULL, sy_sworker, &J) == 0) started++;
    sy_sworker(&J);
    for (int t = 0; t < started; ++t) pthread_join(th[t], NULL);
    pthread_mutex_destroy(&J.mu);
    return J.n_items * sy_block_b(fmt);
}

const char *sy_version(void) { return "synth-1"; }
