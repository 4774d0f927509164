// common.h - device helpers shared by the gfx950 kernels of the routed MoE
// block: block-format decoders, wave64 reductions, number conversions, and
// the workspace layout the host code and the kernels agree on.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe.h"

#define MOE_DEV __device__ __forceinline__

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

namespace moe {

constexpr int kWave = 64;
constexpr int kMaxExperts = 1024;
constexpr int kMaxUsed = 16;

// Block geometry of the three weight formats.
constexpr int kQ2KBytes = 84, kQ8Bytes = 34, kCB2Bytes = 66;

__host__ __device__ inline int64_t fmt_block_weights(int fmt) { return fmt == MOE_Q8_0 ? 32 : 256; }
__host__ __device__ inline int64_t fmt_block_bytes(int fmt) {
    return fmt == MOE_Q2K ? kQ2KBytes : (fmt == MOE_Q8_0 ? kQ8Bytes : kCB2Bytes);
}
__host__ __device__ inline int64_t fmt_bytes(int fmt, int64_t n) {
    return n / fmt_block_weights(fmt) * fmt_block_bytes(fmt);
}

// ---- scalar conversions ---------------------------------------------------

MOE_DEV float half_bits_to_float(uint32_t bits) {
    _Float16 h = __builtin_bit_cast(_Float16, (uint16_t)(bits & 0xFFFFu));
    return (float)h;
}

MOE_DEV float bf16_bits_to_float(uint32_t bits) { return __uint_as_float(bits << 16); }

// fp32 -> bf16 bits, round to nearest even; NaN stays NaN.
MOE_DEV uint32_t float_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// ---- loads ----------------------------------------------------------------

// 16 bytes from a 4-byte aligned address (gfx9 global loads need only dword
// alignment for multi-dword accesses).
MOE_DEV u32x4 load_u32x4(const void *p) {
    u32x4 v;
    __builtin_memcpy(&v, __builtin_assume_aligned(p, 4), 16);
    return v;
}
MOE_DEV uint32_t load_u32(const void *p) { return *(const uint32_t *)__builtin_assume_aligned(p, 4); }

// 8 bytes starting at a 2-byte aligned address, assembled from aligned dwords.
MOE_DEV void load_8_at_even(const uint8_t *p, uint32_t &lo, uint32_t &hi) {
    uintptr_t a = (uintptr_t)p;
    const uint32_t *q = (const uint32_t *)(a & ~(uintptr_t)3);
    uint32_t s = (uint32_t)(a & 3u);  // 0 or 2
    uint32_t w0 = q[0], w1 = q[1];
    if (s == 0) {
        lo = w0;
        hi = w1;
    } else {
        uint32_t w2 = q[2];
        lo = __builtin_amdgcn_alignbyte(w1, w0, s);
        hi = __builtin_amdgcn_alignbyte(w2, w1, s);
    }
}

// ---- wave reductions ------------------------------------------------------

// Sum over groups of `seg` consecutive lanes (seg a power of two <= 64); every
// lane of a group ends with the group's sum.  Fixed butterfly order.
MOE_DEV float seg_sum(float v, int seg) {
    for (int o = seg >> 1; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

// ---- 64-weight chunk decoders ---------------------------------------------
// A lane works on 64 consecutive weights of one row (flat index i0, a multiple
// of 64) and returns sum_i w_i * x_i for its 64 activations x.

// Q2K: 64 weights = 4 groups of 16 inside one 84-byte super-block.
struct Q2KChunk {
    u32x4 qs;     // 16 codes per dword, group g in qs[g]
    uint32_t sm;  // scale/min byte of each of the 4 groups
    uint32_t dd;  // fp16 d (low half) and dmin (high half)
};

MOE_DEV Q2KChunk q2k_load(const uint8_t *base, int64_t i0) {
    const uint8_t *blk = base + (i0 >> 8) * kQ2KBytes;
    int sub = (int)((i0 >> 6) & 3);
    Q2KChunk c;
    c.qs = load_u32x4(blk + 20 + 16 * sub);
    c.sm = load_u32(blk + 4 + 4 * sub);
    c.dd = load_u32(blk);
    return c;
}

// sum_i (d*sc_g*q_i - dmin*m_g) x_i = d * sum_g sc_g (sum_i q_i x_i) - dmin * sum_g m_g (sum_i x_i)
MOE_DEV float q2k_dot(const Q2KChunk &c, const float *x) {
    float d = half_bits_to_float(c.dd), dmin = half_bits_to_float(c.dd >> 16);
    float acc_q = 0.f, acc_m = 0.f;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        uint32_t q = c.qs[g];
        float sq = 0.f, sx = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            uint32_t t = (q >> (2 * j)) & 0x03030303u;  // byte n -> code of weight 4n+j
#pragma unroll
            for (int n = 0; n < 4; ++n) {
                float xv = x[16 * g + 4 * n + j];
                sq = __builtin_fmaf((float)((t >> (8 * n)) & 0xFFu), xv, sq);
                sx += xv;
            }
        }
        uint32_t smb = (c.sm >> (8 * g)) & 0xFFu;
        acc_q = __builtin_fmaf((float)(smb & 15u), sq, acc_q);
        acc_m = __builtin_fmaf((float)(smb >> 4), sx, acc_m);
    }
    return d * acc_q - dmin * acc_m;
}

// Q8_0: 64 weights = 2 blocks of 32 (68 bytes, dword aligned since the chunk
// starts at an even block).
struct Q8Chunk {
    uint32_t w[17];
};

MOE_DEV Q8Chunk q8_load(const uint8_t *base, int64_t i0) {
    const uint8_t *p = base + (i0 >> 5) * kQ8Bytes;
    Q8Chunk c;
    u32x4 a = load_u32x4(p), b = load_u32x4(p + 16), d = load_u32x4(p + 32), e = load_u32x4(p + 48);
    c.w[0] = a[0]; c.w[1] = a[1]; c.w[2] = a[2]; c.w[3] = a[3];
    c.w[4] = b[0]; c.w[5] = b[1]; c.w[6] = b[2]; c.w[7] = b[3];
    c.w[8] = d[0]; c.w[9] = d[1]; c.w[10] = d[2]; c.w[11] = d[3];
    c.w[12] = e[0]; c.w[13] = e[1]; c.w[14] = e[2]; c.w[15] = e[3];
    c.w[16] = load_u32(p + 64);
    return c;
}

MOE_DEV float q8_dot(const Q8Chunk &c, const float *x) {
    float d0 = half_bits_to_float(c.w[0]), d1 = half_bits_to_float(c.w[8] >> 16);
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        uint32_t v = __builtin_amdgcn_alignbyte(c.w[i + 1], c.w[i], 2);  // bytes 2..33
#pragma unroll
        for (int n = 0; n < 4; ++n) s0 = __builtin_fmaf((float)(int8_t)(v >> (8 * n)), x[4 * i + n], s0);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        uint32_t v = c.w[9 + i];  // bytes 36..67
#pragma unroll
        for (int n = 0; n < 4; ++n) s1 = __builtin_fmaf((float)(int8_t)(v >> (8 * n)), x[32 + 4 * i + n], s1);
    }
    return d0 * s0 + d1 * s1;
}

// CB2: 64 weights = 8 groups of 8 inside one 66-byte block; the codebook
// (256 rows x 8 int8) is read from LDS.
struct CB2Chunk {
    uint32_t idx_lo, idx_hi, sg_lo, sg_hi;
    float d;
};

MOE_DEV CB2Chunk cb2_load(const uint8_t *base, int64_t i0) {
    const uint8_t *blk = base + (i0 >> 8) * kCB2Bytes;
    int sub = (int)((i0 >> 6) & 3);
    CB2Chunk c;
    load_8_at_even(blk + 2 + 8 * sub, c.idx_lo, c.idx_hi);
    load_8_at_even(blk + 34 + 8 * sub, c.sg_lo, c.sg_hi);
    uintptr_t a = (uintptr_t)blk;
    uint32_t w = *(const uint32_t *)(a & ~(uintptr_t)3);
    c.d = half_bits_to_float((a & 2u) ? (w >> 16) : w);
    return c;
}

MOE_DEV float cb2_dot(const CB2Chunk &c, const float *x, const uint32_t *cb_lds) {
    float s = 0.f;
#pragma unroll
    for (int g = 0; g < 8; ++g) {
        uint32_t idx = ((g < 4 ? c.idx_lo : c.idx_hi) >> (8 * (g & 3))) & 0xFFu;
        uint32_t sg = ((g < 4 ? c.sg_lo : c.sg_hi) >> (8 * (g & 3))) & 0xFFu;
        uint32_t r0 = cb_lds[2 * idx], r1 = cb_lds[2 * idx + 1];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            int v = (int)(int8_t)((j < 4 ? r0 : r1) >> (8 * (j & 3)));
            float f = (float)v;
            f = __uint_as_float(__float_as_uint(f) ^ (((sg >> j) & 1u) << 31));
            s = __builtin_fmaf(f, x[8 * g + j], s);
        }
    }
    return c.d * s;
}

// Decoded values of the same chunks (exact: every product fits in fp32 and the
// single rounding of the Q2K difference is done by one fused multiply-add).
MOE_DEV void q2k_values(const Q2KChunk &c, float *w) {
    float d = half_bits_to_float(c.dd), dmin = half_bits_to_float(c.dd >> 16);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        uint32_t smb = (c.sm >> (8 * g)) & 0xFFu;
        float off = dmin * (float)(smb >> 4);
        float sc = (float)(smb & 15u);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float q = (float)((c.qs[g] >> (2 * i)) & 3u);
            w[16 * g + i] = __builtin_fmaf(d, sc * q, -off);
        }
    }
}

MOE_DEV void q8_block_values(const uint8_t *blk, float *w) {
    // one 34-byte block at a 2-byte aligned address
    uint32_t dlo, dhi;
    load_8_at_even(blk, dlo, dhi);
    float d = half_bits_to_float(dlo);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint32_t lo, hi;
        load_8_at_even(blk + 2 + 8 * i, lo, hi);
#pragma unroll
        for (int n = 0; n < 4; ++n) {
            w[8 * i + n] = d * (float)(int8_t)(lo >> (8 * n));
            w[8 * i + 4 + n] = d * (float)(int8_t)(hi >> (8 * n));
        }
    }
}

MOE_DEV void cb2_values(const CB2Chunk &c, const uint32_t *cb, float *w) {
#pragma unroll
    for (int g = 0; g < 8; ++g) {
        uint32_t idx = ((g < 4 ? c.idx_lo : c.idx_hi) >> (8 * (g & 3))) & 0xFFu;
        uint32_t sg = ((g < 4 ? c.sg_lo : c.sg_hi) >> (8 * (g & 3))) & 0xFFu;
        uint32_t r0 = cb[2 * idx], r1 = cb[2 * idx + 1];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            int v = (int)(int8_t)((j < 4 ? r0 : r1) >> (8 * (j & 3)));
            if ((sg >> j) & 1u) v = -v;
            w[8 * g + j] = c.d * (float)v;
        }
    }
}

template <int FMT>
MOE_DEV float chunk_dot(const uint8_t *base, int64_t i0, const float *x, const uint32_t *cb_lds) {
    if constexpr (FMT == MOE_Q2K) {
        return q2k_dot(q2k_load(base, i0), x);
    } else if constexpr (FMT == MOE_Q8_0) {
        return q8_dot(q8_load(base, i0), x);
    } else {
        return cb2_dot(cb2_load(base, i0), x, cb_lds);
    }
}

// ---- workspace layout -------------------------------------------------------

struct RouterPlan {
    int kc;      // router rows (k) per partial-sum chunk
    int nchunk;  // D / kc
    int tt;      // tokens per router block
};

__host__ inline RouterPlan router_plan(int T, int D) {
    RouterPlan p;
    if (T <= 4) { p.kc = 16; p.tt = T < 1 ? 1 : T; }
    else if (T <= 64) { p.kc = 64; p.tt = 8; }
    else { p.kc = 1024; p.tt = 32; }
    while (p.kc > D) p.kc >>= 1;
    p.nchunk = D / p.kc;
    return p;
}

struct Workspace {
    double *partial;      // [nchunk][T][E]
    int32_t *topk_idx;    // routing kept in the workspace when the caller gives none
    float *topk_w;
    int32_t *count, *offset, *perm, *pos, *active, *n_active;
    float *h;             // [T*k][F] fp32 (F32 mode) or bf16 pairs (BF16 mode)
    float *hs;            // [T][Fs]
    float *ypart;         // [T*k][D]
    float *ys;            // [T][D]
    size_t bytes;
};

__host__ inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

__host__ inline Workspace workspace_layout(const moe_layer_desc *d, int32_t T, void *base) {
    Workspace w;
    size_t off = 0;
    char *b = (char *)base;
    int32_t E = d->n_expert, k = d->n_expert_used, D = d->n_embd, F = d->n_ff_exp, Fs = d->n_ff_shared;
    int64_t P = (int64_t)T * k;
    RouterPlan rp = router_plan(T, D);
    auto take = [&](size_t n) {
        size_t at = off;
        off = align_up(off + n, 256);
        return b ? (void *)(b + at) : nullptr;
    };
    w.partial = (double *)take(sizeof(double) * (size_t)rp.nchunk * (size_t)T * (size_t)E);
    w.topk_idx = (int32_t *)take(sizeof(int32_t) * (size_t)P);
    w.topk_w = (float *)take(sizeof(float) * (size_t)P);
    w.count = (int32_t *)take(sizeof(int32_t) * (size_t)E);
    w.offset = (int32_t *)take(sizeof(int32_t) * (size_t)(E + 1));
    w.perm = (int32_t *)take(sizeof(int32_t) * (size_t)P);
    w.pos = (int32_t *)take(sizeof(int32_t) * (size_t)P);
    w.active = (int32_t *)take(sizeof(int32_t) * (size_t)E);
    w.n_active = (int32_t *)take(sizeof(int32_t) * 4);
    w.h = (float *)take(sizeof(float) * (size_t)P * (size_t)F);
    w.hs = (float *)take(sizeof(float) * (size_t)T * (size_t)(Fs > 0 ? Fs : 1));
    w.ypart = (float *)take(sizeof(float) * (size_t)P * (size_t)D);
    w.ys = (float *)take(sizeof(float) * (size_t)T * (size_t)D);
    w.bytes = off;
    return w;
}

// ---- launches (defined in the kernel files) -----------------------------------

struct RoutingPtrs {
    int32_t *topk_idx;
    float *topk_w;
    int32_t *count, *offset, *perm, *pos, *active, *n_active;
};

hipError_t launch_route(const moe_layer_desc *d, const void *x, int32_t T, int32_t x_type, const RoutingPtrs &r,
                        const Workspace &ws, hipStream_t s);
hipError_t launch_ffn_decode(const moe_layer_desc *d, const void *x, int32_t T, int32_t x_type,
                             const RoutingPtrs &r, float *y, uint32_t flags, const Workspace &ws, hipStream_t s);
hipError_t launch_rmsnorm(const float *x, const float *gamma, float eps, int32_t T, int32_t D, float *out,
                          hipStream_t s);
hipError_t launch_dequant(int32_t type, const void *src, int64_t n, const int8_t *cb, int32_t out_type, void *dst,
                          hipStream_t s);

}  // namespace moe
