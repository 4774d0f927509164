// common.h - device helpers shared by the gfx950 kernels of the routed MoE
// block: block-format decoders, wave64 reductions, number conversions, and
// the workspace layout the host code and the kernels agree on.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <type_traits>

#include "../../include/moe.h"

#define MOE_DEV __device__ __forceinline__

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

namespace moe {

constexpr int kWave = 64;
constexpr int kMaxExperts = 1024;
constexpr int kMaxUsed = 16;

// Block geometry of the three weight formats.
constexpr int kQ2KBytes = 84, kQ8Bytes = 34, kCB2Bytes = 66, kQ4KBytes = 144;

__host__ __device__ inline int64_t fmt_block_weights(int fmt) { return fmt == MOE_Q8_0 ? 32 : 256; }
__host__ __device__ inline int64_t fmt_block_bytes(int fmt) {
    return fmt == MOE_Q2K ? kQ2KBytes : (fmt == MOE_Q8_0 ? kQ8Bytes : (fmt == MOE_Q4K ? kQ4KBytes : kCB2Bytes));
}
__host__ __device__ inline int64_t fmt_bytes(int fmt, int64_t n) {
    return n / fmt_block_weights(fmt) * fmt_block_bytes(fmt);
}

// ---- scalar conversions ---------------------------------------------------

// two floats -> a bf16 pair (lo in the low half), each rounded to nearest even
MOE_DEV uint32_t bf16x2_rne(float lo, float hi) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2){lo, hi}, b2));
}

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

// Byte N of v as a float, in one instruction (the compiler would extract
// the byte first).
template <int N>
MOE_DEV float byte_to_float(uint32_t v) {
    float f;
    if constexpr (N == 0) __asm__("v_cvt_f32_ubyte0 %0, %1" : "=v"(f) : "v"(v));
    else if constexpr (N == 1) __asm__("v_cvt_f32_ubyte1 %0, %1" : "=v"(f) : "v"(v));
    else if constexpr (N == 2) __asm__("v_cvt_f32_ubyte2 %0, %1" : "=v"(f) : "v"(v));
    else __asm__("v_cvt_f32_ubyte3 %0, %1" : "=v"(f) : "v"(v));
    return f;
}

// 8 bytes starting at a 2-byte aligned address, assembled from aligned dwords.
MOE_DEV void load_8_at_even(const uint8_t *p, uint32_t &lo, uint32_t &hi) {
    // aligned dwords from p rounded down to 4 bytes (a third one only when p
    // is 2 bytes into a dword), then a byte shift; the address is formed by
    // pointer arithmetic on p so that the compiler keeps its address space
    // (an LDS pointer stays an LDS read instead of a flat one)
    const uint32_t s = (uint32_t)((uintptr_t)p & 3u);  // 0 or 2
    const uint32_t *q = (const uint32_t *)(p - s);
    const uint32_t w0 = q[0], w1 = q[1];
    if (s == 0) {
        lo = w0;
        hi = w1;
    } else {
        const uint32_t w2 = q[2];
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

// Q4K: 64 weights = sub-blocks 2s and 2s+1 of one 144-byte block: 32 code
// bytes (weight i in bits 4*(i%2) of byte i/2), the two 6-bit scales and
// mins from the packed 12 bytes, and d, dmin.
struct Q4KChunk {
    u32x4 qa, qb;       // code bytes 0-15 and 16-31 of the chunk
    uint32_t sc, mn;    // scale and min of the two sub-blocks (bytes 0 and 1)
    uint32_t dd;        // fp16 d (low half) and dmin (high half)
};

MOE_DEV uint32_t six_bits(uint32_t w0, uint32_t w1, uint32_t w2, int f) {  // field f of the 96-bit scales
    const int bit = 6 * f, word = bit >> 5, sh = bit & 31;
    const uint32_t lo = word == 0 ? w0 : (word == 1 ? w1 : w2);
    const uint32_t hi = word == 0 ? w1 : (word == 1 ? w2 : 0u);
    const uint32_t v = sh == 0 ? lo : ((lo >> sh) | (hi << (32 - sh)));
    return v & 63u;
}

MOE_DEV Q4KChunk q4k_load(const uint8_t *base, int64_t i0) {
    const uint8_t *blk = base + (i0 >> 8) * kQ4KBytes;
    const int sub = (int)((i0 >> 6) & 3);
    Q4KChunk c;
    c.qa = load_u32x4(blk + 16 + 32 * sub);
    c.qb = load_u32x4(blk + 32 + 32 * sub);
    const uint32_t w0 = load_u32(blk + 4), w1 = load_u32(blk + 8), w2 = load_u32(blk + 12);
    c.sc = six_bits(w0, w1, w2, 2 * sub) | (six_bits(w0, w1, w2, 2 * sub + 1) << 8);
    c.mn = six_bits(w0, w1, w2, 8 + 2 * sub) | (six_bits(w0, w1, w2, 9 + 2 * sub) << 8);
    c.dd = load_u32(blk);
    return c;
}

// code byte j of the chunk (weights 2j, 2j+1)
MOE_DEV uint32_t q4k_byte_word(const Q4KChunk &c, int w) { return w < 4 ? c.qa[w] : c.qb[w - 4]; }

MOE_DEV void q4k_values(const Q4KChunk &c, float *w) {
    const float d = half_bits_to_float(c.dd), dmin = half_bits_to_float(c.dd >> 16);
#pragma unroll
    for (int h = 0; h < 2; ++h) {  // sub-block: weights 32h .. 32h+31
        const float sc = (float)((c.sc >> (8 * h)) & 63u), off = dmin * (float)((c.mn >> (8 * h)) & 63u);
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            const int k = 32 * h + i;
            const float q = (float)((q4k_byte_word(c, k >> 3) >> (8 * ((k >> 1) & 3) + 4 * (k & 1))) & 15u);
            w[k] = __builtin_fmaf(d, sc * q, -off);
        }
    }
}

// sum_i (d*sc_j*q_i - dmin*m_j) x_i over the two sub-blocks, fp32
MOE_DEV float q4k_dot(const Q4KChunk &c, const float *x) {
    const float d = half_bits_to_float(c.dd), dmin = half_bits_to_float(c.dd >> 16);
    float acc = 0.f;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        float sq = 0.f, sx = 0.f;
#pragma unroll
        for (int wd = 0; wd < 4; ++wd) {  // 4 words of code bytes: weights 32h + 8wd .. +7
            const uint32_t v = q4k_byte_word(c, 4 * h + wd);
            const uint32_t ev = v & 0x0F0F0F0Fu, od = (v >> 4) & 0x0F0F0F0Fu;
            const float *xs = x + 32 * h + 8 * wd;
            sq = __builtin_fmaf(byte_to_float<0>(ev), xs[0], sq);
            sq = __builtin_fmaf(byte_to_float<0>(od), xs[1], sq);
            sq = __builtin_fmaf(byte_to_float<1>(ev), xs[2], sq);
            sq = __builtin_fmaf(byte_to_float<1>(od), xs[3], sq);
            sq = __builtin_fmaf(byte_to_float<2>(ev), xs[4], sq);
            sq = __builtin_fmaf(byte_to_float<2>(od), xs[5], sq);
            sq = __builtin_fmaf(byte_to_float<3>(ev), xs[6], sq);
            sq = __builtin_fmaf(byte_to_float<3>(od), xs[7], sq);
#pragma unroll
            for (int i = 0; i < 8; ++i) sx += xs[i];
        }
        const float sc = (float)((c.sc >> (8 * h)) & 63u), mn = (float)((c.mn >> (8 * h)) & 63u);
        acc = __builtin_fmaf(d * sc, sq, acc);
        acc = __builtin_fmaf(-dmin * mn, sx, acc);
    }
    return acc;
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
    const uint32_t s2 = (uint32_t)((uintptr_t)blk & 2u);  // the block starts 0 or 2 bytes into a dword
    const uint32_t w = *(const uint32_t *)(blk - s2);
    c.d = half_bits_to_float(s2 ? (w >> 16) : w);
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

// ---- fp16 dot2 path ------------------------------------------------------
// v_dot2_f32_f16 multiplies two fp16 pairs exactly and accumulates in fp32.
// Weight codes enter as exact fp16 values; the activations as a pair of fp16
// numbers hi + lo (x*S = hi + lo to about 2^-22 relative), scaled per 64-value
// chunk by a power of two S so that nothing overflows.  Q2K codes are taken
// straight from their bit field with one AND: code q at bits 2m..2m+1 of a
// half is the fp16 subnormal q*4^m*2^-24, so the matching activation carries
// the factor 4^-m and every product is q*x*S*2^-24.

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __fp16 fp16x2_t __attribute__((ext_vector_type(2)));

MOE_DEV half2_t as_h2(uint32_t v) { return __builtin_bit_cast(half2_t, v); }

MOE_DEV float dot2(uint32_t a, uint32_t b, float c) { return __builtin_amdgcn_fdot2(as_h2(a), as_h2(b), c, false); }

// hi/lo fp16 pair of (a, b), both already scaled: hi rounds toward zero, lo
// holds the rest (exact in fp32), so hi + lo matches a, b to about 2^-22.
MOE_DEV void split2(float a, float b, uint32_t &hi, uint32_t &lo) {
    fp16x2_t h = __builtin_amdgcn_cvt_pkrtz(a, b);
    hi = __builtin_bit_cast(uint32_t, h);
    lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(a - (float)h[0], b - (float)h[1]));
}

// power-of-two scale for 64 activations: max|x| * S in [2^13, 2^14)
MOE_DEV float chunk_scale(const float *x, float &inv24) {
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < 64; ++i) m = fmaxf(m, fabsf(x[i]));
    int e = m > 0.f ? (int)((__float_as_uint(m) >> 23) & 0xFF) - 127 : 0;
    e = max(-100, min(100, e));
    inv24 = __uint_as_float((uint32_t)(127 + 11 + e) << 23);  // 2^24 / S
    return __uint_as_float((uint32_t)(127 + 13 - e) << 23);   // S
}

// Prepared activations for Q2K rows, in integers: a record of 10 dwords per
// group of 16 values v.  With S = 32512 / max|v|, c_i = rint(v_i * S) is split
// as c_i = 256 * a_i + b_i, a_i in [-127, 127], b_i in [-128, 127]; dword j of
// a[] holds a of positions j, 4+j, 8+j, 12+j in bytes 0..3 (the same order as
// the Q2K codes of one group after a shift by 2j and a byte mask), likewise
// b[].  sx is the fp32 sum of the 16 values, inv = 1 / S.  The dot of 16
// codes with the group is then inv * (256 * sum q*a + sum q*b), the two sums
// from v_dot4_i32_i8; |v_i - inv * c_i| <= inv / 2, a 2^-16 fraction of the
// group's largest magnitude.  A lane's 64 weights use 4 consecutive records.
struct Rec16 {
    uint32_t a[4], b[4];
    float sx, inv;
};
constexpr int kRec16Dwords = 10;
constexpr float kRec16Max = 32512.f;

struct XQ2K {
    Rec16 g[4];
};

// integer code of v for a group scale S, as (a, b) bytes
MOE_DEV void rec16_split(float v, float S, int &hi, int &lo) {
    const int c = (int)__builtin_rintf(v * S);
    hi = (c + 128) >> 8;
    lo = c - 256 * hi;
}

// per-lane preparation of the lane's 64 activations
MOE_DEV void prep_q2k(const float *x, XQ2K &p) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const float *v = x + 16 * g;
        float m = 0.f, s = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            m = fmaxf(m, fabsf(v[i]));
            s += v[i];
        }
        const float S = m > 0.f ? kRec16Max / m : 0.f;
        p.g[g].sx = s;
        p.g[g].inv = m / kRec16Max;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            uint32_t A = 0, B = 0;
#pragma unroll
            for (int n = 0; n < 4; ++n) {
                int hi, lo;
                rec16_split(v[4 * n + j], S, hi, lo);
                A |= (uint32_t)(hi & 0xFF) << (8 * n);
                B |= (uint32_t)(lo & 0xFF) << (8 * n);
            }
            p.g[g].a[j] = A;
            p.g[g].b[j] = B;
        }
    }
}

// Wave-cooperative preparation of ngroups (<= 4) groups: lane l holds the
// value at position l % 16 of group l / 16; the records go to out[(l / 16) *
// 10 ...].  All lanes of the wave must call it.
// NAT: natural byte order instead (byte i % 4 of dword i / 4 holds value i),
// the order of a codebook group's 8 values.
template <bool NAT = false>
MOE_DEV void prep16_wave(float v, uint32_t *out, int ngroups = 4) {
    const int lane = threadIdx.x & 63, pos = lane & 15;
    float m = fabsf(v), s = v;
#pragma unroll
    for (int o = 1; o <= 8; o <<= 1) {  // over the 16 lanes of the group
        m = fmaxf(m, __shfl_xor(m, o, kWave));
        s += __shfl_xor(s, o, kWave);
    }
    const float S = m > 0.f ? kRec16Max / m : 0.f;
    int hi, lo;
    rec16_split(v, S, hi, lo);
    uint32_t A, B;
    if constexpr (NAT) {
        // lanes 4j..4j+3 of the group gather dword j, which then moves to
        // lane j (A) and lane 4 + j (B) of the group
        A = (uint32_t)(hi & 0xFF) << (8 * (pos & 3));
        B = (uint32_t)(lo & 0xFF) << (8 * (pos & 3));
        A |= __shfl_xor(A, 1, kWave);
        B |= __shfl_xor(B, 1, kWave);
        A |= __shfl_xor(A, 2, kWave);
        B |= __shfl_xor(B, 2, kWave);
        const int src = (lane & ~15) + 4 * (pos & 3);
        A = __shfl(A, src, kWave);
        B = __shfl(B, src, kWave);
    } else {
        // byte pos / 4 of dword pos % 4, gathered over the lanes of one residue
        A = (uint32_t)(hi & 0xFF) << (8 * (pos >> 2));
        B = (uint32_t)(lo & 0xFF) << (8 * (pos >> 2));
        A |= __shfl_xor(A, 4, kWave);
        B |= __shfl_xor(B, 4, kWave);
        A |= __shfl_xor(A, 8, kWave);
        B |= __shfl_xor(B, 8, kWave);
    }
    if ((lane >> 4) >= ngroups) return;
    uint32_t *rec = out + (lane >> 4) * kRec16Dwords;
    if (pos < 4) rec[pos] = A;
    else if (pos < 8) rec[pos] = B;  // dword pos - 4 of b[], at offset 4 + (pos - 4)
    else if (pos == 8) rec[8] = __float_as_uint(s);
    else if (pos == 9) rec[9] = __float_as_uint(m / kRec16Max);
}

MOE_DEV void load_q2k_prep(const uint32_t *rec4, XQ2K &p) {
    u32x4 *dst = (u32x4 *)&p;
#pragma unroll
    for (int i = 0; i < 4 * kRec16Dwords / 4; ++i) dst[i] = *(const u32x4 *)(rec4 + 4 * i);
}

MOE_DEV int sdot4(uint32_t a, uint32_t b, int c) { return __builtin_amdgcn_sdot4((int)a, (int)b, c, false); }

// sum_g inv_g * (d*sc_g*sum_i q_i c_i) - dmin * sum_g m_g * sx_g, the integer
// dot of each group exact in int32 (|sum| < 2^21)

// the scale nibbles (low) and min nibbles (high) of the 4 group bytes, each
// byte converted in place
MOE_DEV float q2k_dot2(const Q2KChunk &c, const XQ2K &p) {
    const float d = half_bits_to_float(c.dd), dmin = half_bits_to_float(c.dd >> 16);
    const uint32_t scs = c.sm & 0x0F0F0F0Fu, mns = (c.sm >> 4) & 0x0F0F0F0Fu;
    float acc_q = 0.f, acc_m = 0.f;
    auto group = [&](auto G) {
        constexpr int g = decltype(G)::value;
        const uint32_t q = c.qs[g];
        uint32_t t[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) t[j] = (q >> (2 * j)) & 0x03030303u;
        // sum_i q_i c_i = 256 A + B: the B chain starts from 256 A, so the
        // combination costs one shift and no zeroed accumulator
        int A = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) A = sdot4(t[j], p.g[g].a[j], A);
        int S = A << 8;
#pragma unroll
        for (int j = 0; j < 4; ++j) S = sdot4(t[j], p.g[g].b[j], S);
        const float sq = (float)S;
        acc_q = __builtin_fmaf(byte_to_float<g>(scs) * p.g[g].inv, sq, acc_q);
        acc_m = __builtin_fmaf(byte_to_float<g>(mns), p.g[g].sx, acc_m);
    };
    group(std::integral_constant<int, 0>());
    group(std::integral_constant<int, 1>());
    group(std::integral_constant<int, 2>());
    group(std::integral_constant<int, 3>());
    return d * acc_q - dmin * acc_m;
}

// CB2 chunk against natural-order int16 activation records: per group of 16
// values, the two codebook groups' signed int8 values (picked by byte
// permutes from a table entry {values, negated values}: selector byte j is
// j, or 4 + j when sign bit j is set) dotted with the hi and lo code halves,
// sum = 256 A + B exact in int32 (|values| <= 127), scaled by the group's
// 1/S; d * sum at the end.
MOE_DEV uint32_t cb2_sel(uint32_t nib) { return 0x03020100u + (((nib * 0x00204081u) & 0x01010101u) << 2); }

// bytewise negation of int8 values in [-127, 127]: (b ^ 0x7F) + 1 stays
// below 0x100 in every byte, so no carry crosses a byte
MOE_DEV uint32_t neg_bytes(uint32_t v) { return ((v ^ 0x7F7F7F7Fu) + 0x01010101u) ^ 0x80808080u; }

MOE_DEV float cb2_dot_int(const CB2Chunk &c, const XQ2K &p, const u32x4 *tab) {
    float acc = 0.f;
    auto group = [&](auto G) {
        constexpr int g = decltype(G)::value;
        uint32_t w[4];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const int q = 2 * g + hh;  // codebook group of the chunk
            const uint32_t idx = ((q < 4 ? c.idx_lo : c.idx_hi) >> (8 * (q & 3))) & 0xFFu;
            const uint32_t sg = ((q < 4 ? c.sg_lo : c.sg_hi) >> (8 * (q & 3))) & 0xFFu;
            const u32x4 e = tab[idx];
            w[2 * hh] = __builtin_amdgcn_perm(e[2], e[0], cb2_sel(sg & 15u));
            w[2 * hh + 1] = __builtin_amdgcn_perm(e[3], e[1], cb2_sel(sg >> 4));
        }
        int A = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) A = sdot4(w[j], p.g[g].a[j], A);
        int S = A << 8;
#pragma unroll
        for (int j = 0; j < 4; ++j) S = sdot4(w[j], p.g[g].b[j], S);
        acc = __builtin_fmaf((float)S, p.g[g].inv, acc);
    };
    group(std::integral_constant<int, 0>());
    group(std::integral_constant<int, 1>());
    group(std::integral_constant<int, 2>());
    group(std::integral_constant<int, 3>());
    return c.d * acc;
}

// scale S and 2^24/S for a set whose largest magnitude is m
MOE_DEV float group_scale(float m, float &inv24) {
    int e = m > 0.f ? (int)((__float_as_uint(m) >> 23) & 0xFF) - 127 : 0;
    e = max(-100, min(100, e));
    inv24 = __uint_as_float((uint32_t)(127 + 11 + e) << 23);
    return __uint_as_float((uint32_t)(127 + 13 - e) << 23);
}

// Activations of one lane chunk (64 values) for Q8_0 codes: pair i holds
// (x[2i], x[2i+1]) * S split into hi + lo, S a power of two per chunk; int8
// codes enter as the fp16 subnormal (q+128)*2^-24.  68 dwords: hi[32],
// lo[32], the sums of the two 32-blocks, 2^24 / S, one pad dword.
struct XQ8 {
    uint32_t hi[32], lo[32];
    float sx[2];  // sum of each 32-block of activations
    float inv;
    float pad;
};
constexpr int kXQ8Dwords = 68;

MOE_DEV void prep_q8(const float *x, XQ8 &p) {
    const float S = chunk_scale(x, p.inv);
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < 32; ++i) s += x[32 * b + i];
        p.sx[b] = s;
    }
#pragma unroll
    for (int i = 0; i < 32; ++i) split2(x[2 * i] * S, x[2 * i + 1] * S, p.hi[i], p.lo[i]);
    p.pad = 0.f;
}

// Wave-cooperative XQ8 record of one chunk: lane l holds value l.
MOE_DEV void prep8_wave(float v, uint32_t *rec) {
    const int lane = threadIdx.x & 63;
    float m = fabsf(v), s = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        m = fmaxf(m, __shfl_xor(m, o, kWave));
        if (o < 32) s += __shfl_xor(s, o, kWave);
    }
    float inv;
    const float S = group_scale(m, inv);  // max|v| * S in [2^13, 2^14)
    const float partner = __shfl_down(v, 1, kWave);
    if ((lane & 1) == 0) {
        uint32_t hi, lo;
        split2(v * S, partner * S, hi, lo);
        rec[lane >> 1] = hi;
        rec[32 + (lane >> 1)] = lo;
    }
    if ((lane & 31) == 0) rec[64 + (lane >> 5)] = __float_as_uint(s);
    if (lane == 0) {
        rec[66] = __float_as_uint(inv);
        rec[67] = 0u;
    }
}

// The same records, four chunks per wave at once: row q (16 lanes) of the
// wave takes one chunk, lane m of the row its values 4m..4m+3 in v.  The
// bits are prep8_wave's: the maximum does not depend on order, and each
// 32-value sum is the same tree of pairwise block sums (2, 4, 8, 16, 32
// values, each lane's own block first; fp32 addition is commutative), here
// in registers and DPP moves within the row instead of cross-lane shuffles.
template <int CTRL>
MOE_DEV float dpp_f32(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
MOE_DEV void prep8_rows(f32x4 v, uint32_t *rec) {
    const int m = threadIdx.x & 15;
    float mx = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
    float s = (v[0] + v[1]) + (v[2] + v[3]);
    mx = fmaxf(mx, dpp_f32<0xB1>(mx));  // quad_perm [1,0,3,2]: lane m ^ 1
    s += dpp_f32<0xB1>(s);
    mx = fmaxf(mx, dpp_f32<0x4E>(mx));  // quad_perm [2,3,0,1]: lane m ^ 2
    s += dpp_f32<0x4E>(s);
    mx = fmaxf(mx, dpp_f32<0x141>(mx));  // row_half_mirror: lane 7 - m of its 8
    s += dpp_f32<0x141>(s);
    mx = fmaxf(mx, dpp_f32<0x140>(mx));  // row_mirror: lane 15 - m
    float inv;
    const float S = group_scale(mx, inv);
    uint32_t h0, l0, h1, l1;
    split2(v[0] * S, v[1] * S, h0, l0);
    split2(v[2] * S, v[3] * S, h1, l1);
    *(uint2 *)(rec + 2 * m) = uint2{h0, h1};
    *(uint2 *)(rec + 32 + 2 * m) = uint2{l0, l1};
    if ((m & 7) == 0) rec[64 + (m >> 3)] = __float_as_uint(s);
    if (m == 0) *(uint2 *)(rec + 66) = uint2{__float_as_uint(inv), 0u};
}

MOE_DEV void load_q8_prep(const uint32_t *rec, XQ8 &p) {
    u32x4 *dst = (u32x4 *)&p;
#pragma unroll
    for (int i = 0; i < kXQ8Dwords / 4; ++i) dst[i] = *(const u32x4 *)(rec + 4 * i);
}

MOE_DEV float q8_dot2(const Q8Chunk &c, const XQ8 &p) {
    const float d0 = half_bits_to_float(c.w[0]), d1 = half_bits_to_float(c.w[8] >> 16);
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t v = __builtin_amdgcn_alignbyte(c.w[i + 1], c.w[i], 2) ^ 0x80808080u;  // bytes 2..33
        const uint32_t lo = __builtin_amdgcn_perm(0u, v, 0x0C010C00u), hi = __builtin_amdgcn_perm(0u, v, 0x0C030C02u);
        a0 = dot2(lo, p.hi[2 * i], a0);
        a0 = dot2(lo, p.lo[2 * i], a0);
        a0 = dot2(hi, p.hi[2 * i + 1], a0);
        a0 = dot2(hi, p.lo[2 * i + 1], a0);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t v = c.w[9 + i] ^ 0x80808080u;  // bytes 36..67
        const uint32_t lo = __builtin_amdgcn_perm(0u, v, 0x0C010C00u), hi = __builtin_amdgcn_perm(0u, v, 0x0C030C02u);
        a1 = dot2(lo, p.hi[16 + 2 * i], a1);
        a1 = dot2(lo, p.lo[16 + 2 * i], a1);
        a1 = dot2(hi, p.hi[17 + 2 * i], a1);
        a1 = dot2(hi, p.lo[17 + 2 * i], a1);
    }
    // sum (q+128) x = sum q x + 128 sum x
    return d0 * __builtin_fmaf(p.inv, a0, -128.0f * p.sx[0]) + d1 * __builtin_fmaf(p.inv, a1, -128.0f * p.sx[1]);
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

// Per-slot record for the expert kernels of the few-token schedule: expert
// e (-1: no expert in this slot), its first bucket position j0, its bucket
// size n and the token of each bucket entry, so that one load gives a wave
// everything it needs to address weights and activations.
struct SlotRec {
    int32_t e, j0, n, pad;
    uint32_t tok0, tok1, tok2, tok3;  // byte i of the 16 = token of bucket entry i
};

// The record with every field made wave-uniform (the slot index is uniform).
MOE_DEV SlotRec uniform_slot(const SlotRec *slots, int s) {
    const SlotRec v = slots[s];
    SlotRec r;
    r.e = __builtin_amdgcn_readfirstlane(v.e);
    r.j0 = __builtin_amdgcn_readfirstlane(v.j0);
    r.n = __builtin_amdgcn_readfirstlane(v.n);
    r.pad = 0;
    r.tok0 = (uint32_t)__builtin_amdgcn_readfirstlane((int)v.tok0);
    r.tok1 = (uint32_t)__builtin_amdgcn_readfirstlane((int)v.tok1);
    r.tok2 = (uint32_t)__builtin_amdgcn_readfirstlane((int)v.tok2);
    r.tok3 = (uint32_t)__builtin_amdgcn_readfirstlane((int)v.tok3);
    return r;
}

MOE_DEV int slot_token(const SlotRec &r, int j) {
    const uint64_t w = j < 8 ? ((uint64_t)r.tok1 << 32 | r.tok0) : ((uint64_t)r.tok3 << 32 | r.tok2);
    return (int)((w >> (8 * (j & 7))) & 0xFFu);
}

// Record of expert e, bucket start j0, size n, with the token bytes packed.
MOE_DEV SlotRec make_slot(int e, int j0, int n, uint64_t tlo, uint64_t thi) {
    return SlotRec{e, j0, n, 0, (uint32_t)tlo, (uint32_t)(tlo >> 32), (uint32_t)thi, (uint32_t)(thi >> 32)};
}

// ---- workspace layout -------------------------------------------------------

struct Workspace {
    double *logits;       // [T][E] fp64 router logits
    int32_t *topk_idx;    // routing kept in the workspace when the caller gives none
    float *topk_w;
    int32_t *count, *offset, *perm, *pos, *active, *n_active;
    float *h;             // [T*k][F] fp32
    float *hs;            // [T][Fs]
    float *ypart;         // [T*k][D]
    float *ys;            // [T][D]
    uint32_t *xp16;       // [T][D/16] records: x prepared for Q2K rows
    uint32_t *xq8;        // [T][D/64] records: x prepared for Q8_0 rows
    uint32_t *hp16;       // [T*k][F/16] records: h prepared for Q2K rows
    SlotRec *slots;       // [T*k] per-slot records of the few-token schedule
    // many-row bf16 path: int16 activation codes as two int8 planes per
    // 256-column block ([rows][n/256][512] bytes), group sums as bf16 pairs
    // ([rows][n/256][16] dwords) and scales, for x (gate/up) and h (down)
    uint8_t *pf_xq;
    uint32_t *pf_xs;
    float *pf_xinv;       // [T]
    int4 *pf_tiles;       // {expert, first bucket position, rows, 0}
    int32_t *pf_ntiles;
    uint16_t *pf_shw;     // shared expert weights as bf16 hi (gate, up, down) then lo halves
    uint16_t *pf_hsb;     // [T][Fs] shared h as a bf16 pair: hi = rne(h) here,
    uint16_t *pf_hsb_lo;  //          lo = rne(h - hi) here
    uint8_t *pf_hq;
    uint32_t *pf_hs;
    float *pf_hinv;       // [T*k]
    // shared expert of many fp32 rows on the matrix cores: int16 codes of x
    // (gate/up; their 1/S is pf_xinv) or hs (down), [T][n/64][32 dwords],
    // and hs rows' 1/S
    uint32_t *sg_aq;
    float *sg_ainv;       // [T]
    float *xn;            // [T][D] normalised rows of moe_block_forward (when not fused)
    // the two-pass router of many bf16 rows: per D slice, the logit sums of
    // pass 1 [kRtSplitMax][T][E] and the experts' sums of w^2 [kRtSplitMax][E]
    float *rt_part;
    float *rt_wn;
    size_t bytes;
};

constexpr int kPfTileRows = 64;  // pair rows per tile of the many-row bf16 path
constexpr int kRtSplitMax = 16;  // D slices of the two-pass router's first pass

// Routing of 17 to 127 rows with at most kRouteMidPairs pairs (the pairs
// are then sorted in one block) and at most 256 experts: the fp64 router
// splits the reduction over router_parts blocks per 16 x 16 tile (128
// columns a wave), whose partial sums the top-k selection adds as it reads
// them.  1: the router writes the logits themselves.
constexpr int kRouteMidPairs = 1024;
constexpr int kMaxRouterParts = 8;
__host__ __device__ inline int router_parts(int32_t T, int D, int k, int E) {
    if (T <= 16 || T >= 128 || D % 512 || (int64_t)T * k > kRouteMidPairs || E > 256) return 1;
    return D / 512 < kMaxRouterParts ? D / 512 : kMaxRouterParts;
}

// tiles of at most kPfTileRows pairs over the active experts
__host__ inline int pf_max_tiles(int32_t T, int k, int E) {
    const int64_t P = (int64_t)T * k;
    return (int)((P + kPfTileRows - 1) / kPfTileRows + (P < E ? P : E));
}

__host__ inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

__host__ inline Workspace workspace_layout(const moe_layer_desc *d, int32_t T, void *base) {
    Workspace w;
    size_t off = 0;
    char *b = (char *)base;
    int32_t E = d->n_expert, k = d->n_expert_used, D = d->n_embd, F = d->n_ff_exp, Fs = d->n_ff_shared;
    int64_t P = (int64_t)T * k;
    auto take = [&](size_t n) {
        size_t at = off;
        off = align_up(off + n, 256);
        return b ? (void *)(b + at) : nullptr;
    };
    w.logits = (double *)take(sizeof(double) * (size_t)T * (size_t)E * (size_t)router_parts(T, D, k, E));
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
    w.xp16 = (uint32_t *)take(sizeof(uint32_t) * kRec16Dwords * (size_t)T * (size_t)(D / 16));
    w.xq8 = (uint32_t *)take(sizeof(uint32_t) * kXQ8Dwords * (size_t)T * (size_t)(D / 64));
    w.hp16 = (uint32_t *)take(sizeof(uint32_t) * kRec16Dwords * (size_t)P * (size_t)(F / 16));
    w.slots = (SlotRec *)take(sizeof(SlotRec) * (size_t)P);
    w.pf_xq = (uint8_t *)take((size_t)T * (size_t)D * 2);
    w.pf_xs = (uint32_t *)take((size_t)T * (size_t)(D / 256 + 1) * 64);
    w.pf_xinv = (float *)take(sizeof(float) * (size_t)T);
    w.pf_tiles = (int4 *)take(sizeof(int4) * (size_t)pf_max_tiles(T, k, E));
    w.pf_ntiles = (int32_t *)take(sizeof(int32_t) * 4);
    w.pf_shw = (uint16_t *)take((size_t)6 * (size_t)Fs * (size_t)D * 2);
    w.pf_hsb = (uint16_t *)take((size_t)T * (size_t)Fs * 2);
    w.pf_hsb_lo = (uint16_t *)take((size_t)T * (size_t)Fs * 2);
    w.pf_hq = (uint8_t *)take((size_t)P * (size_t)F * 2);
    w.pf_hs = (uint32_t *)take((size_t)P * (size_t)(F / 256 + 1) * 64);
    w.pf_hinv = (float *)take(sizeof(float) * (size_t)P);
    w.sg_aq = (uint32_t *)take((size_t)T * (size_t)(D > Fs ? D : Fs) * 2);
    w.sg_ainv = (float *)take(sizeof(float) * (size_t)T);
    w.xn = (float *)take(sizeof(float) * (size_t)T * (size_t)D);
    const bool rt = T >= 128;  // the two-pass router may run (bf16 rows)
    w.rt_part = (float *)take(rt ? sizeof(float) * kRtSplitMax * (size_t)T * (size_t)E : 0);
    w.rt_wn = (float *)take(rt ? sizeof(float) * kRtSplitMax * (size_t)E : 0);
    w.bytes = off;
    return w;
}

// ---- launches (defined in the kernel files) -----------------------------------

struct RoutingPtrs {
    int32_t *topk_idx;
    float *topk_w;
    int32_t *count, *offset, *perm, *pos, *active, *n_active;
};

hipError_t launch_router_logits(const moe_layer_desc *d, const void *x, int32_t T, int32_t x_type,
                                 const Workspace &ws, hipStream_t s);
// x, x_type: the rows the logits came from (the two-pass router of many bf16
// rows computes the candidates' logits again from them)
hipError_t launch_route_finish(const moe_layer_desc *d, const void *x, int32_t T, int32_t x_type,
                               const RoutingPtrs &r, const Workspace &ws, hipStream_t s);
hipError_t launch_route(const moe_layer_desc *d, const void *x, int32_t T, int32_t x_type, const RoutingPtrs &r,
                        const Workspace &ws, hipStream_t s);
// decode schedule (few rows): stage 0 = all, 1..4 = its four kernels
bool small_path_ok(const moe_layer_desc *d, int32_t T);
bool small_route_ok(const moe_layer_desc *d, int32_t T);
hipError_t launch_small(const moe_layer_desc *d, const void *x, int32_t T, int32_t x_type, const RoutingPtrs &r,
                        float *y, uint32_t flags, const Workspace &ws, hipStream_t s, int stage, bool route,
                        const float *gamma = nullptr, float eps = 0.f);
// one fp32 token on the schedule without K2; with a gamma (Q2K or codebook
// gate/up rows) K1 also normalises x
bool t1_schedule_ok(const moe_layer_desc *d, int32_t T, int32_t x_type);
// the shared expert (Q8_0) of any number of fp32 rows as two int8 matrix-core
// GEMMs: stage 3 writes hs, stage 4 ys
bool shared_q8_mfma_ok(const moe_layer_desc *d);
hipError_t launch_shared_q8_mfma(const moe_layer_desc *d, int32_t T, const Workspace &ws, const float *ainv,
                                 hipStream_t s, int stage);
// any number of rows: stage 3 = gate/up, 4 = down + combine, 0 = both
hipError_t launch_ffn_large(const moe_layer_desc *d, const void *x, int32_t T, int32_t x_type, const RoutingPtrs &r,
                            float *y, uint32_t flags, const Workspace &ws, hipStream_t s, int stage);
// shared expert alone on the batched kernels: stage 3 writes hs, 4 writes ys
hipError_t launch_ffn_large_shared(const moe_layer_desc *d, const void *x, int32_t T, int32_t x_type,
                                   const RoutingPtrs &r, float *y, uint32_t flags, const Workspace &ws, hipStream_t s,
                                   int stage);
// y = ys + sum_s w_s * ypart[pos] in slot order (+ y when accumulating)
hipError_t launch_combine(const moe_layer_desc *d, const void *x, int32_t T, int32_t x_type, const RoutingPtrs &r,
                          float *y, uint32_t flags, const Workspace &ws, hipStream_t s);
// many rows with Q2K experts (bf16 rows, or fp32 rows beyond the decode
// schedule): MFMA grouped GEMMs
bool prefill_path_ok(const moe_layer_desc *d, int32_t T, int32_t x_type);
// shared_done: bf16 rows whose shared expert runs on another stream
// (launch_prefill_shared_bf16): the shared launches are left out here, and
// the routed down (which adds into the y that the shared down writes) waits
// for this event.
hipError_t launch_prefill(const moe_layer_desc *d, const void *x, int32_t T, int32_t x_type, const RoutingPtrs &r,
                          float *y, uint32_t flags, const Workspace &ws, hipStream_t s, int stage,
                          hipEvent_t shared_done = nullptr);
// bf16 rows: the shared expert alone (its Q8_0 weights split into bf16
// halves, gate/up -> hs, down -> y = ys (+ y)); it needs only x.
hipError_t launch_prefill_shared_bf16(const moe_layer_desc *d, const void *x, int32_t T, float *y, uint32_t flags,
                                      const Workspace &ws, hipStream_t s);
constexpr int kMaxHotlist = 16384;                  // entries one hot-list sort takes
constexpr int64_t kHotCountMax = (int64_t)1 << 39;  // counts are clamped below this in the sort key
hipError_t launch_count_selections(const int32_t *topk_idx, int32_t T, int32_t k, int32_t E, int32_t layer,
                                   int64_t *counts, hipStream_t s);
hipError_t launch_hotlist(const int64_t *counts, int32_t n, int32_t *order, int32_t *n_hot, hipStream_t s);
hipError_t launch_rmsnorm(const float *x, const float *gamma, float eps, int32_t T, int32_t D, float *out,
                          hipStream_t s);
hipError_t launch_dequant(int32_t type, const void *src, int64_t n, const int8_t *cb, int32_t out_type, void *dst,
                          hipStream_t s);
hipError_t launch_read_stream(const void *src, int64_t bytes, uint32_t *sink, int32_t blocks, hipStream_t s);

}  // namespace moe
