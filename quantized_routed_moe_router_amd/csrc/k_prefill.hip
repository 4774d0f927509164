// k_prefill.hip - the routed experts of many token rows (bf16 rows, and fp32
// rows beyond the few-token decode kernels) as grouped GEMMs on the matrix
// cores ("Understanding Dwarf Star", 5.3.7 steps
// 3-5: each active expert's bucket of pairs runs gate/up, SwiGLU, down and a
// weighted scatter into y; 2.8.2 the dequant-dot over 256-weight super-blocks;
// the Q2_K subsection for w = d*sc*q - dmin*m).
//
// A tile is up to 64 pairs of one expert (two 32-row MFMA subtiles).  A block
// of 8 waves streams one 256-weight super-block column of 512 weight rows
// (256 F-rows of gate and of up, or 512 down columns) per step through two
// LDS stages filled by global-to-LDS DMA; each wave owns 64 weight rows (two
// 32-row subtiles) against both pair subtiles, and each activation read from
// LDS feeds both of its row subtiles.  (The small variant: 4 waves, tiles of
// up to 32 pairs.)  Per super-block column:
//   sum_k w_k a_k = d * sum_k (sc*q)_k a_k - sum_g (dmin*m_g) * (sum_{k in g} a_k)
// The first sum runs on v_mfma_i32_32x32x32_i8: the codes sc*q (0..45) are
// exact int8 and the activations are int16 codes c = rint(a*S) split as
// c = 256*hi + lo (two int8 passes).  The integer result, exact in int32, is
// scaled by d in fp32.  The second sum runs on v_mfma_f32_32x32x16_bf16 with
// dmin*m (exact as a bf16 pair) against the group sums (a bf16 pair).
#include <cstddef>
#include <type_traits>

#include "ffn_dev.h"

namespace moe {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int kPfM = 64;                // pair rows per tile
constexpr int kPfWaveRows = 64;         // weight rows per wave (two 32-column MFMA subtiles)
constexpr int kPfARow = 33;             // 16-byte units per code row in LDS: hi 16 + lo 16 + 1 pad
constexpr float kPfCodeMax = 32512.f;   // |c| <= 32512 keeps hi in [-127, 127]

// 4-unit rows (64 bytes): distinct banks for 8 and for 16 consecutive rows
MOE_DEV int sum_swz(int r) { return ((r >> 1) + (r >> 3)) & 3; }

// One super-block column in LDS.  Codes of row r, unit u (0..15 hi, 16..31
// lo) sit at a[33 r + u] (one pad unit per row); group sums of row r, unit u
// (0, 1 sH; 2, 3 sL) at s[4*(r*4 + (u ^ sum_swz(r)))...]; staged weight row R
// (wave R / 64 copies rows 64w..64w+63): scale bytes and codes (the 80 bytes
// after d, dmin) at b[5R..5R+4], d and dmin at dd[R].  The pad and the
// swizzle put the 16-byte reads of 16 consecutive rows on distinct banks
// (and of any 8 consecutive rows).
// W = 8: tiles of up to 64 pairs, 512 weight rows per stage; W = 4 (the
// small variant, when no tile can exceed 32 pairs): 32 pairs, 256 weight
// rows, 40 KB per stage, so that two blocks fit a compute unit.
constexpr int pf_m(int W) { return W == 8 ? 64 : 32; }
template <int W>
struct PfStageT {
    u32x4 a[pf_m(W) * kPfARow];
    uint32_t s[pf_m(W) * 16];
    u32x4 b[kPfWaveRows * W * 5];
    uint32_t dd[kPfWaveRows * W];
};
typedef PfStageT<8> PfStage;

struct PfArgs {
    const uint8_t *w0, *w1;  // gate and up (mode 0) or down (mode 1), expert-major Q2K
    int64_t expert_bytes;
    int n_in;                // reduction length: D (mode 0) or F (mode 1)
    const uint8_t *aq;       // activation codes [rows][n_in/256][512]
    const uint32_t *as;      // group sums in code units [rows][n_in/256][16]
    const float *ainv;       // 1/S of each row: [T] (mode 0) or [T*k] by bucket position (mode 1)
    const int4 *tiles;       // {expert, first bucket position, rows, 0}
    const int32_t *n_tiles;
    const int32_t *perm;
    const float *topk_w;
    int k;
    int D, F;
    float *hf;               // mode 0 output: h in fp32, [T*k][F] by bucket position
    float *y;                // mode 1 output: w * y_pair added into y by atomics
    float *ypart;            // mode 1 output instead, when set: unweighted y_pair rows [T*k][D] by bucket position
};

// Global-to-LDS copies of 16 and 4 bytes per lane (lane l writes lds_wave +
// size * l; lds_wave uniform over the wave), issued as inline assembly: the
// compiler then sees no LDS store to order against the reads of the other
// stage (its own tracking of such copies falls back to waiting for all of
// them), and the kernel counts them with explicit vmcnt waits instead.  One
// wait state separates the m0 write from the copy.

MOE_DEV void pf_dma16(const void *g, void *lds_wave) {
    __asm__ volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                     :
                     : "{m0}"(__builtin_amdgcn_readfirstlane(lds_addr(lds_wave))), "v"(g)
                     : "memory");
}

// a pointer that is the same in every lane, moved to scalar registers
MOE_DEV const void *wave_uniform(const void *p) {
    const uint64_t v = (uint64_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v), hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return (const void *)(((uint64_t)hi << 32) | lo);
}

// The same with a wave-uniform base in scalar registers and a 32-bit lane
// offset.  The base usually comes from v_readfirstlane, and a VALU write of an
// SGPR needs 5 wait states before a vector memory instruction reads that SGPR;
// the compiler cannot see that the assembly is such an instruction, so the
// wait states are part of it (s_nop 4 = 5, which also covers the m0 write).
MOE_DEV void pf_dma16s(const void *base, uint32_t off, void *lds_wave) {
    __asm__ volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %1, %2"
                     :
                     : "{m0}"(__builtin_amdgcn_readfirstlane(lds_addr(lds_wave))), "v"(off), "s"(wave_uniform(base))
                     : "memory");
}

MOE_DEV void pf_dma4s(const void *base, uint32_t off, void *lds_wave) {
    __asm__ volatile("s_nop 4\n\tglobal_load_lds_dword %1, %2"
                     :
                     : "{m0}"(__builtin_amdgcn_readfirstlane(lds_addr(lds_wave))), "v"(off), "s"(wave_uniform(base))
                     : "memory");
}

// the same with the LDS address (m0) already wave-uniform
MOE_DEV void pf_dma16u(const void *base, uint32_t off, uint32_t m0) {
    __asm__ volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %1, %2" : : "{m0}"(m0), "v"(off), "s"(base) : "memory");
}

MOE_DEV void pf_dma4u(const void *base, uint32_t off, uint32_t m0) {
    __asm__ volatile("s_nop 4\n\tglobal_load_lds_dword %1, %2" : : "{m0}"(m0), "v"(off), "s"(base) : "memory");
}

MOE_DEV void pf_dma4(const void *g, void *lds_wave) {
    __asm__ volatile("s_nop 0\n\tglobal_load_lds_dword %1, off"
                     :
                     : "{m0}"(__builtin_amdgcn_readfirstlane(lds_addr(lds_wave))), "v"(g)
                     : "memory");
}

// wait until at most N vector memory operations of the wave are outstanding
// (vmcnt is 6 bits: low 4 at [3:0], high 2 at [15:14])
template <int N>
MOE_DEV void vmem_wait_at_most() {
    static_assert(N >= 0 && N < 64, "vmcnt immediate");
    __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// fp32 -> bf16, round to nearest even (the hardware conversion; inputs here
// are finite)
MOE_DEV uint16_t bf16_rne(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }


// 16 activations -> t-ordered int8 halves (byte 4j+n of the unit holds value
// 4n+j, the order the code dwords of a Q2K group take after >> 2j & 0x03030303)
MOE_DEV void pf_codes16(const float *v, float S, u32x4 &hi, u32x4 &lo) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        uint32_t H = 0, L = 0;
#pragma unroll
        for (int n = 0; n < 4; ++n) {
            const int c = (int)__builtin_rintf(v[4 * n + j] * S);
            const int hv = (c + 128) >> 8;
            H |= (uint32_t)(hv & 0xFF) << (8 * n);
            L |= (uint32_t)((c - 256 * hv) & 0xFF) << (8 * n);
        }
        hi[j] = H;
        lo[j] = L;
    }
}

// Activation codes of rows of n bf16 or fp32 values (x for gate/up, h for
// down): one block per row, a thread per group of 16.  S = 32512 / max|row|; the group
// sums are kept in code units (sum * S), so a whole product stays in code
// units until the row's 1/S at the end.
// 16 consecutive values of a bf16 or fp32 row
template <int XT>
MOE_DEV void pf_load16(const void *x, int64_t i0, float *v) {
    if constexpr (XT == MOE_BF16) {
        const u32x4 *src = (const u32x4 *)((const uint16_t *)x + i0);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const u32x4 w = src[i];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                v[8 * i + 2 * j] = bf16_bits_to_float(w[j] & 0xFFFFu);
                v[8 * i + 2 * j + 1] = bf16_bits_to_float(w[j] >> 16);
            }
        }
    } else {
        const f32x4 *src = (const f32x4 *)((const float *)x + i0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const f32x4 w = src[i];
#pragma unroll
            for (int j = 0; j < 4; ++j) v[4 * i + j] = w[j];
        }
    }
}

// Tiles of at most 64 pairs over the active experts, ascending expert id:
// one wave, 64 experts at a time, tile offsets by a prefix sum over lanes.
MOE_DEV void pf_tiles_wave(const int32_t *active, const int32_t *n_active, const int32_t *count,
                           const int32_t *offset, int4 *tiles, int32_t *n_tiles) {
    const int lane = threadIdx.x & 63, n = n_active[0];
    int base = 0;
    for (int i0 = 0; i0 < n; i0 += 64) {
        const int i = i0 + lane;
        const int e = i < n ? active[i] : 0, c = i < n ? count[e] : 0, o = i < n ? offset[e] : 0;
        const int nt = (c + kPfM - 1) / kPfM;
        int incl = nt;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int v = __shfl_up(incl, d, kWave);
            if (lane >= d) incl += v;
        }
        const int first = base + incl - nt;
        for (int t = 0; t < nt; ++t) tiles[first + t] = make_int4(e, o + t * kPfM, min(kPfM, c - t * kPfM), 0);
        base += __shfl(incl, 63, kWave);
    }
    if (lane == 0) n_tiles[0] = base;
}

// fp32 rows also feed the shared expert's int8 GEMMs (ffn_dev.h): sg_rec,
// when set, takes each row's records at the same scale; blocks from nrows on
// code the rows of rows2 (n2 values each, hs) for those GEMMs alone.  Block
// tiles_block (when >= 0, after all of those) lays out the GEMM tiles
// instead, with its first wave.
struct PfPrepShared {
    uint32_t *sg_rec;     // records of x's rows, or null
    int nrows;            // blocks that code x (the rest code rows2)
    const float *rows2;
    int n2;
    uint32_t *rec2;
    float *inv2;
    int tiles_block;
    const int32_t *active, *n_active, *count, *offset;
    int4 *tiles;
    int32_t *n_tiles;
};

template <int XT>
__global__ void __launch_bounds__(256) pf_prep_rows_kernel(const void *x, int n, uint8_t *xq, uint32_t *xs,
                                                           float *xinv, PfPrepShared extra) {
    __shared__ float wmax[4];
    if ((int)blockIdx.x == extra.tiles_block) {
        if (threadIdx.x < 64)
            pf_tiles_wave(extra.active, extra.n_active, extra.count, extra.offset, extra.tiles, extra.n_tiles);
        return;
    }
    if ((int)blockIdx.x >= extra.nrows) {  // uniform over the block
        const int r = (int)blockIdx.x - extra.nrows;
        sgq_prep_row(extra.rows2 + (int64_t)r * extra.n2, extra.n2,
                     extra.rec2 + (int64_t)r * (extra.n2 / 64) * kSgqPairDw, extra.inv2 + r, wmax);
        return;
    }
    const int t = blockIdx.x, ng = n >> 4;
    float mt = 0.f;
    // rows of up to 4096 values: a thread's one group stays in registers
    // between the two passes (longer rows read theirs again)
    float v0[16];
    if (ng <= 256 && (int)threadIdx.x < ng) {
        pf_load16<XT>(x, (int64_t)t * n + 16 * threadIdx.x, v0);
#pragma unroll
        for (int i = 0; i < 16; ++i) mt = fmaxf(mt, fabsf(v0[i]));
    }
    for (int g = threadIdx.x; ng > 256 && g < ng; g += 256) {
        float v[16];
        pf_load16<XT>(x, (int64_t)t * n + 16 * g, v);
#pragma unroll
        for (int i = 0; i < 16; ++i) mt = fmaxf(mt, fabsf(v[i]));
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) mt = fmaxf(mt, __shfl_xor(mt, o, kWave));
    if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = mt;
    __syncthreads();
    const float m = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
    const float S = m > 0.f ? kPfCodeMax / m : 0.f;
    if (threadIdx.x == 0) xinv[t] = m / kPfCodeMax;
    const int nkb = n >> 8;
    for (int g = threadIdx.x; g < ng; g += 256) {
        float v[16];
        if (ng <= 256) {
#pragma unroll
            for (int i = 0; i < 16; ++i) v[i] = v0[i];
        } else {
            pf_load16<XT>(x, (int64_t)t * n + 16 * g, v);
        }
        const int kb = g >> 4, gi = g & 15;
        float sum = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) sum += v[i];
        const float sc = sum * S;
        const uint16_t sh = bf16_rne(sc);
        const uint16_t sl = bf16_rne(sc - bf16_bits_to_float(sh));
        u32x4 hi, lo;
        pf_codes16(v, S, hi, lo);
        uint8_t *base = xq + ((int64_t)t * nkb + kb) * 512;
        const int unit = 2 * (gi & 7) + (gi >> 3);
        *(u32x4 *)(base + 16 * unit) = hi;
        *(u32x4 *)(base + 256 + 16 * unit) = lo;
        uint16_t *sb = (uint16_t *)(xs + ((int64_t)t * nkb + kb) * 16);
        sb[gi] = sh;
        sb[16 + gi] = sl;
    }
    if constexpr (XT == MOE_F32)
        if (extra.sg_rec)
            sgq_code_row((const float *)x + (int64_t)t * n, n, S, extra.sg_rec + (int64_t)t * (n / 64) * kSgqPairDw);
}

// y = ys (+ y when accumulating), or 0 / y without a shared expert: the
// routed pairs are then added by the down pass.
__global__ void __launch_bounds__(256) pf_y_init_kernel(const float *ys, float *y, int64_t n, int accumulate) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    float v = ys ? ys[i] : 0.f;
    if (accumulate) v += y[i];
    y[i] = v;
}

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// four byte codes (each <= 3) times sc (<= 15) bytewise, no carries: one
// packed 16-bit multiply
MOE_DEV uint32_t mul_bytes(uint32_t t, uint32_t sc) {
    const u16x2 p = __builtin_bit_cast(u16x2, t) * (u16x2){(unsigned short)sc, (unsigned short)sc};
    return __builtin_bit_cast(uint32_t, p);
}

MOE_DEV v8bf as_v8bf(const uint32_t (&w)[4]) {
    v8bf r;
    __builtin_memcpy(&r, w, 16);
    return r;
}

// Barrier for the LDS stages: a compiler-level memory fence only.  Each wave
// has already waited for its own DMA (vmcnt) and consumed its LDS reads, and
// a hardware fence here would also wait for the DMA of the next stage.
MOE_DEV void stage_barrier() {
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
}

// Linear block id -> (tile, column block), so that the column blocks of one
// tile run on one XCD (blocks go round-robin to the 8 XCDs): its activation
// rows are then fetched into that XCD's L2 once instead of into all of them.
// nb = column blocks per tile; the grid holds 8 * ceil(tiles / 8) * nb blocks.
MOE_DEV void xcd_tile_map(int L, int nb, int &tile, int &col) {
    const int xcd = L & 7, j = L >> 3;
    tile = xcd + 8 * (j / nb);
    col = j % nb;
}

// Mode 0: a column block is 256 F-rows; wave w < 4 owns gate rows
// 64w..64w+63, wave w >= 4 the same rows of up; writes h = silu(g) * u in
// fp32.  Mode 1: a column block is 512 D-columns, wave w owns columns
// 64w..64w+63; adds w * y_pair into y (bf16 rows) or writes y_pair (fp32
// rows).
// (two waves per SIMD: for W = 4 that is two blocks per compute unit, which
// also needs the registers of W = 8)
template <int MODE, int W>
__global__ void __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(2, 2))) pf_gemm_kernel(PfArgs a) {
    typedef PfStageT<W> Stage;
    constexpr int PM = pf_m(W), NT = 64 * W, BR = kPfWaveRows * W, AU = PM * kPfARow, SD = PM * 16;
    __shared__ Stage stg[2];
    __shared__ int32_t row_tok[PM];
    __shared__ float row_f[PM];
    constexpr int kColRows = MODE == 0 ? BR / 2 : BR;  // output columns per block
    const int nb = (MODE == 0 ? a.F : a.D) / kColRows;
    int tile, colblk;
    xcd_tile_map(blockIdx.x, nb, tile, colblk);
    if (tile >= a.n_tiles[0]) return;
    const int4 ti = a.tiles[tile];
    const int e = ti.x, start = ti.y, cnt = ti.z;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, c = lane & 31, h = lane >> 5;
    const int nkb = a.n_in >> 8;
    const int o0 = colblk * kColRows;
    const int64_t rowbytes = (int64_t)nkb * kQ2KBytes;

    if (tid < PM) {
        const int pos = start + min(tid, cnt - 1);
        const int pair = a.perm[pos];
        row_tok[tid] = pair / a.k;
        row_f[tid] = MODE == 0 ? a.ainv[pair / a.k] : a.ainv[pos] * (a.ypart ? 1.f : a.topk_w[pair]);
    }
    block_lds_sync();

    // DMA sources, fixed over the columns (32-bit offsets from uniform bases).
    // Code rows: 33 wave copies of 64 units; wave w takes copies w, w+8,
    // w+16, w+24 and wave 0 also copy 32; a pad unit loads a copy of unit 31.
    auto arow = [&](int r) { return MODE == 0 ? row_tok[r] : start + min(r, cnt - 1); };
    // (W = 4: 1056 units, 16.5 copies; the last one is issued by lanes 0-31)
    constexpr int kACopies = (AU + 63) / 64, kAI = kACopies / W + 1, kSI = SD / NT;
    static_assert(kACopies == 4 * W + 1, "A copies");
    uint32_t aoff[kAI], soff[kSI];
#pragma unroll
    for (int i = 0; i < kAI; ++i) {
        const int L = min((i * W + wave) * 64 + lane, AU - 1), r = L / kPfARow, u = min(L % kPfARow, 31);
        aoff[i] = (uint32_t)(arow(r) * nkb * 512 + u * 16);
    }
#pragma unroll
    for (int i = 0; i < kSI; ++i) {
        const int q = i * NT + tid, r = q >> 4;
        const int unit = ((q >> 2) & 3) ^ sum_swz(r);
        soff[i] = (uint32_t)(arow(r) * nkb * 64 + unit * 16 + (q & 3) * 4);
    }
    // Weight rows: wave w copies its own 64 rows (5 units each = 5 copies of
    // 64 units) and their d, dmin (one copy); mode 0 waves 0-3 from gate,
    // 4-7 from up.
    const int wrow0 = MODE == 0 ? (wave % (W / 2)) * kPfWaveRows : wave * kPfWaveRows;  // first row in its matrix block
    const uint8_t *wbm = (MODE == 0 && wave >= W / 2 ? a.w1 : a.w0) + (int64_t)e * a.expert_bytes;
    uint32_t boff[5];
#pragma unroll
    for (int j = 0; j < 5; ++j) {
        const int idx = j * 64 + lane, row = idx / 5, part = idx % 5;
        boff[j] = (uint32_t)((o0 + wrow0 + row) * rowbytes) + 4 + 16 * part;
    }
    const uint32_t ddoff = (uint32_t)((o0 + wrow0 + lane) * rowbytes);

    // uniform (scalar) DMA operands: stage LDS addresses, this wave's
    // destinations within a stage, the weight base of this wave's rows
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    const uint32_t lds_st[2] = {(uint32_t)__builtin_amdgcn_readfirstlane(lds_addr(&stg[0])),
                                (uint32_t)__builtin_amdgcn_readfirstlane(lds_addr(&stg[1]))};
    const uint8_t *wbm_u = (const uint8_t *)wave_uniform(wbm);
    // A tile of at most 32 pairs (one row subtile) copies only code rows
    // 0-31 (copies 0-16: waves take copies w and w + 8, wave 0 also copy 16)
    // and their group sums (the first half): the other rows are never read.
    auto issue = [&](auto nsub_c, int st, int kb) {
        constexpr bool FULL = decltype(nsub_c)::value == 2 || W == 4;  // the small variant's tile is 32 rows
        constexpr int kA = FULL ? kAI - 1 : 2, kS = FULL ? kSI : kSI / 2;
        constexpr int kLast = FULL ? kACopies - 1 : (kACopies - 1) / 2;  // wave 0's extra copy
        const uint8_t *ab = a.aq + kb * 512, *sb = (const uint8_t *)a.as + kb * 64, *wbk = wbm_u + kb * kQ2KBytes;
        const uint32_t L = lds_st[st];
#pragma unroll
        for (int i = 0; i < kA; ++i)
            pf_dma16u(ab, aoff[i], L + (uint32_t)offsetof(Stage, a) + (uint32_t)((i * W + wv) * 64 * 16));
        if (wv == 0) {
            if (W == 8 || lane < AU - 64 * kLast)  // W = 4: the half copy stays inside the array
                pf_dma16u(ab, aoff[kLast / W], L + (uint32_t)offsetof(Stage, a) + (uint32_t)(kLast * 64 * 16));
        }
#pragma unroll
        for (int i = 0; i < kS; ++i)
            pf_dma4u(sb, soff[i], L + (uint32_t)offsetof(Stage, s) + (uint32_t)((i * NT + 64 * wv) * 4));
#pragma unroll
        for (int j = 0; j < 5; ++j)
            pf_dma16u(wbk, boff[j], L + (uint32_t)offsetof(Stage, b) + (uint32_t)((wv * kPfWaveRows * 5 + j * 64) * 16));
        pf_dma4u(wbk, ddoff, L + (uint32_t)offsetof(Stage, dd) + (uint32_t)(wv * kPfWaveRows * 4));
    };
    static_assert(kAI == 5 && kSI == 2, "copy counts of the one-subtile issue");
    auto wait_stage = [&](auto nsub_c) {
        constexpr bool FULL = decltype(nsub_c)::value == 2 || W == 4;
        constexpr int kIssued = (FULL ? (kAI - 1) + kSI : 2 + kSI / 2) + 5 + 1;  // wave 0: one more
        if (wave == 0) vmem_wait_at_most<kIssued + 1>();
        else vmem_wait_at_most<kIssued>();
    };

    const int nsub = W == 8 && cnt > 32 ? 2 : 1;
    v16f tot[2][2];  // [column subtile][row subtile]
#pragma unroll
    for (int n = 0; n < 2; ++n)
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int v = 0; v < 16; ++v) tot[n][q][v] = 0.f;

    auto run = [&](auto nsub_c) {
    constexpr int NSUB = decltype(nsub_c)::value;
    auto compute = [&](Stage &S) {
        // unit 16*pass + 2p + h of row q*32 + c: constant offsets from abase
        const u32x4 *abase = &S.a[c * kPfARow + h];
        // both row subtiles' codes first, so that each activation read
        // feeds the two of them
        v4i bq[2][8];
        uint32_t bmh[2][4], bml[2][4];
        float dsc[2];
#pragma unroll
        for (int n = 0; n < 2; ++n) {
            const int R = wave * kPfWaveRows + 32 * n + c;
            const uint8_t *rb = (const uint8_t *)&S.b[R * 5];
            const uint2 sm = *(const uint2 *)(rb + 8 * h);
            const u32x4 q0 = *(const u32x4 *)(rb + 16 + 32 * h), q1 = *(const u32x4 *)(rb + 32 + 32 * h);
            const uint32_t dd = S.dd[R];
            dsc[n] = half_bits_to_float(dd);
            const float dmin = half_bits_to_float(dd >> 16);
#pragma unroll
            for (int p = 0; p < 8; ++p) {
                const uint32_t Q = p < 4 ? q0[p] : q1[p - 4];
                const uint32_t sc = ((p < 4 ? sm.x : sm.y) >> (8 * (p & 3))) & 15u;
#pragma unroll
                for (int j = 0; j < 4; ++j) bq[n][p][j] = (int)mul_bytes((Q >> (2 * j)) & 0x03030303u, sc);
            }
            // -dmin * m_g of the lane's 8 groups, exactly as bf16 hi + lo
            const uint32_t mA = (sm.x >> 4) & 0x0F0F0F0Fu, mB = (sm.y >> 4) & 0x0F0F0F0Fu;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t mw = i < 2 ? mA : mB;
                const float c0 = -dmin * (float)((mw >> (16 * (i & 1))) & 0xFFu);
                const float c1 = -dmin * (float)((mw >> (16 * (i & 1) + 8)) & 0xFFu);
                const uint32_t hw = bf16x2_rne(c0, c1);
                bmh[n][i] = hw;
                bml[n][i] = bf16x2_rne(c0 - __uint_as_float(hw << 16), c1 - __uint_as_float(hw & 0xFFFF0000u));
            }
        }
        v16i acc[2][2];  // [row subtile][pair subtile]
#pragma unroll
        for (int n = 0; n < 2; ++n)
#pragma unroll
            for (int q = 0; q < 2; ++q)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[n][q][v] = 0;
#pragma unroll
        for (int pass = 0; pass < 2; ++pass) {
            if (pass == 1) {
#pragma unroll
                for (int n = 0; n < 2; ++n)
#pragma unroll
                    for (int q = 0; q < NSUB; ++q)
#pragma unroll
                        for (int v = 0; v < 16; ++v) acc[n][q][v] <<= 8;
            }
#pragma unroll
            for (int p = 0; p < 8; ++p) {
#pragma unroll
                for (int q = 0; q < NSUB; ++q) {
                    const u32x4 av = abase[32 * kPfARow * q + 16 * pass + 2 * p];
                    v4i ai;
                    __builtin_memcpy(&ai, &av, 16);
#pragma unroll
                    for (int n = 0; n < 2; ++n)
                        acc[n][q] = __builtin_amdgcn_mfma_i32_32x32x32_i8(ai, bq[n][p], acc[n][q], 0, 0, 0);
                }
            }
        }
#pragma unroll
        for (int q = 0; q < NSUB; ++q) {
            const int row = q * 32 + c, sw = sum_swz(row);
            const u32x4 shu = *(const u32x4 *)&S.s[4 * (row * 4 + (h ^ sw))];
            const u32x4 slu = *(const u32x4 *)&S.s[4 * (row * 4 + ((2 + h) ^ sw))];
            v8bf sh, sl;
            __builtin_memcpy(&sh, &shu, 16);
            __builtin_memcpy(&sl, &slu, 16);
#pragma unroll
            for (int n = 0; n < 2; ++n) {
#pragma unroll
                for (int v = 0; v < 16; ++v) tot[n][q][v] = __builtin_fmaf((float)acc[n][q][v], dsc[n], tot[n][q][v]);
                const v8bf ch = as_v8bf(bmh[n]), cl = as_v8bf(bml[n]);
                tot[n][q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(sh, ch, tot[n][q], 0, 0, 0);
                tot[n][q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(sl, ch, tot[n][q], 0, 0, 0);
                tot[n][q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(sh, cl, tot[n][q], 0, 0, 0);
            }
        }
    };

    issue(nsub_c, 0, 0);
    if constexpr (W == 8) {
        // One barrier per step: past it every wave's copies of step kb are
        // in LDS and every wave has finished step kb - 1, whose stage then
        // takes the copies of step kb + 1 while step kb computes.  (With
        // many pairs the compute, not the copies, sets the pace, and the
        // second barrier of the scheme below cost about 7%.)
        for (int kb = 0; kb < nkb; ++kb) {
            vmem_wait_at_most<0>();
            stage_barrier();
            if (kb + 1 < nkb) issue(nsub_c, (kb + 1) & 1, kb + 1);
            compute(stg[kb & 1]);
        }
        stage_barrier();  // the stages are free again
    } else {
        // Few pairs: the copies set the pace, so those of step kb + 1 are
        // issued before the wait for step kb, which needs a second barrier
        // (every wave done with the stage they overwrite).
        for (int kb = 0; kb < nkb; kb += 2) {
            if (kb + 1 < nkb) {
                issue(nsub_c, 1, kb + 1);
                wait_stage(nsub_c);
            } else {
                vmem_wait_at_most<0>();
            }
            stage_barrier();
            compute(stg[0]);
            stage_barrier();
            if (kb + 1 >= nkb) break;
            if (kb + 2 < nkb) {
                issue(nsub_c, 0, kb + 2);
                wait_stage(nsub_c);
            } else {
                vmem_wait_at_most<0>();
            }
            stage_barrier();
            compute(stg[1]);
            stage_barrier();
        }
    }
    };
    if constexpr (W == 8) {
        if (nsub == 2) run(std::integral_constant<int, 2>{});
        else run(std::integral_constant<int, 1>{});
    } else {
        run(std::integral_constant<int, 1>{});  // the launch guarantees tiles of at most 32 pairs
    }

    if constexpr (MODE == 0) {
        // up waves hand their values to the gate waves of the same rows
        float *U = (float *)&stg[0];  // [PM rows][kColRows columns]
        static_assert(sizeof(Stage) >= PM * kColRows * sizeof(float), "exchange area");
        if (wave >= W / 2) {
#pragma unroll
            for (int n = 0; n < 2; ++n)
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    if (q == 1 && nsub < 2) continue;
#pragma unroll
                    for (int v = 0; v < 16; ++v)
                        U[(q * 32 + 8 * (v >> 2) + 4 * h + (v & 3)) * kColRows + (wave % (W / 2)) * 64 + 32 * n + c] =
                            tot[n][q][v];
                }
        }
        block_lds_sync();
        if (wave < W / 2) {
#pragma unroll
            for (int n = 0; n < 2; ++n)
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    if (q == 1 && nsub < 2) continue;
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int r = q * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
                        if (r >= cnt) continue;
                        const float f = row_f[r];
                        const int col = wave * 64 + 32 * n + c;
                        const float hv = silu(tot[n][q][v] * f) * (U[r * kColRows + col] * f);
                        a.hf[(int64_t)(start + r) * a.F + o0 + col] = hv;
                    }
                }
        }
    } else {
#pragma unroll
        for (int n = 0; n < 2; ++n)
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                if (q == 1 && nsub < 2) continue;
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int r = q * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
                    if (r >= cnt) continue;
                    const int col = o0 + wave * 64 + 32 * n + c;
                    if (a.ypart) a.ypart[(int64_t)(start + r) * a.D + col] = row_f[r] * tot[n][q][v];
                    else unsafeAtomicAdd(&a.y[(int64_t)row_tok[r] * a.D + col], row_f[r] * tot[n][q][v]);
                }
            }
    }
}

// ---- shared expert: bf16 GEMM on exactly split weights -------------------------
// Each Q8_0 weight w = d*q (at most 18 significant bits) is split once per
// call into bf16 hi = rne(w) and lo = rne(w - hi), so w = hi + lo to 2^-17
// relative; gate/up and down then run as bf16 GEMMs over both halves
// (v_mfma_f32_32x32x16_bf16, fp32 accumulation): bf16 activations times
// either half are exact products.

// One thread per 8 weights (a quarter of a 34-byte block): its 8 codes and
// the block's d come in as aligned dwords (the block starts at a 2-byte
// boundary), and the 8 hi and 8 lo halves go out as one 16-byte store each.
__global__ void __launch_bounds__(256) pf_q8_split_kernel(const uint8_t *src, int64_t nblocks, uint16_t *hi,
                                                          uint16_t *lo) {
    const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x, b = q >> 2;
    if (b >= nblocks) return;
    const int i0 = 8 * (int)(q & 3);
    const uint8_t *blk = src + b * kQ8Bytes;
    const uint32_t s2 = (uint32_t)((uintptr_t)blk & 2u);  // the block starts 0 or 2 bytes into a dword
    const uint32_t dw = *(const uint32_t *)(blk - s2);
    const float d = half_bits_to_float(s2 ? (dw >> 16) : (dw & 0xFFFFu));
    uint32_t c[2];
    load_8_at_even(blk + 2 + i0, c[0], c[1]);
    uint32_t hw[4], lw[4];
#pragma unroll
    for (int j = 0; j < 8; j += 2) {
        uint32_t hh = 0, ll = 0;
#pragma unroll
        for (int z = 0; z < 2; ++z) {
            const int k = j + z;
            const float w = d * (float)(int8_t)(c[k >> 2] >> (8 * (k & 3)));
            const uint16_t wh = bf16_rne(w);
            const uint16_t wl = bf16_rne(w - bf16_bits_to_float(wh));
            hh |= (uint32_t)wh << (16 * z);
            ll |= (uint32_t)wl << (16 * z);
        }
        hw[j / 2] = hh;
        lw[j / 2] = ll;
    }
    *(u32x4 *)(hi + b * 32 + i0) = u32x4{hw[0], hw[1], hw[2], hw[3]};
    *(u32x4 *)(lo + b * 32 + i0) = u32x4{lw[0], lw[1], lw[2], lw[3]};
}

constexpr int kSgM = 128;            // token rows per block (four 32-row subtiles)
constexpr int kSgKc = 32;            // reduction columns per stage
constexpr int kSgRowUnits = kSgKc * 2 / 16;   // 16-byte units per row per stage (4)

// LO: the activations come as a bf16 pair (hi, lo) too (mode 1: the shared
// h, kept to fp32 precision)
template <bool LO>
struct SgStageT {
    u32x4 a[kSgM * kSgRowUnits];       // activation rows: unit u of row r at r*4 + (u ^ sum_swz(r))
    u32x4 al[LO ? kSgM * kSgRowUnits : 1];  // their lo halves, same layout
    u32x4 bh[256 * kSgRowUnits];       // weight rows, hi halves, same swizzle
    u32x4 bl[256 * kSgRowUnits];       // lo halves
};

struct SgArgs {
    const uint16_t *a;          // mode 0: x [T][K] bf16; mode 1: hs hi halves [T][K]
    const uint16_t *a_lo;       // mode 1: hs lo halves [T][K]
    const uint16_t *wh, *wl;    // mode 0: gate rows then up rows [2*Fs][D]; mode 1: down [D][Fs]
    int T, K, Fs, D;
    uint16_t *hs, *hs_lo;       // mode 0 output [T][Fs]: h = silu(g) * u as a bf16 pair hi + lo
    float *y;                   // mode 1 output [T][D]
    int accumulate;
};

MOE_DEV int sg_unit(int r, int u) { return r * kSgRowUnits + (u ^ sum_swz(r)); }

// Mode 0: blockIdx.x = 128 F-rows (waves 0-3 gate, 4-7 up), writes
// h = silu(g) * u as a bf16 pair (hi + lo keeps h to about 2^-17).  Mode 1:
// blockIdx.x = 256 D-columns, both halves of h against both halves of the
// weights (hi*hi, hi*lo, lo*hi; lo*lo is below 2^-16 of the product), y =
// (y if accumulating) + shared output.  blockIdx.y = 128 token rows.
template <int MODE>
__global__ void __launch_bounds__(512) pf_sg_gemm_kernel(SgArgs a) {
    typedef SgStageT<MODE == 1> SgStage;
    __shared__ SgStage stg[2];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, c = lane & 31, h = lane >> 5;
    const int m0 = blockIdx.y * kSgM;
    const int nkc = a.K / kSgKc;
    auto wrow = [&](int R) -> int64_t {
        if (MODE == 0) return (int64_t)((R >> 7) * a.Fs + blockIdx.x * 128 + (R & 127));
        return (int64_t)(blockIdx.x * 256 + R);
    };
    // one 16-byte unit per thread for A (512 units), two for each weight half (1024 units)
    static_assert(kSgM * kSgRowUnits == 512 && 256 * kSgRowUnits == 1024, "stage shape");
    const int ar = tid >> 2;
    const int64_t aoff = (int64_t)min(m0 + ar, a.T - 1) * a.K + 8 * ((tid & 3) ^ sum_swz(ar));
    const uint16_t *asrc = a.a + aoff, *asrc_lo = a.a_lo + aoff;
    int64_t boff[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int u = i * 512 + tid, R = u >> 2;
        boff[i] = wrow(R) * a.K + 8 * ((u & 3) ^ sum_swz(R));
    }
    auto issue = [&](SgStage &S, int kc) {
        pf_dma16(asrc + kc * kSgKc, &S.a[64 * wave]);
        if constexpr (MODE == 1) pf_dma16(asrc_lo + kc * kSgKc, &S.al[64 * wave]);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            pf_dma16(a.wh + boff[i] + kc * kSgKc, &S.bh[i * 512 + 64 * wave]);
            pf_dma16(a.wl + boff[i] + kc * kSgKc, &S.bl[i * 512 + 64 * wave]);
        }
    };
    v16f tot[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int v = 0; v < 16; ++v) tot[q][v] = 0.f;
    const int R = MODE == 0 ? (wave >> 2) * 128 + (wave & 3) * 32 + c : wave * 32 + c;
    auto compute = [&](SgStage &S) {
#pragma unroll
        for (int ks = 0; ks < kSgKc / 16; ++ks) {
            const int u = 2 * ks + h;
            const u32x4 bw = S.bh[sg_unit(R, u)], bx = S.bl[sg_unit(R, u)];
            v8bf bvh, bvl;
            __builtin_memcpy(&bvh, &bw, 16);
            __builtin_memcpy(&bvl, &bx, 16);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const u32x4 aw = S.a[sg_unit(q * 32 + c, u)];
                v8bf av;
                __builtin_memcpy(&av, &aw, 16);
                tot[q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bvh, tot[q], 0, 0, 0);
                tot[q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bvl, tot[q], 0, 0, 0);
                if constexpr (MODE == 1) {
                    const u32x4 alw = S.al[sg_unit(q * 32 + c, u)];
                    v8bf avl;
                    __builtin_memcpy(&avl, &alw, 16);
                    tot[q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(avl, bvh, tot[q], 0, 0, 0);
                }
            }
        }
    };
    // one barrier per step, as in the routed GEMM of many pairs: past it
    // every wave's copies of chunk kc are in LDS and every wave has finished
    // chunk kc - 1, whose stage then takes chunk kc + 1
    issue(stg[0], 0);
    for (int kc = 0; kc < nkc; ++kc) {
        vmem_wait_at_most<0>();
        stage_barrier();
        if (kc + 1 < nkc) issue(stg[(kc + 1) & 1], kc + 1);
        compute(stg[kc & 1]);
    }
    stage_barrier();  // the stages are free again
    if constexpr (MODE == 0) {
        // up waves hand their values to the gate waves, 64 rows at a time
        float *U = (float *)&stg[0];  // [64 rows][128 columns], 32 KB of the 40 KB stage
        static_assert(sizeof(SgStage) >= 64 * 128 * sizeof(float), "exchange area");
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            if (wave >= 4) {
#pragma unroll
                for (int qq = 0; qq < 2; ++qq)
#pragma unroll
                    for (int v = 0; v < 16; ++v)
                        U[(qq * 32 + 8 * (v >> 2) + 4 * h + (v & 3)) * 128 + (wave & 3) * 32 + c] =
                            tot[2 * half + qq][v];
            }
            block_lds_sync();
            if (wave < 4) {
#pragma unroll
                for (int qq = 0; qq < 2; ++qq)
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int rl = qq * 32 + 8 * (v >> 2) + 4 * h + (v & 3), r = 64 * half + rl;
                        if (m0 + r >= a.T) continue;
                        const float hv = silu(tot[2 * half + qq][v]) * U[rl * 128 + wave * 32 + c];
                        const uint16_t hh = bf16_rne(hv);
                        const int64_t o = (int64_t)(m0 + r) * a.Fs + blockIdx.x * 128 + wave * 32 + c;
                        a.hs[o] = hh;
                        a.hs_lo[o] = bf16_rne(hv - bf16_bits_to_float(hh));
                    }
            }
            block_lds_sync();
        }
    } else {
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int r = q * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
                if (m0 + r >= a.T) continue;
                float *dst = a.y + (int64_t)(m0 + r) * a.D + blockIdx.x * 256 + wave * 32 + c;
                *dst = a.accumulate ? *dst + tot[q][v] : tot[q][v];
            }
    }
}

// bf16 rows at any count, and fp32 rows beyond the decode schedule (the caller
// takes that first)
bool prefill_path_ok(const moe_layer_desc *d, int32_t T, int32_t x_type) {
    return (x_type == MOE_BF16 || x_type == MOE_F32) && T > 0 && d->gate_type == MOE_Q2K && d->down_type == MOE_Q2K &&
           d->n_embd % 512 == 0 && d->n_ff_exp % 256 == 0 &&
           (d->n_ff_shared == 0 || (d->shared_type == MOE_Q8_0 && d->n_ff_shared % 128 == 0));
}

// stage 3: x codes, tiles, shared gate/up, routed gate/up; stage 4: h codes,
// shared down, y init, routed down; 0: all; 5: the routed gate/up GEMM alone.
// In both modes the routed GEMMs keep h in fp32 and code it per row for the
// down.  bf16 mode: the shared expert as bf16 GEMMs on exactly split
// weights (h as a bf16 pair), the routed down added into y by atomics.  fp32
// mode: the shared expert on its int8 GEMMs (or the batched kernels), the
// routed down writes one row per pair and the gather adds them in slot
// order, so that two runs give the same bits.
hipError_t launch_prefill_shared_bf16(const moe_layer_desc *d, const void *x, int32_t T, float *y, uint32_t flags,
                                      const Workspace &ws, hipStream_t s) {
    const int D = d->n_embd, Fs = d->n_ff_shared;
    const int64_t nw = (int64_t)Fs * D, nb = nw / 32;
    uint16_t *hi = ws.pf_shw, *lo = ws.pf_shw + 3 * nw;
    const unsigned g = (unsigned)((4 * nb + 255) / 256);  // a thread per 8 weights
    pf_q8_split_kernel<<<g, 256, 0, s>>>((const uint8_t *)d->sh_gate, nb, hi, lo);
    pf_q8_split_kernel<<<g, 256, 0, s>>>((const uint8_t *)d->sh_up, nb, hi + nw, lo + nw);
    pf_q8_split_kernel<<<g, 256, 0, s>>>((const uint8_t *)d->sh_down, nb, hi + 2 * nw, lo + 2 * nw);
    SgArgs sg{};
    sg.a = (const uint16_t *)x;
    sg.wh = hi;
    sg.wl = lo;
    sg.T = T;
    sg.K = D;
    sg.Fs = Fs;
    sg.D = D;
    sg.hs = ws.pf_hsb;
    sg.hs_lo = ws.pf_hsb_lo;
    pf_sg_gemm_kernel<0><<<dim3(Fs / 128, (T + kSgM - 1) / kSgM), 512, 0, s>>>(sg);
    SgArgs dn{};
    dn.a = ws.pf_hsb;
    dn.a_lo = ws.pf_hsb_lo;
    dn.wh = ws.pf_shw + 2 * nw;
    dn.wl = ws.pf_shw + 5 * nw;
    dn.T = T;
    dn.K = Fs;
    dn.Fs = Fs;
    dn.D = D;
    dn.y = y;
    dn.accumulate = (flags & MOE_ACCUMULATE) ? 1 : 0;
    pf_sg_gemm_kernel<1><<<dim3(D / 256, (T + kSgM - 1) / kSgM), 512, 0, s>>>(dn);
    return hipGetLastError();
}

hipError_t launch_prefill(const moe_layer_desc *d, const void *x, int32_t T, int32_t x_type, const RoutingPtrs &r,
                          float *y, uint32_t flags, const Workspace &ws, hipStream_t s, int stage,
                          hipEvent_t shared_done) {
    const bool apart = shared_done != nullptr && x_type == MOE_BF16;  // the shared expert runs elsewhere
    const bool f32 = x_type == MOE_F32;
    const int D = d->n_embd, F = d->n_ff_exp, k = d->n_expert_used, E = d->n_expert, Fs = d->n_ff_shared;
    const int ntmax = pf_max_tiles(T, k, E);
    static_assert(kPfM == kPfTileRows, "tile rows");
    // no expert takes more pairs than there are rows, so with T <= 32 every
    // tile fits the small variant's 32 rows
    const bool small = T <= 32;
    const int64_t P = (int64_t)T * k;
    // fp32 rows with a Q8_0 shared expert: its two int8 matrix-core GEMMs
    const bool sgq = f32 && Fs > 0 && shared_q8_mfma_ok(d);
    PfArgs a{};
    a.tiles = (const int4 *)ws.pf_tiles;
    a.n_tiles = ws.pf_ntiles;
    a.perm = r.perm;
    a.topk_w = r.topk_w;
    a.k = k;
    a.D = D;
    a.F = F;
    a.hf = ws.h;
    a.y = y;
    a.ypart = f32 ? ws.ypart : nullptr;
    a.expert_bytes = fmt_bytes(MOE_Q2K, (int64_t)F * D);
    if (stage == 0 || stage == 3) {
        // fp32 rows: the same launch codes x for the shared expert's int8 GEMMs
        // and one more block lays out the GEMM tiles from the routing
        const PfPrepShared ex{sgq ? ws.sg_aq : nullptr, T, nullptr, 0, nullptr, nullptr, T,
                              r.active, r.n_active, r.count, r.offset, (int4 *)ws.pf_tiles, ws.pf_ntiles};
        if (f32) pf_prep_rows_kernel<MOE_F32><<<T + 1, 256, 0, s>>>(x, D, ws.pf_xq, ws.pf_xs, ws.pf_xinv, ex);
        else pf_prep_rows_kernel<MOE_BF16><<<T + 1, 256, 0, s>>>(x, D, ws.pf_xq, ws.pf_xs, ws.pf_xinv, ex);
        if (Fs > 0 && f32) {
            const hipError_t e = sgq ? launch_shared_q8_mfma(d, T, ws, ws.pf_xinv, s, 3)
                                     : launch_ffn_large_shared(d, x, T, x_type, r, y, flags, ws, s, 3);
            if (e != hipSuccess) return e;
        } else if (Fs > 0 && !apart) {
            // shared weights split into bf16 halves, then the shared gate/up GEMM
            const int64_t nw = (int64_t)Fs * D, nb = nw / 32;
            uint16_t *hi = ws.pf_shw, *lo = ws.pf_shw + 3 * nw;
            const unsigned g = (unsigned)((4 * nb + 255) / 256);  // a thread per 8 weights
            pf_q8_split_kernel<<<g, 256, 0, s>>>((const uint8_t *)d->sh_gate, nb, hi, lo);
            pf_q8_split_kernel<<<g, 256, 0, s>>>((const uint8_t *)d->sh_up, nb, hi + nw, lo + nw);
            pf_q8_split_kernel<<<g, 256, 0, s>>>((const uint8_t *)d->sh_down, nb, hi + 2 * nw, lo + 2 * nw);
            SgArgs sg{};
            sg.a = (const uint16_t *)x;
            sg.wh = hi;
            sg.wl = lo;
            sg.T = T;
            sg.K = D;
            sg.Fs = Fs;
            sg.D = D;
            sg.hs = ws.pf_hsb;
            sg.hs_lo = ws.pf_hsb_lo;
            pf_sg_gemm_kernel<0><<<dim3(Fs / 128, (T + kSgM - 1) / kSgM), 512, 0, s>>>(sg);
        }
    }
    if (stage == 0 || stage == 3 || stage == 5) {  // 5: the routed gate/up GEMM alone, on stage 3's codes and tiles
        PfArgs g = a;
        g.w0 = (const uint8_t *)d->gate;
        g.w1 = (const uint8_t *)d->up;
        g.n_in = D;
        g.aq = ws.pf_xq;
        g.as = ws.pf_xs;
        g.ainv = ws.pf_xinv;
        if (small) pf_gemm_kernel<0, 4><<<(unsigned)(((ntmax + 7) / 8) * 8 * (F / 128)), 256, 0, s>>>(g);
        else pf_gemm_kernel<0, 8><<<(unsigned)(((ntmax + 7) / 8) * 8 * (F / 256)), 512, 0, s>>>(g);
    }
    if (stage == 0 || stage == 4) {
        if (f32) {
            // blocks P.. of the same launch code hs for the shared expert's down
            const PfPrepShared ex{nullptr, (int)P, ws.hs, Fs, ws.sg_aq, ws.sg_ainv, -1,
                                  nullptr, nullptr, nullptr, nullptr, nullptr, nullptr};
            pf_prep_rows_kernel<MOE_F32><<<(unsigned)(P + (sgq ? T : 0)), 256, 0, s>>>(ws.h, F, ws.pf_hq, ws.pf_hs,
                                                                                       ws.pf_hinv, ex);
            if (Fs > 0) {
                const hipError_t e = sgq ? launch_shared_q8_mfma(d, T, ws, ws.sg_ainv, s, 4)
                                         : launch_ffn_large_shared(d, x, T, x_type, r, y, flags, ws, s, 4);
                if (e != hipSuccess) return e;
            }
            PfArgs dn = a;
            dn.w0 = dn.w1 = (const uint8_t *)d->down;
            dn.n_in = F;
            dn.aq = ws.pf_hq;
            dn.as = ws.pf_hs;
            dn.ainv = ws.pf_hinv;
            if (small) pf_gemm_kernel<1, 4><<<(unsigned)(((ntmax + 7) / 8) * 8 * (D / 256)), 256, 0, s>>>(dn);
            else pf_gemm_kernel<1, 8><<<(unsigned)(((ntmax + 7) / 8) * 8 * (D / 512)), 512, 0, s>>>(dn);
            return launch_combine(d, x, T, x_type, r, y, flags, ws, s);
        }
        pf_prep_rows_kernel<MOE_F32><<<(unsigned)P, 256, 0, s>>>(ws.h, F, ws.pf_hq, ws.pf_hs, ws.pf_hinv,
                                                                 PfPrepShared{nullptr, (int)P, nullptr, 0, nullptr, nullptr, -1,
                                                                              nullptr, nullptr, nullptr, nullptr, nullptr,
                                                                              nullptr});
        if (apart) {
            const hipError_t e = hipStreamWaitEvent(s, shared_done, 0);  // y holds the shared expert's rows
            if (e != hipSuccess) return e;
        } else if (Fs > 0) {
            const int64_t nw = (int64_t)Fs * D;
            SgArgs sg{};
            sg.a = ws.pf_hsb;
            sg.a_lo = ws.pf_hsb_lo;
            sg.wh = ws.pf_shw + 2 * nw;
            sg.wl = ws.pf_shw + 5 * nw;
            sg.T = T;
            sg.K = Fs;
            sg.Fs = Fs;
            sg.D = D;
            sg.y = y;
            sg.accumulate = (flags & MOE_ACCUMULATE) ? 1 : 0;
            pf_sg_gemm_kernel<1><<<dim3(D / 256, (T + kSgM - 1) / kSgM), 512, 0, s>>>(sg);
        } else if (!(flags & MOE_ACCUMULATE)) {
            const int64_t n = (int64_t)T * D;
            pf_y_init_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(nullptr, y, n, 0);
        }
        PfArgs dn = a;
        dn.w0 = dn.w1 = (const uint8_t *)d->down;
        dn.n_in = F;
        dn.aq = ws.pf_hq;
        dn.as = ws.pf_hs;
        dn.ainv = ws.pf_hinv;
        if (small) pf_gemm_kernel<1, 4><<<(unsigned)(((ntmax + 7) / 8) * 8 * (D / 256)), 256, 0, s>>>(dn);
        else pf_gemm_kernel<1, 8><<<(unsigned)(((ntmax + 7) / 8) * 8 * (D / 512)), 512, 0, s>>>(dn);
    }
    return hipGetLastError();
}

}  // namespace moe
