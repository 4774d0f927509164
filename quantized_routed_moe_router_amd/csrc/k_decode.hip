// k_decode.hip - the block for a handful of token rows (decode, micro-batched
// decode) in four dependent kernels, each pairing latency-bound routing work
// with bandwidth-bound expert work ("Understanding Dwarf Star", 5.3.7 steps
// 1-5; 5.3.4 the shared expert needs no routing, so it runs beside the
// router and the finisher; 3.5 a schedule built once and replayed per token):
//   K1  router logits (one block per expert row) || x prepared for the routed
//       dot2 path
//   K2  top-k, weights, bucketing (block 0) || shared expert gate/up -> hs
//   K3  routed gate/up + SwiGLU: one block per (active expert, group of 16
//       rows); writes h and, for a Q2K down, its prepared form
//   K4  per block of 16 output rows: routed down of every active expert and
//       the shared expert's down (two rows per wave), then
//       y = shared + sum_s w_s * down_s in slot order
// Routed weight rows are copied into LDS with aligned 16-byte loads (each
// wave instruction reads 1 KB of consecutive bytes) before their 64-weight
// chunks are read from LDS: a 16-byte load per lane straight from the
// 84-byte Q2K blocks would be misaligned and split.
// No routing result ever travels back to the host: the finisher leaves one
// record per slot (expert, bucket start and size, tokens), and each K3/K4
// block reads its slot's record in one load; empty slots return at once.
#include <algorithm>
#include <type_traits>

#include "ffn_dev.h"
#include "route_dev.h"

namespace moe {

constexpr int kDecRows = 16;      // output rows per K4 block
constexpr int kDecWaves = 8;      // waves per K4 block
constexpr int kMaxDecPairs = 256;  // token-slot pairs the decode schedule takes (T*k)
constexpr int kMaxDecTokens = 16;

// Formats the staged decode kernels take for the routed experts (their 16
// rows of gate and up fit in LDS), and the bytes of 16 rows at n_embd or
// n_ff_exp <= 4096.
constexpr bool staged_fmt(int f) { return f == MOE_Q2K || f == MOE_CB2 || f == MOE_Q4K; }
template <int FMT>
constexpr int rows16_bytes_max() {
    return 16 * 16 *
           (FMT == MOE_Q8_0 ? 2 * kQ8Bytes * 4 : (FMT == MOE_CB2 ? kCB2Bytes : (FMT == MOE_Q4K ? kQ4KBytes : kQ2KBytes)));
}
// shared expert rows per wave (gate/up in K1, down in K2)
constexpr int kShGuRows = 2;
// K4: shared expert down rows per wave (kDecRows over kDecWaves waves)
constexpr int kShDownRowsK4 = 2;
// K4: LDS units (16 bytes) a wave stages at once: 16 rows of 2048 Q2K weights
constexpr int kK4WaveUnits = 672;

// The lane's prepared activations (64-column chunk c of row `row` of an
// [.][n] input): from the records written by an earlier kernel (REC: Q2K or
// Q8_0 records), else prepared in the lane from the fp32 / bf16 values.
template <int FMT, bool REC>
MOE_DEV void lane_prep(const uint32_t *rec, const void *src, int src_bf16, int64_t row, int n, int c,
                       typename RawChunk<FMT>::Prep &p) {
    if constexpr (REC && FMT == MOE_Q2K) {
        load_q2k_prep(rec + (row * (n / 16) + 4 * c) * kRec16Dwords, p);
    } else if constexpr (REC && FMT == MOE_Q8_0) {
        load_q8_prep(rec + (row * (n / 64) + c) * kXQ8Dwords, p);
    } else {
        float xf[64];
        load_x64(src, src_bf16, row * n + 64 * c, xf);
        RawChunk<FMT>::prep(xf, p);
    }
}

// A slot record as the decode kernels use it: wave-uniform, and empty (e =
// -1) unless its fields fit the call (expert in [0, E), 1..16 entries inside
// [0, T*k), tokens below T), so that a record that does not belong to this
// call can give a wrong result but never an address outside the buffers.
MOE_DEV SlotRec checked_slot(const FfnArgs &a, int s) {
    SlotRec r = uniform_slot(a.slots, s);
    bool ok = (uint32_t)r.e < (uint32_t)a.E && r.n >= 1 && r.n <= kMaxDecTokens && r.j0 >= 0 &&
              r.j0 + r.n <= a.T * a.k;
    for (int j = 0; ok && j < r.n; ++j) ok = slot_token(r, j) < a.T;
    if (!ok) r = make_slot(-1, 0, 0, 0, 0);
    return r;
}

// Per-slot records from a routing given by the caller (no routing in K1/K2).
MOE_DEV void build_slot_records(const FfnArgs &a) {
    const int na = a.n_active[0];
    for (int s = threadIdx.x; s < a.nslots; s += blockDim.x) {
        SlotRec r = make_slot(-1, 0, 0, 0, 0);
        if (s < na) {
            const int e = a.active[s], j0 = a.offset[e];
            const int n = min(a.count[e], kMaxDecTokens);  // one entry per token at most
            uint64_t tlo = 0, thi = 0;
            for (int i = 0; i < n; ++i) {
                const uint64_t t = (uint64_t)(a.perm[j0 + i] / a.k);
                if (i < 8) tlo |= t << (8 * i);
                else thi |= t << (8 * (i - 8));
            }
            r = make_slot(e, j0, n, tlo, thi);
        }
        a.slots[s] = r;
    }
}

template <int XT>
__global__ void __launch_bounds__(256) dec_k1_kernel(FfnArgs a) {
    __shared__ double part[4 * 16];
    int b = blockIdx.x;
    if (a.build_slots) {
        if (b == 0) {
            build_slot_records(a);
            return;
        }
        b -= 1;
    }
    if (b < a.n_router_blocks) {
        router_row_block<XT>(a.router_w, a.router_bias, a.x, a.T, a.D, a.E, a.logits, b, part);
        return;
    }
    b -= a.n_router_blocks;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int item = b * 4 + wave, per_t = a.D / 64;  // one wave per 64 activations of a token
    if (item >= a.T * per_t) return;
    const int t = item / per_t, c = item % per_t;
    const int64_t i = (int64_t)t * a.D + 64 * c + lane;
    const float v = XT == MOE_BF16 ? bf16_bits_to_float(((const uint16_t *)a.x)[i]) : ((const float *)a.x)[i];
    if (a.xp16) {
        uint32_t *out = a.xp16 + ((int64_t)t * (a.D / 16) + 4 * c) * kRec16Dwords;
        if (a.xp16_nat) prep16_wave<true>(v, out);
        else prep16_wave<false>(v, out);
    }
    if (a.xq8) prep8_wave(v, a.xq8 + ((int64_t)t * (a.D / 64) + c) * kXQ8Dwords);
}

// Column parts of a staged block of 4 waves: P = min(4, n/256) parts of the
// n columns, the 4/P row groups of rows_per_block rows spread over the rest.
struct ColSplit {
    int P, RW, cp, rg, ncol, cpr, rpi;
};
MOE_DEV ColSplit col_split(int n, int rows_per_block, int wave) {
    ColSplit s;
    s.P = min(4, n >> 8);
    s.RW = rows_per_block * s.P / 4;
    s.cp = wave % s.P;
    s.rg = wave / s.P;
    s.ncol = n / s.P;
    s.cpr = s.ncol >> 6;
    s.rpi = 64 / s.cpr;
    return s;
}

// Block 0 (when routing): top-k, weights and bucketing; the other blocks
// run the shared expert's gate/up, kShGuRows rows per wave, fp32
// activations x -> hs.  The finisher's latency hides under the shared
// expert's weight stream.
template <int SFMT>
__global__ void __launch_bounds__(256) dec_k2_kernel(FfnArgs a, int do_route) {
    __shared__ uint32_t cb_lds[SFMT == MOE_CB2 ? 512 : 1];
    __shared__ __align__(16) float red[4][2 * kShGuRows * 64];
    int b = blockIdx.x;
    if (do_route) {
        if (b == 0) {
            route_finish_block(a.logits, a.T, a.E, a.k, a.route_scale, a.w_topk_idx, a.w_topk_w, a.w_count,
                               a.w_offset, a.w_perm, a.w_pos, a.w_active, a.w_n_active, a.slots, a.nslots);
            return;
        }
        b -= 1;
    }
    if constexpr (SFMT == MOE_CB2) load_codebook(a.codebook, cb_lds);  // uniform over the block
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int row0 = (b * 4 + wave) * kShGuRows;
    if (row0 >= a.Fs) return;
    const int nrows = min(kShGuRows, a.Fs - row0), c = lane % (a.D >> 6);
    for (int t = 0; t < a.T; ++t) {
        float *dst = a.hs + (int64_t)t * a.Fs + row0;
        rows_dot_ch<F32Chunk<SFMT>, true, kShGuRows>(
            a.sh_gate, a.sh_up, a.D, 0, a.D, nrows, [&](int l) { return row0 + l; },
            [&](XF32 &xr) { load_x64(a.x, a.x_bf16, (int64_t)t * a.D + 64 * c, xr.x); }, cb_lds, lane, red[wave],
            [&](int l, float gs, float us) { dst[l] = swiglu_h(gs, us); });
    }
}

// K2 with a Q8_0 shared expert at n_embd 4096: block 0 finishes the routing
// (when routing); every other block takes 8 rows of the shared gate and the
// same 8 rows of up, wave w their column quarter w.  Each wave copies into
// its own LDS area, all at once: the first token's prepared x for its
// quarter (16 chunk records), then rows in groups of four ([gate 2q, 2q+1,
// up 2q, 2q+1] for q = 0..3), and starts on each group once it has landed.
// Lane (r, c) dots row r of a group with chunk c of the quarter (packed fp16
// products of the int8 codes with the hi/lo split activations); the 16 lanes
// of a row are added by DPP, the quarters in LDS after the last token (the
// waves run through the tokens without waiting for each other, each loading
// the next token's records while it sums the current one's).
constexpr int kSgXu = 16 * kXQ8Dwords / 4;   // 272 units: 16 chunk records
constexpr int kSgRu = 1024 / 32 * kQ8Bytes / 16;  // 68 units: a row quarter
constexpr int kSgCopies = 22;                 // 272 + 16 x 68 = 1360 units -> 22 copies of 64
static_assert(kSgXu + 16 * kSgRu <= 64 * kSgCopies, "area");

template <int END>
MOE_DEV void sg_wait() {
    __builtin_amdgcn_sched_barrier(0);
    vmem_wait_le<kSgCopies - (END + 63) / 64>();
    __builtin_amdgcn_sched_barrier(0);
}

// do_route 1: block 0 (a block of its own) finishes the routing; 2 (one
// token): a fifth wave of block 0 does, so that the grid is one block per
// 8 shared rows and every block gets a compute unit of its own (the LDS
// areas allow one block per unit).
__global__ void __launch_bounds__(320) dec_k2_q8sg4096_kernel(FfnArgs a, int do_route) {
    __shared__ __align__(16) u32x4 area[4][64 * kSgCopies];
    __shared__ float part[kMaxDecTokens][4][16];
    int b = blockIdx.x;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    if (do_route == 1) {
        if (b == 0) {
            route_finish_block(a.logits, a.T, a.E, a.k, a.route_scale, a.w_topk_idx, a.w_topk_w, a.w_count,
                               a.w_offset, a.w_perm, a.w_pos, a.w_active, a.w_n_active, a.slots, a.nslots);
            return;
        }
        b -= 1;
    }
    if (wave == 4) {  // joins the block's one barrier below
        if (do_route == 2 && b == 0) {
            const int my_e = select_topk(a.logits, a.E, a.k, a.route_scale, a.w_topk_idx, a.w_topk_w);
            bucket_one_token(my_e, a.k, a.E, a.w_count, a.w_offset, a.w_perm, a.w_pos, a.w_active, a.w_n_active,
                             a.slots, a.nslots);
        }
        block_lds_sync();
        return;
    }
    const int row0 = 8 * b;  // rows row0 .. row0 + 7 of gate and of up
    constexpr int RB = 4096 / 32 * kQ8Bytes;  // bytes of a row: 4352
    {
        const uint8_t *xs = (const uint8_t *)(a.xq8 + (int64_t)(16 * wave) * kXQ8Dwords);  // token 0, quarter w
        const uint8_t *gm = a.sh_gate + (int64_t)row0 * RB + 1088 * wave, *um = a.sh_up + (int64_t)row0 * RB + 1088 * wave;
        const uint32_t lb = (uint32_t)__builtin_amdgcn_readfirstlane(lds_addr(area[wave]));
#pragma unroll
        for (int i = 0; i < kSgCopies; ++i) {
            const int u = 64 * i + lane;
            const uint8_t *src;
            if (u < kSgXu) {
                src = xs + 16 * u;
            } else {
                const int v = min(u - kSgXu, 16 * kSgRu - 1), rw = v / kSgRu, o = v - rw * kSgRu;
                const int q = rw >> 2, j = rw & 3;  // group q: gate 2q, 2q+1, up 2q, 2q+1
                src = ((j & 2) ? um : gm) + (int64_t)(2 * q + (j & 1)) * RB + 16 * o;
            }
            dma16_m0(src, lb + 1024 * i);
        }
    }
    const int r = lane >> 4, c = lane & 15;
    const uint8_t *ab = (const uint8_t *)area[wave];
    XQ8 xr;
    float v[4];
    auto group = [&](int q) {
        if (q == 0) load_q8_prep((const uint32_t *)(ab + 272 * c), xr);
        v[q] = q8_dot2(q8_load(ab + 16 * (kSgXu + kSgRu * (4 * q + r)), 64 * c), xr);
        pin_value(v[q]);
    };
    sg_wait<kSgXu + 4 * kSgRu>();
    group(0);
    sg_wait<kSgXu + 8 * kSgRu>();
    group(1);
    sg_wait<kSgXu + 12 * kSgRu>();
    group(2);
    sg_wait<kSgXu + 16 * kSgRu>();
    group(3);
    for (int t = 0;;) {
        // the next token's records (several tokens): issued here and held in
        // registers while this token's sums are written
        // (the pad dword is not loaded: a register whose load is in flight and
        // whose value is never used gets reused, and that reuse waits for the load)
        XQ8 xn;
        const bool more = t + 1 < a.T;
        if (more) {
            const uint32_t *rec = a.xq8 + ((int64_t)(t + 1) * 64 + 16 * wave + c) * kXQ8Dwords;
#pragma unroll
            for (int i = 0; i < 16; ++i) ((u32x4 *)&xn)[i] = *(const u32x4 *)(rec + 4 * i);
            const uint3 tail = *(const uint3 *)(rec + 64);
            xn.sx[0] = __uint_as_float(tail.x);
            xn.sx[1] = __uint_as_float(tail.y);
            xn.inv = __uint_as_float(tail.z);
            xn.pad = 0.f;
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float sv = row16_sum(v[q]);
            if (c == 0) part[t][wave][4 * q + r] = sv;  // [group][gate 2q, 2q+1, up 2q, 2q+1]
        }
        if (!more) break;
        ++t;
        xr = xn;
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = q8_dot2(q8_load(ab + 16 * (kSgXu + kSgRu * (4 * q + r)), 64 * c), xr);
    }
    block_lds_sync();
    for (int o = tid; o < 8 * a.T; o += 256) {  // token o / 8, row o % 8
        const int t = o >> 3, i = o & 7, q = i >> 1, j = i & 1;
        float gs = 0.f, us = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            gs += part[t][w][4 * q + j];
            us += part[t][w][4 * q + 2 + j];
        }
        a.hs[(int64_t)t * a.Fs + row0 + i] = swiglu_h(gs, us);
    }
}

// K2 with a Q8_0 shared expert at n_embd 4096 and 2 to 16 tokens: the
// shared gate/up on the fp32 matrix cores (v_mfma_f32_16x16x4f32, tokens x
// rows), every token at once.  Block b (after the routing block, when
// routing) takes gate rows 8b..8b+7 (columns 0-7) and the same up rows
// (columns 8-15); wave w takes input columns [512 w, 512 w + 512).  Lane l
// (token and row l % 16, quarter l / 16 of the wave's columns) holds 128
// consecutive values of its token's x and of its row's weights d*q (exact in
// fp32); instruction i takes value i of each quarter, so every product
// enters the sum once.  The waves' partial sums meet in LDS and are added in
// wave order, then h = silu(g) * u.
constexpr int kSgmWaves = 8;
__global__ void __launch_bounds__(64 * kSgmWaves) dec_k2_q8sg_mfma_kernel(FfnArgs a, int route) {
    __shared__ float shp[kSgmWaves][16][16];  // [wave][token][gate 0-7, up 8-15]
    int b = blockIdx.x;
    if (route) {
        if (b == 0) {
            route_finish_block(a.logits, a.T, a.E, a.k, a.route_scale, a.w_topk_idx, a.w_topk_w, a.w_count,
                               a.w_offset, a.w_perm, a.w_pos, a.w_active, a.w_n_active, a.slots, a.nslots);
            return;
        }
        b -= 1;
    }
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, n = lane & 15, kq = lane >> 4;
    const int row0 = 8 * b;
    constexpr int RB = 4096 / 32 * kQ8Bytes;  // bytes of a row: 4352
    const int k0 = 512 * wave + 128 * kq;    // the lane's 128 columns: 4 Q8_0 blocks
    float xs[128];
    load_x64(a.x, a.x_bf16, (int64_t)min(n, a.T - 1) * 4096 + k0, xs);
    load_x64(a.x, a.x_bf16, (int64_t)min(n, a.T - 1) * 4096 + k0 + 64, xs + 64);
    const uint8_t *wp = (n < 8 ? a.sh_gate : a.sh_up) + (int64_t)(row0 + (n & 7)) * RB + (k0 / 32) * kQ8Bytes;
    uint32_t wd[34];
#pragma unroll
    for (int j = 0; j < 34; ++j) wd[j] = load_u32(wp + 4 * j);
    float dq[4];
#pragma unroll
    for (int blk = 0; blk < 4; ++blk) {
        const int B = kQ8Bytes * blk;  // d of block blk (fp16, 2-byte aligned)
        dq[blk] = half_bits_to_float((wd[B >> 2] >> (8 * (B & 3))) & 0xFFFFu);
    }
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 128; ++i) {
        const int B = kQ8Bytes * (i >> 5) + 2 + (i & 31);  // byte of code i
        const int q = (int)(int8_t)(wd[B >> 2] >> (8 * (B & 3)));
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(xs[i], dq[i >> 5] * (float)q, acc, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) shp[wave][4 * kq + j][n] = acc[j];
    block_lds_sync();
    if (tid < 8 * a.T) {  // token tid / 8, row tid % 8
        const int t = tid >> 3, i = tid & 7;
        float gs = 0.f, us = 0.f;
#pragma unroll
        for (int w = 0; w < kSgmWaves; ++w) {
            gs += shp[w][t][i];
            us += shp[w][t][8 + i];
        }
        a.hs[(int64_t)t * a.Fs + row0 + i] = swiglu_h(gs, us);
    }
}

// K1 for one fp32 token at n_embd 4096 when the routed gate/up kernel selects
// the top-k itself (no K2): block b computes router logit b and, with a
// Q8_0 shared expert, 8 rows of the shared gate and of up -> hs, so the
// latency-bound router rows run under the shared expert's weight stream.
// Wave w works on column quarter w throughout.  It copies into its own LDS
// area, in this order: x's quarter, router row b's quarter, then the shared
// rows as the K2 kernel above lays them out.  From x in LDS it forms the
// Q8_0 records of its 16 chunks (prep8_rows, the bits of K1's prep8_wave)
// in the place the K2 kernel copies them to, and (blocks 0-15) chunk
// 16 w + b's record for the routed Q2K or codebook rows.  The logit is
// summed exactly as router_row_block sums it (lane l: 16 consecutive
// columns of the quarter in ascending order in fp64, then the lanes by a
// fixed butterfly, then the quarters in wave order), so both schedules give
// the same logits.
constexpr int kT1Xu = 256;                         // units of a 1024-value fp32 quarter
constexpr int kT1WeightCopies = 16 * kSgRu / 64;   // 17
constexpr int kT1Units = kSgXu + 16 * kSgRu + 2 * kT1Xu;  // records, rows, x, router: 1872
static_assert(16 * kSgRu == 64 * kT1WeightCopies, "whole copies of the shared rows");

template <int N>  // at most N of the wave's copies outstanding
MOE_DEV void t1_wait() {
    __builtin_amdgcn_sched_barrier(0);
    vmem_wait_le<N>();
    __builtin_amdgcn_sched_barrier(0);
}
template <int END>  // shared-row units [0, END) of the wave's area (after the records) have landed
MOE_DEV void t1_wait_rows() {
    t1_wait<kT1WeightCopies - (END + 63) / 64>();
}

template <bool NORM>
__global__ void __launch_bounds__(256) dec_k1_t1_kernel(FfnArgs a) {
    __shared__ __align__(16) u32x4 area[4][kT1Units + (NORM ? kT1Xu : 0)];
    __shared__ double rpart[4];
    __shared__ float part[4][16];
    __shared__ float red[4];
    const int b = blockIdx.x, tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const bool router = b < a.E, shared = b < a.Fs / 8;  // uniform over the block
    u32x4 *my = area[wave];
    float *xq = (float *)(my + kSgXu + 16 * kSgRu);  // x, columns 1024 w ..
    float *rq = xq + 1024;                          // router row b, the same columns
    float *gq = xq + 2048;                          // NORM: gamma, the same columns
    const int row0 = 8 * b;
    constexpr int RB = 4096 / 32 * kQ8Bytes;  // bytes of a shared row: 4352
    {
        const uint8_t *xs = (const uint8_t *)a.x + 4096 * wave;
        const uint8_t *rs = (const uint8_t *)(a.router_w + (int64_t)min(b, a.E - 1) * 4096) + 4096 * wave;
        const uint32_t lx = (uint32_t)__builtin_amdgcn_readfirstlane(lds_addr(xq));
        const uint32_t lr = (uint32_t)__builtin_amdgcn_readfirstlane(lds_addr(rq));
#pragma unroll
        for (int i = 0; i < 4; ++i) dma16_m0(xs + 16 * (64 * i + lane), lx + 1024 * i);
        if constexpr (NORM) {
            const uint8_t *gs = (const uint8_t *)a.norm_gamma + 4096 * wave;
            const uint32_t lg = (uint32_t)__builtin_amdgcn_readfirstlane(lds_addr(gq));
#pragma unroll
            for (int i = 0; i < 4; ++i) dma16_m0(gs + 16 * (64 * i + lane), lg + 1024 * i);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) dma16_m0(rs + 16 * (64 * i + lane), lr + 1024 * i);
        if (shared) {
            const uint8_t *gm = a.sh_gate + (int64_t)row0 * RB + 1088 * wave;
            const uint8_t *um = a.sh_up + (int64_t)row0 * RB + 1088 * wave;
            const uint32_t lb = (uint32_t)__builtin_amdgcn_readfirstlane(lds_addr(my + kSgXu));
#pragma unroll
            for (int i = 0; i < kT1WeightCopies; ++i) {
                const int v = 64 * i + lane, rw = v / kSgRu, o = v - rw * kSgRu;
                const int q = rw >> 2, j = rw & 3;  // group q: gate 2q, 2q+1, up 2q, 2q+1
                dma16_m0(((j & 2) ? um : gm) + (int64_t)(2 * q + (j & 1)) * RB + 16 * o, lb + 1024 * i);
            }
        }
    }
    // x's quarter (and gamma's) has landed
    if (shared) t1_wait<4 + kT1WeightCopies>();
    else t1_wait<4>();
    if constexpr (NORM) {
        // x <- gamma * (x / sqrt(mean(x^2) + eps)) in LDS, with the bits of
        // rmsnorm_vec_kernel<4>: thread t sums the squares of its float4s
        // t + 256 i (i = 0..3, one in each quarter) in that order, the lanes
        // by the same butterfly, the waves as (0 + 1) + (2 + 3)
        block_lds_sync();  // every wave's quarter has landed
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const f32x4 v = *(const f32x4 *)((const float *)(area[i] + kSgXu + 16 * kSgRu) + 4 * tid);
#pragma unroll
            for (int j = 0; j < 4; ++j) ss = __builtin_fmaf(v[j], v[j], ss);
        }
        for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o, kWave);
        if (lane == 0) red[wave] = ss;
        block_lds_sync();  // also: every read of x for the squares is done
        const float tot = (red[0] + red[1]) + (red[2] + red[3]);
        const float inv = 1.0f / sqrtf(tot / 4096.f + a.norm_eps);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f32x4 v = *(f32x4 *)(xq + 16 * lane + 4 * i);
            const f32x4 g = *(const f32x4 *)(gq + 16 * lane + 4 * i);
#pragma unroll
            for (int j = 0; j < 4; ++j) v[j] = g[j] * (v[j] * inv);
            *(f32x4 *)(xq + 16 * lane + 4 * i) = v;
        }
    }
    // Q8_0 records of the quarter's 16 chunks, four at a time
    if (shared) {
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            const int c = 4 * r4 + (lane >> 4);
            prep8_rows(*(const f32x4 *)(xq + 64 * c + 4 * (lane & 15)), (uint32_t *)(my + 17 * c));
        }
    }
    // router row b's quarter has landed
    if (shared) t1_wait<kT1WeightCopies>();
    else t1_wait<0>();
    if (router) {
        double acc = 0.0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const f32x4 xv = *(const f32x4 *)(xq + 16 * lane + 4 * i), wv = *(const f32x4 *)(rq + 16 * lane + 4 * i);
#pragma unroll
            for (int j = 0; j < 4; ++j) acc = __builtin_fma((double)xv[j], (double)wv[j], acc);
        }
        acc = seg_sum_f64(acc, kWave);
        if (lane == 0) rpart[wave] = acc;
    }
    // the routed rows' record of chunk 16 w + b (global stores: issued only
    // once every copy of the wave has landed, as vmcnt counts them too)
    auto routed_record = [&]() {
        if (a.xp16 && b < 16) {
            uint32_t *out = a.xp16 + (int64_t)4 * (16 * wave + b) * kRec16Dwords;
            if (a.xp16_nat) prep16_wave<true>(xq[64 * b + lane], out);
            else prep16_wave<false>(xq[64 * b + lane], out);
        }
    };
    if (!shared) {
        routed_record();
        __syncthreads();
        if (router && tid == 0)
            a.logits[b] = (((rpart[0] + rpart[1]) + rpart[2]) + rpart[3]) + (a.router_bias ? (double)a.router_bias[b] : 0.0);
        return;
    }
    const int r = lane >> 4, c = lane & 15;
    const uint8_t *ab = (const uint8_t *)my;
    XQ8 xr;
    float v[4];
    auto group = [&](int q) {
        if (q == 0) load_q8_prep((const uint32_t *)(ab + 272 * c), xr);
        v[q] = q8_dot2(q8_load(ab + 16 * (kSgXu + kSgRu * (4 * q + r)), 64 * c), xr);
        pin_value(v[q]);
    };
    t1_wait_rows<4 * kSgRu>();
    group(0);
    t1_wait_rows<8 * kSgRu>();
    group(1);
    t1_wait_rows<12 * kSgRu>();
    group(2);
    t1_wait_rows<16 * kSgRu>();
    group(3);
    routed_record();
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const float sv = row16_sum(v[q]);
        if (c == 0) part[wave][4 * q + r] = sv;  // [group][gate 2q, 2q+1, up 2q, 2q+1]
    }
    block_lds_sync();
    if (router && tid == 0)
        a.logits[b] = (((rpart[0] + rpart[1]) + rpart[2]) + rpart[3]) + (a.router_bias ? (double)a.router_bias[b] : 0.0);
    if (tid < 8) {
        const int q = tid >> 1, j = tid & 1;
        float gs = 0.f, us = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            gs += part[w][4 * q + j];
            us += part[w][4 * q + 2 + j];
        }
        a.hs[row0 + tid] = swiglu_h(gs, us);
    }
}

// The slot record of a routed gate/up block.  With k3_topk (one token, no
// K2) every wave runs the selection from the router logits, so the slot's
// expert is wave-uniform without a barrier: slot s is the expert of rank s
// among the k (bucket position s, token 0), as the bucketing orders them.
// The slot's first block (g = 0) stores the record for the down kernel, at
// once, before its weight copies go out (a store issued after them could
// be counted in their place by the copy waits).  The down kernel writes the
// rest of the routing.
MOE_DEV int rank_among_k(int my_e, int k) {  // lanes < k: my_e's rank among the k distinct experts
    int rank = 0;
#pragma unroll
    for (int q = 0; q < 16; ++q) rank += q < k && __builtin_amdgcn_readlane(my_e, q) < my_e;
    return rank;
}
MOE_DEV SlotRec k3_slot(const FfnArgs &a, int slot, int g) {
    if (!a.k3_topk) return checked_slot(a, slot);
    const int my_e = select_topk(a.logits, a.E, a.k, a.route_scale, nullptr, nullptr);
    const int lane = threadIdx.x & 63, rank = rank_among_k(my_e, a.k);
    const uint64_t hit = __ballot(lane < a.k && rank == slot);
    const int e = hit ? __builtin_amdgcn_readlane(my_e, (int)__builtin_ctzll(hit)) : -1;
    const SlotRec rec = make_slot(e, slot, 1, 0, 0);
    if (g == 0 && threadIdx.x == 0) a.slots[slot] = rec;
    return rec;
}

// One block per (active slot, group g of 16 rows of the expert's gate and up):
// the 16 rows of both are staged in LDS, wave w takes column part w % P of
// the rows of row group w / P; the parts of a row are added in LDS in column
// order, then wave 0 applies SwiGLU and writes h and the group's prepared
// record.  The staged rows serve every token of the bucket.
template <int GFMT>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 8))) dec_k3_kernel(FfnArgs a) {
    static_assert(staged_fmt(GFMT), "staged formats only");
    constexpr int kU = 2 * rows16_bytes_max<GFMT>() / 16;
    constexpr int kNI = (kU + 255) / 256;
    __shared__ __align__(16) u32x4 wbuf[kU];
    __shared__ uint32_t cb_lds[GFMT == MOE_CB2 ? 512 : 1];
    __shared__ __align__(16) float red[4][2 * 4 * 64];
    __shared__ float part[4][32];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    if constexpr (GFMT == MOE_CB2) load_codebook(a.codebook, cb_lds);
    const int gpe = a.F / 16, slot = blockIdx.x / gpe, g = blockIdx.x % gpe;
    const SlotRec rec = k3_slot(a, slot, g);
    if ((uint32_t)rec.e >= (uint32_t)a.E) return;  // an empty slot (uniform over the block)
    const int U = (int)fmt_bytes(GFMT, (int64_t)16 * a.D) / 16;  // 16 rows in 16-byte units
    const int64_t goff = (int64_t)rec.e * a.gu_expert_bytes + fmt_bytes(GFMT, (int64_t)16 * g * a.D);
    const u32x4 *sg = (const u32x4 *)(a.gate + goff), *su = (const u32x4 *)(a.up + goff);
    const ColSplit cs = col_split(a.D, 16, wave);
    const int col = cs.cp * cs.ncol, chunk = (col >> 6) + lane % cs.cpr;
    typename RawChunk<GFMT>::Prep xr;  // the first token's activations, in flight with the weights
    lane_prep<GFMT, GFMT == MOE_Q2K>(a.xp16, a.x, a.x_bf16, slot_token(rec, 0), a.D, chunk, xr);
    // round i: lane l of wave w copies unit i * 256 + 64 * w + l of gate ++ up
#pragma unroll
    for (int i = 0; i < kNI; ++i) {
        const int u = i * 256 + tid;
        if (u < 2 * U) lds_dma16(u < U ? sg + u : su + (u - U), wbuf + i * 256 + 64 * wave);
    }
    vmem_wait_all();
    block_lds_sync();
    const uint8_t *wb = (const uint8_t *)wbuf;
    for (int j = 0; j < rec.n; ++j) {
        if (j > 0) lane_prep<GFMT, GFMT == MOE_Q2K>(a.xp16, a.x, a.x_bf16, slot_token(rec, j), a.D, chunk, xr);
        lds_rows_dot<GFMT, true, GFMT == MOE_Q2K ? 4 : 2>(wb, wb + U * 16, a.D, cs.rg * cs.RW, col, cs.ncol, cs.RW, xr, cb_lds, lane,
                                    red[wave], [&](int l, float gs, float us) {
                                        part[wave][2 * l] = gs;
                                        part[wave][2 * l + 1] = us;
                                    });
        block_lds_sync();
        if (wave == 0) {
            float hv = 0.f;
            if (lane < 16) {
                const int rg = lane / cs.RW, rl = lane % cs.RW;
                float gs = 0.f, us = 0.f;
                for (int q = 0; q < cs.P; ++q) {
                    gs += part[rg * cs.P + q][2 * rl];
                    us += part[rg * cs.P + q][2 * rl + 1];
                }
                hv = swiglu_h(gs, us);
                a.h[(int64_t)(rec.j0 + j) * a.F + 16 * g + lane] = hv;
            }
            if (a.hp16) prep16_wave(hv, a.hp16 + ((int64_t)(rec.j0 + j) * (a.F / 16) + g) * kRec16Dwords, 1);
        }
        block_lds_sync();
    }
}

// K3 for Q2K gate/up rows of 4096 weights.  The block issues all of its
// copies into LDS at once, in the order [x records of the first token]
// [gate rows 0-15][up rows 0-15] (each a contiguous range of the matrix, so
// a lane's source address is one add per copy): 13 copies of 256 units of
// 16 bytes, lane-contiguous, so that no copy is partial.  The waves then
// work through the 4-row groups in that order, each as soon as
// every copy that covers it has landed (the block's copies land in issue
// order per wave; a barrier joins the waves), so the dot products of one
// group run under the copies of the next.  Wave w takes column quarter w of
// every row: lane (r, c) one 64-weight chunk of row r of the group; the 16
// lanes of a row are added by DPP, the quarters in LDS.
constexpr int kK3PXu = 640;                      // units of one token's records at n_embd 4096
constexpr int kK3PHu = 336;                      // units of 4 rows of 4096 Q2K weights
constexpr int kK3PUnits = kK3PXu + 8 * kK3PHu;  // 3328
constexpr int kK3PCopies = kK3PUnits / 256;      // 13 per lane
static_assert(kK3PUnits % 256 == 0, "whole copies");

// vmcnt that guarantees units [0, end) of the block have landed: a wave's
// copy i covers units [256 i + 64 w, +64), so at most ceil(end / 256) of its
// copies are needed; the rest may still be in flight.
// The scheduling barriers keep the dot products of the previous group in
// front of the wait.
template <int END>
MOE_DEV void k3p_wait() {
    __builtin_amdgcn_sched_barrier(0);
    vmem_wait_le<kK3PCopies - (END + 255) / 256>();
    barrier_only();
    __builtin_amdgcn_sched_barrier(0);
}

__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 8))) dec_k3_q2k4096_kernel(FfnArgs a) {
    __shared__ __align__(16) u32x4 wbuf[kK3PUnits];
    __shared__ float part[4][32];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int gpe = a.F / 16, slot = blockIdx.x / gpe, g = blockIdx.x % gpe;
    const uint32_t lb = (uint32_t)__builtin_amdgcn_readfirstlane(lds_addr(wbuf) + 1024 * wave);
    constexpr int kPre = kK3PXu / 256;  // copies 0-1 hold records only
    // one token (k3_topk): its records do not depend on the slot, so their
    // first copies go out before the selection
    const int first = a.k3_topk ? kPre : 0;
    if (a.k3_topk) {
#pragma unroll
        for (int i = 0; i < kPre; ++i) dma16_m0((const u32x4 *)a.xp16 + 256 * i + tid, lb + 4096 * i);
    }
    const SlotRec rec = k3_slot(a, slot, g);
    if ((uint32_t)rec.e >= (uint32_t)a.E) {  // an empty slot (uniform over the block)
        vmem_wait_all();
        return;
    }
    constexpr int RB = 16 * kQ2KBytes;  // bytes of one row
    const int64_t goff = (int64_t)rec.e * a.gu_expert_bytes + (int64_t)16 * g * RB;
    const uint8_t *gm = a.gate + goff, *um = a.up + goff;
    {
        const u32x4 *xs = (const u32x4 *)(a.xp16 + (int64_t)slot_token(rec, 0) * (4096 / 16) * kRec16Dwords);
#pragma unroll
        for (int i = 0; i < kK3PCopies; ++i) {
            if (i < first) continue;
            const int u = 256 * i + tid;
            const void *src;
            if (u < kK3PXu) src = xs + u;
            else if (u < kK3PXu + 4 * kK3PHu) src = gm + 16 * (u - kK3PXu);
            else src = um + 16 * (u - kK3PXu - 4 * kK3PHu);
            dma16_m0(src, lb + 4096 * i);
        }
    }
    const int c = lane & 15, lr = lane >> 4, cidx = 16 * wave + c;  // chunk of the row: 64 * cidx
    const uint8_t *wb = (const uint8_t *)wbuf;
    XQ2K xr;
    float v[8];
    k3p_wait<kK3PXu>();
    load_q2k_prep((const uint32_t *)wbuf + 40 * cidx, xr);
#pragma unroll
    for (int hgrp = 0; hgrp < 8; ++hgrp) {
        if (hgrp == 0) k3p_wait<kK3PXu + 1 * kK3PHu>();
        if (hgrp == 1) k3p_wait<kK3PXu + 2 * kK3PHu>();
        if (hgrp == 2) k3p_wait<kK3PXu + 3 * kK3PHu>();
        if (hgrp == 3) k3p_wait<kK3PXu + 4 * kK3PHu>();
        if (hgrp == 4) k3p_wait<kK3PXu + 5 * kK3PHu>();
        if (hgrp == 5) k3p_wait<kK3PXu + 6 * kK3PHu>();
        if (hgrp == 6) k3p_wait<kK3PXu + 7 * kK3PHu>();
        if (hgrp == 7) k3p_wait<kK3PXu + 8 * kK3PHu>();
        v[hgrp] = q2k_dot2(q2k_load(wb + 16 * (kK3PXu + kK3PHu * hgrp), (int64_t)lr * 4096 + 64 * cidx), xr);
        pin_value(v[hgrp]);
    }
    for (int j = 0;;) {
#pragma unroll
        for (int hgrp = 0; hgrp < 8; ++hgrp) {
            const float s = row16_sum(v[hgrp]);
            if (c == 0) part[wave][2 * (4 * (hgrp & 3) + lr) + (hgrp >> 2)] = s;  // groups 0-3 gate, 4-7 up
        }
        block_lds_sync();
        if (wave == 0) {
            float hv = 0.f;
            if (lane < 16) {
                float gs = 0.f, us = 0.f;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    gs += part[q][2 * lane];
                    us += part[q][2 * lane + 1];
                }
                hv = swiglu_h(gs, us);
                a.h[(int64_t)(rec.j0 + j) * a.F + 16 * g + lane] = hv;
            }
            if (a.hp16) prep16_wave(hv, a.hp16 + ((int64_t)(rec.j0 + j) * (a.F / 16) + g) * kRec16Dwords, 1);
        }
        if (++j >= rec.n) break;
        block_lds_sync();  // part is rewritten for the next token
        load_q2k_prep(a.xp16 + ((int64_t)slot_token(rec, j) * 256 + 4 * cidx) * kRec16Dwords, xr);
#pragma unroll
        for (int hgrp = 0; hgrp < 8; ++hgrp)
            v[hgrp] = q2k_dot2(q2k_load(wb + 16 * (kK3PXu + kK3PHu * hgrp), (int64_t)lr * 4096 + 64 * cidx), xr);
    }
}

// K3 for CB2 gate/up rows of 4096 weights ("Understanding Dwarf Star", 2.4:
// per 256 weights an fp16 scale, 32 one-byte codebook indices of 8 values and
// one sign bit per weight).  The schedule of the Q2K kernel above: all copies
// issued at once, in the order [the raw codebook][records of the first token]
// [gate rows 0-15][up rows 0-15], and the dot products of each 4-row group as
// soon as it has landed.  Once the codebook has landed, each thread turns one
// entry into {values, negated values} in a table; a group's signed values are
// then two byte permutes, dotted as int8 against the token's int16 codes
// (records in natural byte order, two int8 halves) by v_dot4.  12 copies of
// 256 units: the last one's tail re-reads the final unit into spare LDS.
constexpr int kK3CCbU = 128;                              // codebook: 256 entries x 8 bytes
constexpr int kK3CXu = 640;                               // records of one token at n_embd 4096
constexpr int kK3CHu = 264;                               // 4 rows of 4096 CB2 weights: 64 blocks of 66 bytes
constexpr int kK3CUsed = kK3CCbU + kK3CXu + 8 * kK3CHu;  // 2880
constexpr int kK3CCopies = (kK3CUsed + 255) / 256;        // 12 per lane
constexpr int kK3CUnits = 256 * kK3CCopies;
static_assert(kK3CHu * 16 == 4 * 16 * kCB2Bytes, "4 rows of 16 blocks");

template <int END>
MOE_DEV void k3c_wait() {
    __builtin_amdgcn_sched_barrier(0);
    vmem_wait_le<kK3CCopies - (END + 255) / 256>();
    barrier_only();
    __builtin_amdgcn_sched_barrier(0);
}

template <int HG>
MOE_DEV float k3c_group(const uint8_t *wb, int lr, int cidx, const XQ2K &xr, const u32x4 *tab) {
    return cb2_dot_int(cb2_load(wb + 16 * (kK3CCbU + kK3CXu + kK3CHu * HG), (int64_t)lr * 4096 + 64 * cidx), xr, tab);
}

__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 8))) dec_k3_cb24096_kernel(FfnArgs a) {
    __shared__ __align__(16) u32x4 wbuf[kK3CUnits];
    __shared__ u32x4 cbt[256];
    __shared__ float part[4][32];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int gpe = a.F / 16, slot = blockIdx.x / gpe, g = blockIdx.x % gpe;
    const uint32_t lb = (uint32_t)__builtin_amdgcn_readfirstlane(lds_addr(wbuf) + 1024 * wave);
    const u32x4 *cs = (const u32x4 *)a.codebook;
    constexpr int kPre = (kK3CCbU + kK3CXu) / 256;  // copies 0-2 hold the codebook and records only
    static_assert((kK3CCbU + kK3CXu) % 256 == 0, "whole copies before the rows");
    // one token (k3_topk): the codebook and the token's records do not
    // depend on the slot, so their copies go out before the selection
    const int first = a.k3_topk ? kPre : 0;
    if (a.k3_topk) {
#pragma unroll
        for (int i = 0; i < kPre; ++i) {
            const int u = 256 * i + tid;
            dma16_m0(u < kK3CCbU ? cs + u : (const u32x4 *)a.xp16 + (u - kK3CCbU), lb + 4096 * i);
        }
    }
    const SlotRec rec = k3_slot(a, slot, g);
    if ((uint32_t)rec.e >= (uint32_t)a.E) {  // an empty slot (uniform over the block)
        vmem_wait_all();
        return;
    }
    constexpr int RB = 16 * kCB2Bytes;  // bytes of one row
    const int64_t goff = (int64_t)rec.e * a.gu_expert_bytes + (int64_t)16 * g * RB;
    const uint8_t *gm = a.gate + goff, *um = a.up + goff;
    {
        const u32x4 *xs = (const u32x4 *)(a.xp16 + (int64_t)slot_token(rec, 0) * (4096 / 16) * kRec16Dwords);
#pragma unroll
        for (int i = 0; i < kK3CCopies; ++i) {
            if (i < first) continue;
            const int u = min(256 * i + tid, kK3CUsed - 1);
            const void *src;
            if (u < kK3CCbU) src = cs + u;
            else if (u < kK3CCbU + kK3CXu) src = xs + (u - kK3CCbU);
            else if (u < kK3CCbU + kK3CXu + 4 * kK3CHu) src = gm + 16 * (u - kK3CCbU - kK3CXu);
            else src = um + 16 * (u - kK3CCbU - kK3CXu - 4 * kK3CHu);
            dma16_m0(src, lb + 4096 * i);
        }
    }
    const int c = lane & 15, lr = lane >> 4, cidx = 16 * wave + c;  // chunk of the row: 64 * cidx
    const uint8_t *wb = (const uint8_t *)wbuf;
    k3c_wait<kK3CCbU>();
    {
        const uint2 r = ((const uint2 *)wb)[tid];
        cbt[tid] = u32x4{r.x, r.y, neg_bytes(r.x), neg_bytes(r.y)};
    }
    block_lds_sync();
    XQ2K xr;
    float v[8];
    k3c_wait<kK3CCbU + kK3CXu>();
    load_q2k_prep((const uint32_t *)(wb + 16 * kK3CCbU) + 40 * cidx, xr);
    constexpr int X0 = kK3CCbU + kK3CXu;
    k3c_wait<X0 + 1 * kK3CHu>();
    v[0] = k3c_group<0>(wb, lr, cidx, xr, cbt);
    pin_value(v[0]);
    k3c_wait<X0 + 2 * kK3CHu>();
    v[1] = k3c_group<1>(wb, lr, cidx, xr, cbt);
    pin_value(v[1]);
    k3c_wait<X0 + 3 * kK3CHu>();
    v[2] = k3c_group<2>(wb, lr, cidx, xr, cbt);
    pin_value(v[2]);
    k3c_wait<X0 + 4 * kK3CHu>();
    v[3] = k3c_group<3>(wb, lr, cidx, xr, cbt);
    pin_value(v[3]);
    k3c_wait<X0 + 5 * kK3CHu>();
    v[4] = k3c_group<4>(wb, lr, cidx, xr, cbt);
    pin_value(v[4]);
    k3c_wait<X0 + 6 * kK3CHu>();
    v[5] = k3c_group<5>(wb, lr, cidx, xr, cbt);
    pin_value(v[5]);
    k3c_wait<X0 + 7 * kK3CHu>();
    v[6] = k3c_group<6>(wb, lr, cidx, xr, cbt);
    pin_value(v[6]);
    k3c_wait<X0 + 8 * kK3CHu>();
    v[7] = k3c_group<7>(wb, lr, cidx, xr, cbt);
    pin_value(v[7]);
    for (int j = 0;;) {
#pragma unroll
        for (int hgrp = 0; hgrp < 8; ++hgrp) {
            const float s = row16_sum(v[hgrp]);
            if (c == 0) part[wave][2 * (4 * (hgrp & 3) + lr) + (hgrp >> 2)] = s;  // groups 0-3 gate, 4-7 up
        }
        block_lds_sync();
        if (wave == 0) {
            float hv = 0.f;
            if (lane < 16) {
                float gs = 0.f, us = 0.f;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    gs += part[q][2 * lane];
                    us += part[q][2 * lane + 1];
                }
                hv = swiglu_h(gs, us);
                a.h[(int64_t)(rec.j0 + j) * a.F + 16 * g + lane] = hv;
            }
            if (a.hp16) prep16_wave(hv, a.hp16 + ((int64_t)(rec.j0 + j) * (a.F / 16) + g) * kRec16Dwords, 1);
        }
        if (++j >= rec.n) break;
        block_lds_sync();  // part is rewritten for the next token
        load_q2k_prep(a.xp16 + ((int64_t)slot_token(rec, j) * 256 + 4 * cidx) * kRec16Dwords, xr);
        // one group at a time (the table reads of several would not fit)
        v[0] = k3c_group<0>(wb, lr, cidx, xr, cbt);
        pin_value(v[0]);
        v[1] = k3c_group<1>(wb, lr, cidx, xr, cbt);
        pin_value(v[1]);
        v[2] = k3c_group<2>(wb, lr, cidx, xr, cbt);
        pin_value(v[2]);
        v[3] = k3c_group<3>(wb, lr, cidx, xr, cbt);
        pin_value(v[3]);
        v[4] = k3c_group<4>(wb, lr, cidx, xr, cbt);
        pin_value(v[4]);
        v[5] = k3c_group<5>(wb, lr, cidx, xr, cbt);
        pin_value(v[5]);
        v[6] = k3c_group<6>(wb, lr, cidx, xr, cbt);
        pin_value(v[6]);
        v[7] = k3c_group<7>(wb, lr, cidx, xr, cbt);
        pin_value(v[7]);
    }
}

// One block per 16 output rows, a wave per active slot in turn: the wave
// copies the slot expert's 16 down rows into its own LDS area with aligned
// 16-byte loads (no block barrier: every wave starts on its dots as soon as
// its own rows have landed), then dots them with the prepared h of every
// token of its bucket, into part[bucket position].  Then the combine adds,
// per output, the shared expert's term and the k routed terms in slot order.
// A Q8_0 shared down of width 2048 runs on the fp32 matrix cores
// (v_mfma_f32_16x16x4f32, tokens x rows): wave w takes columns [256 w,
// 256 w + 256) of the block's 16 rows for every token at once; lane l (token
// and row l % 16, quarter l / 16 of the wave's columns) holds 64 consecutive
// values of its token's hs and its row's weights d*q (exact in fp32), and
// instruction i takes value i of each quarter, so every product enters the
// sum once.  The waves' partial sums meet in LDS and the combine adds them
// in wave order.  One token, other shared formats and widths: the rows are
// dotted per token with the routed rows' VALU helpers.
template <int DFMT, int SFMT>
__global__ void __launch_bounds__(64 * kDecWaves) dec_k4_kernel(FfnArgs a) {
    static_assert(staged_fmt(DFMT), "staged formats only");
    static_assert(kDecRows == kShDownRowsK4 * kDecWaves, "shared rows per wave");
    __shared__ __align__(16) u32x4 wstage[kDecWaves][kK4WaveUnits];
    __shared__ uint32_t cb_lds[DFMT == MOE_CB2 || SFMT == MOE_CB2 ? 512 : 1];
    __shared__ __align__(16) float red[kDecWaves][8 * 64];
    __shared__ float part[kMaxDecPairs][kDecRows];
    __shared__ float ysl[kMaxDecTokens][kDecRows];
    __shared__ float wl[kMaxDecPairs];
    __shared__ int32_t posl[kMaxDecPairs];
    constexpr bool kShQ8 = SFMT == MOE_Q8_0;
    __shared__ float shp[kShQ8 ? kDecWaves : 1][kMaxDecTokens][kDecRows];  // matrix-core partial sums
    if constexpr (DFMT == MOE_CB2 || SFMT == MOE_CB2) load_codebook(a.codebook, cb_lds);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int row0 = blockIdx.x * kDecRows;
    const bool sh_mfma = kShQ8 && a.Fs == 256 * kDecWaves && a.T >= 2;  // one token: the VALU pass is shorter
    auto shared_down_mfma = [&]() {
        const int tq = lane & 15, kq = lane >> 4;
        const int k0 = 256 * wave + 64 * kq;
        const f32x4 *hp = (const f32x4 *)(a.hs + (int64_t)min(tq, a.T - 1) * a.Fs + k0);
        f32x4 hv[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) hv[i] = hp[i];
        // two Q8_0 blocks (68 bytes): d, 32 codes, d, 32 codes
        const uint8_t *wp = a.sh_down + (int64_t)(row0 + tq) * (a.Fs / 32 * kQ8Bytes) + (k0 / 32) * kQ8Bytes;
        uint32_t wd[17];
#pragma unroll
        for (int j = 0; j < 17; ++j) wd[j] = load_u32(wp + 4 * j);
        const float d0 = half_bits_to_float(wd[0] & 0xFFFFu), d1 = half_bits_to_float(wd[8] >> 16);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 64; ++i) {
            const int B = i < 32 ? 2 + i : 4 + i;  // byte of code i
            const int q = (int)(int8_t)(wd[B >> 2] >> (8 * (B & 3)));
            const float w = (i < 32 ? d0 : d1) * (float)q;
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(hv[i >> 2][i & 3], w, acc, 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) shp[kShQ8 ? wave : 0][4 * kq + j][tq] = acc[j];  // [token][row]
    };
    // The shared expert's down for rows row0 + 2 wave, +1 and every token
    // (fp32 activations hs), into ysl.  A wave with a routed slot runs it
    // while the copies of its first slot's rows are in flight.
    bool sh_pending = a.Fs > 0;
    auto shared_down = [&]() {
        sh_pending = false;
        if (sh_mfma) {
            shared_down_mfma();
            return;
        }
        const int r0 = row0 + kShDownRowsK4 * wave, c = lane % (a.Fs >> 6);
        for (int t = 0; t < a.T; ++t)
            rows_dot_ch<F32Chunk<SFMT>, false, 1>(
                a.sh_down, nullptr, a.Fs, 0, a.Fs, kShDownRowsK4, [&](int l) { return r0 + l; },
                [&](XF32 &hr) { load_x64(a.hs, 0, (int64_t)t * a.Fs + 64 * c, hr.x); }, cb_lds, lane, red[wave],
                [&](int l, float v, float) { ysl[t][kShDownRowsK4 * wave + l] = v; });
        sh_pending = false;
    };
    for (int p = tid; p < a.T * a.k; p += blockDim.x) {  // for the combine, read early
        wl[p] = a.topk_w[p];
        posl[p] = a.pos[p];
    }
    // rows per staged batch: 16, or fewer when 16 rows exceed the wave's area
    const int64_t b16 = fmt_bytes(DFMT, (int64_t)kDecRows * a.F);
    int rb = kDecRows;  // a power of two that divides kDecRows
    while ((int64_t)rb * b16 > (int64_t)kDecRows * 16 * kK4WaveUnits) rb >>= 1;
    const int c = lane % (a.F >> 6);
    const uint8_t *ws = (const uint8_t *)wstage[wave];
    for (int u = wave; u < a.nslots; u += kDecWaves) {
        const SlotRec rec = checked_slot(a, u);
        if ((uint32_t)rec.e >= (uint32_t)a.E) continue;
        const uint8_t *m = a.down + (int64_t)rec.e * a.down_expert_bytes;
        for (int r0 = 0; r0 < kDecRows; r0 += rb) {
            const int nunits = (int)(fmt_bytes(DFMT, (int64_t)rb * a.F) / 16);
            typename RawChunk<DFMT>::Prep hr;  // the first token's prepared h, in flight with the rows
            lane_prep<DFMT, DFMT == MOE_Q2K>(a.hp16, a.h, 0, rec.j0, a.F, c, hr);
            {
                const u32x4 *src = (const u32x4 *)(m + fmt_bytes(DFMT, (int64_t)(row0 + r0) * a.F));
                constexpr int kNI = (kK4WaveUnits + 63) / 64;
#pragma unroll
                for (int i = 0; i < kNI; ++i)
                    if (i * 64 + lane < nunits) lds_dma16(src + i * 64 + lane, &wstage[wave][i * 64]);
                if (sh_pending) shared_down();
                vmem_wait_all();
                wave_lds_sync();
            }
            for (int j = 0; j < rec.n; ++j) {
                if (j > 0) lane_prep<DFMT, DFMT == MOE_Q2K>(a.hp16, a.h, 0, rec.j0 + j, a.F, c, hr);
                float *dst = part[rec.j0 + j] + r0;
                lds_rows_dot<DFMT, false, 8>(ws, nullptr, a.F, 0, 0, a.F, rb, hr, cb_lds, lane, red[wave],
                                             [&](int l, float s, float) { dst[l] = s; });
            }
            wave_lds_sync();  // the area is rewritten by the next batch
        }
    }
    if (sh_pending) shared_down();
    block_lds_sync();
    for (int i = tid; i < a.T * kDecRows; i += blockDim.x) {
        const int t = i / kDecRows, r = i % kDecRows;
        const int64_t o = (int64_t)t * a.D + row0 + r;
        float acc = 0.f;
        if (sh_mfma) {
#pragma unroll
            for (int w = 0; w < kDecWaves; ++w) acc += shp[kShQ8 ? w : 0][t][r];
        } else if (a.Fs > 0) {
            acc = ysl[t][r];
        }
        for (int s = 0; s < a.k; ++s) {
            const int p = t * a.k + s;
            acc = __builtin_fmaf(wl[p], part[posl[p]][r], acc);
        }
        if (a.flags & MOE_ACCUMULATE) acc += a.y[o];
        a.y[o] = acc;
    }
}

// K4 for one token (k <= 6 slots; routed down Q2K and shared down Q8_0,
// both of width 2048).  Wave s < k takes slot s (16 rows of its expert's
// down matrix); waves 6 and 7 take 8 rows each of the shared expert's down.
// Each wave copies what it reads into its own LDS area, all copies issued at
// once: first the activations (the pair's prepared h row; for the shared
// waves, hs), then its rows in order, and starts on each group of rows as
// soon as the copies covering it have landed.  With one token, slot s
// (ascending expert) holds bucket position s.  The activations are placed
// in LDS permuted (the permutation is applied to the copy sources) so that
// the lanes of a 16-lane group read 16 different bank groups.
constexpr int kK4T1Hu = 320;                // units of a prepared h row of 2048 (32 chunks of 10 units)
constexpr int kK4T1Ru = 672;                // units of 16 Q2K rows of 2048
constexpr int kK4T1SlotCopies = 16;         // (320 + 672 = 992) -> 16 copies of 64 units
constexpr int kK4T1Hsu = 512;               // units of hs: 2048 fp32 (32 chunks of 16 units)
constexpr int kK4T1Su = 8 * 136;            // units of 8 Q8_0 rows of 2048
constexpr int kK4T1ShCopies = 25;           // (512 + 1088 = 1600) -> 25 copies of 64 units
static_assert(kK4T1Hu + kK4T1Ru <= 64 * kK4T1SlotCopies && kK4T1Hsu + kK4T1Su == 64 * kK4T1ShCopies, "areas");

template <int NC, int END>  // the wave's copies covering its units [0, end) have landed
MOE_DEV void k4t1_wait() {
    __builtin_amdgcn_sched_barrier(0);
    vmem_wait_le<NC - (END + 63) / 64>();
    __builtin_amdgcn_sched_barrier(0);
}

MOE_DEV float sum32(float v) {  // over lanes [32 r, 32 r + 32)
    v = row16_sum(v);
    return v + __shfl_xor(v, 16, kWave);
}

// With k3_topk (no K2) a ninth wave selects the top-k again from the logits
// while the others stream, for the combine's weights and bucket positions;
// block 0's also writes the routing (top-k, weights and bucketing).
__global__ void __launch_bounds__(576) dec_k4_t1_kernel(FfnArgs a) {
    __shared__ __align__(16) u32x4 sarea[6][64 * kK4T1SlotCopies];
    __shared__ __align__(16) u32x4 harea[2][64 * kK4T1ShCopies];
    __shared__ float part[6][kDecRows];
    __shared__ float ysl[kDecRows];
    __shared__ float wl[6];
    __shared__ int32_t posl[6];
    __shared__ int32_t sidx[6];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int row0 = blockIdx.x * kDecRows, k = a.k;
    const int r = lane >> 5, c = lane & 31;  // row parity, 64-weight chunk of the row
    if (wave == 8) {
        if (a.k3_topk) {
            const bool out = blockIdx.x == 0;
            const int my_e = select_topk(a.logits, a.E, k, a.route_scale, sidx, wl);
            const int rank = rank_among_k(my_e, k);
            if (lane < k) posl[lane] = rank;
            if (out) {
                if (lane < k) {
                    a.w_topk_idx[lane] = my_e;
                    a.w_topk_w[lane] = wl[lane];
                }
                bucket_one_token(my_e, k, a.E, a.w_count, a.w_offset, a.w_perm, a.w_pos, a.w_active, a.w_n_active,
                                 nullptr, 0);
            }
        }
    } else if (!a.k3_topk && tid < k) {
        wl[tid] = a.topk_w[tid];
        posl[tid] = a.pos[tid];
    }
    if (wave < 6) {
        const SlotRec rec = wave < k ? checked_slot(a, wave) : make_slot(-1, 0, 0, 0, 0);
        if ((uint32_t)rec.e < (uint32_t)a.E) {
            constexpr int RB = 8 * kQ2KBytes;  // bytes of a row
            const uint8_t *hrow = (const uint8_t *)(a.hp16 + (int64_t)rec.j0 * (2048 / 16) * kRec16Dwords);
            const uint8_t *rows = a.down + (int64_t)rec.e * a.down_expert_bytes + (int64_t)row0 * RB;
            const uint32_t lb = (uint32_t)__builtin_amdgcn_readfirstlane(lds_addr(sarea[wave]));
#pragma unroll
            for (int i = 0; i < kK4T1SlotCopies; ++i) {
                const int u = 64 * i + lane;
                const uint8_t *src;
                if (u < kK4T1Hu) {  // record unit m of chunk cc sits at (m + (cc >> 3 & 1)) % 10
                    const int cc = u / 10, m = u - 10 * cc, g = (cc >> 3) & 1;
                    src = hrow + 16 * (10 * cc + (m + 10 - g) % 10);
                } else {
                    src = rows + 16 * min(u - kK4T1Hu, kK4T1Ru - 1);
                }
                dma16_m0(src, lb + 1024 * i);
            }
            const uint8_t *ab = (const uint8_t *)sarea[wave];
            const uint8_t *wb = ab + 16 * kK4T1Hu;
            XQ2K xr;
            float v[8];
            auto group = [&](int gq) {  // rows 4 gq + 2 i + r
                if (gq == 0) {
                    const int g = (c >> 3) & 1;
                    u32x4 *dst = (u32x4 *)&xr;
#pragma unroll
                    for (int m = 0; m < 10; ++m) dst[m] = *(const u32x4 *)(ab + 16 * (10 * c + (m + g) % 10));
                }
#pragma unroll
                for (int i = 0; i < 2; ++i)
                    v[2 * gq + i] = q2k_dot2(q2k_load(wb + RB * (4 * gq + 2 * i + r), 64 * c), xr);
                pin_value(v[2 * gq]);  // computed here, not sunk below the next wait
                pin_value(v[2 * gq + 1]);
            };
            k4t1_wait<kK4T1SlotCopies, kK4T1Hu + 4 * RB / 16>();
            group(0);
            k4t1_wait<kK4T1SlotCopies, kK4T1Hu + 8 * RB / 16>();
            group(1);
            k4t1_wait<kK4T1SlotCopies, kK4T1Hu + 12 * RB / 16>();
            group(2);
            k4t1_wait<kK4T1SlotCopies, kK4T1Hu + 16 * RB / 16>();
            group(3);
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const float sv = sum32(v[q]);
                if (c == 0) part[rec.j0][4 * (q >> 1) + 2 * (q & 1) + r] = sv;
            }
        }
    } else if (wave < 8 && a.Fs > 0) {
        const int h = wave - 6;  // rows row0 + 8 h .. + 8
        constexpr int SB = 2048 / 32 * kQ8Bytes;  // bytes of a row
        const uint8_t *hsb = (const uint8_t *)a.hs;
        const uint8_t *rows = a.sh_down + (int64_t)(row0 + 8 * h) * SB;
        const uint32_t lb = (uint32_t)__builtin_amdgcn_readfirstlane(lds_addr(harea[h]));
#pragma unroll
        for (int i = 0; i < kK4T1ShCopies; ++i) {
            const int u = 64 * i + lane;
            const uint8_t *src;
            if (u < kK4T1Hsu) {  // float4 j of chunk cc sits at j ^ (cc & 15)
                const int cc = u >> 4, j = u & 15;
                src = hsb + 16 * (16 * cc + (j ^ (cc & 15)));
            } else {
                src = rows + 16 * (u - kK4T1Hsu);
            }
            dma16_m0(src, lb + 1024 * i);
        }
        const uint8_t *ab = (const uint8_t *)harea[h];
        const uint8_t *wb = ab + 16 * kK4T1Hsu;
        float xv[64];
        float v[4];
        auto pair = [&](int q) {  // rows 2 q + r
            if (q == 0) {
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const f32x4 t4 = *(const f32x4 *)(ab + 16 * (16 * c + (j ^ (c & 15))));
                    xv[4 * j] = t4[0];
                    xv[4 * j + 1] = t4[1];
                    xv[4 * j + 2] = t4[2];
                    xv[4 * j + 3] = t4[3];
                }
            }
            v[q] = q8_dot(q8_load(wb + SB * (2 * q + r), 64 * c), xv);
            pin_value(v[q]);
        };
        k4t1_wait<kK4T1ShCopies, kK4T1Hsu + 2 * SB / 16>();
        pair(0);
        k4t1_wait<kK4T1ShCopies, kK4T1Hsu + 4 * SB / 16>();
        pair(1);
        k4t1_wait<kK4T1ShCopies, kK4T1Hsu + 6 * SB / 16>();
        pair(2);
        k4t1_wait<kK4T1ShCopies, kK4T1Hsu + 8 * SB / 16>();
        pair(3);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float sv = sum32(v[q]);
            if (c == 0) ysl[8 * h + 2 * q + r] = sv;
        }
    }
    __syncthreads();
    if (tid < kDecRows) {
        const int64_t o = row0 + tid;
        float acc = a.Fs > 0 ? ysl[tid] : 0.f;
        for (int q = 0; q < k; ++q) acc = __builtin_fmaf(wl[q], part[posl[q]][tid], acc);
        if (a.flags & MOE_ACCUMULATE) acc += a.y[o];
        a.y[o] = acc;
    }
}

FfnArgs make_ffn_args(const moe_layer_desc *d, const void *x, int32_t T, int32_t x_type, const RoutingPtrs &r,
                      float *y, uint32_t flags, const Workspace &ws) {
    FfnArgs a{};
    a.gate = (const uint8_t *)d->gate;
    a.up = (const uint8_t *)d->up;
    a.down = (const uint8_t *)d->down;
    a.sh_gate = (const uint8_t *)d->sh_gate;
    a.sh_up = (const uint8_t *)d->sh_up;
    a.sh_down = (const uint8_t *)d->sh_down;
    a.codebook = d->codebook;
    a.x = x;
    a.x_bf16 = x_type == MOE_BF16;
    a.T = T;
    a.D = d->n_embd;
    a.F = d->n_ff_exp;
    a.Fs = d->n_ff_shared;
    a.k = d->n_expert_used;
    a.E = d->n_expert;
    a.gu_expert_bytes = fmt_bytes(d->gate_type, (int64_t)a.F * a.D);
    a.down_expert_bytes = fmt_bytes(d->down_type, (int64_t)a.F * a.D);
    a.topk_idx = a.w_topk_idx = r.topk_idx;
    a.topk_w = a.w_topk_w = r.topk_w;
    a.count = a.w_count = r.count;
    a.offset = a.w_offset = r.offset;
    a.perm = a.w_perm = r.perm;
    a.pos = a.w_pos = r.pos;
    a.active = a.w_active = r.active;
    a.n_active = a.w_n_active = r.n_active;
    a.h = ws.h;
    a.hs = ws.hs;
    a.ypart = ws.ypart;
    a.ys = ws.ys;
    a.y = y;
    a.flags = flags;
    a.router_w = d->router_w;
    a.router_bias = d->router_bias;
    a.route_scale = d->route_scale;
    a.logits = ws.logits;
    a.xp16 = a.xq8 = a.hp16 = nullptr;
    a.k3_topk = 0;
    a.norm_gamma = nullptr;
    a.norm_eps = 0.f;
    return a;
}

bool small_path_ok(const moe_layer_desc *d, int32_t T) {
    return T <= kMaxDecTokens && (int64_t)T * d->n_expert_used <= kMaxDecPairs && staged_fmt(d->gate_type) &&
           staged_fmt(d->down_type);
}

bool small_route_ok(const moe_layer_desc *d, int32_t T) { return route_small_ok(T, d->n_expert, d->n_expert_used); }

// stage 0 = all; 1..4 = K1..K4.  route: also compute the routing (K1's router
// blocks and K2's block 0); otherwise the routing in r is given.
// The one-token schedule without K2 (the routed gate/up blocks select the
// top-k, the down kernel writes the routing), when it applies.
bool t1_schedule_ok(const moe_layer_desc *d, int32_t T, int32_t x_type) {
    const bool has_sh = d->n_ff_shared > 0;
    const bool sg_staged = has_sh && d->shared_type == MOE_Q8_0 && d->n_embd == 4096 && d->n_ff_shared % 8 == 0;
    const bool k4t1 = T == 1 && d->down_type == MOE_Q2K && d->n_ff_exp == 2048 && d->n_expert_used <= 6 &&
                      d->n_embd % kDecRows == 0 &&
                      (d->n_ff_shared == 0 || (d->n_ff_shared == 2048 && d->shared_type == MOE_Q8_0));
    return small_path_ok(d, T) && small_route_ok(d, T) && k4t1 && x_type == MOE_F32 && d->n_embd == 4096 &&
           (!has_sh || sg_staged);
}

hipError_t launch_small(const moe_layer_desc *d, const void *x, int32_t T, int32_t x_type, const RoutingPtrs &r,
                        float *y, uint32_t flags, const Workspace &ws, hipStream_t s, int stage, bool route,
                        const float *gamma, float eps) {
    FfnArgs a = make_ffn_args(d, x, T, x_type, r, y, flags, ws);
    const bool has_sh = a.Fs > 0;
    a.shared_fmt = has_sh ? d->shared_type : MOE_Q8_0;
    a.n_router_blocks = route ? a.E : 0;
    a.slots = ws.slots;
    a.nslots = (int)std::min<int64_t>((int64_t)T * a.k, a.E);
    a.build_slots = route ? 0 : 1;
    if (d->gate_type == MOE_Q2K) a.xp16 = ws.xp16;  // x records for the routed gate/up, written by K1
    const bool cb4096 = d->gate_type == MOE_CB2 && a.D == 4096;
    if (cb4096) {  // natural-order records for the codebook gate/up kernel
        a.xp16 = ws.xp16;
        a.xp16_nat = 1;
    }
    if (d->down_type == MOE_Q2K) a.hp16 = ws.hp16;  // h records for the routed down, written by K3
    // a Q8_0 shared expert at n_embd 4096 takes the staged K2: at one token on
    // x records written by K1, at several on the matrix cores from x itself
    const bool sg_staged = has_sh && a.shared_fmt == MOE_Q8_0 && a.D == 4096 && a.Fs % 8 == 0;
    if (sg_staged && T == 1) a.xq8 = ws.xq8;
    // the one-token down kernel
    const bool k4t1 = T == 1 && d->down_type == MOE_Q2K && a.F == 2048 && a.k <= 6 && a.D % kDecRows == 0 &&
                      (a.Fs == 0 || (a.Fs == 2048 && a.shared_fmt == MOE_Q8_0));
    // one fp32 token at n_embd 4096 with a Q8_0 shared expert (or none) and
    // the one-token down kernel: K1 also runs the shared gate/up, the routed
    // gate/up blocks select the top-k themselves and the down kernel writes
    // the routing, so there is no K2
    const bool t1 = route && k4t1 && x_type == MOE_F32 && a.D == 4096 && (!has_sh || sg_staged);
    if (gamma && !(t1 && (d->gate_type == MOE_Q2K || d->gate_type == MOE_CB2))) return hipErrorInvalidValue;
    if (t1) {
        a.k3_topk = 1;
        a.xq8 = nullptr;
        a.norm_gamma = gamma;
        a.norm_eps = eps;
    }
    a.n_prep_blocks = a.xp16 || a.xq8 ? (T * (a.D / 64) + 3) / 4 : 0;
    a.n_shgu_blocks = has_sh ? (a.Fs + 4 * kShGuRows - 1) / (4 * kShGuRows) : 0;
    const int k1 = t1 ? std::max(std::max(a.E, has_sh ? a.Fs / 8 : 0), 16)
                      : a.build_slots + a.n_router_blocks + a.n_prep_blocks;
    const int k2 = t1 ? 0 : (route ? 1 : 0) + a.n_shgu_blocks;
    const int k3 = a.nslots * (a.F / 16);
    if ((stage == 0 || stage == 1) && k1 > 0)
    {
        if (t1 && gamma) dec_k1_t1_kernel<true><<<k1, 256, 0, s>>>(a);
        else if (t1) dec_k1_t1_kernel<false><<<k1, 256, 0, s>>>(a);
        else if (x_type == MOE_BF16) dec_k1_kernel<MOE_BF16><<<k1, 256, 0, s>>>(a);
        else dec_k1_kernel<MOE_F32><<<k1, 256, 0, s>>>(a);
    }
    if ((stage == 0 || stage == 2) && k2 > 0)
    {
        if (sg_staged && T >= 2) {
            dec_k2_q8sg_mfma_kernel<<<(route ? 1 : 0) + a.Fs / 8, 64 * kSgmWaves, 0, s>>>(a, route ? 1 : 0);
        } else if (sg_staged) {
            const int mode = !route ? 0 : (T == 1 && a.k <= 16 ? 2 : 1);
            dec_k2_q8sg4096_kernel<<<(mode == 1 ? 1 : 0) + a.Fs / 8, 320, 0, s>>>(a, mode);
        }
        else with_fmt(a.shared_fmt, [&](auto S) { dec_k2_kernel<decltype(S)::value><<<k2, 256, 0, s>>>(a, route ? 1 : 0); });
    }
    if (stage == 0 || stage == 3) {
        if (cb4096) dec_k3_cb24096_kernel<<<k3, 256, 0, s>>>(a);
        else if (d->gate_type == MOE_CB2) dec_k3_kernel<MOE_CB2><<<k3, 256, 0, s>>>(a);
        else if (d->gate_type == MOE_Q4K) dec_k3_kernel<MOE_Q4K><<<k3, 256, 0, s>>>(a);
        else if (a.D == 4096) dec_k3_q2k4096_kernel<<<k3, 256, 0, s>>>(a);
        else dec_k3_kernel<MOE_Q2K><<<k3, 256, 0, s>>>(a);
    }
    if (stage == 0 || stage == 4) {
        if (k4t1) dec_k4_t1_kernel<<<a.D / kDecRows, 64 * (kDecWaves + 1), 0, s>>>(a);
        else with_fmt(a.shared_fmt, [&](auto S) {
            constexpr int SF = decltype(S)::value;
            if (d->down_type == MOE_CB2) dec_k4_kernel<MOE_CB2, SF><<<a.D / kDecRows, 64 * kDecWaves, 0, s>>>(a);
            else if (d->down_type == MOE_Q4K) dec_k4_kernel<MOE_Q4K, SF><<<a.D / kDecRows, 64 * kDecWaves, 0, s>>>(a);
            else dec_k4_kernel<MOE_Q2K, SF><<<a.D / kDecRows, 64 * kDecWaves, 0, s>>>(a);
        });
    }
    return hipGetLastError();
}

}  // namespace moe
