// k_shared.hip - the shared expert of a batch of fp32 token rows as two dense
// Q8_0 GEMMs on the matrix cores ("Understanding Dwarf Star", 5.3.7 step 1:
// the shared expert's SwiGLU FFN for every token; 2.8.2 the block-quantized
// dot; the Q8_0 subsection: 32 int8 codes and one fp16 scale d per block).
//
// Per 32-weight block of a weight row and a token row:
//   sum_k w_k x_k = d * sum_k q_k x_k ~= d * (sum_k q_k c_k) / S
// with the token row's int16 codes c = rint(x*S), S = 32512 / max|row|, split
// as c = 256*hi + lo.  The integer sum runs on v_mfma_i32_16x16x32_i8 (one
// instruction per block and plane: K = 32 is exactly one Q8_0 block), exact in
// int32; each lane owns one weight row (the output column) and so applies its
// row's d to every product it holds, in fp32, once per block.
//
// Byte order: a pair of blocks (68 bytes, dword aligned in the row) holds the
// codes of the even block at bytes 2..33 and of the odd block at bytes 36..67.
// The odd block's 8 dwords are used as they are; the even block's are taken as
// dwords 1..7 (codes 2..29) and one dword made of bytes 2, 3 and 32, 33 (codes
// 0, 1, 30, 31).  The activation codes are written in that same order (the
// record layout and writer are in ffn_dev.h; the many-row preparing kernel
// fills them), so the weights reach the matrix cores without any shuffling.
#include "ffn_dev.h"

namespace moe {

typedef int sgq_v4i __attribute__((ext_vector_type(4)));

constexpr int kSgqWaves = 8;       // waves of a block: they split the reduction
constexpr int kSgqRows = 16;       // weight rows of a block (the MFMA's columns)
constexpr int kSgqTileTok = 16;    // token rows of an MFMA tile
constexpr int kSgqTiles = 2;       // token tiles per pass
constexpr int kSgqGroup = 4;       // block pairs a wave loads before it multiplies
constexpr int kSgqChunk = 64;      // block pairs of a staged row: reductions up to 4096 values
constexpr int kSgqRowDw = kSgqChunk * 17 + 4;  // LDS dwords of a staged row (4 more: rows 4 banks apart)
constexpr int kSgqRowU = kSgqRowDw / 4;        // 16-byte units of a staged row
constexpr int kSgqUnits = kSgqRows * kSgqRowU;  // 16-byte units of the staged rows
constexpr int kSgqDmaSlots = ((kSgqUnits + 63) / 64 + kSgqWaves - 1) / kSgqWaves;  // 64-unit copies a wave
// 4-byte copies per thread of a full chunk
constexpr int kSgqStage4 = (kSgqRows * kSgqChunk * 17 + 64 * kSgqWaves - 1) / (64 * kSgqWaves);
struct SgqArgs {
    const uint8_t *w0, *w1;  // MODE 0: gate and up rows [Fs][K]; MODE 1: down rows [D][K]
    const uint32_t *aq;      // token records [T][K/64][32 dwords]
    const float *ainv;       // 1/S of each token row
    int T, K;
    float *out;              // MODE 0: hs [T][Fs]; MODE 1: ys [T][D]
    int ld;                  // row length of out
};

// MODE 0: block b owns gate rows 8b..8b+7 (columns 0-7) and the same up rows
// (columns 8-15) and writes hs = silu(g) * u; MODE 1: down rows 16b..16b+15,
// written to ys.  The block's 16 weight rows are first copied into LDS, up to
// kSgqChunk block pairs of each at a time, by 16-byte global-to-LDS copies
// along the rows, so that the matrix operands come from LDS instead of from
// many narrow global loads.  Wave w takes the block pairs w, w + 8, ... of a
// chunk; the partial sums meet in LDS and are added in wave order.
template <int MODE>
__global__ void __launch_bounds__(64 * kSgqWaves) sgq_gemm_kernel(SgqArgs a) {
    __shared__ float red[kSgqWaves][kSgqTiles][4][64];
    __shared__ u32x4 wst4[kSgqRows * kSgqRowDw / 4];
    uint32_t *const wst = (uint32_t *)wst4;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int j = lane & 15, g = lane >> 4;  // the lane's weight row (column) and k group
    const int64_t rowbytes = (int64_t)(a.K / 32) * kQ8Bytes;
    const int np = a.K / 64;
    auto row_ptr = [&](int r) -> const uint8_t * {
        if (MODE == 0) return (r < 8 ? a.w0 : a.w1) + (int64_t)(8 * blockIdx.x + (r & 7)) * rowbytes;
        return a.w0 + (int64_t)(kSgqRows * blockIdx.x + r) * rowbytes;
    };
    // the 16 rows go to wst (row r at dword r * kSgqRowDw, 17 dwords a block
    // pair); the launcher takes this kernel only for np <= kSgqChunk
    const bool vec = (np & 3) == 0;  // rows and chunk starts 16-byte aligned
    // vec: the copies go straight to LDS (global_load_lds, 64 consecutive
    // 16-byte units an instruction): LDS unit P = 273 r + u holds unit u of
    // row r's chunk; a unit beyond the chunk (the pad, or a short chunk's
    // tail) takes a copy of unit 0 and is never read.
    auto stage_dma = [&]() {
        const int nu = np * 17 >> 2;
        const uint32_t lds0 = lds_addr(wst4);
#pragma unroll
        for (int i = 0; i < kSgqDmaSlots; ++i) {
            const int slot = i * kSgqWaves + wave;
            if (slot * 64 < kSgqUnits) {  // uniform over the wave
                const int P = slot * 64 + lane, r = min(P / kSgqRowU, kSgqRows - 1), u = P - r * kSgqRowU;
                const uint8_t *src = row_ptr(r) + 16 * (u < nu ? u : 0);
                const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds0 + 16u * (uint32_t)(slot * 64));
                if (P < kSgqUnits) dma16_m0(src, m0);
            }
        }
    };
    // rows whose length is not a multiple of 16 bytes (64 or 128 values):
    // dwords through registers, 8 a thread in flight at a time
    auto stage_words = [&]() {
        const int rdw = np * 17;
        for (int i0 = 0; i0 < kSgqStage4; i0 += 8) {
            uint32_t v[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int q = tid + (i0 + i) * 64 * kSgqWaves, r = q / rdw, u = q - r * rdw;
                if (i0 + i < kSgqStage4 && r < kSgqRows) v[i] = load_u32(row_ptr(r) + 4 * u);
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int q = tid + (i0 + i) * 64 * kSgqWaves, r = q / rdw, u = q - r * rdw;
                if (i0 + i < kSgqStage4 && r < kSgqRows) wst[r * kSgqRowDw + u] = v[i];
            }
        }
    };
    if (!vec) {
        stage_words();
        __syncthreads();
    }
    bool staged = !vec;  // every pass over the tokens uses the one staged copy
    const uint32_t *const wrow = wst + j * kSgqRowDw;
    for (int t0 = 0; t0 < a.T; t0 += kSgqTiles * kSgqTileTok) {
        float tot[kSgqTiles][4];
#pragma unroll
        for (int i = 0; i < kSgqTiles; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) tot[i][r] = 0.f;
        // the token rows this lane feeds to the A operand (row j of each tile)
        const uint32_t *arow[kSgqTiles];
        bool aok[kSgqTiles];
#pragma unroll
        for (int i = 0; i < kSgqTiles; ++i) {
            const int t = t0 + kSgqTileTok * i + j;
            aok[i] = t < a.T;
            arow[i] = a.aq + (int64_t)(aok[i] ? t : 0) * np * kSgqPairDw + 4 * g;
        }
        // groups of kSgqGroup pairs: the activation loads of a group are
        // issued before its products, those of the first group also
        // before the weights' copies to LDS, so that both streams are in
        // flight together (every wave runs the first group, even one
        // with no pair in it, so that all of them reach the barriers)
        for (int p0 = wave, first = 1;; p0 += kSgqGroup * kSgqWaves, first = 0) {
            if (!first && p0 >= np) break;  // uniform over the wave
            u32x4 hv[kSgqGroup][kSgqTiles], lv[kSgqGroup][kSgqTiles];
#pragma unroll
            for (int u = 0; u < kSgqGroup; ++u) {
                const int p = p0 + u * kSgqWaves;
                const bool pok = p < np;
#pragma unroll
                for (int i = 0; i < kSgqTiles; ++i) {
                    hv[u][i] = lv[u][i] = u32x4{0u, 0u, 0u, 0u};
                    if (aok[i] && pok) {
                        hv[u][i] = *(const u32x4 *)(arow[i] + p * kSgqPairDw);
                        lv[u][i] = *(const u32x4 *)(arow[i] + p * kSgqPairDw + 16);
                    }
                }
            }
            if (!staged && first) {
                // after the group's activation loads, so that both are in
                // flight at once (every wave passes here)
                stage_dma();
                vmem_wait_le<0>();
                __syncthreads();
                staged = true;
            }
#pragma unroll
            for (int u = 0; u < kSgqGroup; ++u) {
                const int p = p0 + u * kSgqWaves;
                if (p >= np) break;  // uniform over the wave
                const uint32_t *wp = wrow + 17 * p;
                const uint32_t w0 = wp[0], w8 = wp[8];
                uint2 ev = {wp[1 + 2 * g], wp[2 + 2 * g]};
                const uint2 ov = {wp[9 + 2 * g], wp[10 + 2 * g]};
                if (g == 3) ev.y = __builtin_amdgcn_alignbyte(w8, w0, 2);  // codes 0, 1, 30, 31
                const float d0 = half_bits_to_float(w0 & 0xFFFFu), d1 = half_bits_to_float(w8 >> 16);
                long be, bo;
                __builtin_memcpy(&be, &ev, 8);
                __builtin_memcpy(&bo, &ov, 8);
#pragma unroll
                for (int i = 0; i < kSgqTiles; ++i) {
                    long he, ho, le, lo;
                    const uint2 hve = {hv[u][i][0], hv[u][i][1]}, hvo = {hv[u][i][2], hv[u][i][3]};
                    const uint2 lve = {lv[u][i][0], lv[u][i][1]}, lvo = {lv[u][i][2], lv[u][i][3]};
                    __builtin_memcpy(&he, &hve, 8);
                    __builtin_memcpy(&ho, &hvo, 8);
                    __builtin_memcpy(&le, &lve, 8);
                    __builtin_memcpy(&lo, &lvo, 8);
                    const sgq_v4i z = {0, 0, 0, 0};
                    sgq_v4i ce = __builtin_amdgcn_mfma_i32_16x16x32_i8(he, be, z, 0, 0, 0);
                    sgq_v4i co = __builtin_amdgcn_mfma_i32_16x16x32_i8(ho, bo, z, 0, 0, 0);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        ce[r] <<= 8;
                        co[r] <<= 8;
                    }
                    ce = __builtin_amdgcn_mfma_i32_16x16x32_i8(le, be, ce, 0, 0, 0);
                    co = __builtin_amdgcn_mfma_i32_16x16x32_i8(lo, bo, co, 0, 0, 0);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        tot[i][r] = __builtin_fmaf(d0, (float)ce[r], tot[i][r]);
                        tot[i][r] = __builtin_fmaf(d1, (float)co[r], tot[i][r]);
                    }
                }
            }
        }
        // output element of register r: token 4g + r of the tile, column j
#pragma unroll
        for (int i = 0; i < kSgqTiles; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) red[wave][i][r][lane] = tot[i][r];
        __syncthreads();
        if (MODE == 0) {
            // one output per thread: tile i, register r, k group g2, gate column c
            const int tid = threadIdx.x;
            if (tid < kSgqTiles * 4 * 4 * 8) {
                const int i = tid >> 7, r = (tid >> 5) & 3, g2 = (tid >> 3) & 3, c = tid & 7;
                const int t = t0 + kSgqTileTok * i + 4 * g2 + r;
                float gs = 0.f, us = 0.f;
#pragma unroll
                for (int w = 0; w < kSgqWaves; ++w) {
                    gs += red[w][i][r][16 * g2 + c];
                    us += red[w][i][r][16 * g2 + 8 + c];
                }
                if (t < a.T) {
                    const float s = a.ainv[t];
                    a.out[(int64_t)t * a.ld + 8 * blockIdx.x + c] = swiglu_h(gs * s, us * s);
                }
            }
        } else {
            for (int o = threadIdx.x; o < kSgqTiles * 4 * 64; o += 64 * kSgqWaves) {
                const int i = o >> 8, r = (o >> 6) & 3, l = o & 63;
                const int t = t0 + kSgqTileTok * i + 4 * (l >> 4) + r;
                float s = 0.f;
#pragma unroll
                for (int w = 0; w < kSgqWaves; ++w) s += red[w][i][r][l];
                if (t < a.T) a.out[(int64_t)t * a.ld + kSgqRows * blockIdx.x + (l & 15)] = s * a.ainv[t];
            }
        }
        __syncthreads();  // red is rewritten by the next pass
    }
}

bool shared_q8_mfma_ok(const moe_layer_desc *d) {
    return d->n_ff_shared > 0 && d->shared_type == MOE_Q8_0 && d->n_embd % 64 == 0 && d->n_ff_shared % 64 == 0 &&
           d->n_embd <= 64 * kSgqChunk && d->n_ff_shared <= 64 * kSgqChunk;
}

// stage 3: the gate/up GEMM into hs, on x's records; stage 4: the down GEMM
// into ys, on hs's records.  The records (sg_aq) and the rows' 1/S come from
// the many-row preparing kernel (pf_prep_rows_kernel), which codes x for the
// routed GEMMs at the same scale and hs in blocks of its own.
hipError_t launch_shared_q8_mfma(const moe_layer_desc *d, int32_t T, const Workspace &ws, const float *ainv,
                                 hipStream_t s, int stage) {
    const int D = d->n_embd, Fs = d->n_ff_shared;
    SgqArgs a{};
    a.T = T;
    a.aq = ws.sg_aq;
    a.ainv = ainv;
    if (stage == 3) {
        a.w0 = (const uint8_t *)d->sh_gate;
        a.w1 = (const uint8_t *)d->sh_up;
        a.K = D;
        a.out = ws.hs;
        a.ld = Fs;
        sgq_gemm_kernel<0><<<Fs / 8, 64 * kSgqWaves, 0, s>>>(a);
    } else {
        a.w0 = a.w1 = (const uint8_t *)d->sh_down;
        a.K = Fs;
        a.out = ws.ys;
        a.ld = D;
        sgq_gemm_kernel<1><<<D / kSgqRows, 64 * kSgqWaves, 0, s>>>(a);
    }
    return hipGetLastError();
}

}  // namespace moe
