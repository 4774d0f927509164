// ffn_dev.h - device pieces of the expert FFNs for a handful of token rows
// ("Understanding Dwarf Star", 2.8.2 the fused dequant-dot over 256-weight
// blocks; 5.2.4 and 5.3.7 step 4 gate -> activation -> down; 5.3.4 the shared
// expert).  A lane owns 64 consecutive weights of a row (for the 2-bit format
// one 16-byte load of codes plus its scale bytes); the lanes of a row are
// combined with a butterfly; a wave loads all the row chunks it will use
// before it computes any of them.
#pragma once
#include <type_traits>

#include "common.h"

namespace moe {

struct FfnArgs {
    const uint8_t *gate, *up, *down, *sh_gate, *sh_up, *sh_down;
    const int8_t *codebook;
    const void *x;
    int x_bf16;
    int T, D, F, Fs, k, E;
    int64_t gu_expert_bytes, down_expert_bytes;
    const int32_t *topk_idx;
    const float *topk_w;
    const int32_t *count, *offset, *perm, *pos, *active, *n_active;
    float *h, *hs, *ypart, *ys, *y;
    uint32_t flags;
    // routing inputs for the kernels that also run the router
    const float *router_w, *router_bias;
    float route_scale;
    double *logits;
    int n_router_blocks, n_slot_blocks;
    int32_t *w_topk_idx, *w_count, *w_offset, *w_perm, *w_pos, *w_active, *w_n_active;
    float *w_topk_w;
    // prepared activations (NULL when the path does not use them)
    uint32_t *xp16, *hp16;
    int n_prep_blocks;
};

// Load the lane's 64 activations at element offset off of x (fp32 or bf16).
MOE_DEV void load_x64(const void *x, int x_bf16, int64_t off, float *xr) {
    if (x_bf16) {
        const uint16_t *p = (const uint16_t *)x + off;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            u32x4 v = load_u32x4(p + 8 * i);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                xr[8 * i + 2 * j] = bf16_bits_to_float(v[j] & 0xFFFFu);
                xr[8 * i + 2 * j + 1] = bf16_bits_to_float(v[j] >> 16);
            }
        }
    } else {
        const float *p = (const float *)x + off;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            f32x4 v = *(const f32x4 *)(p + 4 * i);
            xr[4 * i] = v[0];
            xr[4 * i + 1] = v[1];
            xr[4 * i + 2] = v[2];
            xr[4 * i + 3] = v[3];
        }
    }
}

MOE_DEV float silu(float z) { return z / (1.0f + expf(-z)); }

MOE_DEV void load_codebook(const int8_t *cb, uint32_t *cb_lds) {
    if (cb)
        for (int i = threadIdx.x; i < 512; i += blockDim.x) cb_lds[i] = ((const uint32_t *)cb)[i];
    __syncthreads();
}

// Row chunk held as raw registers, and the lane's activations prepared for it
// (fp16 hi/lo pairs for the dot2 formats, plain fp32 for the codebook format).
template <int FMT>
struct RawChunk;
template <>
struct RawChunk<MOE_Q2K> {
    typedef XQ2K Prep;
    Q2KChunk c;
    MOE_DEV static void prep(const float *x, Prep &p) { prep_q2k(x, p); }
    MOE_DEV void load(const uint8_t *b, int64_t i0) { c = q2k_load(b, i0); }
    MOE_DEV float dot(const Prep &p, const uint32_t *) const { return q2k_dot2(c, p); }
};
template <>
struct RawChunk<MOE_Q8_0> {
    typedef XQ8 Prep;
    Q8Chunk c;
    MOE_DEV static void prep(const float *x, Prep &p) { prep_q8(x, p); }
    MOE_DEV void load(const uint8_t *b, int64_t i0) { c = q8_load(b, i0); }
    MOE_DEV float dot(const Prep &p, const uint32_t *) const { return q8_dot2(c, p); }
};
struct XF32 {
    float x[64];
};
template <>
struct RawChunk<MOE_CB2> {
    typedef XF32 Prep;
    CB2Chunk c;
    MOE_DEV static void prep(const float *x, Prep &p) {
#pragma unroll
        for (int i = 0; i < 64; ++i) p.x[i] = x[i];
    }
    MOE_DEV void load(const uint8_t *b, int64_t i0) { c = cb2_load(b, i0); }
    MOE_DEV float dot(const Prep &p, const uint32_t *cb) const { return cb2_dot(c, p.x, cb); }
};

// Lane layout over rows of n_in weights: cpr = n_in/64 lanes per row, rpi =
// 64/cpr rows per wave iteration; lane -> (row lane/cpr, chunk lane%cpr).
struct RowPlan {
    int cpr, rpi, lr, c;
};

MOE_DEV RowPlan row_plan(int n_in, int lane) {
    RowPlan p;
    p.cpr = n_in >> 6;
    p.rpi = 64 / p.cpr;
    p.lr = lane / p.cpr;
    p.c = lane % p.cpr;
    return p;
}

// One wave's rows [row0, row0+nrows) of matrix m0 (and m1 when TWO): the
// row chunks are loaded into registers first (load), the dots with the
// lane's prepared activations come after (compute).  All loads are
// unconditional: rows past the end are clamped to the last one.
template <int FMT, bool TWO, int NB>
struct WaveRows {
    RawChunk<FMT> g[NB], u[NB];
    int iters;
    RowPlan rp;

    MOE_DEV void load(const uint8_t *m0, const uint8_t *m1, int n_in, int row0, int nrows, int lane) {
        rp = row_plan(n_in, lane);
        iters = (nrows + rp.rpi - 1) / rp.rpi;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const int r = min(b * rp.rpi + rp.lr, nrows - 1);
            const int64_t i0 = (int64_t)(row0 + r) * n_in + 64 * rp.c;
            g[b].load(m0, i0);
            if constexpr (TWO) u[b].load(m1, i0);
        }
    }

    // emit(r, v0, v1) on the lane holding row r's full sums
    template <typename Emit>
    MOE_DEV void compute(const typename RawChunk<FMT>::Prep &xr, const uint32_t *cb, int nrows, Emit emit) const {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            if (b < iters) {  // uniform over the wave
                const float s0 = seg_sum(g[b].dot(xr, cb), rp.cpr);
                float s1 = 0.f;
                if constexpr (TWO) s1 = seg_sum(u[b].dot(xr, cb), rp.cpr);
                const int r = b * rp.rpi + rp.lr;
                if (rp.c == 0 && r < nrows) emit(r, s0, s1);
            }
        }
    }
};

// Rows of one wave iteration per format: enough to cover the wave's rows in
// one load batch (4 rows of 4096 weights, or 2 rows of 2048 for the down).
template <int FMT>
constexpr int wave_batch() { return FMT == MOE_Q8_0 ? 1 : 4; }

// One wave: dots of rows [row0, row0+nrows) with the lane's activations,
// in batches of wave_batch() row iterations.
template <int FMT, bool TWO, typename Emit>
MOE_DEV void wave_rows(const uint8_t *m0, const uint8_t *m1, int n_in, int row0, int nrows,
                       const typename RawChunk<FMT>::Prep &xr, const uint32_t *cb, int lane, Emit emit) {
    constexpr int NB = wave_batch<FMT>();
    const int rpi = 64 / (n_in >> 6);
    for (int r0 = 0; r0 < nrows; r0 += NB * rpi) {
        WaveRows<FMT, TWO, NB> w;
        const int n = min(nrows - r0, NB * rpi);
        w.load(m0, m1, n_in, row0 + r0, n, lane);
        w.compute(xr, cb, n, [&](int r, float v0, float v1) { emit(r0 + r, v0, v1); });
    }
}

MOE_DEV float swiglu_h(float g, float u, int round_bf16) {
    float hv = silu(g) * u;
    return round_bf16 ? bf16_bits_to_float(float_to_bf16_bits(hv)) : hv;
}

// h rows for one routed expert e (rows [row0, row0+nrows) of its gate/up),
// every token of its bucket.  The weight loads are issued before the
// activations are read.  With prepared x (Q2K) the activations come from the
// workspace records; otherwise each wave prepares its own.
// tile (LDS, 16 floats, or NULL): when set, the block's 4 waves cover the 16
// rows [tile_row0, tile_row0+16) and after each token wave 0 writes the
// prepared h record of those 16 rows (for a Q2K down projection).
template <int FMT, bool PREPPED = false>
MOE_DEV void routed_gateup(const FfnArgs &a, int e, int row0, int nrows, const uint32_t *cb, int lane,
                           float *tile = nullptr, int tile_row0 = 0) {
    const uint8_t *g = a.gate + (int64_t)e * a.gu_expert_bytes, *u = a.up + (int64_t)e * a.gu_expert_bytes;
    const int j0 = a.offset[e], n = a.count[e];
    const RowPlan rp = row_plan(a.D, lane);
    constexpr int NB = wave_batch<FMT>();
    // nrows <= 4: for the formats with NB >= 4 one load batch covers the rows
    // (the weight loads sit inside the token loop so that the compiler does not
    // hoist every decoded code out of it; later tokens hit the cache)
    constexpr bool ONE = NB >= 4;
    for (int j = 0; j < n; ++j) {
        WaveRows<FMT, true, NB> w;
        if constexpr (ONE) w.load(g, u, a.D, row0, nrows, lane);
        const int t = a.perm[j0 + j] / a.k;
        typename RawChunk<FMT>::Prep xr;
        if constexpr (FMT == MOE_Q2K && PREPPED) {
            load_q2k_prep(a.xp16 + ((int64_t)t * (a.D / 16) + 4 * rp.c) * kP16Dwords, xr);
        } else {
            float xf[64];
            load_x64(a.x, a.x_bf16, (int64_t)t * a.D + 64 * rp.c, xf);
            RawChunk<FMT>::prep(xf, xr);
        }
        float *dst = a.h + (int64_t)(j0 + j) * a.F + row0;
        auto emit = [&](int r, float gs, float us) {
            const float hv = swiglu_h(gs, us, a.x_bf16);
            dst[r] = hv;
            if (tile) tile[row0 + r - tile_row0] = hv;
        };
        if constexpr (ONE) w.compute(xr, cb, nrows, emit);
        else wave_rows<FMT, true>(g, u, a.D, row0, nrows, xr, cb, lane, emit);
        if (tile) {  // uniform over the block
            __syncthreads();
            if ((threadIdx.x >> 6) == 0)
                prep16_wave(lane < 16 ? tile[lane] : 0.f,
                            a.hp16 + ((int64_t)(j0 + j) * (a.F / 16) + tile_row0 / 16) * kP16Dwords, 1);
            __syncthreads();
        }
    }
}

// hs rows [row0, row0+nrows) of the shared expert for every token.
template <int FMT>
MOE_DEV void shared_gateup(const FfnArgs &a, int row0, int nrows, const uint32_t *cb, int lane) {
    const RowPlan rp = row_plan(a.D, lane);
    for (int t = 0; t < a.T; ++t) {
        float xf[64];
        load_x64(a.x, a.x_bf16, (int64_t)t * a.D + 64 * rp.c, xf);
        typename RawChunk<FMT>::Prep xr;
        RawChunk<FMT>::prep(xf, xr);
        float *dst = a.hs + (int64_t)t * a.Fs + row0;
        wave_rows<FMT, true>(a.sh_gate, a.sh_up, a.D, row0, nrows, xr, cb, lane,
                             [&](int r, float gs, float us) { dst[r] = swiglu_h(gs, us, a.x_bf16); });
    }
}

// ys rows [row0, row0+nrows) of the shared expert's down projection.
template <int FMT>
MOE_DEV void shared_down(const FfnArgs &a, int row0, int nrows, const uint32_t *cb, int lane) {
    const RowPlan rp = row_plan(a.Fs, lane);
    for (int t = 0; t < a.T; ++t) {
        float xf[64];
        load_x64(a.hs + (int64_t)t * a.Fs, 0, 64 * rp.c, xf);
        typename RawChunk<FMT>::Prep xr;
        RawChunk<FMT>::prep(xf, xr);
        float *dst = a.ys + (int64_t)t * a.D + row0;
        wave_rows<FMT, false>(a.sh_down, nullptr, a.Fs, row0, nrows, xr, cb, lane,
                              [&](int r, float s, float) { dst[r] = s; });
    }
}

// Down rows [row0, row0+nrows) of routed expert e for its bucket, into
// out[q * stride + (row - row0)] for bucket positions q.
template <int FMT, bool PREPPED = false>
MOE_DEV void routed_down(const FfnArgs &a, int e, int row0, int nrows, const uint32_t *cb, int lane, float *out,
                         int stride) {
    const uint8_t *m = a.down + (int64_t)e * a.down_expert_bytes;
    const int j0 = a.offset[e], n = a.count[e];
    const RowPlan rp = row_plan(a.F, lane);
    for (int j = 0; j < n; ++j) {
        typename RawChunk<FMT>::Prep xr;
        if constexpr (FMT == MOE_Q2K && PREPPED) {
            load_q2k_prep(a.hp16 + ((int64_t)(j0 + j) * (a.F / 16) + 4 * rp.c) * kP16Dwords, xr);
        } else {
            float xf[64];
            load_x64(a.h + (int64_t)(j0 + j) * a.F, 0, 64 * rp.c, xf);
            RawChunk<FMT>::prep(xf, xr);
        }
        float *dst = out + (int64_t)(j0 + j) * stride;
        wave_rows<FMT, false>(m, nullptr, a.F, row0, nrows, xr, cb, lane, [&](int r, float s, float) { dst[r] = s; });
    }
}

// Calls fn with std::integral_constant<int, format> for a runtime format.
template <typename Fn>
inline void with_fmt(int f, Fn &&fn) {
    if (f == MOE_Q2K) fn(std::integral_constant<int, MOE_Q2K>{});
    else if (f == MOE_Q8_0) fn(std::integral_constant<int, MOE_Q8_0>{});
    else fn(std::integral_constant<int, MOE_CB2>{});
}

FfnArgs make_ffn_args(const moe_layer_desc *d, const void *x, int32_t T, int32_t x_type, const RoutingPtrs &r,
                      float *y, uint32_t flags, const Workspace &ws);

}  // namespace moe
