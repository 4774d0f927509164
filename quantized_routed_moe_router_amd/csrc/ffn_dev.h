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
    // prepared activations (NULL when the path does not use them): x for Q2K
    // rows ([T][D/16] records), x for Q8_0 rows ([T][D/64] records), h for the
    // routed Q2K down ([T*k][F/16] records)
    uint32_t *xp16, *xq8, *hp16;
    int xp16_nat;       // x records in natural byte order (codebook gate/up)
    int n_prep_blocks;  // K1: x-preparing blocks
    int n_shgu_blocks;  // K2: shared gate/up blocks
    int shared_fmt;
    // per-slot records (few-token schedule) and their number, min(T*k, E)
    SlotRec *slots;
    int nslots;
    int build_slots;  // K1 writes the records from a given routing
    int k3_topk;      // one token: each routed gate/up block selects the top-k itself (no K2)
    // one token: K1 normalises x first (x <- gamma * x / rms(x)) when set
    const float *norm_gamma;
    float norm_eps;
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

template <>
struct RawChunk<MOE_Q4K> {
    typedef XF32 Prep;
    Q4KChunk c;
    MOE_DEV static void prep(const float *x, Prep &p) {
#pragma unroll
        for (int i = 0; i < 64; ++i) p.x[i] = x[i];
    }
    MOE_DEV void load(const uint8_t *b, int64_t i0) { c = q4k_load(b, i0); }
    MOE_DEV float dot(const Prep &p, const uint32_t *) const { return q4k_dot(c, p.x); }
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

// LDS ordering between the lanes of one wave: LDS operations of a wave
// execute in issue order, so only the compiler has to be kept from moving
// them across this point.
// 16 bytes from global memory straight into LDS (no registers held): lane l
// of the wave writes lds_wave + 16 * l.  lds_wave must be the same for every
// lane of the wave; lanes switched off by a branch write nothing.
MOE_DEV void lds_dma16(const void *g, void *lds_wave) {
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)g,
                                     (__attribute__((address_space(3))) void *)lds_wave, 16, 0, 0);
}

// Wait until every vector memory load of the wave, LDS-bound ones included,
// has landed (vmcnt 0; the export and LDS counters left alone).
MOE_DEV void vmem_wait_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// LDS address of a pointer into a __shared__ array.
MOE_DEV uint32_t lds_addr(const void *p) { return (uint32_t)(size_t)(const __attribute__((address_space(3))) void *)p; }

// 16 bytes per lane from global address g into LDS at m0 + 16 * lane (m0
// wave-uniform).  Issued as assembly so that the compiler's wait counting
// does not see it: the caller waits with s_waitcnt on vmcnt itself, counting
// these copies with every vector load issued after them.  The s_nop covers
// the wait state between the write of m0 and the copy that reads it.
MOE_DEV void dma16_m0(const void *g, uint32_t m0) {
    __asm__ volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %1, off" : : "{m0}"(m0), "v"(g) : "memory");
}

// Wait until at most N vector memory loads of the wave are outstanding.
template <int N>
MOE_DEV void vmem_wait_le() {
    static_assert(N >= 0 && N < 64, "vmcnt immediate");
    __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// Block barrier that orders the compiler's memory accesses around it but
// waits for no counter (the copies above are waited for by vmem_wait_le).
MOE_DEV void barrier_only() {
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
}

// Make v appear used and changed here: the compiler then computes it before
// this point and cannot sink the computation below a later wait.
MOE_DEV void pin_value(float &v) { __asm__ volatile("" : "+v"(v)); }

// Sum over the 16 lanes of each row of the wave, returned to all of them
// (DPP row rotations by 8, 4, 2 and 1).
template <int CTRL>
MOE_DEV float dpp_row_f32(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
MOE_DEV float row16_sum(float v) {
    v += dpp_row_f32<0x128>(v);
    v += dpp_row_f32<0x124>(v);
    v += dpp_row_f32<0x122>(v);
    v += dpp_row_f32<0x121>(v);
    return v;
}

MOE_DEV void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Sum of lanes xor 1 and xor 2 (quad permutations) and xor 4.. via shuffles.
MOE_DEV float xor_sum(float s, int L) {
    if (L > 1) s += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, s), 0xB1, 0xF, 0xF, false));
    if (L > 2) s += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, s), 0x4E, 0xF, 0xF, false));
    for (int m = 4; m < L; m <<= 1) s += __shfl_xor(s, m, kWave);
    return s;
}

// Segment sums of NV per-lane partials through a wave-private LDS area red
// (NV * 64 floats, 16-byte aligned).  Lanes form segments of cpr consecutive
// lanes (cpr a power of two <= 64).  Afterwards red[i * 64 + r] holds the sum
// of partial i over segment r (r < 64 / cpr).  The partials of one output are
// added in a fixed order (runs of consecutive lanes, then a fixed butterfly),
// the same for every output.  All lanes of the wave must call it.
template <int NV>
MOE_DEV void seg_reduce_lds(const float (&v)[NV], int cpr, float *red) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < NV; ++i) red[i * 64 + lane] = v[i];
    wave_lds_sync();
    const int rpi = 64 / cpr;
    float res[NV];
    int dst[NV];
#pragma unroll
    for (int j = 0; j < NV; ++j) dst[j] = -1;
    if (cpr >= NV) {  // L lanes per output, each adds a run of NV partials
        const int L = cpr / NV, o = lane / L, sub = lane % L;
        const int i = o / rpi, r = o % rpi;
        const float *p = red + i * 64 + r * cpr + sub * NV;
        float s = 0.f;
        if constexpr (NV % 4 == 0) {
#pragma unroll
            for (int j = 0; j < NV; j += 4) {
                const f32x4 q = *(const f32x4 *)(p + j);
                s += q[0];
                s += q[1];
                s += q[2];
                s += q[3];
            }
        } else {
#pragma unroll
            for (int j = 0; j < NV; ++j) s += p[j];
        }
        res[0] = xor_sum(s, L);
        if (sub == 0) dst[0] = i * 64 + r;
    } else {  // each lane owns NV / cpr outputs and adds all cpr partials of each
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const int o = lane + 64 * j;
            if (o < NV * rpi) {
                const int i = o / rpi, r = o % rpi;
                const float *p = red + i * 64 + r * cpr;
                float s = 0.f;
                for (int q = 0; q < cpr; ++q) s += p[q];
                res[j] = s;
                dst[j] = i * 64 + r;
            }
        }
    }
    wave_lds_sync();
#pragma unroll
    for (int j = 0; j < NV; ++j)
        if (dst[j] >= 0) red[dst[j]] = res[j];
    wave_lds_sync();
}

// One wave: dots of rows rowof(l), l < nrows, of m0 (and m1 when TWO) over
// the columns [col0, col0 + ncols) (rows ld weights apart) with the lane's
// prepared activations.  A lane takes 64 consecutive columns of a row, cpr =
// ncols/64 lanes a row, 64/cpr rows per iteration; NB iterations per load
// batch.  Every weight load of a batch is issued first (unconditionally, rows
// past the end clamped to the last one), then loadprep(xr) issues the loads
// of the activations (first batch only), so that a wave waits for one memory
// round trip, not two.  The partial sums go through red (LDS, 2*NB*64 floats
// per wave, 16-byte aligned); then emit(l, s0, s1) runs once per row, on
// some lane.
template <class CH, bool TWO, int NB, typename RowOf, typename LoadPrep, typename Emit>
MOE_DEV void rows_dot_ch(const uint8_t *m0, const uint8_t *m1, int64_t ld, int col0, int ncols, int nrows, RowOf rowof,
                         LoadPrep loadprep, const uint32_t *cb, int lane, float *red, Emit emit) {
    constexpr int NV = (TWO ? 2 : 1) * NB;
    const int cpr = ncols >> 6, rpi = 64 / cpr, lr = lane / cpr, c = lane % cpr;
    typename CH::Prep xr;
    for (int b0 = 0; b0 < nrows; b0 += NB * rpi) {
        CH g[NB], u[NB];
#pragma unroll
        for (int it = 0; it < NB; ++it) {
            const int l = min(b0 + it * rpi + lr, nrows - 1);
            const int64_t i0 = (int64_t)rowof(l) * ld + col0 + 64 * c;
            g[it].load(m0, i0);
            if constexpr (TWO) u[it].load(m1, i0);
        }
        if (b0 == 0) loadprep(xr);
        float v[NV];
#pragma unroll
        for (int it = 0; it < NB; ++it) {
            const bool ok = b0 + it * rpi < nrows;  // uniform over the wave
            v[(TWO ? 2 : 1) * it] = ok ? g[it].dot(xr, cb) : 0.f;
            if constexpr (TWO) v[2 * it + 1] = ok ? u[it].dot(xr, cb) : 0.f;
        }
        seg_reduce_lds<NV>(v, cpr, red);
        for (int o = lane; o < NB * rpi; o += 64) {
            const int it = o / rpi, r = o % rpi, l = b0 + o;
            if (l < nrows) {
                const float s0 = red[(TWO ? 2 : 1) * it * 64 + r];
                const float s1 = TWO ? red[(2 * it + 1) * 64 + r] : 0.f;
                emit(l, s0, s1);
            }
        }
        wave_lds_sync();
    }
}

template <int FMT, bool TWO, int NB, typename RowOf, typename LoadPrep, typename Emit>
MOE_DEV void rows_dot(const uint8_t *m0, const uint8_t *m1, int64_t ld, int col0, int ncols, int nrows, RowOf rowof,
                      LoadPrep loadprep, const uint32_t *cb, int lane, float *red, Emit emit) {
    rows_dot_ch<RawChunk<FMT>, TWO, NB>(m0, m1, ld, col0, ncols, nrows, rowof, loadprep, cb, lane, red, emit);
}

// A 64-weight chunk of any format dotted with plain fp32 activations (each
// product rounded once in fp32): for the shared expert, whose activations
// are not prepared.
template <int FMT>
struct F32Chunk {
    typedef XF32 Prep;
    typename std::conditional<FMT == MOE_Q2K, Q2KChunk, typename std::conditional<FMT == MOE_Q8_0, Q8Chunk, CB2Chunk>::type>::type c;
    MOE_DEV void load(const uint8_t *b, int64_t i0) {
        if constexpr (FMT == MOE_Q2K) c = q2k_load(b, i0);
        else if constexpr (FMT == MOE_Q8_0) c = q8_load(b, i0);
        else c = cb2_load(b, i0);
    }
    MOE_DEV float dot(const Prep &p, const uint32_t *cb) const {
        if constexpr (FMT == MOE_Q2K) return q2k_dot(c, p.x);
        else if constexpr (FMT == MOE_Q8_0) return q8_dot(c, p.x);
        else return cb2_dot(c, p.x, cb);
    }
};

// Barrier that orders LDS only: global loads still in flight are not waited
// for (a plain __syncthreads also waits for every outstanding global access).
MOE_DEV void block_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// One wave: dots of the rows row0 + l (l < nrows) of matrices staged in LDS
// (m0, and m1 when TWO; rows of n_in weights blocked over the flat index from
// the staged start, as in memory) over the columns [col0, col0 + ncols) with
// the lane's prepared activations.  A lane takes 64 consecutive columns of a
// row, cpr = ncols/64 lanes a row, 64/cpr rows per iteration, NB iterations
// per reduction.  emit(l, s0, s1) runs once per row, on some lane.
template <int FMT, bool TWO, int NB, typename Emit>
MOE_DEV void lds_rows_dot(const uint8_t *m0, const uint8_t *m1, int n_in, int row0, int col0, int ncols, int nrows,
                          const typename RawChunk<FMT>::Prep &xr, const uint32_t *cb, int lane, float *red,
                          Emit emit) {
    constexpr int NV = (TWO ? 2 : 1) * NB;
    const int cpr = ncols >> 6, rpi = 64 / cpr, lr = lane / cpr, col = col0 + 64 * (lane % cpr);
    for (int b0 = 0; b0 < nrows; b0 += NB * rpi) {
        float v[NV];
#pragma unroll
        for (int it = 0; it < NB; ++it) {
            const bool ok = b0 + it * rpi < nrows;  // uniform over the wave
            const int i0 = (row0 + min(b0 + it * rpi + lr, nrows - 1)) * n_in + col;
            RawChunk<FMT> g;
            g.load(m0, i0);
            v[(TWO ? 2 : 1) * it] = ok ? g.dot(xr, cb) : 0.f;
            if constexpr (TWO) {
                RawChunk<FMT> u;
                u.load(m1, i0);
                v[2 * it + 1] = ok ? u.dot(xr, cb) : 0.f;
            }
        }
        seg_reduce_lds<NV>(v, cpr, red);
        for (int o = lane; o < NB * rpi; o += 64) {
            const int it = o / rpi, r = o % rpi, l = b0 + o;
            if (l < nrows) {
                const float s0 = red[(TWO ? 2 : 1) * it * 64 + r];
                const float s1 = TWO ? red[(2 * it + 1) * 64 + r] : 0.f;
                emit(l, s0, s1);
            }
        }
        wave_lds_sync();
    }
}

// Rows of one load batch for the batched (many-token) path.
template <int FMT>
constexpr int wave_batch() { return FMT == MOE_Q8_0 ? 1 : 4; }

// One wave: dots of rows [row0, row0+nrows) with the lane's activations
// (batched path): wave_batch() row iterations per load batch, the lanes of a
// row combined by a butterfly.
template <int FMT, bool TWO, typename Emit>
MOE_DEV void wave_rows(const uint8_t *m0, const uint8_t *m1, int n_in, int row0, int nrows,
                       const typename RawChunk<FMT>::Prep &xr, const uint32_t *cb, int lane, Emit emit) {
    constexpr int NB = wave_batch<FMT>();
    const RowPlan rp = row_plan(n_in, lane);
    for (int b0 = 0; b0 < nrows; b0 += NB * rp.rpi) {
        RawChunk<FMT> g[NB], u[NB];
#pragma unroll
        for (int it = 0; it < NB; ++it)
            if (b0 + it * rp.rpi < nrows) {
                const int64_t i0 = (int64_t)(row0 + min(b0 + it * rp.rpi + rp.lr, nrows - 1)) * n_in + 64 * rp.c;
                g[it].load(m0, i0);
                if constexpr (TWO) u[it].load(m1, i0);
            }
#pragma unroll
        for (int it = 0; it < NB; ++it)
            if (b0 + it * rp.rpi < nrows) {
                const float s0 = seg_sum(g[it].dot(xr, cb), rp.cpr);
                float s1 = 0.f;
                if constexpr (TWO) s1 = seg_sum(u[it].dot(xr, cb), rp.cpr);
                const int l = b0 + it * rp.rpi + rp.lr;
                if (rp.c == 0 && l < nrows) emit(l, s0, s1);
            }
    }
}

// h = silu(g) * u in fp32, never rounded further (in bf16 mode only the
// activations x were cast)
MOE_DEV float swiglu_h(float g, float u) { return silu(g) * u; }

// h rows for one routed expert e (rows [row0, row0+nrows) of its gate/up),
// every token of its bucket, activations prepared in the lane.  The weight
// loads sit inside the token loop so that the compiler does not hoist every
// decoded code out of it; later tokens hit the cache.
template <int FMT>
MOE_DEV void routed_gateup(const FfnArgs &a, int e, int row0, int nrows, const uint32_t *cb, int lane) {
    const uint8_t *g = a.gate + (int64_t)e * a.gu_expert_bytes, *u = a.up + (int64_t)e * a.gu_expert_bytes;
    const int j0 = a.offset[e], n = a.count[e];
    const RowPlan rp = row_plan(a.D, lane);
    for (int j = 0; j < n; ++j) {
        const int t = a.perm[j0 + j] / a.k;
        typename RawChunk<FMT>::Prep xr;
        float xf[64];
        load_x64(a.x, a.x_bf16, (int64_t)t * a.D + 64 * rp.c, xf);
        RawChunk<FMT>::prep(xf, xr);
        float *dst = a.h + (int64_t)(j0 + j) * a.F + row0;
        wave_rows<FMT, true>(g, u, a.D, row0, nrows, xr, cb, lane,
                             [&](int r, float gs, float us) { dst[r] = swiglu_h(gs, us); });
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
                             [&](int r, float gs, float us) { dst[r] = swiglu_h(gs, us); });
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
template <int FMT>
MOE_DEV void routed_down(const FfnArgs &a, int e, int row0, int nrows, const uint32_t *cb, int lane, float *out,
                         int stride) {
    const uint8_t *m = a.down + (int64_t)e * a.down_expert_bytes;
    const int j0 = a.offset[e], n = a.count[e];
    const RowPlan rp = row_plan(a.F, lane);
    for (int j = 0; j < n; ++j) {
        typename RawChunk<FMT>::Prep xr;
        float xf[64];
        load_x64(a.h + (int64_t)(j0 + j) * a.F, 0, 64 * rp.c, xf);
        RawChunk<FMT>::prep(xf, xr);
        float *dst = out + (int64_t)(j0 + j) * stride;
        wave_rows<FMT, false>(m, nullptr, a.F, row0, nrows, xr, cb, lane, [&](int r, float s, float) { dst[r] = s; });
    }
}

// Calls fn with std::integral_constant<int, format> for a runtime format.
template <typename Fn>
inline void with_fmt(int f, Fn &&fn) {
    if (f == MOE_Q2K) fn(std::integral_constant<int, MOE_Q2K>{});
    else if (f == MOE_Q8_0) fn(std::integral_constant<int, MOE_Q8_0>{});
    else if (f == MOE_Q4K) fn(std::integral_constant<int, MOE_Q4K>{});
    else fn(std::integral_constant<int, MOE_CB2>{});
}

// ---- int16 row codes for the shared expert's int8 matrix-core GEMMs ---------
// A token row is coded as c = rint(v*S), S = 32512 / max|row|, c = 256*hi + lo,
// per 64 values (a pair of Q8_0 blocks) as 32 dwords: for each lane group g
// (0..3) four dwords {even 2g, even 2g+1, odd 2g, odd 2g+1} of the hi plane,
// then the same for the lo plane.  Code dword m (0-7 the even block, 8-15 the
// odd block) follows the byte order of the Q8_0 codes in the 68-byte pair:
// the odd block's 8 aligned dwords, the even block's dwords 1..7 and one
// dword of bytes 2, 3, 32, 33 (codes 0, 1, 30, 31).
constexpr int kSgqPairDw = 32;
constexpr float kSgqCodeMax = 32512.f;

// value index (0..63 within the pair) of byte n of code dword m
__host__ __device__ inline int sgq_value_index(int m, int n) {
    if (m < 7) return 4 * m + 2 + n;
    if (m == 7) return n < 2 ? n : 28 + n;
    return 32 + 4 * (m - 8) + n;
}

// position of code dword m within a plane of the pair's record
__host__ __device__ inline int sgq_plane_dword(int m) {
    const int odd = m >= 8, mm = m & 7;
    return 4 * (mm >> 1) + 2 * odd + (mm & 1);
}

// the records of one row of n fp32 values at scale S, a thread per code
// dword of every pair (the whole block takes part)
MOE_DEV void sgq_code_row(const float *row, int n, float S, uint32_t *out) {
    const int np = n / 64;
    for (int i = threadIdx.x; i < np * 16; i += blockDim.x) {
        const int p = i >> 4, md = i & 15;
        uint32_t H = 0, L = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int c = (int)__builtin_rintf(row[64 * p + sgq_value_index(md, b)] * S);
            const int hv = (c + 128) >> 8;
            H |= (uint32_t)(hv & 0xFF) << (8 * b);
            L |= (uint32_t)((c - 256 * hv) & 0xFF) << (8 * b);
        }
        out[p * kSgqPairDw + sgq_plane_dword(md)] = H;
        out[p * kSgqPairDw + 16 + sgq_plane_dword(md)] = L;
    }
}

// S from the row's largest magnitude (a block of 256 threads), then its
// records; inv = 1/S
MOE_DEV void sgq_prep_row(const float *row, int n, uint32_t *rec, float *inv, float *wmax) {
    float mt = 0.f;
    for (int i = threadIdx.x; i < n; i += 256) mt = fmaxf(mt, fabsf(row[i]));
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) mt = fmaxf(mt, __shfl_xor(mt, o, kWave));
    if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = mt;
    __syncthreads();
    const float m = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
    const float S = m > 0.f ? kSgqCodeMax / m : 0.f;
    if (threadIdx.x == 0) *inv = m / kSgqCodeMax;
    sgq_code_row(row, n, S, rec);
}

FfnArgs make_ffn_args(const moe_layer_desc *d, const void *x, int32_t T, int32_t x_type, const RoutingPtrs &r,
                      float *y, uint32_t flags, const Workspace &ws);

}  // namespace moe
