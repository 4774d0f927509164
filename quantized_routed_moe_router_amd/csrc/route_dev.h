// route_dev.h - device pieces of the routing ("Understanding Dwarf Star",
// 5.3.2 router(x) = softmax(x W_router) and the top-k sum; 5.3.7 step 1 and
// the sparse indexing of step 2): fp64 router logits, the wave64 top-k with
// renormalized softmax, and small-batch bucketing.
#pragma once
#include "common.h"

namespace moe {

// Router logits in fp64 from W_r stored expert-major [E][D].  Few tokens:
// one wave per expert row (lane c holds the row's weights [64c, 64c+64) when
// D = 4096; shorter rows put 4096/D experts in one wave), each token's 64
// products per lane summed in fp64 in ascending k, then a fixed butterfly
// over the lanes of the row.  Every expert uses the same reduction tree, so
// equal rows give equal logits.  Products of two fp32 (or bf16 and fp32)
// values are exact in fp64; only the additions round, at 2^-53 relative.
MOE_DEV double seg_sum_f64(double v, int seg) {
    for (int o = seg >> 1; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

template <int XT>
MOE_DEV void router_rows_wave(const float *__restrict__ W, const float *__restrict__ bias, const void *__restrict__ xin,
                              int T, int D, int E, double *__restrict__ logits, int wave_id) {
    const int lane = threadIdx.x & 63;
    const int cpr = D >> 6, rpi = 64 / cpr;
    const int e = wave_id * rpi + lane / cpr, c = lane % cpr;
    const bool ok = e < E;
    const float *wr = W + (int64_t)min(e, E - 1) * D + 64 * c;
    float w[64];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        f32x4 v = *(const f32x4 *)(wr + 4 * i);
        w[4 * i] = v[0];
        w[4 * i + 1] = v[1];
        w[4 * i + 2] = v[2];
        w[4 * i + 3] = v[3];
    }
    const double b = (ok && bias) ? (double)bias[e] : 0.0;
    for (int t = 0; t < T; ++t) {
        double acc = 0.0;
        if constexpr (XT == MOE_BF16) {
            const uint16_t *xp = (const uint16_t *)xin + (int64_t)t * D + 64 * c;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                u32x4 v = load_u32x4(xp + 8 * i);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    acc = __builtin_fma((double)bf16_bits_to_float(v[j] & 0xFFFFu), (double)w[8 * i + 2 * j], acc);
                    acc = __builtin_fma((double)bf16_bits_to_float(v[j] >> 16), (double)w[8 * i + 2 * j + 1], acc);
                }
            }
        } else {
            const float *xp = (const float *)xin + (int64_t)t * D + 64 * c;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                f32x4 v = *(const f32x4 *)(xp + 4 * i);
#pragma unroll
                for (int j = 0; j < 4; ++j) acc = __builtin_fma((double)v[j], (double)w[4 * i + j], acc);
            }
        }
        acc = seg_sum_f64(acc, cpr);
        if (ok && c == 0) logits[(int64_t)t * E + e] = acc + b;
    }
}

// Many tokens: a 16 x 16 tile of (token, expert) logits per 256-thread block,
// 64-wide k slices staged in LDS, each output summed in ascending k in fp64.
template <int XT>
MOE_DEV void router_tile_block(const float *__restrict__ W, const float *__restrict__ bias,
                               const void *__restrict__ xin, int T, int D, int E, double *__restrict__ logits, int tile_t,
                               int tile_e) {
    __shared__ float xs[16][65], wsl[16][65];
    const int r = threadIdx.x / 16, cidx = threadIdx.x % 16;
    const int t = tile_t * 16 + r, e = tile_e * 16 + cidx;
    double acc = 0.0;
    for (int kb = 0; kb < D; kb += 64) {
        __syncthreads();
        for (int i = threadIdx.x; i < 16 * 64; i += 256) {
            const int rr = i / 64, kk = i % 64;
            const int tt = min(tile_t * 16 + rr, T - 1), ee = min(tile_e * 16 + rr, E - 1);
            if constexpr (XT == MOE_BF16) xs[rr][kk] = bf16_bits_to_float(((const uint16_t *)xin)[(int64_t)tt * D + kb + kk]);
            else xs[rr][kk] = ((const float *)xin)[(int64_t)tt * D + kb + kk];
            wsl[rr][kk] = W[(int64_t)ee * D + kb + kk];
        }
        __syncthreads();
#pragma unroll 16
        for (int kk = 0; kk < 64; ++kk) acc = __builtin_fma((double)xs[r][kk], (double)wsl[cidx][kk], acc);
    }
    if (t < T && e < E) logits[(int64_t)t * E + e] = acc + (bias ? (double)bias[e] : 0.0);
}

// a ranks before b: larger logit, then lower expert index
MOE_DEV bool before(double va, int ea, double vb, int eb) { return va > vb || (va == vb && ea < eb); }

// One wave selects the top k of lg[0..E) by (logit desc, index asc): the
// lane's candidates (experts lane, lane+64, ...) sit in registers; each of k
// rounds takes the lane's best untaken candidate and a wave-wide arg-max
// (an empty lane carries index INT_MAX and never wins).  Lane s keeps slot s;
// then w_s = route_scale * exp(l_s - l_0) / sum_j exp(l_j - l_0) in fp64,
// the exponentials computed by lanes 0..k-1 at once.
MOE_DEV void select_topk(const double *lg, int E, int k, float route_scale, int32_t *idx_out, float *w_out,
                         int32_t *sidx, float *sw) {
    const int lane = threadIdx.x & 63;
    constexpr int PER = kMaxExperts / kWave;  // 16 experts per lane at most
    constexpr int NONE = 0x7FFFFFFF;
    double v[PER];
    uint32_t taken = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int e = lane + 64 * i;
        v[i] = lg[min(e, E - 1)];
        if (e >= E) taken |= 1u << i;
    }
    double my_v = 0.0;
    int my_e = 0;
    for (int s = 0; s < k; ++s) {
        double bv = 0.0;
        int be = NONE, bi = -1;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int e = lane + 64 * i;
            if (!((taken >> i) & 1u) && (be == NONE || before(v[i], e, bv, be))) {
                bv = v[i];
                be = e;
                bi = i;
            }
        }
        double wv = bv;
        int we = be;
        for (int o = 32; o > 0; o >>= 1) {
            const double ov = __shfl_xor(wv, o, kWave);
            const int oe = __shfl_xor(we, o, kWave);
            if (oe != NONE && (we == NONE || before(ov, oe, wv, we))) {
                wv = ov;
                we = oe;
            }
        }
        if (bi >= 0 && we == be) taken |= 1u << bi;
        if (lane == s) {
            my_v = wv;
            my_e = we;
        }
    }
    const double mx = __shfl(my_v, 0, kWave);  // slot 0 holds the largest logit
    double ex = lane < k ? exp(my_v - mx) : 0.0;
    double den = ex;
    for (int o = 1; o < 64; o <<= 1) den += __shfl_xor(den, o, kWave);
    if (lane < k) {
        const float w = (float)((double)route_scale * ex / den);
        idx_out[lane] = my_e;
        w_out[lane] = w;
        if (sidx) {
            sidx[lane] = my_e;
            sw[lane] = w;
        }
    }
}

// Bucketing of few pairs (P <= 1024) by one block with the pairs' experts in
// LDS: every count, offset and slot is a plain count over the P pairs, which
// is the stable counting sort without atomics or scans.
MOE_DEV void bucket_small(const int32_t *sidx, int P, int E, int32_t *__restrict__ count,
                          int32_t *__restrict__ offset, int32_t *__restrict__ perm, int32_t *__restrict__ pos,
                          int32_t *__restrict__ active, int32_t *__restrict__ n_active) {
    __shared__ uint8_t isfirst[1024];
    __shared__ int32_t nfirst;
    for (int p = threadIdx.x; p < P; p += blockDim.x) {
        int e = sidx[p];
        bool f = true;
        for (int q = 0; q < p; ++q) f &= sidx[q] != e;
        isfirst[p] = f;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        int n = 0;
        for (int p = 0; p < P; ++p) n += isfirst[p];
        nfirst = n;
        n_active[0] = n;
        offset[E] = P;
    }
    __syncthreads();
    const int na = nfirst;
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        int cnt = 0, below = 0, fb = 0;
        for (int p = 0; p < P; ++p) {
            int ep = sidx[p];
            cnt += ep == e;
            below += ep < e;
            fb += (ep < e) & isfirst[p];
        }
        count[e] = cnt;
        offset[e] = below;
        if (cnt > 0) active[fb] = e;
        if (e >= na) active[e] = -1;
    }
    for (int p = threadIdx.x; p < P; p += blockDim.x) {
        int e = sidx[p], below = 0, rank = 0;
        for (int q = 0; q < P; ++q) {
            below += sidx[q] < e;
            rank += (q < p) & (sidx[q] == e);
        }
        perm[below + rank] = p;
        pos[p] = below + rank;
    }
}

// Routing of a handful of rows (T*E <= 4096, T*k <= 256) by one block:
// top-k (a wave per row) and bucketing.
MOE_DEV void route_finish_small(const double *__restrict__ logits, int T, int E, int k, float route_scale,
                                int32_t *__restrict__ topk_idx,
                                float *__restrict__ topk_w, int32_t *__restrict__ count,
                                int32_t *__restrict__ offset, int32_t *__restrict__ perm, int32_t *__restrict__ pos,
                                int32_t *__restrict__ active, int32_t *__restrict__ n_active) {
    __shared__ double lg[4096];
    __shared__ int32_t sidx[256];
    __shared__ float sw[256];
    for (int i = threadIdx.x; i < T * E; i += blockDim.x) lg[i] = logits[i];
    __syncthreads();
    const int wave = threadIdx.x >> 6;
    for (int t = wave; t < T; t += blockDim.x >> 6)  // a wave per row
        select_topk(lg + t * E, E, k, route_scale, topk_idx + (int64_t)t * k, topk_w + (int64_t)t * k, sidx + t * k,
                    sw + t * k);
    __syncthreads();
    bucket_small(sidx, T * k, E, count, offset, perm, pos, active, n_active);
}

__host__ __device__ inline bool route_small_ok(int T, int E, int k) { return T <= 16 && T * E <= 4096 && T * k <= 256; }

}  // namespace moe
