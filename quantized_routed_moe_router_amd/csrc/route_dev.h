// route_dev.h - device pieces of the routing ("Understanding Dwarf Star",
// 5.3.2 router(x) = softmax(x W_router) and the top-k sum; 5.3.7 step 1 and
// the sparse indexing of step 2): fp64 router partial sums, their reduction,
// the wave64 top-k with renormalized softmax, and small-batch bucketing.
#pragma once
#include "common.h"

namespace moe {

constexpr int kRouterKS = 128;  // router rows staged in LDS at a time
constexpr int kRouterTT = 32;   // tokens per router block at most

// One block (256 threads) of router partial sums in fp64: rows
// k in [c*kc, (c+1)*kc) of W_r [D][E] against tokens [tile*tt, +tt) for the
// 64 experts of `group`.  Thread (row lane r = tid/64, expert group*64 +
// tid%64) walks rows r, r+4, ...; the four row lanes are then added in a
// fixed order.  Products of two fp32 (or bf16 and fp32) values are exact in
// fp64, so only the additions round, at 2^-53 relative.
template <int XT>
MOE_DEV void router_partial_block(const float *__restrict__ W, const void *__restrict__ xin, int T, int D, int E,
                                  int kc, int tt, double *__restrict__ partial, int c, int tile, int group) {
    __shared__ float xs[kRouterTT * kRouterKS];  // [nt][ks]
    __shared__ double red[3][64];
    const int t0 = tile * tt;
    const int nt = min(tt, T - t0);
    const int k0 = c * kc;
    const int rl = threadIdx.x >> 6, el = threadIdx.x & 63;
    const int e = group * 64 + el;
    const bool ok = e < E;
    double acc[kRouterTT];
#pragma unroll
    for (int j = 0; j < kRouterTT; ++j) acc[j] = 0.0;
    const int ks = min(kc, kRouterKS);
    for (int kb = 0; kb < kc; kb += ks) {
        __syncthreads();
        for (int i = threadIdx.x; i < nt * ks; i += blockDim.x) {
            int tl = i / ks, kk = i % ks;
            int64_t gi = (int64_t)(t0 + tl) * D + k0 + kb + kk;
            float v;
            if constexpr (XT == MOE_BF16) v = bf16_bits_to_float(((const uint16_t *)xin)[gi]);
            else v = ((const float *)xin)[gi];
            xs[tl * ks + kk] = v;
        }
        __syncthreads();
        if (ok) {
            // rows rl, rl+4, ... of this sub-chunk; loads issued 16 at a time
            const float *wp = W + (int64_t)(k0 + kb) * E + e;
            for (int kk0 = rl; kk0 < ks; kk0 += 64) {
                float wv[16];
#pragma unroll
                for (int u = 0; u < 16; ++u)  // clamped rows keep the loads unconditional
                    wv[u] = wp[(int64_t)min(kk0 + 4 * u, ks - 1) * E];
#pragma unroll
                for (int u = 0; u < 16; ++u) {
                    int kk = kk0 + 4 * u;
                    if (kk < ks) {
                        double w = (double)wv[u];
#pragma unroll
                        for (int j = 0; j < kRouterTT; ++j)
                            if (j < nt) acc[j] = __builtin_fma((double)xs[j * ks + kk], w, acc[j]);
                    }
                }
            }
        }
    }
#pragma unroll
    for (int j = 0; j < kRouterTT; ++j) {
        if (j < nt) {  // nt is uniform over the block, so the barriers are too
            __syncthreads();
            if (rl > 0) red[rl - 1][el] = acc[j];
            __syncthreads();
            if (rl == 0 && ok)
                partial[((int64_t)c * T + t0 + j) * E + e] = ((acc[j] + red[0][el]) + red[1][el]) + red[2][el];
        }
    }
}

// a ranks before b: larger logit, then lower expert index
MOE_DEV bool before(double va, int ea, double vb, int eb) { return va > vb || (va == vb && ea < eb); }

// lg[tl*E + e] = sum over chunks c (fixed order) of partial[c][t0+tl][e]
// (+ bias) for nt tokens, by the whole block: thread (item, chunk group) sums
// a strided subset of the chunks with 16 loads in flight, then the groups are
// added in order.
MOE_DEV void reduce_logits(const double *__restrict__ partial, const float *__restrict__ bias, int T, int E,
                           int nchunk, int t0, int nt, double *lg) {
    __shared__ double red[1024];
    const int nth = blockDim.x;
    const int items = nt * E;
    int G = 1;
    while (G * 2 * items <= nth && G * 2 <= nchunk) G *= 2;
    const int64_t stride = (int64_t)T * E;
    const int per_pass = nth / G;
    for (int base = 0; base < items; base += per_pass) {
        int it = base + threadIdx.x / G, g = threadIdx.x % G;
        double s = 0.0;
        if (it < items) {
            int tl = it / E, e = it % E;
            const double *p = partial + (int64_t)(t0 + tl) * E + e;
            for (int c0 = g; c0 < nchunk; c0 += 16 * G) {
                double v[16];
#pragma unroll
                for (int u = 0; u < 16; ++u)  // clamped chunks keep the loads unconditional
                    v[u] = p[min(c0 + u * G, nchunk - 1) * stride];
#pragma unroll
                for (int u = 0; u < 16; ++u)
                    if (c0 + u * G < nchunk) s += v[u];
            }
        }
        __syncthreads();
        red[threadIdx.x] = s;
        __syncthreads();
        if (g == 0 && it < items) {
            double v = 0.0;
            for (int j = 0; j < G; ++j) v += red[threadIdx.x + j];
            if (bias) v += (double)bias[it % E];
            lg[it] = v;
        }
    }
    __syncthreads();
}

// One wave selects the top k of lg[0..E) by (logit desc, index asc) with k
// wave-wide arg-max rounds (candidates read from LDS), then forms
// w_s = route_scale * exp(l_s - l_0) / sum_j exp(l_j - l_0) in fp64.
// Lanes 0..k-1 write slot s = lane (and copy to sidx/sw when given).
MOE_DEV void select_topk(const double *lg, int E, int k, float route_scale, int32_t *idx_out, float *w_out,
                         int32_t *sidx, float *sw) {
    const int lane = threadIdx.x & 63;
    constexpr int PER = kMaxExperts / kWave;  // 16 experts per lane at most
    uint32_t taken = 0;
    for (int i = 0; i < PER; ++i)
        if (lane + 64 * i >= E) taken |= 1u << i;
    double mx = 0.0, den = 0.0, my_v = 0.0;
    int my_e = 0;
    for (int s = 0; s < k; ++s) {
        double bv = 0.0;
        int be = 0x7FFFFFFF, bi = -1;
        for (int i = 0; i < PER; ++i) {
            int e = lane + 64 * i;
            if ((taken >> i) & 1u) continue;
            double v = lg[e];
            if (bi < 0 || before(v, e, bv, be)) {
                bv = v;
                be = e;
                bi = i;
            }
        }
        // wave arg-max; a lane without a candidate never wins over one that has
        double wv = bv;
        int we = be;
        bool have = bi >= 0;
        for (int o = 32; o > 0; o >>= 1) {
            double ov = __shfl_xor(wv, o, kWave);
            int oe = __shfl_xor(we, o, kWave);
            int oh = __shfl_xor((int)have, o, kWave);
            if (oh && (!have || before(ov, oe, wv, we))) {
                wv = ov;
                we = oe;
                have = true;
            }
        }
        if (bi >= 0 && we == be) taken |= 1u << bi;
        if (s == 0) mx = wv;  // the first selected logit is the largest
        double ex = exp(wv - mx);
        den += ex;
        if (lane == s) {
            my_v = ex;
            my_e = we;
        }
    }
    if (lane < k) {
        float w = (float)((double)route_scale * my_v / den);
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

// Top-k of every row by rank: candidate (t, e) is selected at slot
// rank = #{e' ranking before e}, which is exactly the (logit desc, index asc)
// order; one pass over E per candidate, spread over the whole block.  Then
// w_s = route_scale * exp(l_s - l_0) / sum_j exp(l_j - l_0) in fp64.
MOE_DEV void select_topk_rank(const double *lg, int T, int E, int k, float route_scale, int32_t *__restrict__ topk_idx,
                              float *__restrict__ topk_w, int32_t *sidx, double *sval) {
    __shared__ int32_t rank_part[1024];
    const int nth = blockDim.x;
    const int items = T * E;
    int G = 1;  // threads per candidate
    while (G * 2 * items <= nth && G * 2 <= 64) G *= 2;
    for (int base = 0; base < items; base += nth / G) {
        const int it = base + threadIdx.x / G, g = threadIdx.x % G;
        int rk = 0;
        if (it < items) {
            const int t = it / E, e = it % E;
            const double v = lg[it];
            const double *row = lg + t * E;
            for (int e2 = g; e2 < E; e2 += G) rk += before(row[e2], e2, v, e);
        }
        rank_part[threadIdx.x] = rk;
        __syncthreads();
        if (g == 0 && it < items) {
            for (int j = 1; j < G; ++j) rk += rank_part[threadIdx.x + j];
            if (rk < k) {
                const int t = it / E;
                sidx[t * k + rk] = it % E;
                sval[t * k + rk] = lg[it];
            }
        }
        __syncthreads();
    }
    for (int i = threadIdx.x; i < T * k; i += nth) {
        const int t = i / k;
        const double mx = sval[t * k];
        double den = 0.0;
        for (int s2 = 0; s2 < k; ++s2) den += exp(sval[t * k + s2] - mx);
        const float w = (float)((double)route_scale * exp(sval[i] - mx) / den);
        topk_idx[i] = sidx[i];
        topk_w[i] = w;
    }
    __syncthreads();
}

// Routing of a handful of rows (T*E <= 4096, T*k <= 256) by one block:
// logits from the partials, top-k by rank, bucketing.
MOE_DEV void route_finish_small(const double *__restrict__ partial, const float *__restrict__ bias, int T, int E,
                                int nchunk, int k, float route_scale, int32_t *__restrict__ topk_idx,
                                float *__restrict__ topk_w, int32_t *__restrict__ count,
                                int32_t *__restrict__ offset, int32_t *__restrict__ perm, int32_t *__restrict__ pos,
                                int32_t *__restrict__ active, int32_t *__restrict__ n_active) {
    __shared__ double lg[4096];
    __shared__ int32_t sidx[256];
    __shared__ double sval[256];
    reduce_logits(partial, bias, T, E, nchunk, 0, T, lg);
    select_topk_rank(lg, T, E, k, route_scale, topk_idx, topk_w, sidx, sval);
    bucket_small(sidx, T * k, E, count, offset, perm, pos, active, n_active);
}

__host__ __device__ inline bool route_small_ok(int T, int E, int k) { return T <= 16 && T * E <= 4096 && T * k <= 256; }

}  // namespace moe
