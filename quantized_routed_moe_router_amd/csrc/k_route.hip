// k_route.hip - routing kernels for moe_route and for batches too large for
// the one-block finisher ("Understanding Dwarf Star", 5.3.2 router and top-k;
// 5.3.7 step 1 and the sparse indexing of step 2).
#include <type_traits>

#include "route_dev.h"

namespace moe {

template <int XT>
__global__ void __launch_bounds__(256) router_row_kernel(const float *__restrict__ W, const float *__restrict__ bias,
                                                         const void *__restrict__ xin, int T, int D, int E,
                                                         double *__restrict__ logits) {
    __shared__ double part[4 * 16];
    router_row_block<XT>(W, bias, xin, T, D, E, logits, blockIdx.x, part);
}

template <int XT>
__global__ void __launch_bounds__(256) router_tile_kernel(const float *__restrict__ W, const float *__restrict__ bias,
                                                          const void *__restrict__ xin, int T, int D, int E,
                                                          double *__restrict__ logits) {
    router_tile_block<XT>(W, bias, xin, T, D, E, logits, blockIdx.x, blockIdx.y);
}

// Many tokens: the logits on the fp64 matrix cores (v_mfma_f64_16x16x4_f64),
// the router contraction of "Understanding Dwarf Star", 5.3.2.  A wave owns a
// 16-token x 16-expert tile over the whole reduction; the 4 waves of a block
// share the token rows and take 4 adjacent expert tiles.  Per 16-wide slice
// of k, lane l loads 4 consecutive values of token row (l & 15) and of expert
// row (l & 15), both at k0 + 4 (l >> 4); matrix instruction j takes component
// j of both, so each product x[t][k] W[e][k] enters the sum exactly once.
// Products of fp32 (or bf16) values are exact in fp64: only the order of the
// fp64 additions differs from a plain ascending sum.  Register r of the
// accumulator holds token (l >> 4) + 4r, expert l & 15.
// Linear block id -> tiles: the blocks of one XCD (ids round-robin over the 8)
// take one contiguous range of token rows, so its L2 holds those rows and the
// router matrix.
typedef double f64x4 __attribute__((ext_vector_type(4)));

// raw 4 activations of one lane (bf16 bits or fp32), converted where used so
// that a load in flight is not waited for before the products that precede
// its use
template <int XT>
using RouterX = typename std::conditional<XT == MOE_BF16, uint2, f32x4>::type;

template <int XT>
MOE_DEV float router_x(const RouterX<XT> &v, int q) {
    if constexpr (XT == MOE_BF16) {
        const uint32_t u = q < 2 ? v.x : v.y;
        return bf16_bits_to_float((q & 1) ? (u >> 16) : (u & 0xFFFFu));
    } else {
        return v[q];
    }
}

// KS = 4 (fewer rows): the 4 waves of a block take quarters of the
// reduction of one 16 x 16 tile instead, and wave 0 adds the four partial
// sums in wave order (fixed, so the result does not vary between runs); the
// blocks then map to tiles in order (n_ttx = token tiles, n_eq = expert
// tiles).  nparts > 1: nparts blocks per tile take consecutive slices of the
// reduction, and block b of a tile writes its sum, without the bias, to
// partial row set b (logits + b*T*E); the selection adds them in order.
template <int XT, int KS>
__global__ void __launch_bounds__(256) router_mfma_kernel(const float *__restrict__ W, const float *__restrict__ bias,
                                                          const void *__restrict__ xin, int T, int D, int E,
                                                          double *__restrict__ logits, int n_ttx, int n_eq,
                                                          int nparts) {
    __shared__ double red[KS == 4 ? 3 : 1][64][4];
    const int L = blockIdx.x, xcd = L & 7, j = L >> 3;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    // expert tiles per wave: with KS = 1 a wave takes two side by side, which
    // share its activation loads and give two independent product chains
    constexpr int NE = KS == 1 ? 2 : 1;
    int tt, e0, kbeg, kend;
    if constexpr (KS == 1) {
        tt = xcd * n_ttx + j / n_eq;
        e0 = ((j % n_eq) * 4 + wave) * 16 * NE;
        kbeg = 0;
        kend = D;
    } else {
        const int tile = L / nparts, part = L % nparts, kw = D / (4 * nparts);
        tt = tile / n_eq;
        e0 = (tile % n_eq) * 16;
        kbeg = (part * 4 + wave) * kw;
        kend = kbeg + kw;
        if (nparts > 1) {
            logits += (int64_t)part * T * E;
            bias = nullptr;
        }
    }
    const int t0 = tt * 16;
    if (t0 >= T || e0 >= E) return;  // uniform over the block when KS = 4
    const int row = lane & 15, kq = 4 * (lane >> 4);
    const int t = min(t0 + row, T - 1);
    const void *xrow = XT == MOE_BF16 ? (const void *)((const uint16_t *)xin + (int64_t)t * D + kq)
                                      : (const void *)((const float *)xin + (int64_t)t * D + kq);
    const float *wrow[NE];
#pragma unroll
    for (int n = 0; n < NE; ++n) wrow[n] = W + (int64_t)min(e0 + 16 * n + row, E - 1) * D + kq;
    f64x4 acc[NE];
#pragma unroll
    for (int n = 0; n < NE; ++n) acc[n] = f64x4{0.0, 0.0, 0.0, 0.0};
    // 64 k per half step from two register sets: the loads of one set are in
    // flight while the other's products run (D is a multiple of 128 here)
    RouterX<XT> xa[4], xb[4];
    f32x4 wa[NE][4], wb[NE][4];
    auto load = [&](RouterX<XT> (&xv)[4], f32x4 (&wv)[NE][4], int k) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            xv[c] = *(const RouterX<XT> *)((const char *)xrow + (int64_t)(k + 16 * c) * (XT == MOE_BF16 ? 2 : 4));
#pragma unroll
            for (int n = 0; n < NE; ++n) wv[n][c] = *(const f32x4 *)(wrow[n] + k + 16 * c);
        }
        __builtin_amdgcn_sched_barrier(0);  // keep the loads ahead of the products
    };
    auto mma = [&](const RouterX<XT> (&xv)[4], const f32x4 (&wv)[NE][4]) {
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const double xd = (double)router_x<XT>(xv[c], q);
#pragma unroll
                for (int n = 0; n < NE; ++n)
                    acc[n] = __builtin_amdgcn_mfma_f64_16x16x4f64(xd, (double)wv[n][c][q], acc[n], 0, 0, 0);
            }
    };
    load(xa, wa, kbeg);
    for (int k0 = kbeg; k0 < kend; k0 += 128) {
        load(xb, wb, k0 + 64);
        mma(xa, wa);
        load(xa, wa, min(k0 + 128, kend - 64));  // the last step re-reads a slice: no branch, so the waits stay exact
        mma(xb, wb);
    }
    if constexpr (KS == 4) {
        if (wave > 0)
#pragma unroll
            for (int r = 0; r < 4; ++r) red[wave - 1][lane][r] = acc[0][r];
        __syncthreads();
        if (wave > 0) return;
#pragma unroll
        for (int r = 0; r < 4; ++r)
            acc[0][r] = ((acc[0][r] + red[0][lane][r]) + red[1][lane][r]) + red[2][lane][r];
    }
#pragma unroll
    for (int n = 0; n < NE; ++n) {
        const int ex = e0 + 16 * n + (lane & 15);
        if (ex >= E) continue;
        const double b = bias ? (double)bias[ex] : 0.0;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int tok = t0 + (lane >> 4) + 4 * r;
            if (tok < T) logits[(int64_t)tok * E + ex] = acc[n][r] + b;
        }
    }
}

__global__ void __launch_bounds__(256) route_finish_small_kernel(const double *__restrict__ logits, int T, int E,
                                                                 int k, float route_scale,
                                                                 int32_t *__restrict__ topk_idx,
                                                                 float *__restrict__ topk_w,
                                                                 int32_t *__restrict__ count,
                                                                 int32_t *__restrict__ offset,
                                                                 int32_t *__restrict__ perm, int32_t *__restrict__ pos,
                                                                 int32_t *__restrict__ active,
                                                                 int32_t *__restrict__ n_active) {
    route_finish_block(logits, T, E, k, route_scale, topk_idx, topk_w, count, offset, perm, pos, active, n_active,
                       nullptr, 0);
}

// One wave per token: top-k of its logit row.  PARTS: the row is the sum of
// nparts partial row sets (the split router's, T*E apart) in order, then the
// bias; the eight reads of a logit are issued at once (past nparts they
// re-read set 0 and add 0).
template <int PER, bool PARTS>
__global__ void __launch_bounds__(256) router_topk_kernel(const double *__restrict__ logits, int nparts,
                                                          const float *__restrict__ bias, int T, int E, int k,
                                                          float route_scale, int32_t *__restrict__ topk_idx,
                                                          float *__restrict__ topk_w) {
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    const double *lt = logits + (int64_t)t * E;
    const int64_t stride = (int64_t)T * E;
    auto logit = [&](int e) {
        if constexpr (!PARTS) {
            return lt[e];
        } else {
            double pv[kMaxRouterParts];
#pragma unroll
            for (int b = 0; b < kMaxRouterParts; ++b) pv[b] = lt[min(b, nparts - 1) * stride + e];
            const double be = bias ? (double)bias[e] : 0.0;
            double v = pv[0];
#pragma unroll
            for (int b = 1; b < kMaxRouterParts; ++b) v += b < nparts ? pv[b] : 0.0;
            return v + be;
        }
    };
    select_topk_load<PER>(logit, E, k, route_scale, topk_idx + (int64_t)t * k, topk_w + (int64_t)t * k);
}

// Stable counting sort of up to 1024 pairs by expert in one block of 16
// waves, in LDS.  Wave w holds pairs 64w..64w+63; ballots over the expert's
// bits rank equal experts inside the wave (the lower pair id first); a
// prefix over the waves per expert, then one scan over the experts of
// (count | active flag << 16), gives each expert's offset and place in the
// active list, and each pair's slot is offset + earlier waves' count + rank.
// The result is a pure function of topk_idx: the same arrays as the other
// sorts.
constexpr int kMidWaves = 16;
constexpr int kMidPairs = 64 * kMidWaves;
static_assert(kMidPairs == kRouteMidPairs, "pairs of the one-block sort");

__global__ void __launch_bounds__(1024) bucket_mid_kernel(const int32_t *__restrict__ topk_idx, int P, int E,
                                                          int32_t *__restrict__ count, int32_t *__restrict__ offset,
                                                          int32_t *__restrict__ perm, int32_t *__restrict__ pos,
                                                          int32_t *__restrict__ active,
                                                          int32_t *__restrict__ n_active) {
    __shared__ int32_t wc[kMidWaves][kMaxExperts];  // per (wave, expert): count, then first slot
    __shared__ int32_t wsum[kMidWaves];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const bool valid = tid < P;
    const int key = valid ? topk_idx[tid] : 0;
    for (int w = 0; w < kMidWaves; ++w)
        if (tid < E) wc[w][tid] = 0;  // blockDim.x = kMaxExperts >= E
    uint64_t same = __ballot(valid);
    const int nbits = 32 - __clz(max(E - 1, 1));
    for (int b = 0; b < nbits; ++b) {
        const uint64_t bal = __ballot(valid && ((key >> b) & 1));
        same &= ((key >> b) & 1) ? bal : ~bal;
    }
    const int rank = __popcll(same & ((1ull << lane) - 1ull));
    __syncthreads();
    if (valid && rank == 0) wc[wave][key] = __popcll(same);
    __syncthreads();

    const int e = tid;
    int tot = 0;
    if (e < E) {
        for (int w = 0; w < kMidWaves; ++w) {
            const int c = wc[w][e];
            wc[w][e] = tot;
            tot += c;
        }
    }
    const int packed = tot | ((tot > 0 ? 1 : 0) << 16);  // both sums stay below 2^16
    int incl = packed;
    for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_up(incl, o, kWave);
        if (lane >= o) incl += v;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    int before = 0, all = 0;
    for (int w = 0; w < kMidWaves; ++w) {
        const int v = wsum[w];
        before += w < wave ? v : 0;
        all += v;
    }
    const int excl = before + incl - packed, first = excl & 0xFFFF, na = all >> 16;
    if (e < E) {
        count[e] = tot;
        offset[e] = first;
        for (int w = 0; w < kMidWaves; ++w) wc[w][e] += first;
        if (tot > 0) active[excl >> 16] = e;  // below na
        if (e >= na) active[e] = -1;
    }
    if (tid == 0) {
        n_active[0] = na;
        offset[E] = P;
    }
    __syncthreads();
    if (valid) {
        const int slot = wc[wave][key] + rank;
        perm[slot] = tid;
        pos[tid] = slot;
    }
}

// Stable counting sort of the P = T*k pairs by expert, one block of 8 waves.
// Wave w owns a contiguous segment of pair ids.  Pass 1 counts per (wave,
// expert); a scan over waves then experts gives each wave's first slot per
// expert; pass 2 walks the segment 64 pairs at a time and ranks equal experts
// inside the wave with ballots, so the result is a pure function of topk_idx.
constexpr int kBucketWaves = 8;
// Pairs whose experts the bucketing block keeps in LDS between its two passes
// (prefill at 2048 rows and top-6 is 12,288): the scatter pass then reads
// them back from LDS instead of one dependent global round trip per 64 pairs.
constexpr int kBucketKeyCache = 16384;
static_assert(kBucketKeyCache % (kBucketWaves * 64) == 0, "whole keys per lane");

__global__ void __launch_bounds__(512) bucket_kernel(const int32_t *__restrict__ topk_idx, int P, int E,
                                                     int32_t *__restrict__ count, int32_t *__restrict__ offset,
                                                     int32_t *__restrict__ perm, int32_t *__restrict__ pos,
                                                     int32_t *__restrict__ active, int32_t *__restrict__ n_active) {
    __shared__ int32_t wc[kBucketWaves][kMaxExperts];
    __shared__ int32_t tot[kMaxExperts];
    __shared__ int32_t scan_tmp[kMaxExperts];
    __shared__ int32_t keys[kBucketKeyCache];  // the experts of the pairs, when P fits
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    for (int i = tid; i < kBucketWaves * kMaxExperts; i += blockDim.x) (&wc[0][0])[i] = 0;
    __syncthreads();
    const int seg = ((P + kBucketWaves - 1) / kBucketWaves + 63) / 64 * 64;
    const int s0 = w * seg, s1 = min(P, s0 + seg);
    const bool cached = P <= kBucketKeyCache;
    if (cached) {
        // every key of the lane's share in flight at once (at most
        // kBucketKeyCache / (kBucketWaves * 64) = 32), then the counts
        constexpr int kPer = kBucketKeyCache / (kBucketWaves * 64);
        int kv[kPer];
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int p = s0 + lane + 64 * i;
            kv[i] = p < s1 ? topk_idx[p] : -1;
        }
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            if (kv[i] >= 0) {
                keys[s0 + lane + 64 * i] = kv[i];  // a wave later reads back only the pairs it wrote
                atomicAdd(&wc[w][kv[i]], 1);
            }
        }
    } else {
        for (int p = s0 + lane; p < s1; p += 64) atomicAdd(&wc[w][topk_idx[p]], 1);
    }
    __syncthreads();
    for (int e = tid; e < E; e += blockDim.x) {  // exclusive prefix over waves
        int run = 0;
        for (int ww = 0; ww < kBucketWaves; ++ww) {
            int c = wc[ww][e];
            wc[ww][e] = run;
            run += c;
        }
        tot[e] = run;
    }
    __syncthreads();
    for (int e = tid; e < kMaxExperts; e += blockDim.x) scan_tmp[e] = e < E ? tot[e] : 0;
    __syncthreads();
    for (int o = 1; o < E; o <<= 1) {  // inclusive scan over experts (entries from E on stay 0)
        int a0 = tid, a1 = tid + 512;
        int v0 = scan_tmp[a0] + (a0 >= o ? scan_tmp[a0 - o] : 0);
        int v1 = scan_tmp[a1] + (a1 >= o ? scan_tmp[a1 - o] : 0);
        __syncthreads();
        scan_tmp[a0] = v0;
        scan_tmp[a1] = v1;
        __syncthreads();
    }
    for (int e = tid; e < E; e += blockDim.x) {
        int excl = scan_tmp[e] - tot[e];
        count[e] = tot[e];
        offset[e] = excl;
        for (int ww = 0; ww < kBucketWaves; ++ww) wc[ww][e] += excl;
    }
    if (tid == 0) offset[E] = scan_tmp[E - 1];
    __syncthreads();
    const int nbits = 32 - __clz(max(E - 1, 1));
    for (int base = s0; base < s1; base += 64) {  // stable scatter
        int p = base + lane;
        bool valid = p < s1;
        int key = valid ? (cached ? keys[p] : topk_idx[p]) : 0;
        uint64_t same = __ballot(valid);
        for (int b = 0; b < nbits; ++b) {
            uint64_t bal = __ballot(valid && ((key >> b) & 1));
            same &= ((key >> b) & 1) ? bal : ~bal;
        }
        int rank = __popcll(same & ((1ull << lane) - 1ull));
        int slot = valid ? wc[w][key] + rank : 0;
        __builtin_amdgcn_wave_barrier();
        if (valid) {
            perm[slot] = p;
            pos[p] = slot;
            if (rank == 0) wc[w][key] = slot + __popcll(same);
        }
        __builtin_amdgcn_wave_barrier();
    }
    __syncthreads();
    for (int e = tid; e < kMaxExperts; e += blockDim.x) scan_tmp[e] = (e < E && tot[e] > 0) ? 1 : 0;
    __syncthreads();
    for (int o = 1; o < E; o <<= 1) {
        int a0 = tid, a1 = tid + 512;
        int v0 = scan_tmp[a0] + (a0 >= o ? scan_tmp[a0 - o] : 0);
        int v1 = scan_tmp[a1] + (a1 >= o ? scan_tmp[a1 - o] : 0);
        __syncthreads();
        scan_tmp[a0] = v0;
        scan_tmp[a1] = v1;
        __syncthreads();
    }
    const int na = scan_tmp[E - 1];
    for (int e = tid; e < E; e += blockDim.x) active[e] = -1;
    __syncthreads();
    for (int e = tid; e < E; e += blockDim.x)
        if (tot[e] > 0) active[scan_tmp[e] - 1] = e;
    if (tid == 0) n_active[0] = na;
}

// one block per expert row for few tokens, 16 x 16 tiles for many
bool router_rows_ok(int T) { return T <= 16; }
// the matrix-core router: a wave per 16 x 16 tile from 128 rows on (the k
// steps need D % 128 == 0); below that, for more rows than the one-block
// router takes, four waves per tile (D % 512 == 0)
bool router_mfma_ok(int T, int D) { return T >= 128 && D % 128 == 0; }
bool router_mfma4_ok(int T, int D) { return T > 16 && D % 512 == 0; }

hipError_t launch_router_logits(const moe_layer_desc *d, const void *x, int32_t T, int32_t x_type,
                                const Workspace &ws, hipStream_t s) {
    const int D = d->n_embd, E = d->n_expert;
    if (router_rows_ok(T)) {
        if (x_type == MOE_BF16)
            router_row_kernel<MOE_BF16><<<E, 256, 0, s>>>(d->router_w, d->router_bias, x, T, D, E, ws.logits);
        else
            router_row_kernel<MOE_F32><<<E, 256, 0, s>>>(d->router_w, d->router_bias, x, T, D, E, ws.logits);
    } else if (router_mfma_ok(T, D)) {
        const int n_tt = (T + 15) / 16, n_ttx = (n_tt + 7) / 8, n_eq = ((E + 15) / 16 + 7) / 8;  // 8 expert tiles a block
        const int grid = 8 * n_ttx * n_eq;
        if (x_type == MOE_BF16)
            router_mfma_kernel<MOE_BF16, 1><<<grid, 256, 0, s>>>(d->router_w, d->router_bias, x, T, D, E, ws.logits,
                                                                  n_ttx, n_eq, 1);
        else
            router_mfma_kernel<MOE_F32, 1><<<grid, 256, 0, s>>>(d->router_w, d->router_bias, x, T, D, E, ws.logits,
                                                                 n_ttx, n_eq, 1);
    } else if (router_mfma4_ok(T, D)) {
        const int n_tt = (T + 15) / 16, n_et = (E + 15) / 16, np = router_parts(T, D, d->n_expert_used, E);
        const unsigned grid = (unsigned)(n_tt * n_et * np);
        if (x_type == MOE_BF16)
            router_mfma_kernel<MOE_BF16, 4><<<grid, 256, 0, s>>>(d->router_w, d->router_bias, x, T, D, E,
                                                                  ws.logits, n_tt, n_et, np);
        else
            router_mfma_kernel<MOE_F32, 4><<<grid, 256, 0, s>>>(d->router_w, d->router_bias, x, T, D, E,
                                                                 ws.logits, n_tt, n_et, np);
    } else {
        dim3 g((T + 15) / 16, (E + 15) / 16);
        if (x_type == MOE_BF16)
            router_tile_kernel<MOE_BF16><<<g, 256, 0, s>>>(d->router_w, d->router_bias, x, T, D, E, ws.logits);
        else
            router_tile_kernel<MOE_F32><<<g, 256, 0, s>>>(d->router_w, d->router_bias, x, T, D, E, ws.logits);
    }
    return hipGetLastError();
}

hipError_t launch_route_finish(const moe_layer_desc *d, int32_t T, const RoutingPtrs &r, const Workspace &ws,
                               hipStream_t s) {
    const int E = d->n_expert, k = d->n_expert_used, P = T * k;
    if (route_small_ok(T, E, k)) {
        route_finish_small_kernel<<<1, 256, 0, s>>>(ws.logits, T, E, k, d->route_scale, r.topk_idx, r.topk_w,
                                                     r.count, r.offset, r.perm, r.pos, r.active, r.n_active);
        return hipGetLastError();
    }
    const int np = router_parts(T, d->n_embd, k, E);
    auto topk = [&](auto kern) {
        kern<<<(T + 3) / 4, 256, 0, s>>>(ws.logits, np, d->router_bias, T, E, k, d->route_scale, r.topk_idx,
                                         r.topk_w);
    };
    if (np > 1) {  // E <= 256 here
        if (E <= 64) topk(router_topk_kernel<1, true>);
        else if (E <= 128) topk(router_topk_kernel<2, true>);
        else topk(router_topk_kernel<4, true>);
    } else {
        if (E <= 64) topk(router_topk_kernel<1, false>);
        else if (E <= 128) topk(router_topk_kernel<2, false>);
        else if (E <= 256) topk(router_topk_kernel<4, false>);
        else if (E <= 512) topk(router_topk_kernel<8, false>);
        else topk(router_topk_kernel<16, false>);
    }
    if (P <= kMidPairs)
        bucket_mid_kernel<<<1, kMaxExperts, 0, s>>>(r.topk_idx, P, E, r.count, r.offset, r.perm, r.pos, r.active,
                                                    r.n_active);
    else
        bucket_kernel<<<1, 512, 0, s>>>(r.topk_idx, P, E, r.count, r.offset, r.perm, r.pos, r.active, r.n_active);
    return hipGetLastError();
}

hipError_t launch_route(const moe_layer_desc *d, const void *x, int32_t T, int32_t x_type, const RoutingPtrs &r,
                        const Workspace &ws, hipStream_t s) {
    hipError_t e = launch_router_logits(d, x, T, x_type, ws, s);
    if (e != hipSuccess) return e;
    return launch_route_finish(d, T, r, ws, s);
}

}  // namespace moe
