// k_route.hip - routing kernels for moe_route and for batches too large for
// the one-block finisher ("Understanding Dwarf Star", 5.3.2 router and top-k;
// 5.3.7 step 1 and the sparse indexing of step 2).
#include <type_traits>

#include "ffn_dev.h"
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

// ---- many bf16 rows: the router in two passes ---------------------------------
// The selection must be that of the fp64 router ("Understanding Dwarf Star",
// 5.3.2: fp32 router weights, the top k by logit, then the softmax over them).
// Pass 1 (router_bf16x3_kernel) bounds every logit cheaply on the bf16 matrix
// cores: x is exact in bf16 and each fp32 weight is split into three bf16
// parts w = w1 + w2 + w3 (8 + 8 + 8 significant bits), so every product is
// exact and only the fp32 accumulation rounds.  A block takes 128 tokens x 128
// experts over one of kRtSplit slices of D; wave w owns experts 32w..32w+31
// against the 4 token subtiles (v_mfma_f32_32x32x16_bf16, three per subtile
// and 16-wide step of k); lane (c, h) loads 8 consecutive values of token row
// c and of expert row c per step, the layout both operands share.  It also
// writes each slice's sum of w^2 per expert.
// Pass 2 (router_refine_kernel, a wave per token) adds the slices per logit and bounds its
// error by eps_e = C |x| |w_e| (Cauchy-Schwarz; C covers the 3 D / kRtSplit
// fp32 roundings of a slice's sum, truncating or not, with a factor 2 to
// spare).  An expert whose upper bound stays below the k-th largest lower
// bound has k experts strictly above it, so only the others can be in the top
// k.  Their logits are computed again exactly as the fp64 router does (exact
// products of bf16 x and fp32 w, fp64 sums plus the bias), and the top k and
// the weights come from those, with the usual order (logit desc, index asc).
constexpr int kRtSplit = kRtSplitMax;       // D slices of pass 1
constexpr int kRtTok = 128, kRtExp = 128;   // block tile of pass 1

bool router_split_ok(int T, int D, int E, int x_type) {
    return x_type == MOE_BF16 && T >= 128 && (D == 1024 || D == 2048 || D == 4096) && E <= 256;
}

// Pass 1 in groups of 64 columns (4 steps of 16): the block's 128 token rows
// of a group are copied into LDS once for its 4 waves (global-to-LDS DMA,
// two stages, the next group's copies in flight under this group's
// products), and each lane loads its expert row's 32 columns of the group
// (one 128-byte line) into registers, also a group ahead.  Columns of step s
// for lane half h: 32 h + 8 s + 0..7 of the group (a permutation of k that
// both operands share).  LDS unit j (16 bytes) of token row r holds the
// row's columns 8 (j ^ (r & 7)) .. + 7, so that the 32 rows one read spans
// fall on different banks.
constexpr int kRtGroupUnits = kRtTok * 8;  // 16-byte units of one group's token rows: 1024
template <int G>  // groups of 64 columns per slice: D / (64 kRtSplit)
__global__ void __launch_bounds__(256) router_bf16x3_kernel(const float *__restrict__ W, const uint16_t *__restrict__ x,
                                                            int T, int D, int E, float *__restrict__ part,
                                                            float *__restrict__ wn) {
    typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
    typedef float v16f __attribute__((ext_vector_type(16)));
    __shared__ __align__(16) u32x4 xs[2][kRtGroupUnits];
    const int tt = blockIdx.x, et = blockIdx.y, sl = blockIdx.z;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, c = lane & 31, h = lane >> 5;
    const int kb = sl * (64 * G);  // the slice's first column
    const int eo = et * kRtExp + 32 * wave + c;  // the lane's expert column
    const float *wr = W + (int64_t)min(eo, E - 1) * D + kb + 32 * h;
    // the DMA sources of the lane's 4 units per group (copy i: units 256 i + 64 wave + lane)
    const uint16_t *xsrc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int p = 256 * i + 64 * wave + lane, r = p >> 3, j = p & 7;
        xsrc[i] = x + (int64_t)min(tt * kRtTok + r, T - 1) * D + kb + 8 * (j ^ (r & 7));
    }
    const uint32_t lbase = (uint32_t)__builtin_amdgcn_readfirstlane(lds_addr(&xs[0][0])) + 1024u * (uint32_t)wave;
    auto issue = [&](int g) {  // 4 copies per wave
        const uint32_t st = lbase + (uint32_t)((g & 1) * kRtGroupUnits * 16);
#pragma unroll
        for (int i = 0; i < 4; ++i) dma16_m0(xsrc[i] + 64 * g, st + 4096u * (uint32_t)i);
    };
    f32x4 wg[2][8];  // the lane's 32 columns of the group, two groups
    auto load_w = [&](int g, int b) {
#pragma unroll
        for (int q = 0; q < 8; ++q) wg[b][q] = *(const f32x4 *)(wr + 64 * g + 4 * q);
        // issued here, in this order after the copies: the copy waits below count them
        __asm__ volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
    };
    v16f acc[4];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[m][v] = 0.f;
    float ss = 0.f;
    issue(0);
    load_w(0, 0);
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const int b = g & 1;
        if (g + 1 < G) {
            issue(g + 1);
            load_w(g + 1, b ^ 1);
            // group g's copies have landed: after them this wave issued its
            // 8 row loads of group g, then 4 copies and 8 loads of group g + 1
            vmem_wait_le<20>();
        } else {
            vmem_wait_le<8>();  // after them: the 8 row loads of group g
        }
        barrier_only();  // every wave's copies of group g are in LDS
        const u32x4 *st = &xs[b][0];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            uint32_t p1[4], p2[4], p3[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float a = wg[b][2 * s + (i >> 1)][2 * (i & 1)], bb = wg[b][2 * s + (i >> 1)][2 * (i & 1) + 1];
                ss = __builtin_fmaf(a, a, ss);
                ss = __builtin_fmaf(bb, bb, ss);
                p1[i] = bf16x2_rne(a, bb);
                const float ra = a - __uint_as_float(p1[i] << 16), rb = bb - __uint_as_float(p1[i] & 0xFFFF0000u);
                p2[i] = bf16x2_rne(ra, rb);
                const float qa = ra - __uint_as_float(p2[i] << 16), qb = rb - __uint_as_float(p2[i] & 0xFFFF0000u);
                p3[i] = bf16x2_rne(qa, qb);
            }
            v8bf w1, w2, w3;
            __builtin_memcpy(&w1, p1, 16);
            __builtin_memcpy(&w2, p2, 16);
            __builtin_memcpy(&w3, p3, 16);
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int r = 32 * m + c;
                const u32x4 av = st[r * 8 + ((4 * h + s) ^ (r & 7))];
                v8bf a;
                __builtin_memcpy(&a, &av, 16);
                acc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, w1, acc[m], 0, 0, 0);
                acc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, w2, acc[m], 0, 0, 0);
                acc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, w3, acc[m], 0, 0, 0);
            }
        }
        barrier_only();  // every wave is done with stage b before group g + 2's copies
    }
    // lane (c, h): expert column c, token rows 8 (v / 4) + 4 h + v % 4 of each subtile
    if (eo < E) {
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int t = tt * kRtTok + 32 * m + 8 * (v >> 2) + 4 * h + (v & 3);
                if (t < T) part[((int64_t)sl * T + t) * E + eo] = acc[m][v];
            }
    }
    ss += __shfl_xor(ss, 32, kWave);  // the two halves of each group's 64 columns
    if (tt == 0 && h == 0 && eo < E) wn[sl * E + eo] = ss;
}

// Pass 2: a wave per token (4 per block); lane l holds the token's V = D / 64
// columns from V l, as bf16 pairs.
template <int PER, int V>
__global__ void __launch_bounds__(256) router_refine_kernel(const float *__restrict__ W, const float *__restrict__ bias,
                                                            const uint16_t *__restrict__ x,
                                                            const float *__restrict__ part,
                                                            const float *__restrict__ wn, int T, int D, int E, int k,
                                                            float route_scale, int32_t *__restrict__ idx_out,
                                                            float *__restrict__ w_out) {
    __shared__ int32_t cand_e[4][256];
    __shared__ double cand_v[4][256];
    __shared__ int32_t by_rank[4][256];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, t = blockIdx.x * 4 + wave;
    if (t >= T) return;  // the whole wave: no block barrier below
    const int q0 = V * lane;
    uint32_t xp[V / 2];
#pragma unroll
    for (int g = 0; g < V / 8; ++g) {
        const u32x4 u = *(const u32x4 *)(x + (int64_t)t * D + q0 + 8 * g);
#pragma unroll
        for (int i = 0; i < 4; ++i) xp[4 * g + i] = u[i];
    }
    double sq = 0.0;
#pragma unroll
    for (int i = 0; i < V / 2; ++i) {
        const double a = (double)__uint_as_float(xp[i] << 16), b = (double)__uint_as_float(xp[i] & 0xFFFF0000u);
        sq = __builtin_fma(a, a, sq);
        sq = __builtin_fma(b, b, sq);
    }
    const double nx = sqrt(seg_sum_f64(sq, kWave)) * (1.0 + 0x1p-40);
    // bounds of the lane's experts l + 64 i
    const double C = 2.0 * 2.0 * 3.0 * (double)(D / kRtSplit) * 0x1p-24;
    double lb[PER], ub[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int e = lane + 64 * i;
        if (e < E) {
            double a = 0.0, n2 = 0.0;
#pragma unroll
            for (int sl = 0; sl < kRtSplit; ++sl) {
                a += (double)part[((int64_t)sl * T + t) * E + e];
                n2 += (double)wn[sl * E + e];
            }
            // the fp32 sums of squares round too: 1 + 2^-10 covers them
            const double eps = C * nx * sqrt(n2 * (1.0 + 0x1p-10)) + 0x1p-100;
            if (bias) a += (double)bias[e];
            lb[i] = a - eps;
            ub[i] = a + eps;
        } else {
            lb[i] = ub[i] = -__builtin_inf();
        }
    }
    // L: the k-th largest lower bound (k rounds of the wave maximum, one
    // lane's copy taken out per round)
    double L = -__builtin_inf();
    {
        uint32_t taken = 0;
        for (int r = 0; r < k; ++r) {
            double best = -__builtin_inf();
            int bi = -1;
#pragma unroll
            for (int i = 0; i < PER; ++i)
                if (!((taken >> i) & 1u) && lb[i] > best) {
                    best = lb[i];
                    bi = i;
                }
            const double m = wave_max_f64(best);
            const uint64_t has = __ballot(bi >= 0 && best == m);
            if (has && lane == (int)__builtin_ctzll(has)) taken |= 1u << bi;
            L = m;
        }
    }
    // the candidates (cnt >= k: every expert whose lower bound reaches L)
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const bool cnd = lane + 64 * i < E && ub[i] >= L;
        const uint64_t m = __ballot(cnd);
        if (cnd) cand_e[wave][cnt + __popcll(m & ((1ull << lane) - 1ull))] = lane + 64 * i;
        cnt += __popcll(m);
    }
    __builtin_amdgcn_wave_barrier();
    // their logits again, exactly: fp64 sums of exact products in column
    // order within the lane, then the fixed butterfly over the lanes
    // Each row in two halves of the lane's columns; the loads of the next two
    // halves are in flight under each half's products.
    constexpr int H = V / 8;  // f32x4 per half
    const float *wb = W + q0;
    auto load_half = [&](int j, f32x4 (&buf)[H]) {
        const float *wr = wb + (int64_t)cand_e[wave][j >> 1] * D + (j & 1) * (V / 2);
#pragma unroll
        for (int g = 0; g < H; ++g) buf[g] = *(const f32x4 *)(wr + 4 * g);
    };
    double acc = 0.0;
    auto half = [&](int j, const f32x4 (&buf)[H]) {
        if (!(j & 1)) acc = 0.0;
#pragma unroll
        for (int g = 0; g < H; ++g) {
            const int i = (j & 1) * (V / 4) + 2 * g;  // the pair index of the half's values
            const uint32_t p0 = xp[i], p1 = xp[i + 1];
            acc = __builtin_fma((double)__uint_as_float(p0 << 16), (double)buf[g][0], acc);
            acc = __builtin_fma((double)__uint_as_float(p0 & 0xFFFF0000u), (double)buf[g][1], acc);
            acc = __builtin_fma((double)__uint_as_float(p1 << 16), (double)buf[g][2], acc);
            acc = __builtin_fma((double)__uint_as_float(p1 & 0xFFFF0000u), (double)buf[g][3], acc);
        }
        if (j & 1) {
            double v = seg_sum_f64(acc, kWave);
            if (bias) v += (double)bias[cand_e[wave][j >> 1]];
            if (lane == 0) cand_v[wave][j >> 1] = v;
        }
    };
    f32x4 ra[H], rb[H], rc[H];  // three halves: two in flight under the products of the third
    const int nh = 2 * cnt;       // even: both halves of every row
    load_half(0, ra);
    load_half(1, rb);
    for (int j = 0; j < nh; j += 3) {
        if (j + 2 < nh) load_half(j + 2, rc);
        half(j, ra);
        if (j + 1 >= nh) break;
        if (j + 3 < nh) load_half(j + 3, ra);
        half(j + 1, rb);
        if (j + 2 >= nh) break;
        if (j + 4 < nh) load_half(j + 4, rb);
        half(j + 2, rc);
    }
    __builtin_amdgcn_wave_barrier();
    // ranks among the candidates (logit descending, then expert ascending)
    for (int c = lane; c < cnt; c += kWave) {
        const double v = cand_v[wave][c];
        const int e = cand_e[wave][c];
        int rank = 0;
        for (int o = 0; o < cnt; ++o) rank += before(cand_v[wave][o], cand_e[wave][o], v, e);
        by_rank[wave][rank] = c;
    }
    __builtin_amdgcn_wave_barrier();
    // slot s = rank s; w_s = route_scale exp(l_s - l_0) / sum_j exp(l_j - l_0)
    // in fp64, as the other selections compute it
    double my_v = 0.0;
    int my_e = 0;
    if (lane < k) {
        const int c = by_rank[wave][lane];
        my_v = cand_v[wave][c];
        my_e = cand_e[wave][c];
    }
    const double mx = __shfl(my_v, 0, kWave);
    const double ex = lane < k ? exp(my_v - mx) : 0.0;
    double den = ex;
    for (int o = 1; o < 64; o <<= 1) den += __shfl_xor(den, o, kWave);
    if (lane < k) {
        idx_out[(int64_t)t * k + lane] = my_e;
        w_out[(int64_t)t * k + lane] = (float)((double)route_scale * ex / den);
    }
}

// one block per expert row for few tokens, 16 x 16 tiles for many
bool router_rows_ok(int T) { return T <= 16; }
// the fp64 matrix-core router: a wave per 16 x 16 tile from 128 rows on (the
// k steps need D % 128 == 0; bf16 rows of the shapes router_split_ok takes
// go to the two-pass router instead); below that, for more rows than the
// one-block router takes, four waves per tile (D % 512 == 0)
bool router_mfma_ok(int T, int D) { return T >= 128 && D % 128 == 0; }
bool router_mfma4_ok(int T, int D) { return T > 16 && D % 512 == 0; }

hipError_t launch_router_logits(const moe_layer_desc *d, const void *x, int32_t T, int32_t x_type,
                                const Workspace &ws, hipStream_t s) {
    const int D = d->n_embd, E = d->n_expert;
    if (router_split_ok(T, D, E, x_type)) {
        const dim3 g((unsigned)((T + kRtTok - 1) / kRtTok), (unsigned)((E + kRtExp - 1) / kRtExp), kRtSplit);
        auto go = [&](auto kern) { kern<<<g, 256, 0, s>>>(d->router_w, (const uint16_t *)x, T, D, E, ws.rt_part, ws.rt_wn); };
        static_assert(1024 % (64 * kRtSplit) == 0, "whole groups of 64 columns per slice");
        if (D == 1024) go(router_bf16x3_kernel<1024 / (64 * kRtSplit)>);
        else if (D == 2048) go(router_bf16x3_kernel<2048 / (64 * kRtSplit)>);
        else go(router_bf16x3_kernel<4096 / (64 * kRtSplit)>);
        return hipGetLastError();
    }
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

template <int PER>
static void launch_refine(const moe_layer_desc *d, const void *x, int32_t T, const RoutingPtrs &r,
                          const Workspace &ws, hipStream_t s) {
    const int D = d->n_embd;
    auto go = [&](auto kern) {
        kern<<<(T + 3) / 4, 256, 0, s>>>(d->router_w, d->router_bias, (const uint16_t *)x, ws.rt_part, ws.rt_wn, T, D,
                                         d->n_expert, d->n_expert_used, d->route_scale, r.topk_idx, r.topk_w);
    };
    if (D == 1024) go(router_refine_kernel<PER, 16>);
    else if (D == 2048) go(router_refine_kernel<PER, 32>);
    else go(router_refine_kernel<PER, 64>);
}

hipError_t launch_route_finish(const moe_layer_desc *d, const void *x, int32_t T, int32_t x_type,
                               const RoutingPtrs &r, const Workspace &ws, hipStream_t s) {
    const int E = d->n_expert, k = d->n_expert_used, P = T * k;
    if (router_split_ok(T, d->n_embd, E, x_type)) {
        if (E <= 64) launch_refine<1>(d, x, T, r, ws, s);
        else if (E <= 128) launch_refine<2>(d, x, T, r, ws, s);
        else launch_refine<4>(d, x, T, r, ws, s);
        if (P <= kMidPairs)
            bucket_mid_kernel<<<1, kMaxExperts, 0, s>>>(r.topk_idx, P, E, r.count, r.offset, r.perm, r.pos, r.active,
                                                        r.n_active);
        else
            bucket_kernel<<<1, 512, 0, s>>>(r.topk_idx, P, E, r.count, r.offset, r.perm, r.pos, r.active,
                                            r.n_active);
        return hipGetLastError();
    }
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
    return launch_route_finish(d, x, T, x_type, r, ws, s);
}

}  // namespace moe
