// k_route.hip - router logits, top-k with renormalized softmax, and the
// stable token-to-expert bucketing ("Understanding Dwarf Star", 5.3.2 router
// and top-k formula; 5.3.7 step 1 and the sparse indexing of step 2).
#include "common.h"

namespace moe {

// Partial router logits in fp64.  Block (chunk c, token tile, expert group):
// rows k in [c*kc, (c+1)*kc) of W_r [D][E] against up to 32 tokens; thread
// e of the group holds one expert's partial sums.  Products of two fp32 (or
// bf16 and fp32) values are exact in fp64, so only the additions round, at
// 2^-53 relative.
constexpr int kRouterKS = 64;

template <int XT>
__global__ void __launch_bounds__(256) router_partial_kernel(const float *__restrict__ W, const void *__restrict__ xin,
                                                             int T, int D, int E, int kc, int tt,
                                                             double *__restrict__ partial) {
    __shared__ double xs[32 * kRouterKS];  // [nt][ks]
    int c = blockIdx.x, t0 = blockIdx.y * tt;
    int nt = min(tt, T - t0);
    int k0 = c * kc;
    int e = blockIdx.z * 256 + threadIdx.x;
    double acc[32];
#pragma unroll
    for (int j = 0; j < 32; ++j) acc[j] = 0.0;
    int ks = min(kc, kRouterKS);
    for (int kb = 0; kb < kc; kb += ks) {
        __syncthreads();
        for (int i = threadIdx.x; i < nt * ks; i += blockDim.x) {
            int tl = i / ks, kk = i % ks;
            int64_t gi = (int64_t)(t0 + tl) * D + k0 + kb + kk;
            double v;
            if constexpr (XT == MOE_BF16) v = (double)bf16_bits_to_float(((const uint16_t *)xin)[gi]);
            else v = (double)((const float *)xin)[gi];
            xs[tl * ks + kk] = v;
        }
        __syncthreads();
        if (e < E) {
            const float *wp = W + (int64_t)(k0 + kb) * E + e;
            for (int kk = 0; kk < ks; ++kk) {
                double w = (double)wp[(int64_t)kk * E];
#pragma unroll
                for (int j = 0; j < 32; ++j)
                    if (j < nt) acc[j] = __builtin_fma(xs[j * ks + kk], w, acc[j]);
            }
        }
    }
    if (e < E)
        for (int j = 0; j < nt; ++j) partial[((int64_t)c * T + t0 + j) * E + e] = acc[j];
}

// a ranks before b: larger logit, then lower expert index
MOE_DEV bool before(double va, int ea, double vb, int eb) { return va > vb || (va == vb && ea < eb); }

// One wave per token: sum the chunk partials in fixed order (+ bias), select
// the top k by (logit desc, index asc) with k wave-wide arg-max rounds, then
// weights = route_scale * exp(l_s - l_0) / sum_j exp(l_j - l_0) in fp64.
__global__ void __launch_bounds__(256) router_topk_kernel(const double *__restrict__ partial,
                                                          const float *__restrict__ bias, int T, int E, int nchunk,
                                                          int k, float route_scale, int32_t *__restrict__ topk_idx,
                                                          float *__restrict__ topk_w) {
    int lane = threadIdx.x & 63;
    int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    constexpr int PER = kMaxExperts / kWave;  // 16 experts per lane at most
    double v[PER];
    uint32_t taken = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        int e = lane + 64 * i;
        double s = 0.0;
        if (e < E) {
            for (int c = 0; c < nchunk; ++c) s += partial[((int64_t)c * T + t) * E + e];
            if (bias) s += (double)bias[e];
        } else {
            taken |= 1u << i;
        }
        v[i] = s;
    }
    double sel_v[kMaxUsed];
    int sel_e[kMaxUsed];
    for (int s = 0; s < k; ++s) {
        // lane-local best among not-yet-taken experts
        double bv = 0.0;
        int be = 0x7FFFFFFF, bi = -1;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            int e = lane + 64 * i;
            if (!((taken >> i) & 1u) && (bi < 0 || before(v[i], e, bv, be))) {
                bv = v[i];
                be = e;
                bi = i;
            }
        }
        // wave arg-max (lanes without a candidate carry e = INT_MAX, never chosen over a real one)
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
        sel_v[s] = wv;
        sel_e[s] = we;
        if (have && we == be && bi >= 0) taken |= 1u << bi;
    }
    if (lane == 0) {
        double mx = sel_v[0], den = 0.0, ex[kMaxUsed];
        for (int s = 0; s < k; ++s) {
            ex[s] = exp(sel_v[s] - mx);
            den += ex[s];
        }
        for (int s = 0; s < k; ++s) {
            topk_idx[(int64_t)t * k + s] = sel_e[s];
            topk_w[(int64_t)t * k + s] = (float)((double)route_scale * ex[s] / den);
        }
    }
}

// Stable counting sort of the P = T*k pairs by expert, one block of 8 waves.
// Wave w owns a contiguous segment of pair ids.  Pass 1 counts per (wave,
// expert); a scan over waves then experts gives each wave's first slot per
// expert; pass 2 walks the segment 64 pairs at a time and ranks equal experts
// inside the wave with ballots, so the result is a pure function of topk_idx.
constexpr int kBucketWaves = 8;

__global__ void __launch_bounds__(512) bucket_kernel(const int32_t *__restrict__ topk_idx, int P, int E,
                                                     int32_t *__restrict__ count, int32_t *__restrict__ offset,
                                                     int32_t *__restrict__ perm, int32_t *__restrict__ pos,
                                                     int32_t *__restrict__ active, int32_t *__restrict__ n_active) {
    __shared__ int32_t wc[kBucketWaves][kMaxExperts];
    __shared__ int32_t tot[kMaxExperts];
    __shared__ int32_t scan_tmp[kMaxExperts];
    int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    for (int i = tid; i < kBucketWaves * kMaxExperts; i += blockDim.x) (&wc[0][0])[i] = 0;
    __syncthreads();
    int seg = ((P + kBucketWaves - 1) / kBucketWaves + 63) / 64 * 64;
    int s0 = w * seg, s1 = min(P, s0 + seg);
    for (int p = s0 + lane; p < s1; p += 64) atomicAdd(&wc[w][topk_idx[p]], 1);
    __syncthreads();
    // per expert: exclusive prefix over waves, total
    for (int e = tid; e < E; e += blockDim.x) {
        int run = 0;
        for (int ww = 0; ww < kBucketWaves; ++ww) {
            int c = wc[ww][e];
            wc[ww][e] = run;
            run += c;
        }
        tot[e] = run;
    }
    __syncthreads();
    // exclusive scan of tot over experts (Hillis-Steele on up to 1024 entries, 2 per thread)
    for (int e = tid; e < kMaxExperts; e += blockDim.x) scan_tmp[e] = e < E ? tot[e] : 0;
    __syncthreads();
    for (int o = 1; o < kMaxExperts; o <<= 1) {
        int a0 = tid, a1 = tid + 512;
        int v0 = scan_tmp[a0] + (a0 >= o ? scan_tmp[a0 - o] : 0);
        int v1 = scan_tmp[a1] + (a1 >= o ? scan_tmp[a1 - o] : 0);
        __syncthreads();
        scan_tmp[a0] = v0;
        scan_tmp[a1] = v1;
        __syncthreads();
    }
    // scan_tmp now inclusive
    for (int e = tid; e < E; e += blockDim.x) {
        int excl = scan_tmp[e] - tot[e];
        count[e] = tot[e];
        offset[e] = excl;
        for (int ww = 0; ww < kBucketWaves; ++ww) wc[ww][e] += excl;
    }
    if (tid == 0) offset[E] = scan_tmp[E - 1];
    __syncthreads();
    // pass 2: stable scatter
    int nbits = 32 - __clz(max(E - 1, 1));
    for (int base = s0; base < s1; base += 64) {
        int p = base + lane;
        bool valid = p < s1;
        int key = valid ? topk_idx[p] : 0;
        uint64_t same = __ballot(valid);
        for (int b = 0; b < nbits; ++b) {
            uint64_t bal = __ballot(valid && ((key >> b) & 1));
            same &= ((key >> b) & 1) ? bal : ~bal;
        }
        uint64_t below = same & ((1ull << lane) - 1ull);
        int rank = __popcll(below);
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
    // active experts, ascending: scan of (count > 0)
    for (int e = tid; e < kMaxExperts; e += blockDim.x) scan_tmp[e] = (e < E && tot[e] > 0) ? 1 : 0;
    __syncthreads();
    for (int o = 1; o < kMaxExperts; o <<= 1) {
        int a0 = tid, a1 = tid + 512;
        int v0 = scan_tmp[a0] + (a0 >= o ? scan_tmp[a0 - o] : 0);
        int v1 = scan_tmp[a1] + (a1 >= o ? scan_tmp[a1 - o] : 0);
        __syncthreads();
        scan_tmp[a0] = v0;
        scan_tmp[a1] = v1;
        __syncthreads();
    }
    int na = scan_tmp[kMaxExperts - 1];
    for (int e = tid; e < E; e += blockDim.x) {
        active[e] = -1;
    }
    __syncthreads();
    for (int e = tid; e < E; e += blockDim.x)
        if (tot[e] > 0) active[scan_tmp[e] - 1] = e;
    if (tid == 0) n_active[0] = na;
}

hipError_t launch_route(const moe_layer_desc *d, const void *x, int32_t T, int32_t x_type, const RoutingPtrs &r,
                        const Workspace &ws, hipStream_t s) {
    int D = d->n_embd, E = d->n_expert, k = d->n_expert_used;
    RouterPlan rp = router_plan(T, D);
    dim3 g1(rp.nchunk, (T + rp.tt - 1) / rp.tt, (E + 255) / 256);
    if (x_type == MOE_BF16)
        router_partial_kernel<MOE_BF16><<<g1, 256, 0, s>>>(d->router_w, x, T, D, E, rp.kc, rp.tt, ws.partial);
    else
        router_partial_kernel<MOE_F32><<<g1, 256, 0, s>>>(d->router_w, x, T, D, E, rp.kc, rp.tt, ws.partial);
    router_topk_kernel<<<(T + 3) / 4, 256, 0, s>>>(ws.partial, d->router_bias, T, E, rp.nchunk, k,
                                                   d->route_scale, r.topk_idx, r.topk_w);
    bucket_kernel<<<1, 512, 0, s>>>(r.topk_idx, T * k, E, r.count, r.offset, r.perm, r.pos, r.active, r.n_active);
    return hipGetLastError();
}

}  // namespace moe
