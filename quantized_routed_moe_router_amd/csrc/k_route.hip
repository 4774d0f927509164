// k_route.hip - routing kernels for moe_route and for batches too large for
// the one-block finisher ("Understanding Dwarf Star", 5.3.2 router and top-k;
// 5.3.7 step 1 and the sparse indexing of step 2).
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

// One wave per token: top-k of its logit row.
__global__ void __launch_bounds__(256) router_topk_kernel(const double *__restrict__ logits, int T, int E, int k,
                                                          float route_scale, int32_t *__restrict__ topk_idx,
                                                          float *__restrict__ topk_w) {
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    select_topk(logits + (int64_t)t * E, E, k, route_scale, topk_idx + (int64_t)t * k, topk_w + (int64_t)t * k);
}

__global__ void __launch_bounds__(1024) bucket_small_kernel(const int32_t *__restrict__ topk_idx, int P, int E,
                                                            int32_t *__restrict__ count, int32_t *__restrict__ offset,
                                                            int32_t *__restrict__ perm, int32_t *__restrict__ pos,
                                                            int32_t *__restrict__ active,
                                                            int32_t *__restrict__ n_active) {
    __shared__ int32_t sidx[1024];
    for (int p = threadIdx.x; p < P; p += blockDim.x) sidx[p] = topk_idx[p];
    __syncthreads();
    bucket_small(sidx, P, E, 1, count, offset, perm, pos, active, n_active, nullptr, 0);
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
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    for (int i = tid; i < kBucketWaves * kMaxExperts; i += blockDim.x) (&wc[0][0])[i] = 0;
    __syncthreads();
    const int seg = ((P + kBucketWaves - 1) / kBucketWaves + 63) / 64 * 64;
    const int s0 = w * seg, s1 = min(P, s0 + seg);
    for (int p = s0 + lane; p < s1; p += 64) atomicAdd(&wc[w][topk_idx[p]], 1);
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
    for (int o = 1; o < kMaxExperts; o <<= 1) {  // inclusive scan over experts
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
        int key = valid ? topk_idx[p] : 0;
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
    for (int o = 1; o < kMaxExperts; o <<= 1) {
        int a0 = tid, a1 = tid + 512;
        int v0 = scan_tmp[a0] + (a0 >= o ? scan_tmp[a0 - o] : 0);
        int v1 = scan_tmp[a1] + (a1 >= o ? scan_tmp[a1 - o] : 0);
        __syncthreads();
        scan_tmp[a0] = v0;
        scan_tmp[a1] = v1;
        __syncthreads();
    }
    const int na = scan_tmp[kMaxExperts - 1];
    for (int e = tid; e < E; e += blockDim.x) active[e] = -1;
    __syncthreads();
    for (int e = tid; e < E; e += blockDim.x)
        if (tot[e] > 0) active[scan_tmp[e] - 1] = e;
    if (tid == 0) n_active[0] = na;
}

// one block per expert row for few tokens, 16 x 16 tiles for many
bool router_rows_ok(int T) { return T <= 16; }

hipError_t launch_router_logits(const moe_layer_desc *d, const void *x, int32_t T, int32_t x_type,
                                const Workspace &ws, hipStream_t s) {
    const int D = d->n_embd, E = d->n_expert;
    if (router_rows_ok(T)) {
        if (x_type == MOE_BF16)
            router_row_kernel<MOE_BF16><<<E, 256, 0, s>>>(d->router_w, d->router_bias, x, T, D, E, ws.logits);
        else
            router_row_kernel<MOE_F32><<<E, 256, 0, s>>>(d->router_w, d->router_bias, x, T, D, E, ws.logits);
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
    router_topk_kernel<<<(T + 3) / 4, 256, 0, s>>>(ws.logits, T, E, k, d->route_scale, r.topk_idx, r.topk_w);
    if (P <= 1024)
        bucket_small_kernel<<<1, 1024, 0, s>>>(r.topk_idx, P, E, r.count, r.offset, r.perm, r.pos, r.active,
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
