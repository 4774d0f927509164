// k_ffn_large.hip - the expert FFNs for batches beyond the decode schedule
// (any T): blockIdx.y is a slot (0 = shared expert when present, then the
// active experts in ascending id), blockIdx.x a block of 16 output rows; the
// down pass writes one row per (token, slot) pair and a gather pass combines
// them in slot order ("Understanding Dwarf Star", 5.3.7 steps 2-5).
#include <algorithm>
#include <type_traits>

#include "ffn_dev.h"

namespace moe {

constexpr int kLargeRows = 16;  // rows per block: 4 waves x 4 rows

template <int GFMT, int SFMT>
__global__ void __launch_bounds__(256) large_gateup_kernel(FfnArgs a) {
    __shared__ uint32_t cb_lds[512];
    const bool has_shared = a.Fs > 0;
    const int slot = blockIdx.y;
    const bool shared = has_shared && slot == 0;
    const int s = slot - (has_shared ? 1 : 0);
    if (!shared && s >= a.n_active[0]) return;
    const int rows = shared ? a.Fs : a.F;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int row0 = blockIdx.x * kLargeRows + wave * 4;
    if (blockIdx.x * kLargeRows >= rows) return;
    load_codebook(a.codebook, cb_lds);
    if (row0 >= rows) return;
    if (shared) shared_gateup<SFMT>(a, row0, min(4, rows - row0), cb_lds, lane);
    else routed_gateup<GFMT>(a, a.active[s], row0, min(4, rows - row0), cb_lds, lane);
}

// Q8 records of rows of n fp32 values (one wave per 64 values), for the
// shared expert's down: prepared once per call instead of in every lane of
// every wave that dots a row with them.
__global__ void __launch_bounds__(256) q8_rows_prep_kernel(const float *__restrict__ rows, int T, int n,
                                                           uint32_t *__restrict__ out) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int item = blockIdx.x * 4 + wave, per_t = n / 64;
    if (item >= T * per_t) return;  // uniform over the wave
    const int t = item / per_t, c = item % per_t;
    prep8_wave(rows[(int64_t)t * n + 64 * c + lane], out + ((int64_t)t * per_t + c) * kXQ8Dwords);
}

// The shared expert's down, rows [row0, row0 + nrows), every token, on the
// Q8 records of hs in a.xq8 ([T][Fs / 64] records).
MOE_DEV void shared_down_q8rec(const FfnArgs &a, int row0, int nrows, int lane) {
    const RowPlan rp = row_plan(a.Fs, lane);
    for (int t = 0; t < a.T; ++t) {
        XQ8 xr;
        load_q8_prep(a.xq8 + ((int64_t)t * (a.Fs / 64) + rp.c) * kXQ8Dwords, xr);
        float *dst = a.ys + (int64_t)t * a.D + row0;
        wave_rows<MOE_Q8_0, false>(a.sh_down, nullptr, a.Fs, row0, nrows, xr, nullptr, lane,
                                   [&](int r, float s, float) { dst[r] = s; });
    }
}

template <int DFMT, int SFMT>
__global__ void __launch_bounds__(256) large_down_kernel(FfnArgs a) {
    __shared__ uint32_t cb_lds[512];
    const bool has_shared = a.Fs > 0;
    const int slot = blockIdx.y;
    const bool shared = has_shared && slot == 0;
    const int s = slot - (has_shared ? 1 : 0);
    if (!shared && s >= a.n_active[0]) return;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int row0 = blockIdx.x * kLargeRows + wave * 4;
    load_codebook(a.codebook, cb_lds);
    if (row0 >= a.D) return;
    if (shared) {
        // blockIdx.z: a contiguous part of the token rows (the shared-only
        // launch spreads its rows over more blocks this way)
        const int tz = (a.T + (int)gridDim.z - 1) / (int)gridDim.z, t0 = (int)blockIdx.z * tz;
        const int tn = min(a.T - t0, tz);
        if (tn <= 0) return;
        FfnArgs b = a;
        b.T = tn;
        b.hs = a.hs + (int64_t)t0 * a.Fs;
        b.ys = a.ys + (int64_t)t0 * a.D;
        if (SFMT == MOE_Q8_0 && a.xq8) {
            b.xq8 = a.xq8 + (int64_t)t0 * (a.Fs / 64) * kXQ8Dwords;
            shared_down_q8rec(b, row0, min(4, a.D - row0), lane);
        } else {
            shared_down<SFMT>(b, row0, min(4, a.D - row0), cb_lds, lane);
        }
    }
    else routed_down<DFMT>(a, a.active[s], row0, min(4, a.D - row0), cb_lds, lane, a.ypart + row0, a.D);
}

// y[t][d] = (y if accumulating) + ys[t][d] + sum_s w[t][s] * ypart[pos[t*k+s]][d]
__global__ void __launch_bounds__(256) combine_kernel(FfnArgs a) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (int64_t)a.T * a.D) return;
    const int t = (int)(i / a.D), d = (int)(i % a.D);
    // every slot's row and weight first, then every slot's value, so that
    // the loads are in flight together; the sum is taken in slot order
    int64_t off[kMaxUsed];
    float w[kMaxUsed], v[kMaxUsed];
#pragma unroll
    for (int s = 0; s < kMaxUsed; ++s)
        if (s < a.k) {
            const int p = t * a.k + s;
            off[s] = (int64_t)a.pos[p] * a.D + d;
            w[s] = a.topk_w[p];
        }
#pragma unroll
    for (int s = 0; s < kMaxUsed; ++s)
        if (s < a.k) v[s] = a.ypart[off[s]];
    float acc = a.Fs > 0 ? a.ys[i] : 0.f;
#pragma unroll
    for (int s = 0; s < kMaxUsed; ++s)
        if (s < a.k) acc = __builtin_fmaf(w[s], v[s], acc);
    if (a.flags & MOE_ACCUMULATE) acc += a.y[i];
    a.y[i] = acc;
}

// stage 3 = gate/up, 4 = down + combine, 0 = both
hipError_t launch_ffn_large(const moe_layer_desc *d, const void *x, int32_t T, int32_t x_type, const RoutingPtrs &r,
                            float *y, uint32_t flags, const Workspace &ws, hipStream_t s, int stage) {
    FfnArgs a = make_ffn_args(d, x, T, x_type, r, y, flags, ws);
    const int max_active = (int)std::min<int64_t>((int64_t)T * a.k, d->n_expert);
    const int slots = max_active + (a.Fs > 0 ? 1 : 0);
    const int sf = a.Fs > 0 ? d->shared_type : MOE_Q8_0;
    dim3 g1((std::max(a.F, a.Fs) + kLargeRows - 1) / kLargeRows, slots);
    dim3 g2((a.D + kLargeRows - 1) / kLargeRows, slots);
    if (stage == 0 || stage == 3)
        with_fmt(d->gate_type, [&](auto G) {
            with_fmt(sf, [&](auto S) { large_gateup_kernel<decltype(G)::value, decltype(S)::value><<<g1, 256, 0, s>>>(a); });
        });
    if (stage == 0 || stage == 4) {
        with_fmt(d->down_type, [&](auto DN) {
            with_fmt(sf, [&](auto S) { large_down_kernel<decltype(DN)::value, decltype(S)::value><<<g2, 256, 0, s>>>(a); });
        });
        const int64_t n = (int64_t)T * a.D;
        combine_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(a);
    }
    return hipGetLastError();
}

// the gather of the per-pair down rows (ypart) in slot order, over the shared
// output ys when there is a shared expert
hipError_t launch_combine(const moe_layer_desc *d, const void *x, int32_t T, int32_t x_type, const RoutingPtrs &r,
                          float *y, uint32_t flags, const Workspace &ws, hipStream_t s) {
    FfnArgs a = make_ffn_args(d, x, T, x_type, r, y, flags, ws);
    const int64_t n = (int64_t)T * a.D;
    combine_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_ffn_large_shared(const moe_layer_desc *d, const void *x, int32_t T, int32_t x_type,
                                   const RoutingPtrs &r, float *y, uint32_t flags, const Workspace &ws, hipStream_t s,
                                   int stage) {
    FfnArgs a = make_ffn_args(d, x, T, x_type, r, y, flags, ws);
    if (a.Fs <= 0) return hipSuccess;
    dim3 g1((a.Fs + kLargeRows - 1) / kLargeRows, 1);
    dim3 g2((a.D + kLargeRows - 1) / kLargeRows, 1, std::min(T, 8));  // down: up to 8 parts of the rows
    const int sf = d->shared_type;
    if (stage == 3)
        with_fmt(d->gate_type, [&](auto G) {
            with_fmt(sf, [&](auto S) { large_gateup_kernel<decltype(G)::value, decltype(S)::value><<<g1, 256, 0, s>>>(a); });
        });
    if (stage == 4) {
        // a Q8_0 down takes records of hs prepared once (the workspace's x
        // records, [T][D / 64], are free again after the gate/up and hold them)
        if (sf == MOE_Q8_0 && a.Fs % 64 == 0 && a.Fs <= a.D) {
            a.xq8 = ws.xq8;
            q8_rows_prep_kernel<<<(T * (a.Fs / 64) + 3) / 4, 256, 0, s>>>(ws.hs, T, a.Fs, ws.xq8);
        }
        with_fmt(d->down_type, [&](auto DN) {
            with_fmt(sf, [&](auto S) { large_down_kernel<decltype(DN)::value, decltype(S)::value><<<g2, 256, 0, s>>>(a); });
        });
    }
    return hipGetLastError();
}

}  // namespace moe
