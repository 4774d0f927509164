// k_ffn_decode.hip - the expert FFNs for a handful of token rows: grouped
// dequant-GEMV over the active experts' 2-bit blocks with the SwiGLU fused
// into the gate/up pass, the down pass, and the gather combine
// ("Understanding Dwarf Star", 2.8.2 fused dequant-dot; 5.3.7 steps 2-5;
// 5.3.4 the shared expert, always on).
//
// Work split: blockIdx.y is a slot (0 = shared expert when present, then the
// active experts in ascending id), blockIdx.x a block of 16 output rows.  A
// lane owns 64 consecutive weights of a row (one 16-byte load of 2-bit codes
// plus its scales); the lanes of a row are combined with a butterfly.  The
// grid is sized for the largest possible number of active experts; blocks
// whose slot is not active return at once, so no routing data ever comes back
// to the host.
#include <algorithm>
#include <type_traits>

#include "common.h"

namespace moe {

constexpr int kRowsPerBlock = 16;

struct FfnArgs {
    const uint8_t *gate, *up, *down, *sh_gate, *sh_up, *sh_down;
    const int8_t *codebook;
    const void *x;
    int x_bf16;
    int T, D, F, Fs, k;
    int64_t gu_expert_bytes, down_expert_bytes;
    const int32_t *topk_idx;
    const float *topk_w;
    const int32_t *count, *offset, *perm, *pos, *active, *n_active;
    float *h, *hs, *ypart, *ys, *y;
    uint32_t flags;
};

// Which rows/tokens/matrices a block works on.
struct SlotView {
    bool shared;
    int rows;         // output rows of this matrix set
    int ntok;         // tokens in the bucket
    int j0;           // first bucket position (routed) or 0 (shared)
    const uint8_t *m0, *m1;
};

MOE_DEV bool slot_view(const FfnArgs &a, bool gateup, SlotView &v) {
    int slot = blockIdx.y;
    bool has_shared = a.Fs > 0;
    if (has_shared && slot == 0) {
        v.shared = true;
        v.rows = gateup ? a.Fs : a.D;
        v.ntok = a.T;
        v.j0 = 0;
        v.m0 = gateup ? a.sh_gate : a.sh_down;
        v.m1 = gateup ? a.sh_up : nullptr;
        return true;
    }
    int s = slot - (has_shared ? 1 : 0);
    if (s >= a.n_active[0]) return false;
    int e = a.active[s];
    v.shared = false;
    v.rows = gateup ? a.F : a.D;
    v.ntok = a.count[e];
    v.j0 = a.offset[e];
    v.m0 = gateup ? a.gate + (int64_t)e * a.gu_expert_bytes : a.down + (int64_t)e * a.down_expert_bytes;
    v.m1 = gateup ? a.up + (int64_t)e * a.gu_expert_bytes : nullptr;
    return true;
}

// Load the lane's 64 activations starting at column c0 of a row of x (fp32 or bf16).
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
    if (cb) {
        for (int i = threadIdx.x; i < 512; i += blockDim.x) cb_lds[i] = ((const uint32_t *)cb)[i];
    }
    __syncthreads();
}

// gate/up pass: h[j][f] = silu(W_gate[f] . x_j) * (W_up[f] . x_j)
template <int GFMT, int SFMT>
__global__ void __launch_bounds__(256) gateup_gemv_kernel(FfnArgs a) {
    __shared__ uint32_t cb_lds[512];
    SlotView v;
    if (!slot_view(a, true, v)) return;
    int row0 = blockIdx.x * kRowsPerBlock;
    if (row0 >= v.rows) return;
    load_codebook(a.codebook, cb_lds);
    const int n_in = a.D;
    const int cpr = n_in >> 6;              // 64-weight chunks per row (<= 64)
    const int rpi = 64 / cpr;               // rows per wave iteration
    int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int lr = lane / cpr, c = lane % cpr;
    int nrows = min(kRowsPerBlock, v.rows - row0);
    const int Fo = v.shared ? a.Fs : a.F;
    for (int j = 0; j < v.ntok; ++j) {
        int t = v.shared ? j : a.perm[v.j0 + j] / a.k;
        float xr[64];
        load_x64(a.x, a.x_bf16, (int64_t)t * n_in + 64 * c, xr);
        for (int it = wave; it * rpi < nrows; it += 4) {
            int r = it * rpi + lr;
            bool ok = r < nrows;
            int64_t row = row0 + (ok ? r : 0);
            int64_t i0 = row * n_in + 64 * c;
            float g, u;
            if (v.shared) {
                g = chunk_dot<SFMT>(v.m0, i0, xr, cb_lds);
                u = chunk_dot<SFMT>(v.m1, i0, xr, cb_lds);
            } else {
                g = chunk_dot<GFMT>(v.m0, i0, xr, cb_lds);
                u = chunk_dot<GFMT>(v.m1, i0, xr, cb_lds);
            }
            g = seg_sum(g, cpr);
            u = seg_sum(u, cpr);
            if (ok && c == 0) {
                float hv = silu(g) * u;
                if (a.x_bf16) hv = bf16_bits_to_float(float_to_bf16_bits(hv));
                float *dst = v.shared ? a.hs + (int64_t)j * Fo : a.h + (int64_t)(v.j0 + j) * Fo;
                dst[row] = hv;
            }
        }
    }
}

// down pass: ypart[j][d] = W_down[d] . h_j (routed) or ys[t][d] (shared)
template <int DFMT, int SFMT>
__global__ void __launch_bounds__(256) down_gemv_kernel(FfnArgs a) {
    __shared__ uint32_t cb_lds[512];
    SlotView v;
    if (!slot_view(a, false, v)) return;
    int row0 = blockIdx.x * kRowsPerBlock;
    if (row0 >= v.rows) return;
    load_codebook(a.codebook, cb_lds);
    const int n_in = v.shared ? a.Fs : a.F;
    const int cpr = n_in >> 6;
    const int rpi = 64 / cpr;
    int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int lr = lane / cpr, c = lane % cpr;
    int nrows = min(kRowsPerBlock, v.rows - row0);
    for (int j = 0; j < v.ntok; ++j) {
        const float *hv = v.shared ? a.hs + (int64_t)j * n_in : a.h + (int64_t)(v.j0 + j) * n_in;
        float xr[64];
        load_x64(hv, 0, 64 * c, xr);
        for (int it = wave; it * rpi < nrows; it += 4) {
            int r = it * rpi + lr;
            bool ok = r < nrows;
            int64_t row = row0 + (ok ? r : 0);
            int64_t i0 = row * n_in + 64 * c;
            float s = v.shared ? chunk_dot<SFMT>(v.m0, i0, xr, cb_lds) : chunk_dot<DFMT>(v.m0, i0, xr, cb_lds);
            s = seg_sum(s, cpr);
            if (ok && c == 0) {
                float *dst = v.shared ? a.ys + (int64_t)j * a.D : a.ypart + (int64_t)(v.j0 + j) * a.D;
                dst[row] = s;
            }
        }
    }
}

// y[t][d] = (y[t][d] if accumulating) + ys[t][d] + sum_s w[t][s] * ypart[pos[t*k+s]][d]
__global__ void __launch_bounds__(256) combine_kernel(FfnArgs a) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (int64_t)a.T * a.D) return;
    int t = (int)(i / a.D), d = (int)(i % a.D);
    float acc = a.Fs > 0 ? a.ys[i] : 0.f;
    for (int s = 0; s < a.k; ++s) {
        int p = t * a.k + s;
        acc = __builtin_fmaf(a.topk_w[p], a.ypart[(int64_t)a.pos[p] * a.D + d], acc);
    }
    if (a.flags & MOE_ACCUMULATE) acc += a.y[i];
    a.y[i] = acc;
}

template <int GFMT, int SFMT>
static void launch_gateup(dim3 g, const FfnArgs &a, hipStream_t s) {
    gateup_gemv_kernel<GFMT, SFMT><<<g, 256, 0, s>>>(a);
}

template <int DFMT, int SFMT>
static void launch_down(dim3 g, const FfnArgs &a, hipStream_t s) {
    down_gemv_kernel<DFMT, SFMT><<<g, 256, 0, s>>>(a);
}

// Calls fn with std::integral_constant<int, format> for a runtime format.
template <typename Fn>
static void with_fmt(int f, Fn &&fn) {
    if (f == MOE_Q2K) fn(std::integral_constant<int, MOE_Q2K>{});
    else if (f == MOE_Q8_0) fn(std::integral_constant<int, MOE_Q8_0>{});
    else fn(std::integral_constant<int, MOE_CB2>{});
}

hipError_t launch_ffn_decode(const moe_layer_desc *d, const void *x, int32_t T, int32_t x_type,
                             const RoutingPtrs &r, float *y, uint32_t flags, const Workspace &ws, hipStream_t s) {
    FfnArgs a;
    a.gate = (const uint8_t *)d->gate;
    a.up = (const uint8_t *)d->up;
    a.down = (const uint8_t *)d->down;
    a.sh_gate = (const uint8_t *)d->sh_gate;
    a.sh_up = (const uint8_t *)d->sh_up;
    a.sh_down = (const uint8_t *)d->sh_down;
    a.codebook = d->codebook;
    a.x = x;
    a.x_bf16 = x_type == MOE_BF16;
    a.T = T;
    a.D = d->n_embd;
    a.F = d->n_ff_exp;
    a.Fs = d->n_ff_shared;
    a.k = d->n_expert_used;
    a.gu_expert_bytes = fmt_bytes(d->gate_type, (int64_t)a.F * a.D);
    a.down_expert_bytes = fmt_bytes(d->down_type, (int64_t)a.F * a.D);
    a.topk_idx = r.topk_idx;
    a.topk_w = r.topk_w;
    a.count = r.count;
    a.offset = r.offset;
    a.perm = r.perm;
    a.pos = r.pos;
    a.active = r.active;
    a.n_active = r.n_active;
    a.h = ws.h;
    a.hs = ws.hs;
    a.ypart = ws.ypart;
    a.ys = ws.ys;
    a.y = y;
    a.flags = flags;
    int max_active = (int)std::min<int64_t>((int64_t)T * a.k, d->n_expert);
    int slots = max_active + (a.Fs > 0 ? 1 : 0);
    int gu_rows = std::max(a.F, a.Fs), dn_rows = a.D;
    dim3 g1((gu_rows + kRowsPerBlock - 1) / kRowsPerBlock, slots);
    dim3 g2((dn_rows + kRowsPerBlock - 1) / kRowsPerBlock, slots);
    int sf = a.Fs > 0 ? d->shared_type : MOE_Q8_0;
    with_fmt(d->gate_type, [&](auto G) {
        with_fmt(sf, [&](auto S) { launch_gateup<decltype(G)::value, decltype(S)::value>(g1, a, s); });
    });
    with_fmt(d->down_type, [&](auto DN) {
        with_fmt(sf, [&](auto S) { launch_down<decltype(DN)::value, decltype(S)::value>(g2, a, s); });
    });
    int64_t n = (int64_t)T * a.D;
    combine_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace moe
