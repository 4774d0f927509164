// k_decode.hip - the block for a handful of token rows (decode, micro-batched
// decode) in four dependent kernels, each pairing latency-bound routing work
// with bandwidth-bound expert work ("Understanding Dwarf Star", 5.3.7 steps
// 1-5; 5.3.4 the shared expert runs alongside the routed ones; 3.5 a
// schedule built once and replayed per token):
//   K1  router logits (a wave per expert row) + x prepared for the dot2 path
//   K2  top-k, weights, bucketing (block 0)  || shared expert gate/up -> hs
//   K3  routed gate/up + SwiGLU (4 waves x 4 rows of one active expert per
//       block; writes h and its prepared form) || shared expert down -> ys
//   K4  routed down, then y = ys + sum_s w_s * down_s in slot order
//       (block = 4 output rows x every active expert, combined in LDS)
// No routing result ever travels back to the host: K3/K4 read n_active and
// the active list from device memory and idle blocks return at once.
#include <algorithm>
#include <type_traits>

#include "ffn_dev.h"
#include "route_dev.h"

namespace moe {

constexpr int kGatherRows = 4;    // output rows per K4 block
constexpr int kGatherWaves = 8;   // waves per K4 block, one active expert each at a time
constexpr int kMaxGatherPairs = 1024;

template <int XT>
__global__ void __launch_bounds__(256) dec_k1_kernel(FfnArgs a) {
    int b = blockIdx.x;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    if (b < a.n_router_blocks) {
        router_rows_wave<XT>(a.router_w, a.router_bias, a.x, a.T, a.D, a.E, a.logits, b * 4 + wave);
        return;
    }
    b -= a.n_router_blocks;
    const int item = b * 4 + wave, per_t = a.D / 64;  // x prepared for the routed Q2K gate/up
    if (item < a.T * per_t) {
        const int t = item / per_t, c = item % per_t;
        const float v = XT == MOE_BF16 ? bf16_bits_to_float(((const uint16_t *)a.x)[(int64_t)t * a.D + 64 * c + lane])
                                       : ((const float *)a.x)[(int64_t)t * a.D + 64 * c + lane];
        prep16_wave(v, a.xp16 + ((int64_t)t * (a.D / 16) + 4 * c) * kP16Dwords);
    }
}

template <int SFMT>
__global__ void __launch_bounds__(256) dec_k2_kernel(FfnArgs a, int do_route) {
    __shared__ uint32_t cb_lds[512];
    int b = blockIdx.x;
    if (do_route) {
        if (b == 0) {
            route_finish_small(a.logits, a.T, a.E, a.k, a.route_scale, a.w_topk_idx, a.w_topk_w, a.w_count,
                               a.w_offset, a.w_perm, a.w_pos, a.w_active, a.w_n_active);
            return;
        }
        b -= 1;
    }
    load_codebook(SFMT == MOE_CB2 ? a.codebook : nullptr, cb_lds);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int rpw = 4096 / a.D;  // rows per wave: one wave iteration
    const int row0 = (b * 4 + wave) * rpw;
    if (row0 >= a.Fs) return;
    shared_gateup<SFMT>(a, row0, min(rpw, a.Fs - row0), cb_lds, lane);
}

// blocks [0, n_slot_blocks): 16 rows of one active expert; then shared down
template <int GFMT, int SFMT>
__global__ void __launch_bounds__(256) dec_k3_kernel(FfnArgs a) {
    __shared__ uint32_t cb_lds[512];
    __shared__ float tile[16];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    int b = blockIdx.x;
    if (b < a.n_slot_blocks) {
        const int nrb = a.F / 16, slot = b / nrb, rb = b % nrb;
        if (slot >= a.n_active[0]) return;
        load_codebook(GFMT == MOE_CB2 ? a.codebook : nullptr, cb_lds);
        const int row0 = rb * 16 + wave * 4;  // F is a multiple of 64: every wave has its 4 rows
        routed_gateup<GFMT, GFMT == MOE_Q2K>(a, a.active[slot], row0, 4, cb_lds, lane, a.hp16 ? tile : nullptr,
                                             rb * 16);
        return;
    }
    b -= a.n_slot_blocks;
    load_codebook(SFMT == MOE_CB2 ? a.codebook : nullptr, cb_lds);
    const int rpw = 4096 / a.Fs;
    const int row0 = (b * 4 + wave) * rpw;
    if (row0 >= a.D) return;
    shared_down<SFMT>(a, row0, min(rpw, a.D - row0), cb_lds, lane);
}

template <int DFMT>
__global__ void __launch_bounds__(64 * kGatherWaves) dec_k4_kernel(FfnArgs a) {
    __shared__ uint32_t cb_lds[512];
    __shared__ float part[kMaxGatherPairs * kGatherRows];
    load_codebook(DFMT == MOE_CB2 ? a.codebook : nullptr, cb_lds);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int row0 = blockIdx.x * kGatherRows;
    const int nrows = min(kGatherRows, a.D - row0);
    const int na = a.n_active[0];
    for (int s = wave; s < na; s += kGatherWaves)
        routed_down<DFMT, DFMT == MOE_Q2K>(a, a.active[s], row0, nrows, cb_lds, lane, part, kGatherRows);
    __syncthreads();
    for (int i = threadIdx.x; i < a.T * nrows; i += blockDim.x) {
        const int t = i / nrows, r = i % nrows;
        const int64_t o = (int64_t)t * a.D + row0 + r;
        float acc = a.Fs > 0 ? a.ys[o] : 0.f;
        for (int s = 0; s < a.k; ++s) {
            const int p = t * a.k + s;
            acc = __builtin_fmaf(a.topk_w[p], part[a.pos[p] * kGatherRows + r], acc);
        }
        if (a.flags & MOE_ACCUMULATE) acc += a.y[o];
        a.y[o] = acc;
    }
}

FfnArgs make_ffn_args(const moe_layer_desc *d, const void *x, int32_t T, int32_t x_type, const RoutingPtrs &r,
                      float *y, uint32_t flags, const Workspace &ws) {
    FfnArgs a{};
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
    a.E = d->n_expert;
    a.gu_expert_bytes = fmt_bytes(d->gate_type, (int64_t)a.F * a.D);
    a.down_expert_bytes = fmt_bytes(d->down_type, (int64_t)a.F * a.D);
    a.topk_idx = a.w_topk_idx = r.topk_idx;
    a.topk_w = a.w_topk_w = r.topk_w;
    a.count = a.w_count = r.count;
    a.offset = a.w_offset = r.offset;
    a.perm = a.w_perm = r.perm;
    a.pos = a.w_pos = r.pos;
    a.active = a.w_active = r.active;
    a.n_active = a.w_n_active = r.n_active;
    a.h = ws.h;
    a.hs = ws.hs;
    a.ypart = ws.ypart;
    a.ys = ws.ys;
    a.y = y;
    a.flags = flags;
    a.router_w = d->router_w;
    a.router_bias = d->router_bias;
    a.route_scale = d->route_scale;
    a.logits = ws.logits;
    a.xp16 = nullptr;
    a.hp16 = nullptr;
    return a;
}

bool small_path_ok(const moe_layer_desc *d, int32_t T) {
    return T <= 16 && (int64_t)T * d->n_expert_used <= kMaxGatherPairs;
}

bool small_route_ok(const moe_layer_desc *d, int32_t T) { return route_small_ok(T, d->n_expert, d->n_expert_used); }

// stage 0 = all; 1..4 = K1..K4.  route: also compute the routing (K1's router
// waves and K2's block 0); otherwise the routing in r is given.
hipError_t launch_small(const moe_layer_desc *d, const void *x, int32_t T, int32_t x_type, const RoutingPtrs &r,
                        float *y, uint32_t flags, const Workspace &ws, hipStream_t s, int stage, bool route) {
    FfnArgs a = make_ffn_args(d, x, T, x_type, r, y, flags, ws);
    const int sf = a.Fs > 0 ? d->shared_type : MOE_Q8_0;
    a.n_router_blocks = route ? (a.E + 4 * (4096 / a.D) - 1) / (4 * (4096 / a.D)) : 0;
    int prep_blocks = 0;
    if (d->gate_type == MOE_Q2K) {  // x prepared once per token for the routed gate/up
        a.xp16 = ws.xp16;
        prep_blocks = (T * (a.D / 64) + 3) / 4;
    }
    if (d->down_type == MOE_Q2K) a.hp16 = ws.hp16;  // h prepared by K3 for the routed down
    const int max_slots = (int)std::min<int64_t>((int64_t)T * a.k, a.E);
    a.n_slot_blocks = max_slots * (a.F / 16);
    const int sh_gu_blocks = a.Fs > 0 ? (a.Fs + 4 * (4096 / a.D) - 1) / (4 * (4096 / a.D)) : 0;
    const int sh_dn_blocks = a.Fs > 0 ? (a.D + 4 * (4096 / a.Fs) - 1) / (4 * (4096 / a.Fs)) : 0;
    const int k1 = a.n_router_blocks + prep_blocks, k2 = (route ? 1 : 0) + sh_gu_blocks;
    if ((stage == 0 || stage == 1) && k1 > 0) {
        if (x_type == MOE_BF16) dec_k1_kernel<MOE_BF16><<<k1, 256, 0, s>>>(a);
        else dec_k1_kernel<MOE_F32><<<k1, 256, 0, s>>>(a);
    }
    if ((stage == 0 || stage == 2) && k2 > 0)
        with_fmt(sf, [&](auto S) { dec_k2_kernel<decltype(S)::value><<<k2, 256, 0, s>>>(a, route ? 1 : 0); });
    if (stage == 0 || stage == 3)
        with_fmt(d->gate_type, [&](auto G) {
            with_fmt(sf, [&](auto S) {
                dec_k3_kernel<decltype(G)::value, decltype(S)::value><<<a.n_slot_blocks + sh_dn_blocks, 256, 0, s>>>(a);
            });
        });
    if (stage == 0 || stage == 4)
        with_fmt(d->down_type, [&](auto DN) {
            dec_k4_kernel<decltype(DN)::value><<<(a.D + kGatherRows - 1) / kGatherRows, 64 * kGatherWaves, 0, s>>>(a);
        });
    return hipGetLastError();
}

}  // namespace moe
