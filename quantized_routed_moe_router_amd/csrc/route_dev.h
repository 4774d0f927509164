// route_dev.h - device pieces of the routing ("Understanding Dwarf Star",
// 5.3.2 router(x) = softmax(x W_router) and the top-k sum; 5.3.7 step 1 and
// the sparse indexing of step 2): fp64 router logits, the wave64 top-k with
// renormalized softmax, and small-batch bucketing.
#pragma once
#include "common.h"

namespace moe {

// Sum over groups of `seg` consecutive lanes in fp64, fixed butterfly order.
MOE_DEV double seg_sum_f64(double v, int seg) {
    for (int o = seg >> 1; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

// Router logits in fp64 from W_r stored expert-major [E][D], one expert row
// per block of 4 waves (few tokens).  Wave w owns columns [w D/4, (w+1) D/4);
// lane l of it the D/256 consecutive columns from w D/4 + l D/256.  Each
// token's products are summed in fp64 in ascending column inside the lane,
// then over the lanes by a fixed butterfly, then over the 4 waves in wave
// order.  Every expert row takes the same path, so equal rows give equal
// logits.  Products of two fp32 (or bf16 and fp32) values are exact in fp64;
// only the additions round, at 2^-53 relative.  part: LDS [4][16] doubles.
template <int XT>
MOE_DEV void router_row_block(const float *__restrict__ W, const float *__restrict__ bias,
                              const void *__restrict__ xin, int T, int D, int E, double *__restrict__ logits, int e,
                              double *part) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int per = D >> 8;  // 1..16 columns per lane
    const int k0 = wave * (D >> 2) + lane * per;
    const float *wr = W + (int64_t)e * D + k0;
    float w[16];
    if ((per & 3) == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (4 * i < per) {
                const f32x4 v = *(const f32x4 *)(wr + 4 * i);
                w[4 * i] = v[0];
                w[4 * i + 1] = v[1];
                w[4 * i + 2] = v[2];
                w[4 * i + 3] = v[3];
            }
    } else {
#pragma unroll
        for (int i = 0; i < 16; ++i)
            if (i < per) w[i] = wr[i];
    }
    for (int t = 0; t < T; ++t) {
        float xv[16];
        if constexpr (XT == MOE_BF16) {
            const uint16_t *xp = (const uint16_t *)xin + (int64_t)t * D + k0;
            if ((per & 7) == 0) {
#pragma unroll
                for (int i = 0; i < 2; ++i)
                    if (8 * i < per) {
                        const u32x4 v = load_u32x4(xp + 8 * i);
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            xv[8 * i + 2 * j] = bf16_bits_to_float(v[j] & 0xFFFFu);
                            xv[8 * i + 2 * j + 1] = bf16_bits_to_float(v[j] >> 16);
                        }
                    }
            } else {
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if (i < per) xv[i] = bf16_bits_to_float(xp[i]);
            }
        } else {
            const float *xp = (const float *)xin + (int64_t)t * D + k0;
            if ((per & 3) == 0) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (4 * i < per) {
                        const f32x4 v = *(const f32x4 *)(xp + 4 * i);
                        xv[4 * i] = v[0];
                        xv[4 * i + 1] = v[1];
                        xv[4 * i + 2] = v[2];
                        xv[4 * i + 3] = v[3];
                    }
            } else {
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if (i < per) xv[i] = xp[i];
            }
        }
        double acc = 0.0;
#pragma unroll
        for (int i = 0; i < 16; ++i)
            if (i < per) acc = __builtin_fma((double)xv[i], (double)w[i], acc);
        acc = seg_sum_f64(acc, kWave);
        if (lane == 0) part[wave * 16 + t] = acc;
    }
    __syncthreads();
    if ((int)threadIdx.x < T) {
        const int t = threadIdx.x;
        const double l = ((part[t] + part[16 + t]) + part[32 + t]) + part[48 + t];
        logits[(int64_t)t * E + e] = l + (bias ? (double)bias[e] : 0.0);
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

// Cross-lane moves by DPP patterns; lanes of rows outside ROWMASK keep `old`.
// The quad permutations and row rotations stay inside a row of 16 lanes;
// row_bcast15 / row_bcast31 pass lane 15 of each row to the next row and
// lane 31 to rows 2 and 3, so no lane reads outside the wave.
template <int CTRL, int ROWMASK>
MOE_DEV int dpp_i32(int old, int v) {
    return __builtin_amdgcn_update_dpp(old, v, CTRL, ROWMASK, 0xF, false);
}
template <int CTRL, int ROWMASK>
MOE_DEV double dpp_f64(double old, double v) {
    const uint64_t o = (uint64_t)__double_as_longlong(old), b = (uint64_t)__double_as_longlong(v);
    const uint32_t lo = (uint32_t)dpp_i32<CTRL, ROWMASK>((int)(uint32_t)o, (int)(uint32_t)b);
    const uint32_t hi = (uint32_t)dpp_i32<CTRL, ROWMASK>((int)(uint32_t)(o >> 32), (int)(uint32_t)(b >> 32));
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Wave-wide maximum of a double, the same value returned to every lane:
// inside each row by xor 1, xor 2 and rotations by 4 and 8, then rows folded
// into lane 63 by the two row broadcasts.
MOE_DEV double wave_max_f64(double v) {
    const double ninf = -__builtin_inf();
    v = fmax(v, dpp_f64<0xB1, 0xF>(v, v));   // quad_perm [1,0,3,2]
    v = fmax(v, dpp_f64<0x4E, 0xF>(v, v));   // quad_perm [2,3,0,1]
    v = fmax(v, dpp_f64<0x124, 0xF>(v, v));  // row_ror 4
    v = fmax(v, dpp_f64<0x128, 0xF>(v, v));  // row_ror 8
    v = fmax(v, dpp_f64<0x142, 0xA>(ninf, v));  // row_bcast15 into rows 1, 3
    v = fmax(v, dpp_f64<0x143, 0xC>(ninf, v));  // row_bcast31 into rows 2, 3
    const uint64_t b = (uint64_t)__double_as_longlong(v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, 63);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), 63);
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Wave-wide minimum of an int, the same value returned to every lane.
MOE_DEV int wave_min_i32(int v) {
    constexpr int big = 0x7FFFFFFF;
    v = min(v, dpp_i32<0xB1, 0xF>(v, v));
    v = min(v, dpp_i32<0x4E, 0xF>(v, v));
    v = min(v, dpp_i32<0x124, 0xF>(v, v));
    v = min(v, dpp_i32<0x128, 0xF>(v, v));
    v = min(v, dpp_i32<0x142, 0xA>(big, v));
    v = min(v, dpp_i32<0x143, 0xC>(big, v));
    return __builtin_amdgcn_readlane(v, 63);
}

// One wave selects the top k of the logit row lg[0..E) (global or LDS) by
// (logit desc, index asc).  Lane l holds candidates l, l+64, ..., PER of
// them (E <= 64 PER), in registers and keeps its best untaken one.  Each of
// the k rounds takes the wave's largest logit, then the lowest index among
// the lanes offering it; only the lane that supplied the winner rescans its
// candidates.  Lane s keeps slot s; then w_s = route_scale * exp(l_s - l_0) /
// sum_j exp(l_j - l_0) in fp64, the exponentials computed by lanes 0..k-1 at
// once.  Writes idx_out[s], w_out[s] unless idx_out is null; returns the
// lane's slot expert (lanes < k).
// (select_topk_load: the same with logit(e) from a loader, e < E.)
template <int PER, class Load>
MOE_DEV int select_topk_load(Load logit, int E, int k, float route_scale, int32_t *idx_out, float *w_out) {
    const int lane = threadIdx.x & 63;
    constexpr int NONE = 0x7FFFFFFF;
    double v[PER];
    uint32_t avail = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int e = lane + 64 * i;
        v[i] = logit(min(e, E - 1));
        if (e < E) avail |= 1u << i;
    }
    double bv = -__builtin_inf();
    int be = NONE;
    auto rescan = [&]() {
        bv = -__builtin_inf();
        be = NONE;
#pragma unroll
        for (int i = 0; i < PER; ++i)
            if (((avail >> i) & 1u) && before(v[i], lane + 64 * i, bv, be)) {
                bv = v[i];
                be = lane + 64 * i;
            }
    };
    rescan();
    double my_v = 0.0;
    int my_e = 0;
    for (int s = 0; s < k; ++s) {
        const double wv = wave_max_f64(bv);
        // Usually one lane offers the maximum: take its expert by ballot;
        // only an exact tie needs the lowest index across lanes.
        const uint64_t tied = __ballot(bv == wv);
        const int we = __popcll(tied) == 1 ? __builtin_amdgcn_readlane(be, (int)__builtin_ctzll(tied))
                                           : wave_min_i32(bv == wv ? be : NONE);
        if (we == be) {  // the one lane whose candidate won
            avail &= ~(1u << ((be - lane) >> 6));
            rescan();
        }
        if (lane == s) {
            my_v = wv;
            my_e = we;
        }
    }
    if (!idx_out) return my_e;  // the selection only (uniform over the wave)
    const double mx = __shfl(my_v, 0, kWave);  // slot 0 holds the largest logit
    const double ex = lane < k ? exp(my_v - mx) : 0.0;
    double den = ex;
    for (int o = 1; o < 64; o <<= 1) den += __shfl_xor(den, o, kWave);
    if (lane < k) {
        idx_out[lane] = my_e;
        w_out[lane] = (float)((double)route_scale * ex / den);
    }
    return my_e;
}

template <int PER>
MOE_DEV int select_topk_per(const double *lg, int E, int k, float route_scale, int32_t *idx_out, float *w_out) {
    return select_topk_load<PER>([&](int e) { return lg[e]; }, E, k, route_scale, idx_out, w_out);
}

MOE_DEV int select_topk(const double *lg, int E, int k, float route_scale, int32_t *idx_out, float *w_out) {
    if (E <= 64) return select_topk_per<1>(lg, E, k, route_scale, idx_out, w_out);
    if (E <= 128) return select_topk_per<2>(lg, E, k, route_scale, idx_out, w_out);
    if (E <= 256) return select_topk_per<4>(lg, E, k, route_scale, idx_out, w_out);
    if (E <= 512) return select_topk_per<8>(lg, E, k, route_scale, idx_out, w_out);
    return select_topk_per<16>(lg, E, k, route_scale, idx_out, w_out);
}

// Bucketing of P <= 16 pairs by one wave: lane p < P holds the expert of
// pair p.  Every count, offset and slot is a count over the P pairs (the
// stable counting sort); the active list comes from ballots in expert order.
// slots (optional): records of slots [0, nslots).
// Bucketing of one token's k distinct experts by one wave (lanes < k hold
// slot s's expert ep): rank = number of selected experts below ep is the
// pair's bucket position; count and offset of every expert come from k
// comparisons each.  Same outputs as bucket_wave with P = k.
MOE_DEV void bucket_one_token(int ep, int k, int E, int32_t *__restrict__ count, int32_t *__restrict__ offset,
                              int32_t *__restrict__ perm, int32_t *__restrict__ pos, int32_t *__restrict__ active,
                              int32_t *__restrict__ n_active, SlotRec *__restrict__ slots, int nslots) {
    const int lane = threadIdx.x & 63;
    int eq[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) eq[q] = q < k ? __builtin_amdgcn_readlane(ep, q) : 0x7FFFFFFF;
    if (lane < k) {
        int rank = 0;
#pragma unroll
        for (int q = 0; q < 16; ++q) rank += eq[q] < ep;
        perm[rank] = lane;
        pos[lane] = rank;
        active[rank] = ep;
        if (slots && rank < nslots) slots[rank] = make_slot(ep, rank, 1, 0, 0);
    }
    for (int e = lane; e < E; e += 64) {
        int below = 0, hit = 0;
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            below += eq[q] < e;
            hit += eq[q] == e;
        }
        count[e] = hit;
        offset[e] = below;
        if (e >= k) active[e] = -1;
    }
    if (slots)
        for (int s = k + lane; s < nslots; s += 64) slots[s] = make_slot(-1, 0, 0, 0, 0);
    if (lane == 0) {
        n_active[0] = k;
        offset[E] = k;
    }
}

MOE_DEV void bucket_wave(int ep, int P, int E, int k, int32_t *__restrict__ count, int32_t *__restrict__ offset,
                         int32_t *__restrict__ perm, int32_t *__restrict__ pos, int32_t *__restrict__ active,
                         int32_t *__restrict__ n_active, SlotRec *__restrict__ slots, int nslots) {
    const int lane = threadIdx.x & 63;
    constexpr int NONE = 0x7FFFFFFF;  // never equal to, nor below, an expert index
    const int epv = lane < P ? ep : NONE;
    int eq[16];  // the P experts, the same in every lane, padded with NONE
#pragma unroll
    for (int q = 0; q < 16; ++q) eq[q] = __builtin_amdgcn_readlane(epv, q);
    int below = 0, rank = 0;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        below += eq[q] < ep;
        rank += (q < lane) & (eq[q] == ep);
    }
    if (lane < P) {
        perm[below + rank] = lane;
        pos[lane] = below + rank;
    }
    int base = 0;
    for (int e0 = 0; e0 < E; e0 += 64) {
        const int e = e0 + lane;
        int cnt = 0, bl = 0;
        uint64_t tlo = 0, thi = 0;  // tokens of the bucket, one byte each
        int t = 0, sl = 0;
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const bool hit = eq[q] == e;
            if (hit) {
                if (cnt < 8) tlo |= (uint64_t)t << (8 * cnt);
                else thi |= (uint64_t)t << (8 * (cnt - 8));
            }
            cnt += hit;
            bl += eq[q] < e;
            if (++sl == k) {
                sl = 0;
                ++t;
            }
        }
        const bool on = e < E && cnt > 0;
        const uint64_t act = __ballot(on);
        if (e < E) {
            count[e] = cnt;
            offset[e] = bl;
        }
        if (on) {
            const int s = base + __popcll(act & ((1ull << lane) - 1ull));
            active[s] = e;
            if (slots && s < nslots) slots[s] = make_slot(e, bl, cnt, tlo, thi);
        }
        base += __popcll(act);
    }
    for (int e = base + lane; e < E; e += 64) active[e] = -1;
    if (slots)
        for (int s = base + lane; s < nslots; s += 64) slots[s] = make_slot(-1, 0, 0, 0, 0);
    if (lane == 0) {
        n_active[0] = base;
        offset[E] = P;
    }
}

// Bucketing of P <= 256 pairs by a whole block with the pairs' experts in
// LDS: every count, offset and slot is a plain count over the P pairs.
MOE_DEV void bucket_small(const int32_t *sidx, int P, int E, int k, int32_t *__restrict__ count,
                          int32_t *__restrict__ offset, int32_t *__restrict__ perm, int32_t *__restrict__ pos,
                          int32_t *__restrict__ active, int32_t *__restrict__ n_active, SlotRec *__restrict__ slots,
                          int nslots) {
    __shared__ uint8_t isfirst[1024];
    int nf = 0;
    for (int p0 = 0; p0 < P; p0 += blockDim.x) {
        const int p = p0 + threadIdx.x;
        bool f = false;
        if (p < P) {
            const int e = sidx[p];
            f = true;
            for (int q = 0; q < p; ++q) f &= sidx[q] != e;
            isfirst[p] = f;
        }
        nf += __syncthreads_count(f);
    }
    const int na = nf;
    if (threadIdx.x == 0) {
        n_active[0] = na;
        offset[E] = P;
    }
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        int cnt = 0, below = 0, fb = 0;
        for (int p = 0; p < P; ++p) {
            const int ep = sidx[p];
            cnt += ep == e;
            below += ep < e;
            fb += (ep < e) & isfirst[p];
        }
        count[e] = cnt;
        offset[e] = below;
        if (cnt > 0) active[fb] = e;
        if (e >= na) active[e] = -1;
        if (slots && cnt > 0 && fb < nslots) {  // a bucket holds at most one entry per token, so <= 16 here
            uint64_t tlo = 0, thi = 0;
            int n = 0;
            for (int p = 0; p < P && n < 16; ++p)
                if (sidx[p] == e) {
                    const uint64_t t = (uint64_t)(p / k);
                    if (n < 8) tlo |= t << (8 * n);
                    else thi |= t << (8 * (n - 8));
                    ++n;
                }
            slots[fb] = make_slot(e, below, cnt, tlo, thi);
        }
    }
    if (slots)
        for (int s = na + threadIdx.x; s < nslots; s += blockDim.x) slots[s] = make_slot(-1, 0, 0, 0, 0);
    for (int p = threadIdx.x; p < P; p += blockDim.x) {
        const int e = sidx[p];
        int below = 0, rank = 0;
        for (int q = 0; q < P; ++q) {
            below += sidx[q] < e;
            rank += (q < p) & (sidx[q] == e);
        }
        perm[below + rank] = p;
        pos[p] = below + rank;
    }
}

// Routing of a handful of rows (T <= 16, T*k <= 256) by one block: a wave
// per token row selects its top k straight from the logits in memory, then
// the pairs are bucketed (by wave 0 alone when T = 1 and k <= 16).  slots
// (optional): the per-slot records of slots [0, nslots).
MOE_DEV void route_finish_block(const double *__restrict__ logits, int T, int E, int k, float route_scale,
                                int32_t *__restrict__ topk_idx, float *__restrict__ topk_w,
                                int32_t *__restrict__ count, int32_t *__restrict__ offset, int32_t *__restrict__ perm,
                                int32_t *__restrict__ pos, int32_t *__restrict__ active,
                                int32_t *__restrict__ n_active, SlotRec *__restrict__ slots, int nslots) {
    __shared__ int32_t sidx[256];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, nw = blockDim.x >> 6;
    const int P = T * k;
    if (T == 1 && k <= 16) {
        if (wave == 0) {
            const int my_e = select_topk(logits, E, k, route_scale, topk_idx, topk_w);
            bucket_one_token(my_e, k, E, count, offset, perm, pos, active, n_active, slots, nslots);
        }
        return;
    }
    for (int t = wave; t < T; t += nw) {
        const int my_e = select_topk(logits + (int64_t)t * E, E, k, route_scale, topk_idx + (int64_t)t * k,
                                     topk_w + (int64_t)t * k);
        if (lane < k) sidx[t * k + lane] = my_e;
    }
    __syncthreads();
    if (P <= 16) {
        if (wave == 0)
            bucket_wave(lane < P ? sidx[lane] : 0, P, E, k, count, offset, perm, pos, active, n_active, slots, nslots);
    } else {
        bucket_small(sidx, P, E, k, count, offset, perm, pos, active, n_active, slots, nslots);
    }
}

__host__ __device__ inline bool route_small_ok(int T, int E, int k) { return T <= 16 && T * k <= 256 && E >= 1; }

}  // namespace moe
