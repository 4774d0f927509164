// api.hip - the C ABI declared in include/moe.h: argument validation (all of
// it before anything is enqueued), workspace sizing, and the launches.
#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <mutex>

#include "common.h"

using namespace moe;

// The static scratch of moe_layer_forward_noalloc (see below).
constexpr size_t kScratchBytes = (size_t)8 << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

int fail(char *err, size_t errlen, int code, const char *fmt, ...) {
    if (err && errlen) {
        va_list ap;
        va_start(ap, fmt);
        vsnprintf(err, errlen, fmt, ap);
        va_end(ap);
    }
    return code;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
bool pow2(int v) { return v > 0 && (v & (v - 1)) == 0; }
bool block_fmt(int f) { return f == MOE_Q2K || f == MOE_Q8_0 || f == MOE_CB2; }
bool routed_fmt(int f) { return block_fmt(f) || f == MOE_Q4K; }

// Rows are split into 64-weight chunks, one per lane, up to 64 lanes per row.
bool row_ok(int n_in) { return n_in > 0 && n_in % 64 == 0 && pow2(n_in / 64) && n_in / 64 <= 64; }

int check_desc(const moe_layer_desc *d, char *err, size_t errlen) {
    if (!d) return fail(err, errlen, MOE_EINVAL, "desc is NULL");
    int D = d->n_embd, E = d->n_expert, k = d->n_expert_used, F = d->n_ff_exp, Fs = d->n_ff_shared;
    if (D <= 0 || E <= 0 || k <= 0 || F <= 0 || Fs < 0)
        return fail(err, errlen, MOE_EINVAL, "sizes must be positive (D=%d E=%d k=%d F=%d Fs=%d)", D, E, k, F, Fs);
    if (E > kMaxExperts || k > kMaxUsed || k > E)
        return fail(err, errlen, MOE_EUNSUPPORTED, "need 1 <= k <= min(16, E) and E <= 1024 (E=%d k=%d)", E, k);
    if (D % 256 || !row_ok(D) || !row_ok(F) || (Fs && !row_ok(Fs)))
        return fail(err, errlen, MOE_EUNSUPPORTED,
                    "D must be a multiple of 256 and D, F, Fs of the form 64*2^j <= 4096 (D=%d F=%d Fs=%d)", D, F,
                    Fs);
    if (!routed_fmt(d->gate_type) || d->up_type != d->gate_type || !routed_fmt(d->down_type) ||
        (Fs && !block_fmt(d->shared_type)))
        return fail(err, errlen, MOE_EUNSUPPORTED,
                    "formats: gate = up and down in {Q2K, Q8_0, CB2, Q4K}, shared in {Q2K, Q8_0, CB2}");
    if (!d->router_w || !d->gate || !d->up || !d->down)
        return fail(err, errlen, MOE_EINVAL, "router_w, gate, up and down must be set");
    if (Fs && (!d->sh_gate || !d->sh_up || !d->sh_down))
        return fail(err, errlen, MOE_EINVAL, "n_ff_shared > 0 needs sh_gate, sh_up and sh_down");
    bool cb = d->gate_type == MOE_CB2 || d->down_type == MOE_CB2 || (Fs && d->shared_type == MOE_CB2);
    if (cb && !d->codebook) return fail(err, errlen, MOE_EINVAL, "a CB2 format needs the codebook");
    const void *ptrs[] = {d->router_w, d->router_bias, d->gate, d->up, d->down, d->sh_gate, d->sh_up, d->sh_down,
                          d->codebook};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return fail(err, errlen, MOE_EALIGN, "weight pointers must be 16-byte aligned");
    return MOE_OK;
}

size_t ws_bytes_for(const moe_layer_desc *d, int32_t T) {
    return workspace_layout(d, T, nullptr).bytes;
}

int check_call(const moe_layer_desc *d, const void *x, int32_t T, int32_t x_type, void *ws, size_t ws_bytes,
               char *err, size_t errlen) {
    int rc = check_desc(d, err, errlen);
    if (rc) return rc;
    if (T < 0) return fail(err, errlen, MOE_EINVAL, "T must be >= 0 (T=%d)", T);
    if (x_type != MOE_F32 && x_type != MOE_BF16)
        return fail(err, errlen, MOE_EUNSUPPORTED, "x_type must be MOE_F32 or MOE_BF16");
    if (T == 0) return MOE_OK;
    // The grouped GEMMs address the activation codes of x ([T][D]) and of h
    // ([T*k][F]), 2 bytes per value, with 32-bit offsets from one base.
    if ((int64_t)T * d->n_embd * 2 > INT32_MAX || (int64_t)T * d->n_expert_used * d->n_ff_exp * 2 > INT32_MAX)
        return fail(err, errlen, MOE_EUNSUPPORTED,
                    "T=%d rows is too many for one call: T*n_embd and T*k*n_ff_exp must stay below 2^30 "
                    "(split the rows over several calls)",
                    T);
    if (!x) return fail(err, errlen, MOE_EINVAL, "x is NULL");
    if (!aligned16(x)) return fail(err, errlen, MOE_EALIGN, "x must be 16-byte aligned");
    size_t need = ws_bytes_for(d, T);
    if (!ws || ws_bytes < need)
        return fail(err, errlen, MOE_EWORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws ? ws_bytes : 0);
    if (!aligned16(ws)) return fail(err, errlen, MOE_EALIGN, "workspace must be 16-byte aligned");
    return MOE_OK;
}

int check_routing(const moe_routing *r, char *err, size_t errlen) {
    if (!r) return fail(err, errlen, MOE_EINVAL, "routing is NULL");
    if (!r->topk_idx || !r->topk_w || !r->count || !r->offset || !r->perm || !r->pos || !r->active || !r->n_active)
        return fail(err, errlen, MOE_EINVAL, "every routing array must be set");
    return MOE_OK;
}

RoutingPtrs from_routing(const moe_routing *r) {
    return RoutingPtrs{r->topk_idx, r->topk_w, r->count, r->offset, r->perm, r->pos, r->active, r->n_active};
}

RoutingPtrs from_ws(const Workspace &w) {
    return RoutingPtrs{w.topk_idx, w.topk_w, w.count, w.offset, w.perm, w.pos, w.active, w.n_active};
}

// ---- a second stream for the bf16 rows' shared expert ------------------------
// The shared expert needs only x, so on the many-row bf16 path it runs on a
// stream of its own beside the router, the bucketing and the routed gate/up
// GEMM; the routed down, which adds into the y that the shared down writes,
// waits for it.  One stream and two events per device, made on first use
// (not while the caller's stream is being captured: that call runs the
// shared expert in line).  The lock is held from the fork to the join's wait,
// so that the join event a call waits on is the one it recorded.
constexpr int kMaxSideDevices = 64;

struct SideStream {
    hipStream_t s = nullptr;
    hipEvent_t fork = nullptr, join = nullptr;
};

std::mutex side_mu;
SideStream side_of[kMaxSideDevices];

// nullptr: run in line (no device, capture before first use, or no stream)
SideStream *side_stream_locked(hipStream_t main) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxSideDevices) return nullptr;
    SideStream &ss = side_of[dev];
    if (ss.s && ss.fork && ss.join) return &ss;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(main, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) return nullptr;
    if (!ss.s && hipStreamCreateWithFlags(&ss.s, hipStreamNonBlocking) != hipSuccess) ss.s = nullptr;
    if (!ss.fork && hipEventCreateWithFlags(&ss.fork, hipEventDisableTiming) != hipSuccess) ss.fork = nullptr;
    if (!ss.join && hipEventCreateWithFlags(&ss.join, hipEventDisableTiming) != hipSuccess) ss.join = nullptr;
    return ss.s && ss.fork && ss.join ? &ss : nullptr;
}

// The many-row bf16 block with the shared expert on the side stream; route:
// the router and the bucketing run first (stage 0), else r is given.
hipError_t prefill_bf16_overlapped(const moe_layer_desc *d, const void *x, int32_t T, const RoutingPtrs &r, float *y,
                                   uint32_t flags, const Workspace &w, hipStream_t s, bool route, bool *done) {
    *done = false;
    std::lock_guard<std::mutex> lock(side_mu);
    SideStream *ss = side_stream_locked(s);
    if (!ss) return hipSuccess;
    hipError_t e = hipEventRecord(ss->fork, s);
    if (e == hipSuccess) e = hipStreamWaitEvent(ss->s, ss->fork, 0);
    if (e != hipSuccess) return e;
    *done = true;
    hipError_t es = launch_prefill_shared_bf16(d, x, T, y, flags, w, ss->s);
    const hipError_t ej = hipEventRecord(ss->join, ss->s);
    if (es == hipSuccess) es = ej;
    if (es != hipSuccess) {
        (void)hipStreamWaitEvent(s, ss->join, 0);  // the caller's stream still joins what was enqueued
        return es;
    }
    if (route) e = launch_router_logits(d, x, T, MOE_BF16, w, s);
    if (route && e == hipSuccess) e = launch_route_finish(d, x, T, MOE_BF16, r, w, s);
    if (e == hipSuccess) return launch_prefill(d, x, T, MOE_BF16, r, y, flags, w, s, 0, ss->join);
    (void)hipStreamWaitEvent(s, ss->join, 0);
    return e;
}

bool overlap_shared(const moe_layer_desc *d, int32_t T, int32_t x_type) {
    return x_type == MOE_BF16 && d->n_ff_shared > 0 && prefill_path_ok(d, T, x_type);
}

// The whole block (stage 0) or one of its four stages.  Few rows: the decode
// schedule; otherwise router logits, top-k + bucketing, gate/up, down.
hipError_t forward(const moe_layer_desc *d, const void *x, int32_t T, int32_t x_type, const RoutingPtrs &r, float *y,
                   uint32_t flags, const Workspace &w, hipStream_t s, int stage) {
    // stage 5 (the routed gate/up kernel alone) differs from stage 3 on the
    // grouped-GEMM path only
    const int st3 = stage == 5 ? 3 : stage;
    if (small_path_ok(d, T) && small_route_ok(d, T)) return launch_small(d, x, T, x_type, r, y, flags, w, s, st3, true);
    hipError_t e = hipSuccess;
    if (stage == 0 && overlap_shared(d, T, x_type)) {
        bool done = false;
        e = prefill_bf16_overlapped(d, x, T, r, y, flags, w, s, true, &done);
        if (done || e != hipSuccess) return e;
    }
    if (stage == 0 || stage == 1) e = launch_router_logits(d, x, T, x_type, w, s);
    if (e == hipSuccess && (stage == 0 || stage == 2)) e = launch_route_finish(d, x, T, x_type, r, w, s);
    if (e == hipSuccess && (stage == 0 || stage >= 3))
        e = prefill_path_ok(d, T, x_type) ? launch_prefill(d, x, T, x_type, r, y, flags, w, s, stage)
                                          : launch_ffn_large(d, x, T, x_type, r, y, flags, w, s, st3);
    return e;
}

int device_status(hipError_t e, char *err, size_t errlen) {
    if (e == hipSuccess) return MOE_OK;
    return fail(err, errlen, MOE_EDEVICE, "HIP: %s", hipGetErrorString(e));
}

// ---- scratch of the entry point that allocates nothing -----------------------
// A file-scope device array: every GPU the library runs on holds its own copy
// until the process ends.  Host code never uses the array's name as an
// address: its device address comes from hipGetSymbolAddress, once per
// device, with that device current.
constexpr int kMaxDevices = 64;

std::mutex scratch_mu;
void *scratch_addr[kMaxDevices];

int scratch_of_current_device(void **out, char *err, size_t errlen) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return device_status(e, err, errlen);
    if (dev < 0 || dev >= kMaxDevices) return fail(err, errlen, MOE_EDEVICE, "device %d out of range", dev);
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_addr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return device_status(e, err, errlen);
        if (!p) return fail(err, errlen, MOE_EDEVICE, "no device address for the scratch array");
        scratch_addr[dev] = p;
    }
    *out = scratch_addr[dev];
    return MOE_OK;
}

// Bytes of workspace the few-row schedule reads and writes: it uses only the
// buffers laid out before the many-row ones.
size_t few_row_ws_bytes(const moe_layer_desc *d, int32_t T) {
    char *const base = (char *)(uintptr_t)4096;  // any aligned address: only offsets are taken
    return (size_t)((char *)workspace_layout(d, T, base).pf_xq - base);
}

}  // namespace

extern "C" {

size_t moe_workspace_size(const moe_layer_desc *d, int32_t max_rows, int32_t x_type) {
    if (check_desc(d, nullptr, 0) || max_rows < 0 || (x_type != MOE_F32 && x_type != MOE_BF16)) return 0;
    if (max_rows == 0) return 256;
    // the router's chunking changes with T, so cover every plan up to max_rows
    size_t b = ws_bytes_for(d, max_rows);
    b = std::max(b, ws_bytes_for(d, std::min<int32_t>(max_rows, 4)));
    b = std::max(b, ws_bytes_for(d, std::min<int32_t>(max_rows, 64)));
    // the largest row count whose router writes partial sums
    const int32_t split_top = std::min<int32_t>(127, kRouteMidPairs / d->n_expert_used);
    b = std::max(b, ws_bytes_for(d, std::min<int32_t>(max_rows, split_top)));
    return b;
}

int moe_route(const moe_layer_desc *d, const void *x, int32_t T, int32_t x_type, const moe_routing *out, void *ws,
              size_t ws_bytes, void *stream, char *err, size_t errlen) {
    int rc = check_call(d, x, T, x_type, ws, ws_bytes, err, errlen);
    if (rc) return rc;
    if ((rc = check_routing(out, err, errlen))) return rc;
    if (T == 0) return MOE_OK;
    Workspace w = workspace_layout(d, T, ws);
    return device_status(launch_route(d, x, T, x_type, from_routing(out), w, (hipStream_t)stream), err, errlen);
}

int moe_expert_ffn(const moe_layer_desc *d, const void *x, int32_t T, int32_t x_type, const moe_routing *r,
                   float *y, uint32_t flags, void *ws, size_t ws_bytes, void *stream, char *err, size_t errlen) {
    int rc = check_call(d, x, T, x_type, ws, ws_bytes, err, errlen);
    if (rc) return rc;
    if ((rc = check_routing(r, err, errlen))) return rc;
    if (flags & ~(uint32_t)MOE_ACCUMULATE) return fail(err, errlen, MOE_EINVAL, "unknown flags 0x%x", flags);
    if (T == 0) return MOE_OK;
    if (!y) return fail(err, errlen, MOE_EINVAL, "y is NULL");
    if (!aligned16(y)) return fail(err, errlen, MOE_EALIGN, "y must be 16-byte aligned");
    Workspace w = workspace_layout(d, T, ws);
    hipStream_t s = (hipStream_t)stream;
    if (!small_path_ok(d, T) && overlap_shared(d, T, x_type)) {
        bool done = false;
        const hipError_t e = prefill_bf16_overlapped(d, x, T, from_routing(r), y, flags, w, s, false, &done);
        if (done || e != hipSuccess) return device_status(e, err, errlen);
    }
    hipError_t e = small_path_ok(d, T)                ? launch_small(d, x, T, x_type, from_routing(r), y, flags, w, s, 0, false)
                   : prefill_path_ok(d, T, x_type) ? launch_prefill(d, x, T, x_type, from_routing(r), y, flags, w, s, 0)
                                                   : launch_ffn_large(d, x, T, x_type, from_routing(r), y, flags, w, s, 0);
    return device_status(e, err, errlen);
}

int moe_layer_forward(const moe_layer_desc *d, const void *x, int32_t T, int32_t x_type, float *y, uint32_t flags,
                      const moe_routing *routing, void *ws, size_t ws_bytes, void *stream, char *err,
                      size_t errlen) {
    int rc = check_call(d, x, T, x_type, ws, ws_bytes, err, errlen);
    if (rc) return rc;
    if (routing && (rc = check_routing(routing, err, errlen))) return rc;
    if (flags & ~(uint32_t)MOE_ACCUMULATE) return fail(err, errlen, MOE_EINVAL, "unknown flags 0x%x", flags);
    if (T == 0) return MOE_OK;
    if (!y) return fail(err, errlen, MOE_EINVAL, "y is NULL");
    if (!aligned16(y)) return fail(err, errlen, MOE_EALIGN, "y must be 16-byte aligned");
    Workspace w = workspace_layout(d, T, ws);
    RoutingPtrs r = routing ? from_routing(routing) : from_ws(w);
    return device_status(forward(d, x, T, x_type, r, y, flags, w, (hipStream_t)stream, 0), err, errlen);
}

int moe_layer_forward_stage(const moe_layer_desc *d, const void *x, int32_t T, int32_t x_type, float *y,
                            uint32_t flags, const moe_routing *routing, int32_t stage, void *ws, size_t ws_bytes,
                            void *stream, char *err, size_t errlen) {
    if (stage < 1 || stage > 5) return fail(err, errlen, MOE_EINVAL, "stage must be 1 to 5 (got %d)", stage);
    int rc = check_call(d, x, T, x_type, ws, ws_bytes, err, errlen);
    if (rc) return rc;
    if (routing && (rc = check_routing(routing, err, errlen))) return rc;
    if (flags & ~(uint32_t)MOE_ACCUMULATE) return fail(err, errlen, MOE_EINVAL, "unknown flags 0x%x", flags);
    if (T == 0) return MOE_OK;
    if (!y) return fail(err, errlen, MOE_EINVAL, "y is NULL");
    if (!aligned16(y)) return fail(err, errlen, MOE_EALIGN, "y must be 16-byte aligned");
    Workspace w = workspace_layout(d, T, ws);
    RoutingPtrs r = routing ? from_routing(routing) : from_ws(w);
    return device_status(forward(d, x, T, x_type, r, y, flags, w, (hipStream_t)stream, stage), err, errlen);
}

int moe_layer_forward_noalloc(const moe_layer_desc *d, const void *x, int32_t T, int32_t x_type, float *y,
                              uint32_t flags, const moe_routing *routing, void *stream, char *err, size_t errlen) {
    int rc = check_desc(d, err, errlen);
    if (rc) return rc;
    if (T < 0) return fail(err, errlen, MOE_EINVAL, "T must be >= 0 (T=%d)", T);
    if (x_type != MOE_F32 && x_type != MOE_BF16)
        return fail(err, errlen, MOE_EUNSUPPORTED, "x_type must be MOE_F32 or MOE_BF16");
    if (routing && (rc = check_routing(routing, err, errlen))) return rc;
    if (flags & ~(uint32_t)MOE_ACCUMULATE) return fail(err, errlen, MOE_EINVAL, "unknown flags 0x%x", flags);
    if (T == 0) return MOE_OK;
    if (!(small_path_ok(d, T) && small_route_ok(d, T)))
        return fail(err, errlen, MOE_EUNSUPPORTED,
                    "the entry point without allocation takes the few-row schedule only: T <= 16, T*k <= 256, "
                    "Q2K, CB2 or Q4K experts (T=%d k=%d)",
                    T, d->n_expert_used);
    const size_t need = few_row_ws_bytes(d, T);
    if (need > kScratchBytes)
        return fail(err, errlen, MOE_EWORKSPACE, "%zu bytes of scratch needed, the static scratch holds %zu", need,
                    kScratchBytes);
    if (!x || !y) return fail(err, errlen, MOE_EINVAL, "x and y must be set");
    if (!aligned16(x) || !aligned16(y)) return fail(err, errlen, MOE_EALIGN, "x and y must be 16-byte aligned");
    void *ws = nullptr;
    if ((rc = scratch_of_current_device(&ws, err, errlen))) return rc;
    Workspace w = workspace_layout(d, T, ws);
    RoutingPtrs r = routing ? from_routing(routing) : from_ws(w);
    return device_status(forward(d, x, T, x_type, r, y, flags, w, (hipStream_t)stream, 0), err, errlen);
}

int moe_block_forward(const moe_layer_desc *d, const float *gamma, float eps, float *x, int32_t T,
                      const moe_routing *routing, void *ws, size_t ws_bytes, void *stream, char *err, size_t errlen) {
    int rc = check_call(d, x, T, MOE_F32, ws, ws_bytes, err, errlen);
    if (rc) return rc;
    if (routing && (rc = check_routing(routing, err, errlen))) return rc;
    if (!(eps >= 0.f)) return fail(err, errlen, MOE_EINVAL, "eps must be >= 0");
    if (T == 0) return MOE_OK;
    if (!gamma) return fail(err, errlen, MOE_EINVAL, "gamma is NULL");
    if (!aligned16(gamma)) return fail(err, errlen, MOE_EALIGN, "gamma must be 16-byte aligned");
    Workspace w = workspace_layout(d, T, ws);
    RoutingPtrs r = routing ? from_routing(routing) : from_ws(w);
    hipStream_t s = (hipStream_t)stream;
    // one token with Q2K or codebook gate/up rows: the first kernel normalises
    // x itself and the last adds the block's output into x
    if (t1_schedule_ok(d, T, MOE_F32) && (d->gate_type == MOE_Q2K || d->gate_type == MOE_CB2))
        return device_status(launch_small(d, x, T, MOE_F32, r, x, MOE_ACCUMULATE, w, s, 0, true, gamma, eps), err,
                             errlen);
    hipError_t e = launch_rmsnorm(x, gamma, eps, T, d->n_embd, w.xn, s);
    if (e == hipSuccess) e = forward(d, w.xn, T, MOE_F32, r, x, MOE_ACCUMULATE, w, s, 0);
    return device_status(e, err, errlen);
}

int moe_count_selections(const int32_t *topk_idx, int32_t T, int32_t k, int32_t E, int32_t layer, int64_t *counts,
                         void *stream, char *err, size_t errlen) {
    if (T < 0 || k < 1 || E < 1 || layer < 0)
        return fail(err, errlen, MOE_EINVAL, "need T >= 0, k >= 1, E >= 1, layer >= 0 (T=%d k=%d E=%d layer=%d)", T, k,
                    E, layer);
    if (T == 0) return MOE_OK;
    if (!topk_idx || !counts) return fail(err, errlen, MOE_EINVAL, "topk_idx and counts must be set");
    return device_status(launch_count_selections(topk_idx, T, k, E, layer, counts, (hipStream_t)stream), err,
                         errlen);
}

int moe_hotlist(const int64_t *counts, int32_t n, int32_t *order, int32_t *n_hot, void *stream, char *err,
                size_t errlen) {
    if (n < 0 || n > kMaxHotlist)
        return fail(err, errlen, MOE_EINVAL, "n must be in [0, %d] (got %d)", kMaxHotlist, n);
    if (n == 0) return MOE_OK;
    if (!counts || !order || !n_hot) return fail(err, errlen, MOE_EINVAL, "counts, order and n_hot must be set");
    return device_status(launch_hotlist(counts, n, order, n_hot, (hipStream_t)stream), err, errlen);
}

int moe_rmsnorm(const float *x, const float *gamma, float eps, int32_t T, int32_t D, float *out, void *stream,
                char *err, size_t errlen) {
    if (T < 0 || D <= 0) return fail(err, errlen, MOE_EINVAL, "need T >= 0 and D > 0 (T=%d D=%d)", T, D);
    if (!(eps >= 0.f)) return fail(err, errlen, MOE_EINVAL, "eps must be >= 0");
    if (T == 0) return MOE_OK;
    if (!x || !gamma || !out) return fail(err, errlen, MOE_EINVAL, "x, gamma and out must be set");
    return device_status(launch_rmsnorm(x, gamma, eps, T, D, out, (hipStream_t)stream), err, errlen);
}

int moe_dequant(int32_t type, const void *src, int64_t n, const int8_t *codebook, int32_t out_type, void *dst,
                void *stream, char *err, size_t errlen) {
    if (!routed_fmt(type)) return fail(err, errlen, MOE_EUNSUPPORTED, "type must be Q2K, Q8_0, CB2 or Q4K");
    if (out_type != MOE_F32 && out_type != MOE_BF16)
        return fail(err, errlen, MOE_EUNSUPPORTED, "out_type must be MOE_F32 or MOE_BF16");
    int64_t unit = type == MOE_Q8_0 ? 32 : 256;
    if (n < 0 || n % unit) return fail(err, errlen, MOE_EINVAL, "n_weights must be a multiple of %lld", (long long)unit);
    if (n == 0) return MOE_OK;
    if (!src || !dst) return fail(err, errlen, MOE_EINVAL, "src and dst must be set");
    if (type == MOE_CB2 && !codebook) return fail(err, errlen, MOE_EINVAL, "CB2 needs the codebook");
    if (((uintptr_t)src & 3u) || ((uintptr_t)dst & 3u) || (codebook && ((uintptr_t)codebook & 3u)))
        return fail(err, errlen, MOE_EALIGN, "src, dst and codebook must be 4-byte aligned");
    return device_status(launch_dequant(type, src, n, codebook, out_type, dst, (hipStream_t)stream), err, errlen);
}

int moe_read_stream(const void *src, int64_t bytes, uint32_t *sink, int32_t sink_words, void *stream, char *err,
                    size_t errlen) {
    if (bytes < 0 || bytes % 16) return fail(err, errlen, MOE_EINVAL, "bytes must be a multiple of 16 (got %lld)",
                                             (long long)bytes);
    if (sink_words < 4 || sink_words % 4)
        return fail(err, errlen, MOE_EINVAL, "sink_words must be a positive multiple of 4 (got %d)", sink_words);
    if (bytes == 0) return MOE_OK;
    if (!src || !sink) return fail(err, errlen, MOE_EINVAL, "src and sink must be set");
    if (!aligned16(src)) return fail(err, errlen, MOE_EALIGN, "src must be 16-byte aligned");
    return device_status(launch_read_stream(src, bytes, sink, sink_words / 4, (hipStream_t)stream), err, errlen);
}

const char *moe_version(void) { return "moe-gfx950 0.1"; }

}  // extern "C"
