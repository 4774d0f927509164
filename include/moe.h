/*
 * moe.h - C ABI of the routed mixture-of-experts block on one MI355X (gfx950).
 *
 * The block (pages: "Understanding Dwarf Star", 5.3.2 MoE formula, 5.3.4 the
 * shared expert, 5.3.5 routing, 5.3.7 the MoE kernel's five steps; "The
 * sparsity that pays for everything else in DwarfStar", "Where the parameters
 * actually are"):
 *
 *   logits  l[t][e] = sum_k x[t][k] * W_r[e][k] (+ bias[e])        fp64 accumulation
 *   top-k   the k experts of largest logit, ties to the lower index, slot 0 best
 *   weights w[t][s] = route_scale * softmax over the k chosen logits
 *   FFN_e   y = W_down[e] (silu(W_gate[e] x) * (W_up[e] x))           SwiGLU
 *   shared  S(x) = the same FFN with the shared expert's weights, always on
 *   y[t]    = S(x_t) + sum_s w[t][s] * FFN_{idx[t][s]}(x_t)
 *
 * Weights stay in 2-bit / 8-bit blocks and are decoded on the fly inside the
 * kernels ("Understanding Dwarf Star", 2.8.1-2.8.2).  Block layouts (this
 * library's own byte order; no GGUF compatibility is claimed):
 *   MOE_Q2K  84 B / 256 weights: fp16 d @0, fp16 dmin @2, 16 bytes @4 with a
 *            4-bit scale (low nibble) and 4-bit min (high nibble) per group of
 *            16 weights, 64 bytes of 2-bit codes @20 (weight i in bits
 *            2*(i%4) of byte i/4).  w = d*scale*q - dmin*min.
 *            ("Understanding Dwarf Star", Q2_K subsection.)
 *   MOE_Q8_0 34 B / 32 weights: fp16 d @0, 32 int8 @2.  w = d*q.
 *            ("Understanding Dwarf Star", 2.4 table: 8-bit shared expert.)
 *   MOE_CB2  66 B / 256 weights: fp16 d @0, 32 codebook indices @2 (one per 8
 *            weights), 32 sign masks @34 (bit j negates weight j of the 8).
 *            w = d * (+/-) codebook[idx][j], codebook int8 [256][8].
 *            ("Understanding Dwarf Star", 2.3.4: 66 bytes per 256 weights.)
 *   MOE_Q4K  144 B / 256 weights: fp16 d @0, fp16 dmin @2, 12 bytes @4 holding
 *            sixteen 6-bit fields (field f in bits 6f..6f+5 of the 96-bit
 *            little-endian integer; f = j is the scale and f = 8 + j the min
 *            of sub-block j of 32 weights), 128 bytes of 4-bit codes @16
 *            (weight i in bits 4*(i%2) of byte i/2).  w = d*scale*q - dmin*min.
 *            Routed gate/up/down only.  ("Understanding Dwarf Star", 2.3.2,
 *            the Q4_K block layout.)
 * A matrix [n_out][n_in] is flattened row-major and cut into consecutive
 * blocks, so blocks run along the reduction dimension.  Expert tensors are
 * expert-major: gate/up [E][F][D], down [E][D][F]; shared [Fs][D], [Fs][D],
 * [D][Fs]; router [E][D] fp32 (the D x E router matrix stored with each
 * expert's D weights contiguous).
 *
 * Conventions ("Understanding Dwarf Star", 3.3.3 opaque types, 3.7.1-3.7.2
 * return codes and the caller's error buffer, 3.2.2-3.2.3 scratch buffers
 * allocated once and reused):
 *  - Every pointer argument that names tensor data is a DEVICE pointer unless
 *    the comment says host.  The caller owns every buffer, including the
 *    workspace; the library allocates nothing on these calls and keeps no
 *    pointer after returning.
 *  - Calls validate all arguments first; on error nothing is enqueued.  Work
 *    is enqueued on `stream` (a hipStream_t; NULL = the null stream) and the
 *    call returns without synchronizing; device faults surface at the
 *    caller's next synchronization.  No host<->device copy happens inside.
 *  - Return 0 (MOE_OK) or a negative moe_status; err (host, may be NULL)
 *    receives a NUL-terminated message of at most errlen bytes.
 *  - T = 0 is valid and enqueues nothing.
 *  - Reentrant.  Global state: a lazily filled per-device property cache,
 *    and per device one second stream of the library's (default priority,
 *    made on first use) with two events.  On the many-row bf16 path
 *    (moe_layer_forward, moe_expert_ffn) the shared expert runs on that
 *    stream, forked from `stream` and joined back into it by the events, so
 *    every result is still ordered on `stream` (under graph capture the fork
 *    and the join are captured as edges; a call made while `stream` is being
 *    captured before that stream exists runs the shared expert in line).
 *    Host threads that call on one device take turns over the fork and join.
 *  - Limits: 1 <= k <= 16, k <= E <= 1024, D % 256 == 0, F % 64 == 0, the
 *    64-weight chunks of a row (n_in/64) a power of two up to 64 or a
 *    multiple of 64, weight and activation base addresses 16-byte aligned,
 *    and T * D and T * k * F below 2^30 per call (MOE_EUNSUPPORTED beyond:
 *    split the rows over several calls).
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_EINVAL = -1,       /* NULL where data is required, bad size, k > E ... */
    MOE_EALIGN = -2,       /* a base address is not 16-byte aligned */
    MOE_EWORKSPACE = -3,   /* workspace NULL or smaller than moe_workspace_size */
    MOE_EUNSUPPORTED = -4, /* a format or shape outside the limits above */
    MOE_EDEVICE = -5       /* a HIP call failed (message carries hipGetErrorString) */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_Q2K = 2, MOE_Q8_0 = 3, MOE_CB2 = 4, MOE_Q4K = 5 } moe_dtype;

enum { MOE_ACCUMULATE = 1u }; /* y += block(x) instead of y = block(x) */

/* One MoE layer.  A host struct whose pointer fields are device pointers. */
typedef struct {
    int32_t n_embd;        /* D: model width */
    int32_t n_expert;      /* E: routed experts */
    int32_t n_expert_used; /* k: experts per token */
    int32_t n_ff_exp;      /* F: routed expert FFN width */
    int32_t n_ff_shared;   /* Fs: shared expert FFN width, 0 = no shared expert */
    int32_t gate_type, up_type, down_type, shared_type; /* moe_dtype block formats */
    const float *router_w;    /* [E][D] fp32, expert-major: row e = the D weights of expert e */
    const float *router_bias; /* [E] fp32 added to the logits before top-k, or NULL */
    float route_scale;        /* multiplies the renormalized weights (1.0 = plain) */
    const void *gate, *up;    /* [E][F][D] in gate_type / up_type blocks */
    const void *down;         /* [E][D][F] in down_type blocks */
    const void *sh_gate, *sh_up, *sh_down; /* [Fs][D], [Fs][D], [D][Fs] or NULL */
    const int8_t *codebook;   /* [256][8] int8 when any format is MOE_CB2, else NULL; entries in
                                 [-127, 127] (the decode kernels negate them bytewise) */
} moe_layer_desc;

/* Routing of T token rows: caller-owned device arrays. */
typedef struct {
    int32_t *topk_idx; /* [T][k] expert ids, slot 0 = largest logit */
    float *topk_w;     /* [T][k] weights */
    int32_t *count;    /* [E] pairs routed to each expert */
    int32_t *offset;   /* [E+1] exclusive prefix sum of count */
    int32_t *perm;     /* [T*k] pair ids t*k+s sorted by (expert, t, s) */
    int32_t *pos;      /* [T*k] inverse of perm */
    int32_t *active;   /* [E] experts with count > 0, ascending; -1 after n_active */
    int32_t *n_active; /* [1] */
} moe_routing;

/* Bytes of workspace the calls below need for up to max_rows token rows with
 * activations of type x_type (MOE_F32 or MOE_BF16).  Returns 0 if the
 * descriptor is invalid.  Host-only; enqueues nothing. */
size_t moe_workspace_size(const moe_layer_desc *desc, int32_t max_rows, int32_t x_type);

/* Router logits, top-k, renormalized weights and expert bucketing of T rows
 * ("Understanding Dwarf Star", 5.3.2 router(x) = softmax(x W_router), top-k;
 * 5.3.7 step 1 and the sparse indexing of step 2).
 * x: [T][D] fp32 (x_type MOE_F32) or bf16 (MOE_BF16).  out: every array set.
 * The logits are accumulated in fp64 so that the selected indices do not
 * depend on the summation order.  From 128 bf16 rows on (n_embd 1024, 2048
 * or 4096, at most 256 experts) they are first bounded on the bf16 matrix
 * cores, and only the experts whose bound can still reach the top k are
 * summed in fp64: the indices and weights are those of the fp64 sums. */
int moe_route(const moe_layer_desc *desc, const void *x, int32_t T, int32_t x_type, const moe_routing *out,
              void *ws, size_t ws_bytes, void *stream, char *err, size_t errlen);

/* Expert FFNs, shared expert and weighted combine for a routing produced by
 * moe_route on the same x ("Understanding Dwarf Star", 5.3.7 steps 2-5; 5.3.4).
 * y: [T][D] fp32.  flags: MOE_ACCUMULATE adds to y.
 * Numerics: in both modes the products take the exact integer codes of the
 * weights against activations coded as int16 (c = rint(v * 32512 / max|v|))
 * per group of 16 values (few rows) or per row (many rows, on the matrix
 * cores), accumulated exactly in int32 and scaled in fp32.  x_type MOE_F32
 * keeps x, h and y in fp32, and two calls give the same bits.  MOE_BF16
 * takes bf16 x (coded per row like fp32 rows); h stays fp32 and is coded
 * per row for the down projection, and the routed down rows are added into y
 * with atomics (the order of those additions varies between calls). */
int moe_expert_ffn(const moe_layer_desc *desc, const void *x, int32_t T, int32_t x_type, const moe_routing *r,
                   float *y, uint32_t flags, void *ws, size_t ws_bytes, void *stream, char *err, size_t errlen);

/* moe_route followed by moe_expert_ffn.  routing may be NULL (kept in the
 * workspace) or caller arrays to receive the routing. */
int moe_layer_forward(const moe_layer_desc *desc, const void *x, int32_t T, int32_t x_type, float *y,
                      uint32_t flags, const moe_routing *routing, void *ws, size_t ws_bytes, void *stream,
                      char *err, size_t errlen);

/* The four stages moe_layer_forward runs, callable one by one with the same
 * arguments (so that each can be timed with events on the caller's stream);
 * running stages 1, 2, 3, 4 in order equals one moe_layer_forward call.
 *   1  router logits
 *   2  top-k, weights, bucketing (for a few rows, also the shared expert's
 *      gate/up)
 *   3  gate/up with SwiGLU
 *   4  down projection and the weighted combine into y (for a few rows, also
 *      the shared expert's down)
 *   5  the routed gate/up kernel of stage 3 alone: on the grouped-GEMM path
 *      (many rows, Q2K experts) it reuses the activation codes and tiles a
 *      stage 3 call with the same x and routing left in the workspace;
 *      elsewhere it equals stage 3.  For timing that kernel by itself. */
int moe_layer_forward_stage(const moe_layer_desc *desc, const void *x, int32_t T, int32_t x_type, float *y,
                            uint32_t flags, const moe_routing *routing, int32_t stage, void *ws, size_t ws_bytes,
                            void *stream, char *err, size_t errlen);

/* One block of the stack ("Understanding Dwarf Star", 5.6.2: the layers
 * applied in turn, each normalising its input first; 5.2.1 RMSNorm):
 * x <- x + MoE(RMSNorm(x) * gamma), in place on the residual stream.
 * x: [T][D] fp32, read and then overwritten; gamma: [D] fp32, 16-byte
 * aligned; eps >= 0.  The normalised rows have the bits of moe_rmsnorm and
 * the MoE output those of moe_layer_forward on them with MOE_ACCUMULATE.  One
 * token with Q2K or codebook gate/up rows runs in three launches (the first
 * normalises x itself, the last adds into x); otherwise moe_rmsnorm into the
 * workspace, then moe_layer_forward.  routing may be NULL.  Workspace from
 * moe_workspace_size (which covers the normalised rows). */
int moe_block_forward(const moe_layer_desc *desc, const float *gamma, float eps, float *x, int32_t T,
                      const moe_routing *routing, void *ws, size_t ws_bytes, void *stream, char *err,
                      size_t errlen);

/* moe_layer_forward without a workspace argument, for callers that cannot
 * allocate device memory (code under graph capture, tight serving loops,
 * harnesses that forbid allocation): the buffers live in a static scratch of
 * 8 MiB per device (a file-scope device array, held until the process ends),
 * so the call allocates nothing.  It takes the few-row schedule only: T <= 16
 * and T*k <= 256 with Q2K, CB2 or Q4K routed experts (MOE_EUNSUPPORTED
 * otherwise), and shapes whose buffers fit the scratch (MOE_EWORKSPACE
 * otherwise; the DeepSeek-V4-Flash shape needs about 3.6 MB at 16 rows).
 * The stream's device must be current.  Every call on one GPU shares that
 * GPU's scratch, so calls that overlap on one GPU (other streams, other
 * threads) race; nothing in the scratch needs to start at zero.  Arguments,
 * errors and results as moe_layer_forward (the same kernels, so the same
 * bits). */
int moe_layer_forward_noalloc(const moe_layer_desc *desc, const void *x, int32_t T, int32_t x_type, float *y,
                              uint32_t flags, const moe_routing *routing, void *stream, char *err, size_t errlen);

/* Expert selection counts for the hot list ("The sparsity that pays for
 * everything else in DwarfStar", "Some experts run far more often than
 * others": a run counts expert selections per {layer, expert} and merges
 * them into an existing profile).
 * topk_idx: [T][k] int32, the routing of one layer (moe_routing.topk_idx).
 * counts: [n_layer][E] int64, caller-owned and caller-initialised (zeros, or
 * a profile loaded earlier): counts[layer][e] += the number of (t, s) with
 * topk_idx[t][s] == e.  Entries outside [0, E) are not counted.  The adds
 * are integer, so the result does not depend on their order.  T = 0
 * enqueues nothing. */
int moe_count_selections(const int32_t *topk_idx, int32_t T, int32_t k, int32_t E, int32_t layer, int64_t *counts,
                         void *stream, char *err, size_t errlen);

/* The hot list (same section: the profile's entries sorted by hits, which
 * the engine walks to seed its expert cache).  counts: [n] int64 (n =
 * n_layer * E, entry layer*E + e); order: [n] int32 receives the entry
 * indices sorted by count descending, equal counts by index ascending;
 * n_hot: [1] int32 receives the number of entries with a positive count (the
 * list's length).  Counts are ordered as if clamped to [0, 2^39).  n must be
 * in [0, 16384]; n = 0 enqueues nothing.  One workgroup sorts the entries in
 * LDS. */
int moe_hotlist(const int64_t *counts, int32_t n, int32_t *order, int32_t *n_hot, void *stream, char *err,
                size_t errlen);

/* out[t][i] = gamma[i] * x[t][i] / sqrt(mean_i x[t][i]^2 + eps), fp32 in and
 * out, accumulated in fp32 ("Understanding Dwarf Star", 5.2.1 and 5.6.2:
 * RMSNorm before each block).  out may equal x. */
int moe_rmsnorm(const float *x, const float *gamma, float eps, int32_t T, int32_t D, float *out, void *stream,
                char *err, size_t errlen);

/* Decode n_weights of a block tensor (type MOE_Q2K, MOE_Q8_0, MOE_CB2 or MOE_Q4K) to
 * fp32 (out_type MOE_F32) or bf16 (MOE_BF16, round to nearest even).  The
 * fp32 result is exact: every product in the formats fits in fp32.  A test
 * hook for the decoders the kernels use ("Understanding Dwarf Star", 2.8.2
 * steps 1-3). */
int moe_dequant(int32_t type, const void *src, int64_t n_weights, const int8_t *codebook, int32_t out_type,
                void *dst, void *stream, char *err, size_t errlen);

/* A plain read of `bytes` (a multiple of 16) of device memory at src, every
 * 16-byte unit once, by sink_words / 4 workgroups of 256 threads; sink
 * (device, sink_words words, a multiple of 4) receives one XOR-fold per wave
 * so that no read is dropped.  The bandwidth one launch of a pure stream
 * reaches, beside the 8 TB/s HBM figure, for judging the kernels' rooflines
 * (the measurement plan of the block: the achievable HBM bandwidth next to
 * the specification).  bytes = 0 enqueues nothing. */
int moe_read_stream(const void *src, int64_t bytes, uint32_t *sink, int32_t sink_words, void *stream, char *err,
                    size_t errlen);

/* Library version string (static storage). */
const char *moe_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
