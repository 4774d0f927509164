// k_hot.hip - expert selection counts per {layer, expert} and the hot list
// ("The sparsity that pays for everything else in DwarfStar", "Some experts
// run far more often than others": a run counts selections per {layer,
// expert}, merges them with an existing profile and writes the entries
// sorted by hits; the engine seeds its expert cache in that order).
#include "common.h"

namespace moe {

// One lane per (token, slot) pair: an integer add per selection, so the
// counts do not depend on the order in which lanes land.
__global__ void __launch_bounds__(256) count_selections_kernel(const int32_t *__restrict__ topk_idx, int64_t P, int E,
                                                               int layer, int64_t *__restrict__ counts) {
    const int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (p >= P) return;
    const int e = topk_idx[p];
    if (e >= 0 && e < E) atomicAdd((unsigned long long *)(counts + (int64_t)layer * E + e), 1ull);
}

// The hot list by ranks: every entry has a unique 64-bit key (the clamped
// count in the high 40 bits, 2^24 - 1 - index in the low 24 bits: more hits
// first, equal hits by lower index), and its place in the list is the number
// of keys above it.  A block stages all keys in LDS and takes 64 entries, one
// per lane; its 16 waves count over a sixteenth of the keys each (the same
// key is read by all lanes at once, an LDS broadcast), and the parts are
// added.  n^2 compares spread over the chip take a few microseconds for the
// 11,008 {layer, expert} entries of the stack, where one workgroup sorting
// in LDS took 266 us.
MOE_DEV uint64_t hot_key(const int64_t *counts, int i) {
    const int64_t c = counts[i];
    const uint64_t cc = c < 0 ? 0 : (c >= kHotCountMax ? (uint64_t)kHotCountMax - 1 : (uint64_t)c);
    return (cc << 24) | (uint64_t)(0xFFFFFF - i);
}

typedef unsigned long long u64x2 __attribute__((ext_vector_type(2)));

__global__ void __launch_bounds__(1024) hotlist_kernel(const int64_t *__restrict__ counts, int n,
                                                       int32_t *__restrict__ order, int32_t *__restrict__ n_hot) {
    __shared__ __align__(16) uint64_t key[kMaxHotlist + 16];
    __shared__ int part[16][64];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int n16 = (n + 15) & ~15;  // padded with keys of 0, below every entry's key
    for (int i = tid; i < n16; i += 1024) key[i] = i < n ? hot_key(counts, i) : 0ull;
    __syncthreads();
    const int i = blockIdx.x * 64 + lane;
    const uint64_t ki = i < n ? key[i] : ~0ull;
    // wave w counts over its sixteenth of the keys, 8 keys (4 LDS reads of
    // two) per step so that the reads overlap
    const int q = ((n16 >> 4) + 1) & ~1, j0 = min(n16, wave * q), j1 = min(n16, j0 + q);  // even: 16-byte reads
    int above = 0;
    int j = j0;
    for (; j + 8 <= j1; j += 8) {
        const u64x2 a = *(const u64x2 *)&key[j], b = *(const u64x2 *)&key[j + 2];
        const u64x2 c = *(const u64x2 *)&key[j + 4], d = *(const u64x2 *)&key[j + 6];
        above += (a[0] > ki) + (a[1] > ki) + (b[0] > ki) + (b[1] > ki) + (c[0] > ki) + (c[1] > ki) + (d[0] > ki) +
                 (d[1] > ki);
    }
    for (; j < j1; ++j) above += key[j] > ki;
    part[wave][lane] = above;
    __syncthreads();
    if (wave == 0 && i < n) {
        int r = 0;
#pragma unroll
        for (int w = 0; w < 16; ++w) r += part[w][lane];
        order[r] = i;
    }
    if (blockIdx.x == 0) {  // the list's length: entries with a positive count
        int hot = 0;
        for (int t = tid; t < n; t += 1024) hot += counts[t] > 0;
        for (int o = 32; o > 0; o >>= 1) hot += __shfl_xor(hot, o, kWave);
        __syncthreads();
        if (lane == 0) part[wave][0] = hot;
        __syncthreads();
        if (tid == 0) {
            int h = 0;
            for (int w = 0; w < 16; ++w) h += part[w][0];
            n_hot[0] = h;
        }
    }
}

hipError_t launch_count_selections(const int32_t *topk_idx, int32_t T, int32_t k, int32_t E, int32_t layer,
                                   int64_t *counts, hipStream_t s) {
    const int64_t P = (int64_t)T * k;
    count_selections_kernel<<<(unsigned)((P + 255) / 256), 256, 0, s>>>(topk_idx, P, E, layer, counts);
    return hipGetLastError();
}

hipError_t launch_hotlist(const int64_t *counts, int32_t n, int32_t *order, int32_t *n_hot, hipStream_t s) {
    hotlist_kernel<<<(n + 63) / 64, 1024, 0, s>>>(counts, n, order, n_hot);
    return hipGetLastError();
}

}  // namespace moe
