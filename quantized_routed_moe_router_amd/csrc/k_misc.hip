// k_misc.hip - RMSNorm before each block ("Understanding Dwarf Star", 5.2.1
// norm + residual, 5.6.2 step 1), the dequantization test hook
// ("Understanding Dwarf Star", 2.8.2 steps 1-3), and a plain read stream
// that measures the HBM bandwidth one launch can reach.
#include "common.h"

namespace moe {

// One block per row: sum of squares in fp32 (fixed reduction tree), then
// out = gamma * x / sqrt(mean + eps).
__global__ void __launch_bounds__(256) rmsnorm_kernel(const float *__restrict__ x, const float *__restrict__ gamma,
                                                      float eps, int D, float *__restrict__ out) {
    __shared__ float red[4];
    int t = blockIdx.x;
    const float *xr = x + (int64_t)t * D;
    float ss = 0.f;
#pragma unroll 4
    for (int i = threadIdx.x; i < D; i += 256) ss = __builtin_fmaf(xr[i], xr[i], ss);
    for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o, kWave);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    float tot = (red[0] + red[1]) + (red[2] + red[3]);
    float inv = 1.0f / sqrtf(tot / (float)D + eps);
    __syncthreads();  // all reads of x done before an in-place write
    for (int i = threadIdx.x; i < D; i += 256) out[(int64_t)t * D + i] = gamma[i] * (xr[i] * inv);
}

// D = 1024 NV with 16-byte aligned rows: every load of a thread (NV x and NV
// gamma, 16 bytes each) is issued before the first is used, and the values
// stay in registers for the output, so the row costs one memory round trip
// instead of one per element a thread holds.  A thread writes only the
// elements it read, so out may be x.
template <int NV>
__global__ void __launch_bounds__(256) rmsnorm_vec_kernel(const float *__restrict__ x, const float *__restrict__ gamma,
                                                          float eps, float *__restrict__ out) {
    __shared__ float red[4];
    constexpr int D = 1024 * NV;
    const int t = blockIdx.x;
    const f32x4 *xr = (const f32x4 *)(x + (int64_t)t * D), *gr = (const f32x4 *)gamma;
    f32x4 v[NV], g[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) v[i] = xr[threadIdx.x + 256 * i];
#pragma unroll
    for (int i = 0; i < NV; ++i) g[i] = gr[threadIdx.x + 256 * i];
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) ss = __builtin_fmaf(v[i][j], v[i][j], ss);
    for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o, kWave);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    const float tot = (red[0] + red[1]) + (red[2] + red[3]);
    const float inv = 1.0f / sqrtf(tot / (float)D + eps);
    f32x4 *orow = (f32x4 *)(out + (int64_t)t * D);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        f32x4 r;
#pragma unroll
        for (int j = 0; j < 4; ++j) r[j] = g[i][j] * (v[i][j] * inv);
        orow[threadIdx.x + 256 * i] = r;
    }
}

hipError_t launch_rmsnorm(const float *x, const float *gamma, float eps, int32_t T, int32_t D, float *out,
                          hipStream_t s) {
    const bool al = ((uintptr_t)x % 16 == 0) && ((uintptr_t)gamma % 16 == 0) && ((uintptr_t)out % 16 == 0);
    if (al && D == 4096) rmsnorm_vec_kernel<4><<<T, 256, 0, s>>>(x, gamma, eps, out);
    else if (al && D == 2048) rmsnorm_vec_kernel<2><<<T, 256, 0, s>>>(x, gamma, eps, out);
    else if (al && D == 1024) rmsnorm_vec_kernel<1><<<T, 256, 0, s>>>(x, gamma, eps, out);
    else rmsnorm_kernel<<<T, 256, 0, s>>>(x, gamma, eps, D, out);
    return hipGetLastError();
}

MOE_DEV void store_vals(void *dst, int out_bf16, int64_t at, const float *w, int n) {
    if (out_bf16) {
        uint16_t *o = (uint16_t *)dst + at;
        for (int i = 0; i < n; ++i) o[i] = (uint16_t)float_to_bf16_bits(w[i]);
    } else {
        float *o = (float *)dst + at;
        for (int i = 0; i < n; ++i) o[i] = w[i];
    }
}

// One thread per 64-weight chunk (Q2K, CB2, Q4K) or per 32-weight block (Q8_0).
__global__ void __launch_bounds__(256) dequant_kernel(int type, const uint8_t *__restrict__ src, int64_t nunits,
                                                      const int8_t *__restrict__ cb, int out_bf16, void *dst) {
    __shared__ uint32_t cb_lds[512];
    if (type == MOE_CB2) {
        for (int i = threadIdx.x; i < 512; i += blockDim.x) cb_lds[i] = ((const uint32_t *)cb)[i];
    }
    __syncthreads();
    int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (u >= nunits) return;
    float w[64];
    if (type == MOE_Q2K) {
        q2k_values(q2k_load(src, 64 * u), w);
        store_vals(dst, out_bf16, 64 * u, w, 64);
    } else if (type == MOE_CB2) {
        cb2_values(cb2_load(src, 64 * u), cb_lds, w);
        store_vals(dst, out_bf16, 64 * u, w, 64);
    } else if (type == MOE_Q4K) {
        q4k_values(q4k_load(src, 64 * u), w);
        store_vals(dst, out_bf16, 64 * u, w, 64);
    } else {
        q8_block_values(src + u * kQ8Bytes, w);
        store_vals(dst, out_bf16, 32 * u, w, 32);
    }
}

hipError_t launch_dequant(int32_t type, const void *src, int64_t n, const int8_t *cb, int32_t out_type, void *dst,
                          hipStream_t s) {
    int64_t units = type == MOE_Q8_0 ? n / 32 : n / 64;
    dequant_kernel<<<(unsigned)((units + 255) / 256), 256, 0, s>>>(type, (const uint8_t *)src, units, cb,
                                                                 out_type == MOE_BF16, dst);
    return hipGetLastError();
}

// Plain read stream: every 16-byte unit of src read once (four loads in
// flight per thread, the grid striding over the buffer), folded by XOR into
// one word per wave so that no load can be dropped.  sink: gridDim.x * 4
// words.
__global__ void __launch_bounds__(256) read_stream_kernel(const u32x4 *__restrict__ src, int64_t n16,
                                                          uint32_t *__restrict__ sink) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    uint32_t acc = 0;
    int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const u32x4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
        acc ^= a[0] ^ a[1] ^ a[2] ^ a[3] ^ b[0] ^ b[1] ^ b[2] ^ b[3] ^ c[0] ^ c[1] ^ c[2] ^ c[3] ^ d[0] ^ d[1] ^
               d[2] ^ d[3];
    }
    for (; i < n16; i += stride) {
        const u32x4 a = src[i];
        acc ^= a[0] ^ a[1] ^ a[2] ^ a[3];
    }
    for (int o = 32; o > 0; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o, kWave);
    if ((threadIdx.x & 63) == 0) sink[blockIdx.x * 4 + (threadIdx.x >> 6)] = acc;
}

hipError_t launch_read_stream(const void *src, int64_t bytes, uint32_t *sink, int32_t blocks, hipStream_t s) {
    read_stream_kernel<<<blocks, 256, 0, s>>>((const u32x4 *)src, bytes / 16, sink);
    return hipGetLastError();
}

}  // namespace moe
