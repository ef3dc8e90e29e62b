// Measurement probes: the streaming rate of HBM and the bf16 MFMA rate that the
// chip sustains on the card in use, the denominators of the measured roofline
// fractions next to the nominal ones (8 TB/s, 2.5 PFLOP/s dense bf16).
//
//  - probe_read_kernel: every workgroup streams a contiguous share of a buffer
//    with 16-byte loads, four in flight per lane, and folds them into one word
//    (so that no load is dead).  A buffer far larger than the 256 MB last-level
//    cache gives the HBM read rate, the bound of the decode kernels.
//  - probe_copy_kernel: the same access pattern, storing what it reads.
//  - probe_mfma_kernel: each wave issues independent 16x16x32 bf16 MFMAs into
//    eight accumulators from four operand pairs of pseudo-random bits (the
//    multiplier inputs change from one MFMA to the next, as in a GEMM, so the
//    power draw and hence the clock are those of real work).  Two waves per
//    SIMD on every compute unit.
#include "common.cuh"
#include "kernels.h"

namespace llb {

namespace {

// Workgroup g streams the contiguous 16-byte units [beg, end) of the buffer,
// 16 KB per iteration (four 4 KB rows of the workgroup's 256 lanes).
struct Share {
    size_t beg, end;
};
LLB_DEV Share share_of(size_t n16) {
    const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
    const size_t beg = min((size_t)blockIdx.x * per, n16);
    return {beg, min(beg + per, n16)};
}

__global__ void __launch_bounds__(256) probe_read_kernel(const uint4* __restrict__ src, size_t n16,
                                                         uint32_t* __restrict__ sink) {
    const Share sh = share_of(n16);
    size_t i = sh.beg + threadIdx.x;
    uint32_t acc = 0;
    for (; i + 768 < sh.end; i += 1024) {
        const uint4 a = src[i], b = src[i + 256], c = src[i + 512], d = src[i + 768];
        acc ^= (a.x ^ a.y ^ a.z ^ a.w) ^ (b.x ^ b.y ^ b.z ^ b.w) ^ (c.x ^ c.y ^ c.z ^ c.w) ^
               (d.x ^ d.y ^ d.z ^ d.w);
    }
    for (; i < sh.end; i += 256) {
        const uint4 a = src[i];
        acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    // one word per workgroup: the xor over its lanes
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) acc ^= __shfl_xor(acc, o, 64);
    __shared__ uint32_t s[4];
    if ((threadIdx.x & 63) == 0) s[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = s[0] ^ s[1] ^ s[2] ^ s[3];
}

__global__ void __launch_bounds__(256) probe_copy_kernel(uint4* __restrict__ dst, const uint4* __restrict__ src,
                                                         size_t n16) {
    const Share sh = share_of(n16);
    size_t i = sh.beg + threadIdx.x;
    for (; i + 768 < sh.end; i += 1024) {
        const uint4 a = src[i], b = src[i + 256], c = src[i + 512], d = src[i + 768];
        dst[i] = a;
        dst[i + 256] = b;
        dst[i + 512] = c;
        dst[i + 768] = d;
    }
    for (; i < sh.end; i += 256) dst[i] = src[i];
}

// bf16 bits with a pseudo-random sign and mantissa and an exponent in [2^-4, 2^3]:
// finite products, and accumulators that stay finite over the probe.
LLB_DEV uint32_t rand_bf16x2(uint32_t h) {
    h ^= h >> 15;
    h *= 0x2c1b3c6du;
    h ^= h >> 12;
    const uint32_t lo = (h & 0x807fu) | ((123u + ((h >> 7) & 7u)) << 7);
    const uint32_t hi = ((h >> 16) & 0x807fu) | ((123u + ((h >> 23) & 7u)) << 7);
    return lo | (hi << 16);
}

__global__ void __launch_bounds__(256) probe_mfma_kernel(float* __restrict__ sink, int iters) {
    const uint32_t id = blockIdx.x * 256 + threadIdx.x;
    bf16x8 a[4], b[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        uint4 ua, ub;
        ua.x = rand_bf16x2(id * 16 + 8 * k + 0); ua.y = rand_bf16x2(id * 16 + 8 * k + 1);
        ua.z = rand_bf16x2(id * 16 + 8 * k + 2); ua.w = rand_bf16x2(id * 16 + 8 * k + 3);
        ub.x = rand_bf16x2(id * 16 + 8 * k + 4); ub.y = rand_bf16x2(id * 16 + 8 * k + 5);
        ub.z = rand_bf16x2(id * 16 + 8 * k + 6); ub.w = rand_bf16x2(id * 16 + 8 * k + 7);
        a[k] = as_bf16x8(ua);
        b[k] = as_bf16x8(ub);
    }
    f32x4 acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    // The MFMAs are written as instructions that accumulate in place in AGPRs:
    // from the builtin, the register allocator rotated the accumulators between
    // iterations and chained consecutive MFMAs through the copies.
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
            asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0"
                         : "+a"(acc[j])
                         : "v"(a[j & 3]), "v"(b[(j + (j >> 2)) & 3]));
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
    s = warp_sum(s);
    if ((threadIdx.x & 63) == 0) sink[blockIdx.x * 4 + (threadIdx.x >> 6)] = s;
}

}  // namespace

hipError_t probe_read_launch(const void* src, size_t bytes, uint32_t* sink, int n_wg, hipStream_t s) {
    if (!src || !sink || bytes % 16 != 0 || n_wg <= 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL(probe_read_kernel, dim3(n_wg), dim3(256), 0, s, (const uint4*)src, bytes / 16, sink);
    return hipGetLastError();
}

hipError_t probe_copy_launch(void* dst, const void* src, size_t bytes, int n_wg, hipStream_t s) {
    if (!src || !dst || bytes % 16 != 0 || n_wg <= 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL(probe_copy_kernel, dim3(n_wg), dim3(256), 0, s, (uint4*)dst, (const uint4*)src, bytes / 16);
    return hipGetLastError();
}

hipError_t probe_mfma_launch(float* sink, int n_wg, int iters, hipStream_t s) {
    if (!sink || n_wg <= 0 || iters <= 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL(probe_mfma_kernel, dim3(n_wg), dim3(256), 0, s, sink, iters);
    return hipGetLastError();
}

}  // namespace llb
