// The model around the blocks: the token embedding gather and the rows that
// reach the LM head ("Llama 3.1 70B", the embedding and LM head sections: the
// embedding looks up one row of the table per token; the head applies the final
// RMSNorm and one linear map to the vocabulary).
#include "common.cuh"
#include "kernels.h"

namespace llb {

namespace {

// x[m, :] = fp32(E[tok[m], :]) for the bf16 table E [vocab, d]; 8 columns per
// thread (one 16-byte load, two 16-byte stores).  An id outside [0, vocab)
// yields a row of NaN, so the table is never read out of range.
__global__ void __launch_bounds__(256)
embed_kernel(const int* __restrict__ tok, const bf16_t* __restrict__ E, float* __restrict__ x, int M,
             int d, int vocab) {
    const int cpr = d / 8;
    const long idx = (long)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (long)M * cpr) return;
    const int m = (int)(idx / cpr);
    const int c = (int)(idx % cpr) * 8;
    const int t = tok[m];
    float v[8];
    if (t >= 0 && t < vocab) {
        unpack_bf16x8(*(const uint4*)(E + (size_t)t * d + c), v);
    } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = __builtin_nanf("");
    }
    float* dst = x + (size_t)m * d + c;
    *(float4*)dst = make_float4(v[0], v[1], v[2], v[3]);
    *(float4*)(dst + 4) = make_float4(v[4], v[5], v[6], v[7]);
}

// dst[b, :] = src[b * T + T - 1, :] (fp32, 4 columns per thread).
__global__ void __launch_bounds__(256)
last_rows_kernel(const float* __restrict__ src, float* __restrict__ dst, int B, int T, int d) {
    const int cpr = d / 4;
    const long idx = (long)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (long)B * cpr) return;
    const int b = (int)(idx / cpr);
    const int c = (int)(idx % cpr) * 4;
    *(float4*)(dst + (size_t)b * d + c) = *(const float4*)(src + ((size_t)b * T + T - 1) * d + c);
}

}  // namespace

hipError_t embed_launch(const int* tok, const void* E, float* x, int M, int d, int vocab, hipStream_t s) {
    if (M <= 0 || d <= 0 || d % 8 != 0 || vocab <= 0) return hipErrorInvalidValue;
    const long n = (long)M * (d / 8);
    hipLaunchKernelGGL(embed_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, tok,
                       (const bf16_t*)E, x, M, d, vocab);
    return hipGetLastError();
}

hipError_t last_rows_launch(const float* src, float* dst, int B, int T, int d, hipStream_t s) {
    if (B <= 0 || T <= 0 || d <= 0 || d % 4 != 0) return hipErrorInvalidValue;
    const long n = (long)B * (d / 4);
    hipLaunchKernelGGL(last_rows_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, src, dst, B,
                       T, d);
    return hipGetLastError();
}

}  // namespace llb
