// fp32 path: projections and attention for blocks whose weights and cache are
// fp32 (small shapes; launch-latency bound).  Same epilogues and the same
// fused RMSNorm as the bf16 path, computed on the vector ALU without rounding.
#include "common.cuh"
#include "epilogue.cuh"
#include "kernels.h"

namespace llb {

namespace {

// 64x64 output tile, K step 16, 256 threads.  Thread (tx, ty) owns rows
// 4ty..4ty+3 and columns {2tx, 2tx+1, 32+2tx, 33+2tx}: RoPE pairs (2tx, 2tx+1)
// and SwiGLU gate/up pairs (c, c+32) are both inside one thread.
template <bool NORM, int EPI>
__global__ void __launch_bounds__(256) gemm_f32_kernel(GemmArgs args) {
    __shared__ float sA[16][64 + 4];
    __shared__ float sB[16][64 + 4];
    __shared__ float sScale[64];
    const int M = args.M, N = args.N, K = args.K;
    const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
    const int tid = threadIdx.x;
    const float* __restrict__ A = (const float*)args.A;
    const float* __restrict__ W = (const float*)args.W;

    if constexpr (NORM) {
        const int r = tid >> 2, q = tid & 3;
        float s = 0.f;
        if (m0 + r < M) {
            const float* row = A + (size_t)(m0 + r) * K;
            for (int k = q; k < K; k += 4) s += row[k] * row[k];
        }
        s += __shfl_xor(s, 1, 64);
        s += __shfl_xor(s, 2, 64);
        if (q == 0) sScale[r] = inv_rms(s, K, args.eps);
        __syncthreads();
    }

    const int tx = tid & 15, ty = tid >> 4;
    float acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;
    const int cols[4] = {2 * tx, 2 * tx + 1, 32 + 2 * tx, 33 + 2 * tx};

    const int lr = tid >> 2, lk = (tid & 3) * 4;
    for (int k0 = 0; k0 < K; k0 += 16) {
        float4 av = make_float4(0.f, 0.f, 0.f, 0.f);
        if (m0 + lr < M) av = *(const float4*)(A + (size_t)(m0 + lr) * K + k0 + lk);
        if constexpr (NORM) {
            const float4 gv = *(const float4*)(args.gain + k0 + lk);
            av.x *= gv.x; av.y *= gv.y; av.z *= gv.z; av.w *= gv.w;
        }
        const float4 bv = *(const float4*)(W + (size_t)(n0 + lr) * K + k0 + lk);
        sA[lk + 0][lr] = av.x; sA[lk + 1][lr] = av.y; sA[lk + 2][lr] = av.z; sA[lk + 3][lr] = av.w;
        sB[lk + 0][lr] = bv.x; sB[lk + 1][lr] = bv.y; sB[lk + 2][lr] = bv.z; sB[lk + 3][lr] = bv.w;
        __syncthreads();
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            float a[4], bb[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = sA[k][ty * 4 + i];
#pragma unroll
            for (int j = 0; j < 4; ++j) bb[j] = sB[k][cols[j]];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] += a[i] * bb[j];
        }
        __syncthreads();
    }

    const Epilogue& e = args.epi;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int rl = ty * 4 + i;
        const int m = m0 + rl;
        if (m >= M) continue;
        const float sc = NORM ? sScale[rl] : 1.0f;
        float v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = acc[i][j] * sc;
        if constexpr (EPI == EPI_QKV) {
#pragma unroll
            for (int p = 0; p < 4; p += 2) {
                const int n = n0 + cols[p];
                epi_qkv<float>(e, m, n, v[p], v[p + 1]);
                epi_qkv<float>(e, m, n + 1, v[p + 1], v[p]);
            }
        } else if constexpr (EPI == EPI_SWIGLU) {
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                const int f = (n0 >> 1) + cols[p];
                epi_swiglu<float>(e, m, f, N >> 1, v[p], v[p + 2]);
            }
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) epi_resid(e, m, n0 + cols[j], N, v[j]);
        }
    }
}

// One wave per (query, head, sequence): online softmax over key blocks of 64.
__global__ void __launch_bounds__(64) attn_f32_kernel(AttnArgs a) {
    __shared__ float sq[128];
    __shared__ float sp[64];
    const int t = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int lane = threadIdx.x;
    const int hd = a.hd;
    const int G = a.n_heads / a.n_kv;
    const int g = h / G;
    const int pos = seq_start(a, b) + t;
    const int L = pos + 1;
    const float* q = (const float*)a.q + (((size_t)b * a.n_heads + h) * a.T + t) * hd;
    const size_t head_off = ((size_t)b * a.n_kv + g) * a.cap * hd;
    const float* Kg = (const float*)a.k_cache + head_off;
    const float* Vg = (const float*)a.v_cache + head_off;
    for (int j = lane; j < hd; j += 64) sq[j] = q[j];
    __syncthreads();
    const float scale = 1.0f / sqrtf((float)hd);
    float m_run = -INFINITY, l_run = 0.f, o0 = 0.f, o1 = 0.f;
    for (int kb = 0; kb < L; kb += 64) {
        const int key = kb + lane;
        float s = -INFINITY;
        if (key < L) {
            const float* kr = Kg + (size_t)key * hd;
            float d = 0.f;
            for (int j = 0; j < hd; ++j) d += sq[j] * kr[j];
            s = d * scale;
        }
        const float m_new = fmaxf(m_run, warp_max(s));
        const float alpha = expf(m_run - m_new);
        const float p = key < L ? expf(s - m_new) : 0.f;
        l_run = l_run * alpha + warp_sum(p);
        m_run = m_new;
        sp[lane] = p;
        __syncthreads();
        const int n = min(64, L - kb);
        float a0 = 0.f, a1 = 0.f;
        for (int i = 0; i < n; ++i) {
            const float* vr = Vg + (size_t)(kb + i) * hd;
            a0 += sp[i] * vr[lane];
            if (lane + 64 < hd) a1 += sp[i] * vr[lane + 64];
        }
        o0 = o0 * alpha + a0;
        o1 = o1 * alpha + a1;
        __syncthreads();
    }
    float* orow = (float*)a.o + ((size_t)b * a.T + t) * ((size_t)a.n_heads * hd) + (size_t)h * hd;
    if (lane < hd) orow[lane] = o0 / l_run;
    if (lane + 64 < hd) orow[lane + 64] = o1 / l_run;
}

template <bool NORM, int EPI>
hipError_t launch_f32(const GemmArgs& a, hipStream_t s) {
    hipLaunchKernelGGL((gemm_f32_kernel<NORM, EPI>), dim3(a.N / 64, (a.M + 63) / 64), dim3(256), 0,
                       s, a);
    return hipGetLastError();
}

__global__ void __launch_bounds__(256)
kv_append_kernel(uint4* __restrict__ kc, uint4* __restrict__ vc, const uint4* __restrict__ kn,
                 const uint4* __restrict__ vn, int B, int n_kv, int cap, int pos0, int n_new,
                 int row_chunks) {
    const long idx = (long)blockIdx.x * 256 + threadIdx.x;
    const long total = (long)B * n_kv * n_new * row_chunks;
    if (idx >= total) return;
    const int c = (int)(idx % row_chunks);
    const long r = idx / row_chunks;  // (bg, t)
    const int t = (int)(r % n_new);
    const long bg = r / n_new;
    const size_t dst = ((size_t)bg * cap + pos0 + t) * row_chunks + c;
    kc[dst] = kn[idx];
    vc[dst] = vn[idx];
}

}  // namespace

hipError_t gemm_f32_launch(const GemmArgs& a, hipStream_t s) {
    if (a.M <= 0 || a.N % 64 != 0 || a.K % 16 != 0) return hipErrorInvalidValue;
    if (a.epi.kind == EPI_QKV && a.norm) return launch_f32<true, EPI_QKV>(a, s);
    if (a.epi.kind == EPI_SWIGLU && a.norm) return launch_f32<true, EPI_SWIGLU>(a, s);
    if (a.epi.kind == EPI_RESID && !a.norm) return launch_f32<false, EPI_RESID>(a, s);
    return hipErrorInvalidValue;
}

hipError_t attn_f32_launch(const AttnArgs& a, hipStream_t s) {
    if (a.hd > 128 || a.n_kv <= 0 || a.n_heads % a.n_kv != 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL(attn_f32_kernel, dim3(a.T, a.n_heads, a.B), dim3(64), 0, s, a);
    return hipGetLastError();
}

namespace {
// Up to 64 host integers carried in the kernel's arguments (copied at launch,
// so the host array is free as soon as the launch returns).
struct IntChunk {
    int n;
    int v[64];
};
__global__ void __launch_bounds__(64) store_ints_kernel(int* __restrict__ dst, IntChunk c) {
    if ((int)threadIdx.x < c.n) dst[threadIdx.x] = c.v[threadIdx.x];
}
}  // namespace

hipError_t store_ints_launch(int* dst, const int* src, int n, hipStream_t s) {
    for (int i = 0; i < n; i += 64) {
        IntChunk c;
        c.n = n - i < 64 ? n - i : 64;
        for (int j = 0; j < c.n; ++j) c.v[j] = src[i + j];
        hipLaunchKernelGGL(store_ints_kernel, dim3(1), dim3(64), 0, s, dst + i, c);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t kv_append_launch(void* kc, void* vc, const void* kn, const void* vn, int B, int n_kv,
                            int cap, int pos0, int n_new, int hd, int elem_bytes, hipStream_t s) {
    const int row_bytes = hd * elem_bytes;
    if (row_bytes % 16 != 0) return hipErrorInvalidValue;
    const int row_chunks = row_bytes / 16;
    const long total = (long)B * n_kv * n_new * row_chunks;
    if (total == 0) return hipSuccess;
    hipLaunchKernelGGL(kv_append_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s,
                       (uint4*)kc, (uint4*)vc, (const uint4*)kn, (const uint4*)vn, B, n_kv, cap,
                       pos0, n_new, row_chunks);
    return hipGetLastError();
}

}  // namespace llb
