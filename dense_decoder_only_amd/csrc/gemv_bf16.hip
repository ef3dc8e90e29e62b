// Small-M bf16 projection for decode (M = batch <= 64 tokens): weight streaming.
//
// Decode multiplies a few token rows by every weight once, so the time is the
// weight bytes over HBM bandwidth.  Each workgroup streams a 64-row x KS slab
// of W straight from global memory into MFMA operand registers (W rows are
// K-contiguous, so a 32x32x16 fragment is one 16-byte load per lane); the
// token fragments (bf16, a few hundred KB in total) come from L2.  Per wave the
// loads of one 64-wide k step are issued in the order [tokens(it), W(it + 1)],
// so the wait for this step's operands leaves the next step's weights in
// flight.  The 4 waves of a workgroup split the slab's K range and are summed
// through LDS; workgroups along grid.y split K further and write fp32
// partials, which a second kernel sums in split order and passes through the
// epilogue.
#include "common.cuh"
#include "epilogue.cuh"
#include "kernels.h"

namespace llb {

namespace {

constexpr int GV_ROWS = 64;    // W rows per workgroup
constexpr int GV_UNROLL = 4;   // k-steps of 16 per pipeline step (64 k)
constexpr int GV_KQUANT = 4 * 16 * GV_UNROLL;  // K granularity of one split (256)

template <int MT>
__global__ void __launch_bounds__(256)
gemv_bf16_kernel(GemmArgs args, int KS, float* __restrict__ part) {
    constexpr int MS = MT / 32;
    constexpr int U = GV_UNROLL;
    __shared__ float sRed[4][MT * GV_ROWS];

    const int M = args.M, N = args.N, K = args.K;
    const int n0 = blockIdx.x * GV_ROWS;
    const int split = blockIdx.y;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int KW = KS / 4;
    const int kw0 = split * KS + wave * KW;
    const int kl = 8 * (lane >> 5);
    const int n_it = KW / (16 * U);

    const bf16_t* __restrict__ W = (const bf16_t*)args.W;
    const bf16_t* __restrict__ A = (const bf16_t*)args.A;
    const bf16_t* wrow0 = W + (size_t)(n0 + (lane & 31)) * K + kw0 + kl;
    const bf16_t* wrow1 = wrow0 + (size_t)32 * K;
    const bf16_t* arow[MS];
    bool tok_ok[MS];
#pragma unroll
    for (int ms = 0; ms < MS; ++ms) {
        const int tok = ms * 32 + (lane & 31);
        tok_ok[ms] = tok < M;
        arow[ms] = A + (size_t)(tok_ok[ms] ? tok : 0) * K + kw0 + kl;
    }

    f32x16 acc[MS][2];
#pragma unroll
    for (int ms = 0; ms < MS; ++ms)
#pragma unroll
        for (int ns = 0; ns < 2; ++ns)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[ms][ns][r] = 0.f;

    uint4 wa[U][2], wb[U][2];
    auto load_w = [&](uint4 (&w)[U][2], int it) {
        const int k = it * 16 * U;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            w[u][0] = *(const uint4*)(wrow0 + k + 16 * u);
            w[u][1] = *(const uint4*)(wrow1 + k + 16 * u);
        }
    };
    auto load_a = [&](bf16x8 (&af)[U][MS], int it) {
        const int k = it * 16 * U;
#pragma unroll
        for (int ms = 0; ms < MS; ++ms)
#pragma unroll
            for (int u = 0; u < U; ++u)
                af[u][ms] = as_bf16x8(tok_ok[ms] ? *(const uint4*)(arow[ms] + k + 16 * u)
                                                 : make_uint4(0, 0, 0, 0));
    };
    auto mma = [&](const uint4 (&w)[U][2], const bf16x8 (&af)[U][MS]) {
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int ms = 0; ms < MS; ++ms)
#pragma unroll
                for (int ns = 0; ns < 2; ++ns)
                    acc[ms][ns] = mfma32(af[u][ms], as_bf16x8(w[u][ns]), acc[ms][ns]);
    };

    load_w(wa, 0);
    for (int it = 0; it < n_it; it += 2) {
        bf16x8 af[U][MS];
        load_a(af, it);
        if (it + 1 < n_it) load_w(wb, it + 1);
        mma(wa, af);
        if (it + 1 < n_it) {
            load_a(af, it + 1);
            if (it + 2 < n_it) load_w(wa, it + 2);
            mma(wb, af);
        }
    }

    // acc[ms][ns]: lane -> W row n0 + 32*ns + (lane & 31); reg r -> token
    // 32*ms + 8*(r/4) + 4*(lane/32) + r%4.
#pragma unroll
    for (int ms = 0; ms < MS; ++ms)
#pragma unroll
        for (int ns = 0; ns < 2; ++ns)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int tok = ms * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                sRed[wave][tok * GV_ROWS + ns * 32 + (lane & 31)] = acc[ms][ns][r];
            }
    __syncthreads();
    for (int e = threadIdx.x; e < MT * GV_ROWS; e += 256) {
        const int tok = e / GV_ROWS;
        const int nl = e % GV_ROWS;
        if (tok < M) {
            const float v = (sRed[0][e] + sRed[1][e]) + (sRed[2][e] + sRed[3][e]);
            part[((size_t)split * M + tok) * N + n0 + nl] = v;
        }
    }
}

LLB_DEV float row_scale(const GemmArgs& a, int m) {
    float s = 0.f;
    for (int p = 0; p < a.ssq_count; ++p) s += a.ssq_in[(size_t)p * a.M + m];
    return inv_rms(s, a.K, a.eps);
}

// Sums the split partials in split order, applies the row's inverse RMS (QKV,
// SwiGLU) and the epilogue.  One thread per RoPE pair (QKV), output (RESID) or
// SwiGLU feature (SWIGLU).
template <int EPI>
__global__ void __launch_bounds__(256)
splitk_epilogue_kernel(GemmArgs args, int splits, const float* __restrict__ part) {
    const int M = args.M, N = args.N;
    const int per_row = (EPI == EPI_RESID) ? N : (N >> 1);
    const long idx = (long)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (long)M * per_row) return;
    const int m = (int)(idx / per_row);
    const int c = (int)(idx - (long)m * per_row);
    const float sc = (EPI == EPI_RESID) ? 1.0f : row_scale(args, m);
    auto sum_col = [&](int n) {
        float v = 0.f;
        for (int sp = 0; sp < splits; ++sp) v += part[((size_t)sp * M + m) * N + n];
        return v * sc;
    };
    const Epilogue& e = args.epi;
    if constexpr (EPI == EPI_QKV) {
        const int n = 2 * c;
        const float v0 = sum_col(n), v1 = sum_col(n + 1);
        epi_qkv<bf16_t>(e, m, n, v0, v1);
        epi_qkv<bf16_t>(e, m, n + 1, v1, v0);
    } else if constexpr (EPI == EPI_SWIGLU) {
        const int ng = (c >> 5) * 64 + (c & 31);
        epi_swiglu<bf16_t>(e, m, c, N >> 1, sum_col(ng), sum_col(ng + 32));
    } else {
        epi_resid(e, m, c, N, sum_col(c));
    }
}

// EPI_RESID_NORM for decode: one workgroup per row; h = resid + sum of the
// partials, the next RMSNorm's operand bf16(h * g) and the full row sum of h^2.
__global__ void __launch_bounds__(256)
splitk_resid_norm_kernel(GemmArgs args, int splits, const float* __restrict__ part) {
    __shared__ float sRed[4];
    const int M = args.M, N = args.N;
    const int m = blockIdx.x;
    const Epilogue& e = args.epi;
    float ss = 0.f;
    for (int n = threadIdx.x; n < N; n += 256) {
        float v = 0.f;
        for (int sp = 0; sp < splits; ++sp) v += part[((size_t)sp * M + m) * N + n];
        const float h = epi_resid(e, m, n, N, v);
        epi_norm_operand(e, m, n, N, h);
        ss += h * h;
    }
    ss = warp_sum(ss);
    if ((threadIdx.x & 63) == 0) sRed[threadIdx.x >> 6] = ss;
    __syncthreads();
    if (threadIdx.x == 0) e.ssq_out[m] = (sRed[0] + sRed[1]) + (sRed[2] + sRed[3]);
}

template <int MT>
hipError_t launch_main(const GemmArgs& a, int splits, float* part, hipStream_t s) {
    const int KS = a.K / splits;
    hipLaunchKernelGGL((gemv_bf16_kernel<MT>), dim3(a.N / GV_ROWS, splits), dim3(256), 0, s, a,
                       KS, part);
    return hipGetLastError();
}

template <int EPI>
hipError_t launch_epi(const GemmArgs& a, int splits, const float* part, hipStream_t s) {
    const long per_row = (EPI == EPI_RESID) ? a.N : (a.N >> 1);
    const long total = (long)a.M * per_row;
    hipLaunchKernelGGL((splitk_epilogue_kernel<EPI>), dim3((unsigned)((total + 255) / 256)),
                       dim3(256), 0, s, a, splits, part);
    return hipGetLastError();
}

}  // namespace

// Split count: enough workgroups to cover the GPU (>= ~512), each split a
// multiple of 256 in K.
int gemv_bf16_splits(int M, int N, int K) {
    (void)M;
    const int tiles = N / GV_ROWS;
    const int want = (512 + tiles - 1) / tiles;
    const int qmax = K / GV_KQUANT;
    for (int s = want; s <= qmax; ++s)
        if (qmax % s == 0) return s;
    for (int s = want; s >= 1; --s)
        if (qmax % s == 0) return s;
    return 1;
}

size_t gemv_bf16_ws_bytes(int M, int N, int splits) {
    return (size_t)splits * M * N * sizeof(float);
}

hipError_t gemv_bf16_launch(const GemmArgs& a, int splits, float* ws, hipStream_t s) {
    if (a.M <= 0 || a.M > 64 || a.N % GV_ROWS != 0 || splits < 1 ||
        a.K % (splits * GV_KQUANT) != 0)
        return hipErrorInvalidValue;
    hipError_t err = a.M <= 32 ? launch_main<32>(a, splits, ws, s) : launch_main<64>(a, splits, ws, s);
    if (err != hipSuccess) return err;
    switch (a.epi.kind) {
        case EPI_QKV: return launch_epi<EPI_QKV>(a, splits, ws, s);
        case EPI_SWIGLU: return launch_epi<EPI_SWIGLU>(a, splits, ws, s);
        case EPI_RESID: return launch_epi<EPI_RESID>(a, splits, ws, s);
        case EPI_RESID_NORM:
            hipLaunchKernelGGL(splitk_resid_norm_kernel, dim3(a.M), dim3(256), 0, s, a, splits, ws);
            return hipGetLastError();
        default: return hipErrorInvalidValue;
    }
}

// ---------------------------------------------------------------------------
// RMSNorm operand: one wave per row.  a[m, j] = bf16(x[m, j] * g[j]) (one
// rounding) and ssq[m] = sum_j x[m, j]^2 accumulated in fp32 across the wave
// ("Llama 3.1 70B", section "RMSNorm": the reduction is done in fp32).  The
// inverse RMS itself is applied to the fp32 results of the projection.
__global__ void __launch_bounds__(256)
norm_rows_kernel(const float* __restrict__ x, const float* __restrict__ g, bf16_t* __restrict__ a,
                 float* __restrict__ ssq, int M, int d) {
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= M) return;
    const float* xr = x + (size_t)row * d;
    bf16_t* ar = a + (size_t)row * d;
    float s = 0.f;
    for (int j = lane * 8; j < d; j += 64 * 8) {
        const float4 v0 = *(const float4*)(xr + j);
        const float4 v1 = *(const float4*)(xr + j + 4);
        const float4 g0 = *(const float4*)(g + j);
        const float4 g1 = *(const float4*)(g + j + 4);
        s += v0.x * v0.x + v0.y * v0.y + v0.z * v0.z + v0.w * v0.w;
        s += v1.x * v1.x + v1.y * v1.y + v1.z * v1.z + v1.w * v1.w;
        uint4 p;
        p.x = pack_bf16x2(v0.x * g0.x, v0.y * g0.y);
        p.y = pack_bf16x2(v0.z * g0.z, v0.w * g0.w);
        p.z = pack_bf16x2(v1.x * g1.x, v1.y * g1.y);
        p.w = pack_bf16x2(v1.z * g1.z, v1.w * g1.w);
        *(uint4*)(ar + j) = p;
    }
    s = warp_sum(s);
    if (lane == 0) ssq[row] = s;
}

hipError_t norm_rows_launch(const float* x, const float* g, void* a, float* ssq, int M, int d,
                            hipStream_t s) {
    if (M <= 0 || d % 8 != 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL(norm_rows_kernel, dim3((M + 3) / 4), dim3(256), 0, s, x, g, (bf16_t*)a, ssq,
                       M, d);
    return hipGetLastError();
}

}  // namespace llb
