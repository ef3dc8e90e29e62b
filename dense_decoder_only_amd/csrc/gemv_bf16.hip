// Small-M bf16 projection for decode (M = batch <= 64 tokens): weight streaming.
//
// Decode multiplies a few token rows by every weight once, so the time is the
// weight bytes over HBM bandwidth.  Each workgroup streams a 64-row x KS slab
// of W straight from global memory into MFMA operand registers (W rows are
// K-contiguous, so a 32x32x16 fragment is one 16-byte load per lane); the
// token fragments come from L2 (the activations are a few hundred KB).  The 4
// waves of a workgroup split the slab's K range and are summed through LDS;
// workgroups along grid.y split K further and write fp32 partials, which a
// second kernel sums in a fixed order and passes through the epilogue.
//
// NORM variant: A is the fp32 residual stream; tokens are multiplied by the
// gain and rounded once to bf16 for the MFMA, and each split also emits its
// rows' partial sum of squares so the epilogue can apply the inverse RMS
// ("Llama 3.1 70B", section "RMSNorm", fp32 reduction).
#include "common.cuh"
#include "epilogue.cuh"
#include "kernels.h"

namespace llb {

namespace {

constexpr int GV_ROWS = 64;    // W rows per workgroup
constexpr int GV_UNROLL = 4;   // k-steps of 16 in flight per wave
constexpr int GV_KQUANT = 4 * 16 * GV_UNROLL;  // K granularity of one split (256)

template <int MT, bool NORM>
__global__ void __launch_bounds__(256)
gemv_bf16_kernel(GemmArgs args, int KS, float* __restrict__ part, float* __restrict__ stats) {
    constexpr int MS = MT / 32;
    __shared__ float sRed[4][MT * GV_ROWS];
    __shared__ float sSsq[4][MT];

    const int M = args.M, N = args.N, K = args.K;
    const int n0 = blockIdx.x * GV_ROWS;
    const int split = blockIdx.y;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int KW = KS / 4;
    const int kw0 = split * KS + wave * KW;
    const int kl = 8 * (lane >> 5);

    const bf16_t* __restrict__ W = (const bf16_t*)args.W;
    const bf16_t* wrow0 = W + (size_t)(n0 + (lane & 31)) * K + kl;
    const bf16_t* wrow1 = wrow0 + (size_t)32 * K;

    f32x16 acc[MS][2];
#pragma unroll
    for (int ms = 0; ms < MS; ++ms)
#pragma unroll
        for (int ns = 0; ns < 2; ++ns)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[ms][ns][r] = 0.f;
    float ssq[MS];
#pragma unroll
    for (int ms = 0; ms < MS; ++ms) ssq[ms] = 0.f;

    for (int k = kw0; k < kw0 + KW; k += 16 * GV_UNROLL) {
        uint4 wf[GV_UNROLL][2];
#pragma unroll
        for (int u = 0; u < GV_UNROLL; ++u) {
            wf[u][0] = *(const uint4*)(wrow0 + k + 16 * u);
            wf[u][1] = *(const uint4*)(wrow1 + k + 16 * u);
        }
        bf16x8 af[GV_UNROLL][MS];
#pragma unroll
        for (int ms = 0; ms < MS; ++ms) {
            const int tok = ms * 32 + (lane & 31);
#pragma unroll
            for (int u = 0; u < GV_UNROLL; ++u) {
                const int kk = k + 16 * u + kl;
                if (tok < M) {
                    if constexpr (NORM) {
                        const float* xr = (const float*)args.A + (size_t)tok * K + kk;
                        const float4 x0 = *(const float4*)xr;
                        const float4 x1 = *(const float4*)(xr + 4);
                        const float4 g0 = *(const float4*)(args.gain + kk);
                        const float4 g1 = *(const float4*)(args.gain + kk + 4);
                        ssq[ms] += x0.x * x0.x + x0.y * x0.y + x0.z * x0.z + x0.w * x0.w +
                                   x1.x * x1.x + x1.y * x1.y + x1.z * x1.z + x1.w * x1.w;
                        const float v[8] = {x0.x * g0.x, x0.y * g0.y, x0.z * g0.z, x0.w * g0.w,
                                            x1.x * g1.x, x1.y * g1.y, x1.z * g1.z, x1.w * g1.w};
                        af[u][ms] = to_bf16x8(v);
                    } else {
                        af[u][ms] = as_bf16x8(
                            *(const uint4*)((const bf16_t*)args.A + (size_t)tok * K + kk));
                    }
                } else {
                    af[u][ms] = as_bf16x8(make_uint4(0, 0, 0, 0));
                }
            }
        }
#pragma unroll
        for (int u = 0; u < GV_UNROLL; ++u)
#pragma unroll
            for (int ms = 0; ms < MS; ++ms)
#pragma unroll
                for (int ns = 0; ns < 2; ++ns)
                    acc[ms][ns] = mfma32(af[u][ms], as_bf16x8(wf[u][ns]), acc[ms][ns]);
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
    if constexpr (NORM) {
#pragma unroll
        for (int ms = 0; ms < MS; ++ms) {
            const float s = ssq[ms] + __shfl_xor(ssq[ms], 32, 64);
            if (lane < 32) sSsq[wave][ms * 32 + lane] = s;
        }
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
    if constexpr (NORM) {
        if (blockIdx.x == 0 && threadIdx.x < M) {
            const int t = threadIdx.x;
            stats[(size_t)split * M + t] = (sSsq[0][t] + sSsq[1][t]) + (sSsq[2][t] + sSsq[3][t]);
        }
    }
}

// Sums the split partials in split order, applies the row's inverse RMS (NORM)
// and the epilogue.  One thread per RoPE pair (QKV), output (RESID) or SwiGLU
// feature (SWIGLU).
template <int EPI, bool NORM>
__global__ void __launch_bounds__(256)
splitk_epilogue_kernel(GemmArgs args, int splits, const float* __restrict__ part,
                       const float* __restrict__ stats) {
    const int M = args.M, N = args.N;
    const int per_row = (EPI == EPI_RESID) ? N : (N >> 1);
    const long idx = (long)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (long)M * per_row) return;
    const int m = (int)(idx / per_row);
    const int c = (int)(idx - (long)m * per_row);
    float sc = 1.0f;
    if constexpr (NORM) {
        float s = 0.f;
        for (int sp = 0; sp < splits; ++sp) s += stats[(size_t)sp * M + m];
        sc = inv_rms(s, args.K, args.eps);
    }
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

template <int MT, bool NORM>
hipError_t launch_main(const GemmArgs& a, int splits, float* part, float* stats, hipStream_t s) {
    const int KS = a.K / splits;
    hipLaunchKernelGGL((gemv_bf16_kernel<MT, NORM>), dim3(a.N / GV_ROWS, splits), dim3(256), 0,
                       s, a, KS, part, stats);
    return hipGetLastError();
}

template <int EPI, bool NORM>
hipError_t launch_epi(const GemmArgs& a, int splits, const float* part, const float* stats,
                      hipStream_t s) {
    const long per_row = (EPI == EPI_RESID) ? a.N : (a.N >> 1);
    const long total = (long)a.M * per_row;
    hipLaunchKernelGGL((splitk_epilogue_kernel<EPI, NORM>), dim3((unsigned)((total + 255) / 256)),
                       dim3(256), 0, s, a, splits, part, stats);
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
    return (size_t)splits * M * N * sizeof(float) + (size_t)splits * M * sizeof(float);
}

hipError_t gemv_bf16_launch(const GemmArgs& a, int splits, float* ws, hipStream_t s) {
    if (a.M <= 0 || a.M > 64 || a.N % GV_ROWS != 0 || splits < 1 ||
        a.K % (splits * GV_KQUANT) != 0)
        return hipErrorInvalidValue;
    float* part = ws;
    float* stats = ws + (size_t)splits * a.M * a.N;
    hipError_t err;
    const bool norm = a.norm != 0;
    if (a.M <= 32)
        err = norm ? launch_main<32, true>(a, splits, part, stats, s)
                   : launch_main<32, false>(a, splits, part, stats, s);
    else
        err = norm ? launch_main<64, true>(a, splits, part, stats, s)
                   : launch_main<64, false>(a, splits, part, stats, s);
    if (err != hipSuccess) return err;
    switch (a.epi.kind) {
        case EPI_QKV: return norm ? launch_epi<EPI_QKV, true>(a, splits, part, stats, s)
                                  : hipErrorInvalidValue;
        case EPI_SWIGLU: return norm ? launch_epi<EPI_SWIGLU, true>(a, splits, part, stats, s)
                                     : hipErrorInvalidValue;
        default: return norm ? hipErrorInvalidValue
                             : launch_epi<EPI_RESID, false>(a, splits, part, stats, s);
    }
}

}  // namespace llb
