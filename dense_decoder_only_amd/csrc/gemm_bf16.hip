// Large-M bf16 projection C = A . W^T on gfx950 MFMA (v_mfma_f32_32x32x16_bf16).
//
// Block tile BM x BN, K step 64, double-buffered LDS; both operands are
// K-contiguous ([rows][K] row-major), so every MFMA fragment is one 16-byte LDS
// read.  LDS rows are 128 bytes; the 16-byte chunk index is XOR-swizzled with
// (row & 7) so that the 32 lanes reading one fragment column hit distinct banks.
//
// NORM variant (RMSNorm fused into the prologue, "Llama 3.1 70B", section
// "RMSNorm": y = x / sqrt(mean(x^2) + eps) * g, reduction in fp32): A is the fp32
// residual stream.  While staging a tile the loader multiplies x by the gain,
// rounds once to bf16 for the MFMA, and accumulates sum(x^2) of its rows in
// fp32.  The K loop covers whole rows (K = d_model), so after the loop each
// row's inverse RMS is known and is applied to the fp32 accumulators in the
// epilogue: C = r_m * sum_k bf16(x_mk g_k) W_nk.
#include "common.cuh"
#include "epilogue.cuh"
#include "kernels.h"

namespace llb {

namespace {

constexpr int BK = 64;

template <int BM, int BN, int WAVES_M, int WAVES_N, bool NORM, int EPI>
__global__ void __launch_bounds__(64 * WAVES_M * WAVES_N)
gemm_bf16_kernel(GemmArgs args) {
    constexpr int NT = 64 * WAVES_M * WAVES_N;
    constexpr int WTM = BM / WAVES_M;
    constexpr int WTN = BN / WAVES_N;
    constexpr int TM = WTM / 32;
    constexpr int TN = WTN / 32;
    constexpr int A_PER_T = NORM ? (BM * 16) / NT : (BM * 8) / NT;  // 16-byte chunks per thread
    constexpr int B_PER_T = (BN * 8) / NT;
    static_assert(A_PER_T >= 1 && B_PER_T >= 1, "tile too small for the thread count");
    static_assert(EPI != EPI_SWIGLU || (WTN % 64) == 0, "SwiGLU needs gate/up pairs in a wave");

    __shared__ __attribute__((aligned(16))) bf16_t sA[2][BM * BK];
    __shared__ __attribute__((aligned(16))) bf16_t sB[2][BN * BK];
    __shared__ float sScale[NORM ? BM : 1];

    const int M = args.M, N = args.N, K = args.K;
    const int tiles_m = (M + BM - 1) / BM;
    const int tiles_n = N / BN;
    const int tile = xcd_remap(blockIdx.x, tiles_m * tiles_n);
    const int m0 = (tile % tiles_m) * BM;
    const int n0 = (tile / tiles_m) * BN;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave % WAVES_M;
    const int wn = wave / WAVES_M;

    const bf16_t* __restrict__ W = (const bf16_t*)args.W;

    uint4 ra[A_PER_T];
    uint4 rb[B_PER_T];
    float4 rg = make_float4(0.f, 0.f, 0.f, 0.f);
    float ssq[NORM ? A_PER_T : 1];
#pragma unroll
    for (int i = 0; i < (NORM ? A_PER_T : 1); ++i) ssq[i] = 0.f;

    auto load_tile = [&](int kt) {
        const int k0 = kt * BK;
        if constexpr (NORM) {
            const float* __restrict__ A = (const float*)args.A;
            const int c4 = tid & 15;
            rg = *(const float4*)(args.gain + k0 + c4 * 4);
#pragma unroll
            for (int i = 0; i < A_PER_T; ++i) {
                const int gm = m0 + (tid >> 4) + i * (NT / 16);
                ra[i] = gm < M ? *(const uint4*)(A + (size_t)gm * K + k0 + c4 * 4)
                               : make_uint4(0, 0, 0, 0);
            }
        } else {
            const bf16_t* __restrict__ A = (const bf16_t*)args.A;
            const int c8 = tid & 7;
#pragma unroll
            for (int i = 0; i < A_PER_T; ++i) {
                const int gm = m0 + (tid >> 3) + i * (NT / 8);
                ra[i] = gm < M ? *(const uint4*)(A + (size_t)gm * K + k0 + c8 * 8)
                               : make_uint4(0, 0, 0, 0);
            }
        }
        const int c8 = tid & 7;
#pragma unroll
        for (int i = 0; i < B_PER_T; ++i) {
            const int row = (tid >> 3) + i * (NT / 8);
            rb[i] = *(const uint4*)(W + (size_t)(n0 + row) * K + k0 + c8 * 8);
        }
    };

    auto store_tile = [&](int buf) {
        if constexpr (NORM) {
            const int c4 = tid & 15;
            const int c = c4 >> 1, half = c4 & 1;
#pragma unroll
            for (int i = 0; i < A_PER_T; ++i) {
                const int row = (tid >> 4) + i * (NT / 16);
                const float4 v = __builtin_bit_cast(float4, ra[i]);
                ssq[i] += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
                uint2 p;
                p.x = pack_bf16x2(v.x * rg.x, v.y * rg.y);
                p.y = pack_bf16x2(v.z * rg.z, v.w * rg.w);
                *(uint2*)&sA[buf][row * BK + ((c ^ (row & 7)) << 3) + (half << 2)] = p;
            }
        } else {
            const int c = tid & 7;
#pragma unroll
            for (int i = 0; i < A_PER_T; ++i) {
                const int row = (tid >> 3) + i * (NT / 8);
                *(uint4*)&sA[buf][row * BK + ((c ^ (row & 7)) << 3)] = ra[i];
            }
        }
        const int c = tid & 7;
#pragma unroll
        for (int i = 0; i < B_PER_T; ++i) {
            const int row = (tid >> 3) + i * (NT / 8);
            *(uint4*)&sB[buf][row * BK + ((c ^ (row & 7)) << 3)] = rb[i];
        }
    };

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    auto compute = [&](int buf) {
        const bf16_t* a_s = sA[buf];
        const bf16_t* b_s = sB[buf];
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            const int c = kk * 2 + (lane >> 5);
            bf16x8 af[TM], bfr[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const int r = wm * WTM + i * 32 + (lane & 31);
                af[i] = as_bf16x8(*(const uint4*)&a_s[r * BK + ((c ^ (r & 7)) << 3)]);
            }
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int r = wn * WTN + j * 32 + (lane & 31);
                bfr[j] = as_bf16x8(*(const uint4*)&b_s[r * BK + ((c ^ (r & 7)) << 3)]);
            }
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) acc[i][j] = mfma32(af[i], bfr[j], acc[i][j]);
        }
    };

    const int nk = K / BK;
    load_tile(0);
    store_tile(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) load_tile(kt + 1);
        compute(cur);
        if (kt + 1 < nk) store_tile(cur ^ 1);
        __syncthreads();
    }

    if constexpr (NORM) {
#pragma unroll
        for (int i = 0; i < A_PER_T; ++i) {
            float s = ssq[i];
            s += __shfl_xor(s, 1, 64);
            s += __shfl_xor(s, 2, 64);
            s += __shfl_xor(s, 4, 64);
            s += __shfl_xor(s, 8, 64);
            if ((tid & 15) == 0) sScale[(tid >> 4) + i * (NT / 16)] = inv_rms(s, K, args.eps);
        }
        __syncthreads();
    }

    const Epilogue& e = args.epi;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int rl = wm * WTM + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            const int m = m0 + rl;
            const float sc = NORM ? sScale[rl] : 1.0f;
            if constexpr (EPI == EPI_SWIGLU) {
#pragma unroll
                for (int j = 0; j < TN; j += 2) {
                    const float g = acc[i][j][r] * sc;
                    const float u = acc[i][j + 1][r] * sc;
                    const int ng = n0 + wn * WTN + j * 32;  // multiple of 64
                    const int f = (ng >> 1) + (lane & 31);
                    if (m < M) epi_swiglu<bf16_t>(e, m, f, N >> 1, g, u);
                }
            } else {
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    const int n = n0 + wn * WTN + j * 32 + (lane & 31);
                    const float v = acc[i][j][r] * sc;
                    if constexpr (EPI == EPI_QKV) {
                        const float partner = __shfl_xor(v, 1, 64);
                        if (m < M) epi_qkv<bf16_t>(e, m, n, v, partner);
                    } else {
                        if (m < M) epi_resid(e, m, n, N, v);
                    }
                }
            }
        }
    }
}

struct TileCfg {
    int bm, bn, wm, wn;
};
constexpr TileCfg kTiles[] = {
    {256, 256, 2, 4},  // 8 waves, wave tile 128x64
    {256, 128, 4, 2},  // 8 waves, wave tile 64x64
    {128, 128, 2, 2},  // 4 waves, wave tile 64x64
};
constexpr int kNumTiles = sizeof(kTiles) / sizeof(kTiles[0]);

template <int BM, int BN, int WM, int WN, bool NORM, int EPI>
hipError_t launch_one(const GemmArgs& a, hipStream_t s) {
    const int tiles = ((a.M + BM - 1) / BM) * (a.N / BN);
    hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WM, WN, NORM, EPI>), dim3(tiles),
                       dim3(64 * WM * WN), 0, s, a);
    return hipGetLastError();
}

template <int BM, int BN, int WM, int WN>
hipError_t launch_cfg(const GemmArgs& a, hipStream_t s) {
    const int kind = a.epi.kind;
    if (kind == EPI_QKV && a.norm) return launch_one<BM, BN, WM, WN, true, EPI_QKV>(a, s);
    if (kind == EPI_SWIGLU && a.norm) return launch_one<BM, BN, WM, WN, true, EPI_SWIGLU>(a, s);
    if (kind == EPI_RESID && !a.norm) return launch_one<BM, BN, WM, WN, false, EPI_RESID>(a, s);
    return hipErrorInvalidValue;
}

}  // namespace

int gemm_bf16_num_tile_cfgs() { return kNumTiles; }

void gemm_bf16_tile(int cfg, int* bm, int* bn, int* threads) {
    *bm = kTiles[cfg].bm;
    *bn = kTiles[cfg].bn;
    *threads = 64 * kTiles[cfg].wm * kTiles[cfg].wn;
}

hipError_t gemm_bf16_launch(const GemmArgs& a, int cfg, hipStream_t s) {
    if (cfg < 0 || cfg >= kNumTiles) return hipErrorInvalidValue;
    const TileCfg t = kTiles[cfg];
    if (a.M <= 0 || a.N % t.bn != 0 || a.K % BK != 0) return hipErrorInvalidValue;
    switch (cfg) {
        case 0: return launch_cfg<256, 256, 2, 4>(a, s);
        case 1: return launch_cfg<256, 128, 4, 2>(a, s);
        default: return launch_cfg<128, 128, 2, 2>(a, s);
    }
}

}  // namespace llb
