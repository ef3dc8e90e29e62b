// Small-M bf16 projection for decode (M = batch <= 64 tokens): weight streaming.
//
// Decode multiplies a few token rows by every weight once, so the time is the
// weight bytes over HBM bandwidth; the MFMA work is small.  Each workgroup owns
// 128 W rows (one 32-row MFMA column block per wave) and a contiguous range of
// 64-wide k-tiles (split-K).  Every k-tile of W (128 rows x 128 bytes: whole
// cache lines) and of the token rows is copied global -> LDS by the DMA path,
// GV_NSTAGE tiles ahead, so about 100 KB per CU are in flight.  With one split
// the workgroup applies the epilogue itself; with several, each writes an fp32
// partial tile and a second kernel sums the partials in split order and
// applies the epilogue (one workgroup per column tile and pair/quad of rows).
#include <algorithm>

#include "common.cuh"
#include "epilogue.cuh"
#include "kernels.h"

namespace llb {

namespace {

constexpr int GV_BN = 128;     // W rows per workgroup (4 waves x 32)
constexpr int GV_BK = 64;      // k per pipeline stage (128-byte rows)
constexpr int GV_NSTAGE = 6;

// 16-byte chunk c of a 128-byte LDS row r sits at c ^ ((r >> 1) & 7): the 16
// lanes of a ds_read_b128 phase (16 consecutive rows, one chunk) hit distinct
// banks.
LLB_DEV int gv_swz(int r) { return (r >> 1) & 7; }

LLB_DEV float row_scale(const GemmArgs& a, int m) {
    float s = 0.f;
#pragma unroll 8
    for (int p = 0; p < a.ssq_count; ++p) s += a.ssq_in[(size_t)p * a.M + m];
    return inv_rms(s, a.K, a.eps);
}

template <int MS, int EPI>
__global__ void __launch_bounds__(256)
gemv_bf16_kernel(GemmArgs args, int splits, float* __restrict__ part) {
    constexpr int MT = 32 * MS;                      // token rows held (M <= MT)
    constexpr int W_BLK = GV_BN * GV_BK * 2 / 1024;  // 1 KB copy blocks of W per stage
    constexpr int A_BLK = MT * GV_BK * 2 / 1024;     // ... of the token rows
    constexpr int BLK = W_BLK + A_BLK;
    constexpr int DPW = BLK / 4;                     // copies per wave per stage
    constexpr int STAGE = BLK * 1024;
    static_assert(BLK % 4 == 0, "copy split");
    static_assert((GV_NSTAGE - 2) * DPW < 64, "vmcnt range");
    __shared__ __attribute__((aligned(1024))) char smem[GV_NSTAGE * STAGE];

    const int M = args.M, N = args.N, K = args.K;
    const int tiles = N / GV_BN;
    const int tile = blockIdx.x % tiles;
    const int split = blockIdx.x / tiles;
    const int n0 = tile * GV_BN;
    const int nkt = K / GV_BK;
    const int kt0 = (int)((long)split * nkt / splits);
    const int nk = (int)((long)(split + 1) * nkt / splits) - kt0;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    const bf16_t* __restrict__ W = (const bf16_t*)args.W;
    const bf16_t* __restrict__ A = (const bf16_t*)args.A;
    // Copy block j of a stage: rows 8j..8j+7 of [W tile; token rows], lane ->
    // (row 8j + lane/8, LDS chunk lane%8), holding global chunk (lane%8) ^ swz(row).
    const bf16_t* src[DPW];
#pragma unroll
    for (int i = 0; i < DPW; ++i) {
        const int blk = i * 4 + wave;
        const int row = blk * 8 + (lane >> 3);
        const int chunk = (lane & 7) ^ gv_swz(row);
        // W: tile (tile, kt0 + j) is one contiguous 16 KB block (128-row x 64-column
        // tiled layout), so a stage streams whole pages of it
        if (blk < W_BLK) src[i] = W + ((size_t)tile * nkt + kt0) * 8192 + row * 64 + chunk * 8;
        else src[i] = A + (size_t)min(row - GV_BN, M - 1) * K + (size_t)kt0 * GV_BK + chunk * 8;
    }
    const uint32_t lds_base = lds_offset(smem);
    auto issue = [&](int j) {  // k-tile kt0 + j into stage j % GV_NSTAGE
        const uint32_t st = lds_base + (uint32_t)(j % GV_NSTAGE) * STAGE;
#pragma unroll
        for (int i = 0; i < DPW; ++i) {
            const int blk = i * 4 + wave;
            dma16(src[i] + (size_t)j * (blk < W_BLK ? 8192 : GV_BK), st + (uint32_t)blk * 1024);
        }
    };
    // wait until k-tile j has landed: min(GV_NSTAGE - 2, nk - 1 - j) later ones may stay in flight
    auto wait_for = [&](int j) {
        const int later = min(GV_NSTAGE - 2, nk - 1 - j);
        if (later >= 4) wait_vm_lgkm<4 * DPW>();
        else if (later == 3) wait_vm_lgkm<3 * DPW>();
        else if (later == 2) wait_vm_lgkm<2 * DPW>();
        else if (later == 1) wait_vm_lgkm<DPW>();
        else wait_vm_lgkm<0>();
    };

    // row scale of the normalised-operand epilogues, loaded before the copies
    // start (its loads are retired before the first wait on them)
    constexpr bool SCALED = (EPI == EPI_QKV || EPI == EPI_SWIGLU || EPI == EPI_LOGITS);
    float my_scale = 1.0f;
    if (SCALED && tid < M) my_scale = row_scale(args, tid);

    f32x16 acc[MS];
#pragma unroll
    for (int ms = 0; ms < MS; ++ms)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[ms][r] = 0.f;

    // fragment addresses within a stage: W rows 32*wave + lane%32, token rows
    // 32*ms + lane%32 (after the W region), chunk 2*kk + lane/32
    const int wr = wave * 32 + (lane & 31);
    typedef bf16x8 __attribute__((address_space(3))) * lds_frag_ptr;

    for (int j = 0; j < GV_NSTAGE - 1 && j < nk; ++j) issue(j);
    for (int j = 0; j < nk; ++j) {
        wait_for(j);
        barrier();  // every wave is past k-tile j-1: its stage is free
        if (j + GV_NSTAGE - 1 < nk) issue(j + GV_NSTAGE - 1);
        const uint32_t st = lds_base + (uint32_t)(j % GV_NSTAGE) * STAGE;
#pragma unroll
        for (int kk = 0; kk < GV_BK / 16; ++kk) {
            const int c = 2 * kk + (lane >> 5);
            const bf16x8 wf = *(lds_frag_ptr)(uintptr_t)(st + wr * 128 + ((c ^ gv_swz(wr)) << 4));
#pragma unroll
            for (int ms = 0; ms < MS; ++ms) {
                const int ar = ms * 32 + (lane & 31);
                const bf16x8 af = *(lds_frag_ptr)(uintptr_t)(
                    st + W_BLK * 1024 + ar * 128 + ((c ^ gv_swz(ar)) << 4));
                acc[ms] = mfma32(af, wf, acc[ms]);
            }
        }
    }

    // With several splits: this split's fp32 partial tile [M x 128]; lane ->
    // column 32*wave + lane%32, register r -> token 32*ms + 8*(r/4) +
    // 4*(lane/32) + r%4.  The reduction kernel applies the epilogue.
    if (splits > 1) {
        float* my = part + ((size_t)tile * splits + split) * MT * GV_BN;
#pragma unroll
        for (int ms = 0; ms < MS; ++ms)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int tok = ms * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                if (tok < M) my[tok * GV_BN + wr] = acc[ms][r];
            }
        return;
    }
    // One split: the tile [M x 128] goes through LDS (fp32, reusing the stages)
    // to the epilogue.
    float* sred = (float*)smem;
    static_assert(MT * GV_BN * 4 + MT * 4 <= GV_NSTAGE * STAGE, "tile fits in LDS");
    float* sscale = sred + MT * GV_BN;
    __syncthreads();  // every wave is done with the stages
#pragma unroll
    for (int ms = 0; ms < MS; ++ms)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int tok = ms * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            sred[tok * GV_BN + wr] = acc[ms][r];
        }
    if (SCALED && tid < M) sscale[tid] = my_scale;
    __syncthreads();

    const Epilogue& e = args.epi;
    if constexpr (EPI == EPI_RESID_NORM) {
        // two rows per pass, 128 threads (two waves) per row
        __shared__ float s_ss[4];
        for (int m0r = 0; m0r < M; m0r += 2) {
            const int m = m0r + (tid >> 7);
            const int c = tid & 127;
            float ss = 0.f;
            if (m < M) {
                const float h = epi_resid(e, m, n0 + c, N, sred[m * GV_BN + c]);
                epi_norm_operand(e, m, n0 + c, N, h);
                ss = h * h;
            }
            ss = warp_sum(ss);
            if (lane == 0) s_ss[wave] = ss;
            __syncthreads();
            if (tid == 0 || tid == 128) {
                const int w0 = tid >> 6;
                if (m < M) e.ssq_out[(size_t)tile * M + m] = s_ss[w0] + s_ss[w0 + 1];
            }
            __syncthreads();
        }
    } else if constexpr (EPI == EPI_RESID) {
        for (int idx = tid; idx < M * GV_BN; idx += 256) {
            const int m = idx / GV_BN, c = idx % GV_BN;
            epi_resid(e, m, n0 + c, N, sred[idx]);
        }
    } else if constexpr (EPI == EPI_LOGITS) {
        for (int idx = tid; idx < M * GV_BN; idx += 256) {
            const int m = idx / GV_BN, c = idx % GV_BN;
            e.out[(size_t)m * N + n0 + c] = sred[idx] * sscale[m];
        }
    } else if constexpr (EPI == EPI_SWIGLU) {
        // 128 columns = two groups [gate 32 | up 32]: 64 features per row
        for (int idx = tid; idx < M * 64; idx += 256) {
            const int m = idx / 64, j = idx % 64;
            const int cg = (j >> 5) * 64 + (j & 31);
            const float sc = sscale[m];
            epi_swiglu<bf16_t>(e, m, n0 / 2 + j, N >> 1, sred[m * GV_BN + cg] * sc,
                               sred[m * GV_BN + cg + 32] * sc);
        }
    } else {  // EPI_QKV: RoPE pairs
        for (int idx = tid; idx < M * 64; idx += 256) {
            const int m = idx / 64, c = 2 * (idx % 64);
            const float sc = sscale[m];
            const float v0 = sred[m * GV_BN + c] * sc, v1 = sred[m * GV_BN + c + 1] * sc;
            epi_qkv<bf16_t>(e, m, n0 + c, v0, v1);
            epi_qkv<bf16_t>(e, m, n0 + c + 1, v1, v0);
        }
    }
}

// Sums the split partials of one column tile in split order and applies the
// epilogue, for RPW rows per workgroup (256 / RPW threads per row): RPW = 2 for
// the element-wise epilogues (128 columns), 4 for RoPE pairs and SwiGLU
// features (64 per row).
template <int EPI>
__global__ void __launch_bounds__(256)
gemv_reduce_kernel(GemmArgs args, int splits, const float* __restrict__ part) {
    constexpr int RPW = (EPI == EPI_RESID || EPI == EPI_RESID_NORM || EPI == EPI_LOGITS) ? 2 : 4;
    constexpr int TPR = 256 / RPW;
    const int M = args.M, N = args.N;
    const int MT = M <= 32 ? 32 : 64;
    const int tiles = N / GV_BN;
    const int tile = blockIdx.x % tiles;
    const int m = (blockIdx.x / tiles) * RPW + threadIdx.x / TPR;
    const int j = threadIdx.x % TPR;
    const int n0 = tile * GV_BN;
    const float* tp = part + (size_t)tile * splits * MT * GV_BN + (size_t)m * GV_BN;
    auto col = [&](int c) {
        float v = 0.f;
        for (int sp = 0; sp < splits; ++sp) v += tp[(size_t)sp * MT * GV_BN + c];
        return v;
    };
    const Epilogue& e = args.epi;
    if constexpr (EPI == EPI_RESID_NORM) {
        __shared__ float s_ss[4];
        float ss = 0.f;
        if (m < M) {
            const float h = epi_resid(e, m, n0 + j, N, col(j));
            epi_norm_operand(e, m, n0 + j, N, h);
            ss = h * h;
        }
        ss = warp_sum(ss);
        const int wave = threadIdx.x >> 6;
        if ((threadIdx.x & 63) == 0) s_ss[wave] = ss;
        __syncthreads();
        if (j == 0 && m < M) e.ssq_out[(size_t)tile * M + m] = s_ss[2 * (wave >> 1)] + s_ss[2 * (wave >> 1) + 1];
    } else if constexpr (EPI == EPI_RESID) {
        if (m < M) epi_resid(e, m, n0 + j, N, col(j));
    } else if constexpr (EPI == EPI_LOGITS) {
        if (m < M) e.out[(size_t)m * N + n0 + j] = col(j) * row_scale(args, m);
    } else if constexpr (EPI == EPI_SWIGLU) {
        if (m < M) {
            const int cg = (j >> 5) * 64 + (j & 31);
            const float sc = row_scale(args, m);
            epi_swiglu<bf16_t>(e, m, n0 / 2 + j, N >> 1, col(cg) * sc, col(cg + 32) * sc);
        }
    } else {
        if (m < M) {
            const int c = 2 * j;
            const float sc = row_scale(args, m);
            const float v0 = col(c) * sc, v1 = col(c + 1) * sc;
            epi_qkv<bf16_t>(e, m, n0 + c, v0, v1);
            epi_qkv<bf16_t>(e, m, n0 + c + 1, v1, v0);
        }
    }
}

template <int EPI>
hipError_t launch_epi(const GemmArgs& a, int splits, float* part, hipStream_t s) {
    const dim3 grid((a.N / GV_BN) * splits);
    if (a.M <= 32)
        hipLaunchKernelGGL((gemv_bf16_kernel<1, EPI>), grid, dim3(256), 0, s, a, splits, part);
    else
        hipLaunchKernelGGL((gemv_bf16_kernel<2, EPI>), grid, dim3(256), 0, s, a, splits, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || splits == 1) return e;
    constexpr int RPW = (EPI == EPI_RESID || EPI == EPI_RESID_NORM || EPI == EPI_LOGITS) ? 2 : 4;
    const dim3 rgrid((a.N / GV_BN) * ((a.M + RPW - 1) / RPW));
    hipLaunchKernelGGL((gemv_reduce_kernel<EPI>), rgrid, dim3(256), 0, s, a, splits, part);
    return hipGetLastError();
}

size_t partial_bytes(int M, int N, int splits) {
    const int mt = M <= 32 ? 32 : 64;
    return ((size_t)(N / GV_BN) * splits * mt * GV_BN * sizeof(float) + 255) & ~(size_t)255;
}

}  // namespace

// Split count, from measurements on MI355X: the fewest splits that give at
// least 192 workgroups; more splits only add partial traffic and reduction
// work.  Every split keeps at least 4 k-tiles of 64.
int gemv_bf16_splits(int M, int N, int K) {
    const int tiles = N / GV_BN;
    const int nkt = K / GV_BK;
    const int target = 192;
    int s = (target + tiles - 1) / tiles;
    s = std::max(1, std::min(s, nkt / 4));
    return s;
}

size_t gemv_bf16_ws_bytes(int M, int N, int splits) {
    return partial_bytes(M, N, splits);
}

hipError_t gemv_bf16_launch(const GemmArgs& a, int splits, float* ws, hipStream_t s) {
    if (a.M <= 0 || a.M > 64 || a.N % GV_BN != 0 || a.K % GV_BK != 0 || splits < 1 ||
        splits > a.K / GV_BK)
        return hipErrorInvalidValue;
    switch (a.epi.kind) {
        case EPI_QKV: return launch_epi<EPI_QKV>(a, splits, ws, s);
        case EPI_SWIGLU: return launch_epi<EPI_SWIGLU>(a, splits, ws, s);
        case EPI_RESID: return launch_epi<EPI_RESID>(a, splits, ws, s);
        case EPI_RESID_NORM: return launch_epi<EPI_RESID_NORM>(a, splits, ws, s);
        case EPI_LOGITS: return launch_epi<EPI_LOGITS>(a, splits, ws, s);
        default: return hipErrorInvalidValue;
    }
}

int gemv_bf16_ssq_parts(int N) { return N / GV_BN; }

// ---------------------------------------------------------------------------
// RMSNorm operand: one workgroup per row.  a[m, j] = bf16(x[m, j] * g[j]) (one
// rounding) and ssq[m] = sum_j x[m, j]^2 accumulated in fp32 across the
// workgroup ("Llama 3.1 70B", section "RMSNorm": the reduction is done in
// fp32).  The inverse RMS itself is applied to the fp32 results of the
// projection.
__global__ void __launch_bounds__(256)
norm_rows_kernel(const float* __restrict__ x, const float* __restrict__ g, bf16_t* __restrict__ a,
                 float* __restrict__ ssq, int M, int d) {
    __shared__ float s_red[4];
    const int row = blockIdx.x;
    const int lane = threadIdx.x & 63;
    const float* xr = x + (size_t)row * d;
    bf16_t* ar = a + (size_t)row * d;
    float s = 0.f;
#pragma unroll 4
    for (int j = threadIdx.x * 8; j < d; j += 256 * 8) {
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
    if (lane == 0) s_red[threadIdx.x >> 6] = s;
    __syncthreads();
    if (threadIdx.x == 0) ssq[row] = (s_red[0] + s_red[1]) + (s_red[2] + s_red[3]);
}

hipError_t norm_rows_launch(const float* x, const float* g, void* a, float* ssq, int M, int d,
                            hipStream_t s) {
    if (M <= 0 || d % 8 != 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL(norm_rows_kernel, dim3(M), dim3(256), 0, s, x, g, (bf16_t*)a, ssq, M, d);
    return hipGetLastError();
}

}  // namespace llb
