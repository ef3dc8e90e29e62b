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
constexpr int GV_MAXSPLIT = 8;  // most k-splits of one projection

// 16-byte chunk c of a 128-byte LDS row r sits at c ^ ((r >> 1) & 7): the 16
// lanes of a ds_read_b128 phase (16 consecutive rows, one chunk) hit distinct
// banks.
LLB_DEV int gv_swz(int r) { return (r >> 1) & 7; }

// Partial sums of squares of the decode projections are laid out [P][MT]:
// partial p of token row m at ssq[p * MT + m], MT = 32 or 64 token rows held
// by the kernels (an RMSNorm operand with one partial is the plain [M] row).

// Serial inverse RMS of row m from P partials (the split-K reduction kernel).
LLB_DEV float row_scale(const GemmArgs& a, int m, int MT) {
    float s = 0.f;
#pragma unroll 8
    for (int p = 0; p < a.ssq_count; ++p) s += a.ssq_in[(size_t)p * MT + m];
    return inv_rms(s, a.K, a.eps);
}

// The row scales of a normalised operand, gathered by the whole workgroup:
// thread t loads partials p = g, g + G, ... (g = t / (MT/4), G = 1024 / MT)
// of rows 4q..4q+3 (q = t % (MT/4)) with SL float4 loads, all issued at once
// (partials past P re-read partial P-1 and are dropped), so that their latency
// hides behind the weight copies.  finish() sums them in a fixed order into
// out[m] = 1/rms of row m.  Needs P <= SL * G.
template <int MT, int SL>
struct RowScales {
    static constexpr int Q = MT / 4, G = 256 / Q;
    float4 v[SL];
    LLB_DEV void issue(const GemmArgs& a) {
        const int q = threadIdx.x % Q, g = threadIdx.x / Q;
#pragma unroll
        for (int i = 0; i < SL; ++i) {
            const int p = min(g + i * G, a.ssq_count - 1);
            v[i] = *(const float4*)(a.ssq_in + (size_t)p * MT + 4 * q);
        }
    }
    // part: LDS scratch of 256 * 4 floats; out: LDS [MT].  Ends with a barrier.
    LLB_DEV void finish(const GemmArgs& a, float* part, float* out) {
        const int q = threadIdx.x % Q, g = threadIdx.x / Q;
        float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int i = 0; i < SL; ++i)
            if (g + i * G < a.ssq_count) {
                s.x += v[i].x; s.y += v[i].y; s.z += v[i].z; s.w += v[i].w;
            }
        *(float4*)(part + g * MT + 4 * q) = s;
        __syncthreads();
        if (threadIdx.x < MT) {
            float t = 0.f;
            for (int k = 0; k < G; ++k) t += part[k * MT + threadIdx.x];
            out[threadIdx.x] = inv_rms(t, a.K, a.eps);
        }
        __syncthreads();
    }
};

// s_waitcnt for a pipeline whose k-tiles are DPW copies each: `later` k-tiles
// (0..MAXL) issued after the awaited one may stay in flight, plus EXTRA loads
// issued after it.
template <int DPW, int EXTRA, int MAXL>
LLB_DEV void wait_later(int later) {
    if constexpr (MAXL > 0) {
        if (later >= MAXL) {
            wait_vm_lgkm<MAXL * DPW + EXTRA>();
            return;
        }
        wait_later<DPW, EXTRA, MAXL - 1>(later);
    } else {
        wait_vm_lgkm<EXTRA>();
    }
}

// The epilogue of one 128-column tile whose fp32 result sits in LDS: sred[tok *
// 128 + c] for token rows tok < M, with the row scales in sscale[tok] (the
// normalised-operand epilogues).  Called by all 256 threads of the workgroup.
template <int MS, int EPI>
LLB_DEV void gemv_tile_epilogue(const GemmArgs& args, const float* sred, const float* sscale, int tile) {
    constexpr int MT = 32 * MS;
    const int M = args.M, N = args.N;
    const int n0 = tile * GV_BN;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const Epilogue& e = args.epi;
    if constexpr (EPI == EPI_RESID_NORM) {
        // two rows per pass, 128 threads (two waves) per row; a thread's column
        // (and gain) is the same in every pass
        __shared__ float s_ss[4];
        const float g = e.gain[n0 + (tid & 127)];
        for (int m0r = 0; m0r < M; m0r += 2) {
            const int m = m0r + (tid >> 7);
            const int c = tid & 127;
            float ss = 0.f;
            if (m < M) {
                const float h = epi_resid(e, m, n0 + c, N, sred[m * GV_BN + c]);
                epi_norm_operand_g(e, m, n0 + c, N, h, g);
                ss = h * h;
            }
            ss = warp_sum(ss);
            if (lane == 0) s_ss[wave] = ss;
            __syncthreads();
            if (tid == 0 || tid == 128) {
                const int w0 = tid >> 6;
                if (m < M) e.ssq_out[(size_t)tile * MT + m] = s_ss[w0] + s_ss[w0 + 1];
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
    // Row scales of the normalised-operand epilogues (one split only; with
    // several the reduction kernel applies them): their loads go out right
    // after the first copies, so the waits on those copies allow SL more.
    constexpr bool SCALED = (EPI == EPI_QKV || EPI == EPI_SWIGLU || EPI == EPI_LOGITS);
    constexpr int SL = EPI == EPI_SWIGLU ? 16 : 4;
    static_assert((GV_NSTAGE - 2) * DPW + SL < 64, "vmcnt range");
    const bool scaled = SCALED && splits == 1;
    RowScales<MT, SL> rs;
    // wait until k-tile j has landed: min(GV_NSTAGE - 2, nk - 1 - j) later ones
    // may stay in flight, and the row-scale loads when j was issued before them
    auto wait_for = [&](int j) {
        const int later = min(GV_NSTAGE - 2, nk - 1 - j);
        if (scaled && j < GV_NSTAGE - 1) wait_later<DPW, SL, GV_NSTAGE - 2>(later);
        else wait_later<DPW, 0, GV_NSTAGE - 2>(later);
    };

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
    if (scaled) rs.issue(args);
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
    static_assert(MT * GV_BN * 4 + MT * 4 + 1024 * 4 <= GV_NSTAGE * STAGE, "tile fits in LDS");
    float* sscale = sred + MT * GV_BN;
    __syncthreads();  // every wave is done with the stages
    if (SCALED) rs.finish(args, sscale + MT, sscale);
#pragma unroll
    for (int ms = 0; ms < MS; ++ms)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int tok = ms * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            sred[tok * GV_BN + wr] = acc[ms][r];
        }
    __syncthreads();

    gemv_tile_epilogue<MS, EPI>(args, sred, sscale, tile);
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
    const float* tp = part + (size_t)tile * splits * MT * GV_BN + (size_t)min(m, M - 1) * GV_BN;
    // the partials of up to GV_MAXSPLIT splits are loaded together (one memory
    // round trip), then summed in split order
    auto col = [&](int c) {
        float p[GV_MAXSPLIT];
#pragma unroll
        for (int sp = 0; sp < GV_MAXSPLIT; ++sp) p[sp] = tp[(size_t)min(sp, splits - 1) * MT * GV_BN + c];
        float v = p[0];
#pragma unroll
        for (int sp = 1; sp < GV_MAXSPLIT; ++sp)
            if (sp < splits) v += p[sp];
        return v;
    };
    const Epilogue& e = args.epi;
    if constexpr (EPI == EPI_RESID_NORM) {
        __shared__ float s_ss[4];
        float ss = 0.f;
        const float g = e.gain[n0 + j];
        if (m < M) {
            const float h = epi_resid(e, m, n0 + j, N, col(j));
            epi_norm_operand_g(e, m, n0 + j, N, h, g);
            ss = h * h;
        }
        ss = warp_sum(ss);
        const int wave = threadIdx.x >> 6;
        if ((threadIdx.x & 63) == 0) s_ss[wave] = ss;
        __syncthreads();
        if (j == 0 && m < M)
            e.ssq_out[(size_t)tile * MT + m] = s_ss[2 * (wave >> 1)] + s_ss[2 * (wave >> 1) + 1];
    } else if constexpr (EPI == EPI_RESID) {
        if (m < M) epi_resid(e, m, n0 + j, N, col(j));
    } else if constexpr (EPI == EPI_LOGITS) {
        if (m < M) e.out[(size_t)m * N + n0 + j] = col(j) * row_scale(args, m, MT);
    } else if constexpr (EPI == EPI_SWIGLU) {
        if (m < M) {
            const int cg = (j >> 5) * 64 + (j & 31);
            const float sc = row_scale(args, m, MT);
            epi_swiglu<bf16_t>(e, m, n0 / 2 + j, N >> 1, col(cg) * sc, col(cg + 32) * sc);
        }
    } else {
        if (m < M) {
            const int c = 2 * j;
            const float sc = row_scale(args, m, MT);
            const float v0 = col(c) * sc, v1 = col(c + 1) * sc;
            epi_qkv<bf16_t>(e, m, n0 + c, v0, v1);
            epi_qkv<bf16_t>(e, m, n0 + c + 1, v1, v0);
        }
    }
}

// ---------------------------------------------------------------------------
// Narrow weight streaming: one workgroup per RW (16 or 32) weight rows over the
// whole of K, for projections whose N / 128 row tiles alone would not fill the
// chip (a decode step's QKV, O and down projections).  Its four waves each
// stream one quarter of K as independent pipelines: a wave copies its own
// k-tiles (RW weight rows and the MT token rows, 64 columns each) global ->
// LDS into a private ring of NS stages and multiplies them, with no workgroup
// barrier in the main loop.  The four fp32 partial tiles are then summed
// through LDS in wave order and the workgroup applies the epilogue itself, so
// no partial ever leaves the CU.  RW = 16 uses 16x16x32 MFMAs, RW = 32 the
// 32x32x16 ones.

// Bytes of one wave's pipeline stage: RW weight rows and the MT token rows of
// a 64-wide k-tile, as bf16 operands or (NORM) as fp32 rows of x plus the
// k-tile's 64 RMSNorm gains.
constexpr int narrow_stage(int rw, int ms, bool norm) {
    return norm ? (rw / 8 + 32 * ms / 4) * 1024 + 256 : (rw + 32 * ms) * GV_BK * 2;
}

// Ring depth: as deep as LDS allows, for one workgroup per CU or (TWO) two.
constexpr int narrow_ns(int rw, int ms, bool two, bool norm = false) {
    const int ns = (two ? 75 * 1024 : 150 * 1024) / (4 * narrow_stage(rw, ms, norm));
    return ns > 6 ? 6 : ns < 2 ? 2 : ns;
}

// NORM (EPI_QKV): the attention RMSNorm is formed inside the kernel.  A is the
// fp32 residual stream x and args.gain its gain: each wave copies the fp32 x
// rows and the 64 gains of its k-tiles into its ring, and the fragment reads
// form the operand bf16(x * g) (rounded once, as the separate norm kernel
// would) while summing x^2 for the row's 1/rms ("Llama 3.1 70B", section
// "RMSNorm": one fp32 reduction per token).  Each element of a wave's k-range
// enters exactly one lane's sum; the lanes of a row and then the four waves are
// added in a fixed order, so the result is deterministic.
template <int MS, int EPI, int RW, int NS, bool NORM>
__global__ void __launch_bounds__(256)
gemv_narrow_kernel(GemmArgs args) {
    constexpr int MT = 32 * MS;
    constexpr int W_BLK = RW / 8;       // 1 KB copy blocks per stage: 8 rows of 128 bytes
    constexpr int A_BLK = NORM ? MT / 4 : MT / 8;   // fp32 rows: 4 per 1 KB block
    constexpr int DPW = W_BLK + A_BLK;  // a wave issues every copy of its stages
    constexpr int VPS = DPW + (NORM ? 1 : 0);       // vector-memory ops per stage (+ the gains)
    constexpr int STAGE = narrow_stage(RW, MS, NORM);
    constexpr bool SCALED = EPI == EPI_QKV;
    constexpr int SL = NORM ? 0 : 4;
    static_assert(EPI == EPI_QKV || EPI == EPI_RESID || EPI == EPI_RESID_NORM, "epilogue");
    static_assert(!NORM || (EPI == EPI_QKV && MS == 1), "in-kernel RMSNorm: QKV over at most 32 token rows");
    static_assert((NS - 2) * VPS + SL < 64, "vmcnt range");
    static_assert(MT * RW * 4 <= NS * STAGE, "partial tile fits in a wave's ring");
    __shared__ __attribute__((aligned(1024))) char smem[4 * NS * STAGE];
    __shared__ __attribute__((aligned(16))) float s_part[1024];
    __shared__ float sscale[MT];

    const int M = args.M, N = args.N, K = args.K;
    const int n0 = blockIdx.x * RW;
    const int nkt = K / GV_BK;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kt0 = wave * nkt / 4;
    const int nk = (wave + 1) * nkt / 4 - kt0;

    const bf16_t* __restrict__ W = (const bf16_t*)args.W;
    const bf16_t* __restrict__ A = (const bf16_t*)args.A;
    const float* __restrict__ X = (const float*)args.A;
    // Copy block i of a stage: LDS rows 8i..8i+7 of [W rows; token rows], lane ->
    // (row 8i + lane/8, LDS chunk lane%8) holding global chunk (lane%8) ^ swz(row).
    // The RW rows of one k-tile are RW * 128 contiguous bytes of the 128 x 64
    // tiled weight layout.  NORM: after the W blocks, fp32 token rows of 256
    // bytes (sixteen 16-byte chunks, chunk c of row r at position c ^ (r & 15)),
    // 4 rows per block, then the k-tile's 64 gains.
    const char* src[DPW];
#pragma unroll
    for (int i = 0; i < DPW; ++i) {
        if (i < W_BLK) {
            const int row = i * 8 + (lane >> 3);
            const int chunk = (lane & 7) ^ gv_swz(row);
            src[i] = (const char*)(W + ((size_t)(n0 >> 7) * nkt + kt0) * 8192 + ((n0 & 127) + row) * 64 + chunk * 8);
        } else if constexpr (NORM) {
            const int row = (i - W_BLK) * 4 + (lane >> 4);
            const int chunk = (lane & 15) ^ (row & 15);
            src[i] = (const char*)(X + (size_t)min(row, M - 1) * K + (size_t)kt0 * GV_BK + chunk * 4);
        } else {
            const int row = i * 8 + (lane >> 3);
            const int chunk = (lane & 7) ^ gv_swz(row);
            src[i] = (const char*)(A + (size_t)min(row - RW, M - 1) * K + (size_t)kt0 * GV_BK + chunk * 8);
        }
    }
    const float* gsrc = NORM ? args.gain + (size_t)kt0 * GV_BK + lane : nullptr;
    const uint32_t ring = lds_offset(smem) + (uint32_t)wave * NS * STAGE;
    auto issue = [&](int j) {  // k-tile kt0 + j into stage j % NS of this wave's ring
        const uint32_t st = ring + (uint32_t)(j % NS) * STAGE;
#pragma unroll
        for (int i = 0; i < DPW; ++i)
            dma16(src[i] + (size_t)j * (i < W_BLK ? 8192 * 2 : NORM ? GV_BK * 4 : GV_BK * 2),
                  st + (uint32_t)i * 1024);
        if constexpr (NORM) dma4(gsrc + (size_t)j * GV_BK, st + (uint32_t)DPW * 1024);
    };

    RowScales<MT, SL == 0 ? 1 : SL> rs;
    for (int j = 0; j < NS - 1 && j < nk; ++j) issue(j);
    if (SCALED && !NORM) rs.issue(args);

    constexpr int NACC = RW == 32 ? MS : 2 * MS;
    f32x16 acc32[RW == 32 ? MS : 1];
    f32x4 acc16[RW == 16 ? 2 * MS : 1];
#pragma unroll
    for (int i = 0; i < NACC; ++i) {
        if constexpr (RW == 32) {
#pragma unroll
            for (int r = 0; r < 16; ++r) acc32[i][r] = 0.f;
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) acc16[i][r] = 0.f;
        }
    }
    typedef bf16x8 __attribute__((address_space(3))) * lds_frag_ptr;
    typedef f32x4 __attribute__((address_space(3))) * lds_f4_ptr;
    auto frag = [&](uint32_t st, int row, int c) {
        return *(lds_frag_ptr)(uintptr_t)(st + row * 128 + ((c ^ gv_swz(row)) << 4));
    };
    // token-row operand fragment: row trow (of MT), 8-element chunk c of the
    // k-tile.  NORM: bf16(x * g) from the staged fp32 row and gains, adding the
    // eight x^2 to ss.
    constexpr int NSS = RW == 32 ? MS : 2 * MS;
    float ss[NSS];
#pragma unroll
    for (int i = 0; i < NSS; ++i) ss[i] = 0.f;
    auto afrag = [&](uint32_t st, int trow, int c, float& acc_ss) -> bf16x8 {
        if constexpr (NORM) {
            const uint32_t rb = st + W_BLK * 1024 + trow * 256;
            const f32x4 x0 = *(lds_f4_ptr)(uintptr_t)(rb + (((2 * c) ^ (trow & 15)) << 4));
            const f32x4 x1 = *(lds_f4_ptr)(uintptr_t)(rb + (((2 * c + 1) ^ (trow & 15)) << 4));
            const uint32_t gb = st + DPW * 1024 + c * 32;
            const f32x4 g0 = *(lds_f4_ptr)(uintptr_t)(gb);
            const f32x4 g1 = *(lds_f4_ptr)(uintptr_t)(gb + 16);
            acc_ss += x0[0] * x0[0] + x0[1] * x0[1] + x0[2] * x0[2] + x0[3] * x0[3];
            acc_ss += x1[0] * x1[0] + x1[1] * x1[1] + x1[2] * x1[2] + x1[3] * x1[3];
            const float v[8] = {x0[0] * g0[0], x0[1] * g0[1], x0[2] * g0[2], x0[3] * g0[3],
                                x1[0] * g1[0], x1[1] * g1[1], x1[2] * g1[2], x1[3] * g1[3]};
            return to_bf16x8(v);
        } else {
            (void)acc_ss;
            return frag(st, RW + trow, c);
        }
    };

    for (int j = 0; j < nk; ++j) {
        // k-tile j has landed once at most min(NS - 2, nk - 1 - j) later k-tiles
        // (and the row-scale loads, when j was issued before them) are in flight;
        // the wait also retires this wave's LDS reads of the stage refilled next
        const int later = min(NS - 2, nk - 1 - j);
        if (SCALED && !NORM && j < NS - 1) wait_later<VPS, SL, NS - 2>(later);
        else wait_later<VPS, 0, NS - 2>(later);
        if (j + NS - 1 < nk) issue(j + NS - 1);
        const uint32_t st = ring + (uint32_t)(j % NS) * STAGE;
        if constexpr (RW == 32) {
            // lane: W row lane%32 / token row lane%32, chunk 2*kk + lane/32
#pragma unroll
            for (int kk = 0; kk < GV_BK / 16; ++kk) {
                const int c = 2 * kk + (lane >> 5);
                const bf16x8 wf = frag(st, lane & 31, c);
#pragma unroll
                for (int ms = 0; ms < MS; ++ms)
                    acc32[ms] = mfma32(afrag(st, ms * 32 + (lane & 31), c, ss[ms]), wf, acc32[ms]);
            }
        } else {
            // lane: W row lane%16 / token row lane%16, chunk 4*kk + lane/16
#pragma unroll
            for (int kk = 0; kk < GV_BK / 32; ++kk) {
                const int c = 4 * kk + (lane >> 4);
                const bf16x8 wf = frag(st, lane & 15, c);
#pragma unroll
                for (int tb = 0; tb < 2 * MS; ++tb)
                    acc16[tb] = mfma16(afrag(st, tb * 16 + (lane & 15), c, ss[tb]), wf, acc16[tb]);
            }
        }
    }

    // This wave's partial tile [MT][RW] (fp32) into its own ring: its copies
    // have all landed and its reads have completed (the last wait was vmcnt(0)
    // lgkmcnt(0)).  D layouts: 32x32 -> lane column lane%32, register r row
    // 8*(r/4) + 4*(lane/32) + r%4; 16x16 -> lane column lane%16, register r row
    // 4*(lane/16) + r.
    float* part = (float*)(smem + wave * NS * STAGE);
    if constexpr (RW == 32) {
#pragma unroll
        for (int ms = 0; ms < MS; ++ms)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                part[(ms * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)) * RW + (lane & 31)] = acc32[ms][r];
    } else {
#pragma unroll
        for (int tb = 0; tb < 2 * MS; ++tb)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                part[(tb * 16 + 4 * (lane >> 4) + r) * RW + (lane & 15)] = acc16[tb][r];
    }
    if constexpr (NORM) {
        // each row's sum of x^2: the lanes holding the row (lane ^ 32 for the
        // 32-row fragments, lane ^ 16, ^ 32 for the 16-row ones), then the waves
        // in order
#pragma unroll
        for (int i = 0; i < NSS; ++i) {
            if constexpr (RW == 16) ss[i] += __shfl_xor(ss[i], 16, 64);
            ss[i] += __shfl_xor(ss[i], 32, 64);
        }
        constexpr int RB = RW == 32 ? 32 : 16;   // rows per fragment block
        if (lane < RB) {
#pragma unroll
            for (int i = 0; i < NSS; ++i) s_part[wave * MT + i * RB + lane] = ss[i];
        }
    }
    __syncthreads();
    if constexpr (NORM) {
        if (tid < MT)
            sscale[tid] = inv_rms(((s_part[tid] + s_part[MT + tid]) + s_part[2 * MT + tid]) + s_part[3 * MT + tid],
                                  K, args.eps);
        __syncthreads();
    } else if (SCALED) {
        rs.finish(args, s_part, sscale);
    }

    // C[m, n0 + c] for 8 columns c0..c0+7, summed over the waves in order
    const float* p0 = (const float*)smem;
    auto cols8 = [&](int m, int c0, float* v) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int i = m * RW + c0 + k;
            float s = p0[i];
#pragma unroll
            for (int w = 1; w < 4; ++w) s += p0[w * (NS * STAGE / 4) + i];
            v[k] = s;
        }
    };
    const Epilogue& e = args.epi;
    constexpr int TPR = RW / 8;  // threads per token row, 8 columns each
    const int m = tid / TPR, c0 = (tid % TPR) * 8;
    static_assert(256 / TPR >= 64, "one pass covers every token row");
    float v[8];
    if constexpr (EPI == EPI_QKV) {
        if (m < M) {
            cols8(m, c0, v);
            const float sc = sscale[m];
#pragma unroll
            for (int k = 0; k < 8; ++k) v[k] *= sc;
            epi_qkv8(e, m, n0 + c0, v);
        }
    } else if constexpr (EPI == EPI_RESID) {
        if (m < M) {
            cols8(m, c0, v);
            epi_resid8(e, m, n0 + c0, N, v);
        }
    } else {  // EPI_RESID_NORM: h, the next RMSNorm's operand, sum of h^2 over the RW columns
        float ss = 0.f;
        float g[8];
        epi_gain8(e, n0 + c0, g);
        if (m < M) {
            cols8(m, c0, v);
            epi_resid8(e, m, n0 + c0, N, v);
            ss = epi_norm_operand8g(e, m, n0 + c0, N, v, g);
        }
#pragma unroll
        for (int o = TPR / 2; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, 64);
        if (m < M && c0 == 0) e.ssq_out[(size_t)blockIdx.x * MT + m] = ss;
    }
}

template <int MS, int EPI, int RW, bool TWO>
hipError_t launch_narrow(const GemmArgs& a, hipStream_t s) {
    if constexpr (EPI == EPI_QKV && MS == 1 && !TWO) {
        if (a.norm) {
            hipLaunchKernelGGL((gemv_narrow_kernel<1, EPI_QKV, RW, narrow_ns(RW, 1, false, true), true>),
                               dim3(a.N / RW), dim3(256), 0, s, a);
            return hipGetLastError();
        }
    }
    if (a.norm) return hipErrorInvalidValue;
    hipLaunchKernelGGL((gemv_narrow_kernel<MS, EPI, RW, narrow_ns(RW, MS, TWO), false>), dim3(a.N / RW),
                       dim3(256), 0, s, a);
    return hipGetLastError();
}

template <int MS, int EPI>
hipError_t launch_narrow_rw(const GemmArgs& a, int rw, bool two, hipStream_t s) {
    if (rw == 16) return two ? launch_narrow<MS, EPI, 16, true>(a, s) : launch_narrow<MS, EPI, 16, false>(a, s);
    return two ? launch_narrow<MS, EPI, 32, true>(a, s) : launch_narrow<MS, EPI, 32, false>(a, s);
}

template <int EPI>
hipError_t launch_narrow_epi(const GemmArgs& a, int rw, bool two, hipStream_t s) {
    return a.M <= 32 ? launch_narrow_rw<1, EPI>(a, rw, two, s) : launch_narrow_rw<2, EPI>(a, rw, two, s);
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
    s = std::max(1, std::min(std::min(s, nkt / 4), GV_MAXSPLIT));
    return s;
}

size_t gemv_bf16_ws_bytes(int M, int N, int splits) {
    return partial_bytes(M, N, splits);
}

hipError_t gemv_bf16_launch(const GemmArgs& a, int splits, float* ws, hipStream_t s) {
    if (a.M <= 0 || a.M > 64 || a.N % GV_BN != 0 || a.K % GV_BK != 0 || splits < 1 ||
        splits > a.K / GV_BK || splits > GV_MAXSPLIT)
        return hipErrorInvalidValue;
    // one split gathers the row scales with RowScales: 16 (SwiGLU) or 4 loads per thread
    const int groups = a.M <= 32 ? 32 : 16;
    const bool scaled = a.epi.kind == EPI_QKV || a.epi.kind == EPI_SWIGLU || a.epi.kind == EPI_LOGITS;
    if (scaled && splits == 1 && a.ssq_count > (a.epi.kind == EPI_SWIGLU ? 16 : 4) * groups)
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

bool gemv_narrow_supports(int M, int N, int K, int epi, int rw) {
    return M >= 1 && M <= 64 && (rw == 16 || rw == 32) && N % GV_BN == 0 && K % GV_BK == 0 &&
           K / GV_BK >= 4 && (epi == EPI_QKV || epi == EPI_RESID || epi == EPI_RESID_NORM);
}

bool gemv_narrow_norm_supports(int M, int N, int K, int rw, int num_cus) {
    return gemv_narrow_supports(M, N, K, EPI_QKV, rw) && M <= 32 && N / rw <= num_cus;
}

hipError_t gemv_narrow_launch(const GemmArgs& a, int rw, int num_cus, hipStream_t s) {
    if (!gemv_narrow_supports(a.M, a.N, a.K, a.epi.kind, rw)) return hipErrorInvalidValue;
    if (a.norm && !gemv_narrow_norm_supports(a.M, a.N, a.K, rw, num_cus)) return hipErrorInvalidValue;
    if (a.epi.kind == EPI_QKV && !a.norm && a.ssq_count > 4 * (a.M <= 32 ? 32 : 16)) return hipErrorInvalidValue;
    const bool two = a.N / rw > num_cus;  // more workgroups than CUs: two fit per CU
    switch (a.epi.kind) {
        case EPI_QKV: return launch_narrow_epi<EPI_QKV>(a, rw, two, s);
        case EPI_RESID: return launch_narrow_epi<EPI_RESID>(a, rw, two, s);
        default: return launch_narrow_epi<EPI_RESID_NORM>(a, rw, two, s);
    }
}

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
