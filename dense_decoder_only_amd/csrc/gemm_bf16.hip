// Large-M bf16 projection C = A . W^T on gfx950 MFMA (v_mfma_f32_32x32x16_bf16
// or v_mfma_f32_16x16x32_bf16, per schedule).
//
// Both operands are bf16 and K-contiguous: A row-major [M][K], W in 128-row x
// 64-column tiles (see tile_weights_launch), so that one k-tile of a 128-row
// block of W is 16 KB of contiguous memory.  Tiles of BM x BK (A) and BN x BK
// (W) are copied global -> LDS by the DMA path of the vector memory unit
// (global_load_lds_dwordx4: each lane's 16 bytes land in LDS without passing
// through registers), STAGES - 1 k-tiles ahead of the MFMAs.  The only
// synchronisation per k-tile is one `s_waitcnt vmcnt(n)` that retires the
// oldest stage's copies and one workgroup barrier.
//
// LDS rows are BK bf16 (BK = 32: 64 bytes, four 16-byte chunks).  Chunk c of
// row r is stored at chunk position c ^ f(r) (see swz), so the lanes reading
// one MFMA fragment column (32 consecutive rows, one chunk) hit distinct banks.
// The DMA writes 1 KB per wave instruction; lane i fetches the global chunk
// that belongs at its fixed LDS slot, which realises the swizzle for free.
//
// Epilogues (see epilogue.cuh) run on the fp32 accumulators:
//   EPI_QKV        rows scaled by 1/rms(x) from the row-norm kernel's sum of
//                  squares, RoPE, Q/K/V scattered to the query buffer and cache;
//   EPI_RESID      out = resid + C;
//   EPI_RESID_NORM out = h = resid + C, plus the operand of the next RMSNorm,
//                  bf16(h * g), and this tile's partial sum of h^2 per row;
//   EPI_SWIGLU     rows scaled by 1/rms(h) from those partials, SiLU(gate)*up.
#include <type_traits>

#include "common.cuh"
#include "epilogue.cuh"
#include "kernels.h"

namespace llb {

namespace {


// Chunk swizzle of LDS rows (measured conflict-free for ds_read_b128 on gfx950,
// whose LDS serves 16 lanes x 16 bytes per cycle from 64 four-byte banks):
// BK = 32 (four 16-byte chunks per 64-byte row): chunk c of row r sits at
// c ^ ((r >> 2) & 3); BK = 64 (eight chunks per 128-byte row): c ^ ((r >> 1) & 7).
template <int BK>
LLB_DEV int swz(int r) {
    if constexpr (BK == 32) return (r >> 2) & 3;
    else return (r >> 1) & 7;
}

// Main-loop schedules: SCHED_PLAIN (per k-tile: wait, barrier, copies,
// fragment reads and MFMAs, with latency hidden by the other waves of the
// SIMD), SCHED_INTERLEAVE (one wave per SIMD, its LDS reads and copies
// threaded between its MFMAs) and SCHED_INTERLEAVE_PF (the same, plus an L2
// prefetch of the operand lines two k-tiles ahead of the copies), all on
// 32x32x16 MFMAs; SCHED_I16 and SCHED_I16_PF are the interleaved schedules on
// 16x16x32 MFMAs, which do the same work at a lower power draw (more clock
// under the chip's power limit, measured on random operands).  Flags:
// SCHED_SPREAD (below) and SCHED_PF_W_ONLY, which prefetches the W lines only,
// for projections whose A panels the last-level cache already holds.
constexpr int SCHED_PLAIN = 0, SCHED_INTERLEAVE = 1, SCHED_INTERLEAVE_PF = 2, SCHED_I16 = 3,
              SCHED_I16_PF = 4, SCHED_SPREAD = 8, SCHED_PF_W_ONLY = 16;

template <int BM, int BN, int WAVES_M, int WAVES_N, int BK, int STAGES, int OCC, int EPI, int SCHED>
__global__ void __launch_bounds__(64 * WAVES_M * WAVES_N) __attribute__((amdgpu_waves_per_eu(OCC)))
gemm_bf16_kernel(GemmArgs args) {
    constexpr int NW = WAVES_M * WAVES_N;
    constexpr int CPR_K = BK / 8;              // 16-byte chunks per LDS row
    constexpr int RPB = 64 / CPR_K;            // rows per 1 KB DMA block
    constexpr int WTM = BM / WAVES_M;
    constexpr int WTN = BN / WAVES_N;
    constexpr int TM = WTM / 32;
    constexpr int TN = WTN / 32;
    constexpr int STAGE_ELEMS = (BM + BN) * BK;
    constexpr int BLOCKS = (BM + BN) / RPB;  // 1 KB DMA blocks per stage
    constexpr int L = BLOCKS / NW;            // DMA instructions per wave per stage
    static_assert(BLOCKS % NW == 0 && BM % RPB == 0, "DMA split");
    static_assert((STAGES - 2) * L < 64, "vmcnt range");
    constexpr int BASE = SCHED & 7;
    constexpr bool INTERLEAVED = BASE != SCHED_PLAIN;
    constexpr bool M16 = BASE == SCHED_I16 || BASE == SCHED_I16_PF;   // 16x16x32 MFMAs
    constexpr int PF_DIST = (BASE == SCHED_INTERLEAVE_PF || BASE == SCHED_I16_PF) ? 2 : 0;  // in k-tiles
    // SCHED_SPREAD: a k-tile's copies start in the second half of the last
    // k-step two k-tiles earlier (the stage is free from that barrier on) and
    // continue through the first k-step one k-tile earlier, so that the CU's
    // copy path (about 1 KB per 16 cycles) is never asked for a k-tile's 64 KB
    // within a quarter of a k-tile.
    constexpr bool SPREAD = (SCHED & SCHED_SPREAD) != 0;
    constexpr int MB = M16 ? 16 : 32;          // MFMA block edge
    constexpr int KSTEP = M16 ? 32 : 16;       // k per MFMA
    constexpr int TMB = WTM / MB, TNB = WTN / MB;
    static_assert(WTM % MB == 0 && WTN % MB == 0 && BK % KSTEP == 0, "MFMA blocks");
    static_assert(STAGES >= 2 && STAGES <= (INTERLEAVED ? 5 : 4), "pipeline depth");
    static_assert(EPI != EPI_SWIGLU || (WTN % 64) == 0, "SwiGLU needs gate/up pairs in a wave");

    // the stages, then (prefetching schedule) 256 B per wave that the L2
    // prefetch copies land in and nothing reads
    __shared__ __attribute__((aligned(1024))) bf16_t smem[STAGES * STAGE_ELEMS + (PF_DIST > 0 ? NW * 128 : 0)];

    const int M = args.M, N = args.N, K = args.K;
    const int tiles_m = (M + BM - 1) / BM;
    const int n_begin = args.n_begin;
    const int tiles_n = ((args.n_end ? args.n_end : N) - n_begin) / BN;
    // Tile order.  Workgroups are dispatched round-robin over the 8 XCDs, and
    // each XCD runs about 32 tiles at a time.  The 32 tiles of an XCD form an
    // 8 x 4 block of the tile grid (8 row panels x 4 column panels: the fewest
    // operand panels that 32 tiles can share in the XCD's L2).  The 256 tiles
    // of the chip form one (8 XR) x (4 XC) block (XR x XC = 8 XCDs, as square
    // as the grid allows), so that the operand panels the XCDs refill from
    // beyond their L2 are largely the same panels, served by the shared last
    // level cache rather than by HBM; the blocks walk the columns of a band of
    // 8 XR row panels, every other band from the right, so that a band starts
    // on the W panels the previous one ended on (measured 0.25% faster on the
    // 70B prefill).  The gate/up projection (SwiGLU epilogue) takes the taller
    // 32 x 8 block where it divides the grid: its band of A panels (128 MB)
    // stays in the last-level cache, and each round then fetches 8 W panels
    // from HBM instead of 16 (measured 0.6% faster on the 70B prefill; the
    // residual projections, whose A streams, are faster on 16 x 16).  Grids
    // that no such block divides fall back to XCDs
    // owning the columns n = x (mod 8) and walking groups of 8 row panels
    // together, or to consecutive ids per XCD (xcd_remap).
    constexpr int GM = 8;
    const int xr = (EPI == EPI_SWIGLU && tiles_m % 32 == 0 && tiles_n % 8 == 0) ? 4
                   : (tiles_m % 16 == 0 && tiles_n % 16 == 0) ? 2
                   : (tiles_m % 32 == 0 && tiles_n % 8 == 0) ? 4
                   : (tiles_m % 8 == 0 && tiles_n % 32 == 0) ? 1 : 0;
    int m0, n0;
    if (xr) {
        const int xc = 8 / xr;
        const int x = blockIdx.x % 8, j = blockIdx.x / 8;
        const int r = j / 32, w = j % 32;          // chip block, place in the XCD's 8 x 4
        const int ncb = tiles_n / (4 * xc);
        const int rb = r / ncb, cb = (rb & 1) ? ncb - 1 - r % ncb : r % ncb;
        m0 = (rb * 8 * xr + (x % xr) * 8 + w % 8) * BM;
        n0 = n_begin + (cb * 4 * xc + (x / xr) * 4 + w / 8) * BN;
    } else if (tiles_n % 8 == 0) {
        const int x = blockIdx.x % 8, j = blockIdx.x / 8;
        const int ncx = tiles_n / 8;
        const int group = j / (GM * ncx);
        const int first_m = group * GM;
        const int gm = min(tiles_m - first_m, GM);
        const int in_group = j - group * (GM * ncx);
        m0 = (first_m + in_group % gm) * BM;
        n0 = n_begin + ((in_group / gm) * 8 + x) * BN;
    } else {
        const int tile = xcd_remap(blockIdx.x, tiles_m * tiles_n);
        const int group = tile / (GM * tiles_n);
        const int first_m = group * GM;
        const int gm = min(tiles_m - first_m, GM);
        const int in_group = tile - group * (GM * tiles_n);
        m0 = (first_m + in_group % gm) * BM;
        n0 = n_begin + (in_group / gm) * BN;
    }

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    static_assert(!INTERLEAVED || (NW == 4 && (BK == 32 || BK == 64) && STAGES >= 2), "interleaved shape");
    const int wm = wave % WAVES_M;
    const int wn = wave / WAVES_M;

    const bf16_t* __restrict__ A = (const bf16_t*)args.A;
    const bf16_t* __restrict__ W = (const bf16_t*)args.W;

    // Per-lane global source of each of this wave's DMA blocks (k0 = 0).  A is
    // row-major [M, K]; W is stored in 128-row x 64-column tiles (see
    // tile_weights_launch): element (n, k) at
    // ((n / 128) * (K / 64) + k / 64) * 8192 + (n % 128) * 64 + k % 64.
    const bf16_t* src[L];
    bool is_w[L];
#pragma unroll
    for (int i = 0; i < L; ++i) {
        const int blk = wave + i * NW;
        const int row = blk * RPB + lane / CPR_K;        // row in the [A; W] stage
        const int chunk = (lane % CPR_K) ^ swz<BK>(row);
        is_w[i] = blk * RPB >= BM;
        if (!is_w[i]) {
            const int gm = min(m0 + row, M - 1);         // rows past M: any valid row
            src[i] = A + (size_t)gm * K + chunk * 8;
        } else {
            const int wr = n0 + row - BM;
            src[i] = W + (size_t)(wr >> 7) * (K / 64) * 8192 + (wr & 127) * 64 + chunk * 8;
        }
    }
    // element offset of k-tile kt from a block's k0 = 0 source
    auto k_off = [&](int i, int kt) -> size_t {
        if (!is_w[i]) return (size_t)kt * BK;
        if constexpr (BK == 64) return (size_t)kt * 8192;
        else return (size_t)(kt >> 1) * 8192 + (kt & 1) * 32;
    };
    // Copies of k-tile kt into stage `st` (a compile-time constant at every call:
    // the stage offsets must be constants for the compiler to see that the LDS
    // reads of one stage do not depend on the copies in flight to another).
    const uint32_t lds_base = lds_offset(smem);
    auto issue = [&](int kt, int st) {
#pragma unroll
        for (int i = 0; i < L; ++i) {
            const int blk = wave + i * NW;
            dma16(src[i] + k_off(i, kt),
                  lds_base + (uint32_t)((st * STAGE_ELEMS + blk * RPB * BK) * sizeof(bf16_t)));
        }
    };

    static_assert(BM <= 64 * NW, "one thread per tile row");
    constexpr bool SCALED = (EPI == EPI_QKV || EPI == EPI_SWIGLU || EPI == EPI_LOGITS);
    const int nk = K / BK;
#pragma unroll
    for (int st = 0; st < STAGES - 1; ++st)
        if (st < nk) issue(st, st);

    // Row scale of the normalised-operand epilogues (one thread per tile row),
    // loaded after the first copies so that its loads wait alongside theirs;
    // the partial sums of squares are fetched eight at a time and added in
    // index order.  Parked in LDS after the main loop.
    float row_scale = 1.0f;
    if constexpr (SCALED) {
        const int m = m0 + tid;
        if (tid < BM && m < M) {
            const float* ssq = args.ssq_in + m;
            float s = 0.f;
            int p = 0;
            for (; p + 8 <= args.ssq_count; p += 8) {
                float v[8];
#pragma unroll
                for (int q = 0; q < 8; ++q) v[q] = ssq[(size_t)(p + q) * M];
#pragma unroll
                for (int q = 0; q < 8; ++q) s += v[q];
            }
            for (; p < args.ssq_count; ++p) s += ssq[(size_t)p * M];
            row_scale = inv_rms(s, K, args.eps);
        }
    }

    // accumulators: 32x32 blocks (acc) or 16x16 blocks (acc16); the other is unused
    f32x16 acc[M16 ? 1 : TM][M16 ? 1 : TN];
    f32x4 acc16[M16 ? TMB : 1][M16 ? TNB : 1];
    if constexpr (M16) {
#pragma unroll
        for (int i = 0; i < TMB; ++i)
#pragma unroll
            for (int j = 0; j < TNB; ++j) acc16[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    } else {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    }

    auto compute = [&](int st) {
        const bf16_t* a_s = smem + st * STAGE_ELEMS;
        const bf16_t* b_s = a_s + BM * BK;
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            const int c = 2 * kk + (lane >> 5);
            bf16x8 af[TM], bfr[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const int r = wm * WTM + i * 32 + (lane & 31);
                af[i] = as_bf16x8(*(const uint4*)&a_s[r * BK + ((c ^ swz<BK>(r)) << 3)]);
            }
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int r = wn * WTN + j * 32 + (lane & 31);
                bfr[j] = as_bf16x8(*(const uint4*)&b_s[r * BK + ((c ^ swz<BK>(r)) << 3)]);
            }
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) acc[i][j] = mfma32(af[i], bfr[j], acc[i][j]);
        }
    };
    if constexpr (!INTERLEAVED) {
        // One k-tile: retire its copies (the STAGES-2 later ones stay in flight),
        // barrier, refill the stage that was read one step earlier, multiply.
        auto step = [&](int kt, int rd, int wr) {
            const int later = min(STAGES - 2, nk - 1 - kt);
            if (STAGES >= 4 && later >= 2) wait_vm_lgkm<(STAGES >= 4 ? 2 : 0) * L>();
            else if (STAGES >= 3 && later >= 1) wait_vm_lgkm<(STAGES >= 3 ? 1 : 0) * L>();
            else wait_vm_lgkm<0>();
            barrier();
            if (kt + STAGES - 1 < nk) issue(kt + STAGES - 1, wr);
            compute(rd);
        };
        // unrolled over the stages so that every stage offset is a constant
        for (int kt = 0; kt < nk; kt += STAGES) {
    #pragma unroll
            for (int st = 0; st < STAGES; ++st)
                if (kt + st < nk) step(kt + st, st, (st + STAGES - 1) % STAGES);
        }
    } else {
        // Interleaved: one wave per SIMD owns a WTM x WTN block (TMB x TNB MFMA
        // blocks of MB x MB, NM = TMB*TNB MFMAs per k-step of KSTEP, NR =
        // TMB+TNB fragment reads).  Within k-tile t, the MFMAs of steps 0..KS-2 are threaded with
        // the reads of the next step's fragments (first) and this k-tile's share
        // of the copies of k-tile t+STAGES-1 into the stage of k-tile t-1; the
        // MFMAs of the last step are split around the wait + barrier that
        // publishes k-tile t+1, after which step 0's fragments of k-tile t+1 are
        // read between the remaining MFMAs.  Every element is pinned in place
        // with a scheduling barrier.
        constexpr int NM = TMB * TNB, NR = TMB + TNB;
        constexpr int KS = BK / KSTEP;
        // the copies ride on k-steps 0..KS-2 (a tile of one k-step, 16x16x32
        // MFMAs at BK 32, computed wrong results when tried: not supported)
        static_assert(KS > 1, "interleaved schedules need at least two k-steps per k-tile");
        static_assert(NR <= NM, "reads ride on the MFMAs");
        bf16x8 fa[2][TMB], fb[2][TNB];
        uint32_t a_off[KS], b_off[KS];
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
            // fragment of an MB-row block: lane -> row lane % MB, 16-byte k-chunk
            // (KSTEP / 8) kk + lane / MB
            const int c = (KSTEP / 8) * kk + lane / MB;
            const int ra = wm * WTM + lane % MB, rb = wn * WTN + lane % MB;
            a_off[kk] = lds_base + (uint32_t)((ra * BK + ((c ^ swz<BK>(ra)) << 3)) * 2);
            b_off[kk] = lds_base + (uint32_t)((BM * BK + rb * BK + ((c ^ swz<BK>(rb)) << 3)) * 2);
        }
        constexpr uint32_t STAGE_BYTES = STAGE_ELEMS * 2;
        typedef bf16x8 __attribute__((address_space(3))) * lds_frag_ptr;
        // n-th of the NR fragment reads of one k-step, in the order the MFMAs
        // (i-major) first use them: A0 B0 .. B(TNB-1) A1 .. A(TMB-1).  ab / bb:
        // that k-step's fragment-0 addresses in the stage (the swizzle of row
        // r + MB i equals that of r: MB i / 2 is a multiple of 8).
        auto rd = [&](uint32_t ab, uint32_t bb, int fbuf, int n) {
            if (n == 0) fa[fbuf][0] = *(lds_frag_ptr)(uintptr_t)(ab);
            else if (n <= TNB) fb[fbuf][n - 1] = *(lds_frag_ptr)(uintptr_t)(bb + (n - 1) * MB * BK * 2);
            else fa[fbuf][n - TNB] = *(lds_frag_ptr)(uintptr_t)(ab + (n - TNB) * MB * BK * 2);
        };
        // n-th of the NM MFMAs of a k-step, in serpentine order (odd block rows
        // walk j downwards, so consecutive MFMAs always share an operand:
        // measured 0.4% faster on the 70B gate/up than plain row order)
        auto mf = [&](int fbuf, int n) {
            const int i = n / TNB, j = (i & 1) ? TNB - 1 - n % TNB : n % TNB;
            if constexpr (M16) acc16[i][j] = mfma16(fa[fbuf][i], fb[fbuf][j], acc16[i][j]);
            else acc[i][j] = mfma32(fa[fbuf][i], fb[fbuf][j], acc[i][j]);
        };
        // Copies with a scalar base per operand and k-tile and a fixed per-lane
        // offset: copy i moves A rows for i < NA, W rows after (BM/RPB rows
        // blocks of A are a multiple of the wave count).
        constexpr int NA = BM / (RPB * NW);
        static_assert(BM % (RPB * NW) == 0, "copy i is all-A or all-W");
        uint32_t voff[L];
#pragma unroll
        for (int i = 0; i < L; ++i)
            voff[i] = (uint32_t)((const char*)src[i] - (const char*)(i < NA ? A : W));
        // The c-th copy a k-tile issues moves block i: the W blocks go first.
        // W is the operand that streams from HBM (the A panels of a band stay
        // in the last-level cache), so its copies get the most time to land
        // before the wait (measured 1.3% faster on the 70B prefill than A
        // first, 0.7% on the 8B).
        auto dma_one = [&](int kt, int st, int c) {
            const int i = c < L - NA ? NA + c : c - (L - NA);
            const int blk = wave + i * NW;
            const char* sb = i < NA ? (const char*)A + (size_t)kt * BK * 2 : (const char*)W + k_off(NA, kt) * 2;
            dma16_s(voff[i], sb, lds_base + (uint32_t)((st * STAGE_ELEMS + blk * RPB * BK) * sizeof(bf16_t)));
        };
        // L2 prefetch (SCHED_INTERLEAVE_PF): each lane touches one 128-byte line
        // of the k-tile PF_DIST ahead of the copies, in one of this wave's 64 A
        // rows and 64 W rows, with a 4-byte LDS copy into the wave's scratch
        // slot.  The copies of k-tile t+1 then mostly hit in L2.  The two
        // prefetch loads are issued after the tile's copies, so waiting for the
        // copies leaves them in flight (vector memory loads complete in order).
        // SCHED_PF_W_ONLY drops the A line: where a band's A panels stay in the
        // last-level cache (the gate/up projection walks 7 to 14 column blocks
        // per band; an 8B prefill's whole A is 16 MB) its prefetch only adds
        // traffic and a load for the waits to cover.
        constexpr bool PF_A = (SCHED & SCHED_PF_W_ONLY) == 0;
        constexpr int NPF = PF_DIST > 0 ? (PF_A ? 2 : 1) : 0;
        const bf16_t* pf_a = A + (size_t)min(m0 + (wave * 64 + lane) % BM, M - 1) * K;
        const int pf_n = n0 + (wave * 64 + lane) % BN;
        const bf16_t* pf_w = W + (size_t)(pf_n >> 7) * (K / 64) * 8192 + (pf_n & 127) * 64;
        const uint32_t pf_lds = lds_base + (uint32_t)(STAGES * STAGE_ELEMS * 2) + wave * 256;
        auto prefetch = [&](int kt) {
            if constexpr (PF_A) dma4(pf_a + (size_t)kt * BK, pf_lds);
            dma4(pf_w + (size_t)(BK == 64 ? kt : kt >> 1) * 8192, pf_lds);
        };
        // the prologue issued k-tiles 0..STAGES-2 (clamped copies for small K
        // keep the count): k-tile 0 landed once (STAGES-2) L copies are pending
        for (int t = nk; t < STAGES - 1; ++t)
            for (int i = 0; i < L; ++i) dma_one(nk - 1, t, i);
        // SPREAD: the first CA copies of k-tile STAGES-1, as the second half of
        // a previous k-tile would have issued them (an eighth of the copies:
        // with W first, a quarter or more was slower, none no faster)
        constexpr int CA = SPREAD ? L / 8 : 0;
        static_assert(!SPREAD || KS >= 2, "spread copies: two or more k-steps");
        if constexpr (SPREAD)
            for (int i = 0; i < CA; ++i) dma_one(min(STAGES - 1, nk - 1), STAGES - 1, i);
        wait_vm_lgkm<(STAGES - 2) * L + CA>();
        barrier();
#pragma unroll
        for (int n = 0; n < NR; ++n) rd(a_off[0], b_off[0], 0, n);
        // copies per step of 0..KS-2 (the last step carries none)
        constexpr int CPS = (L - CA + KS - 2) / (KS - 1);
        // MFMAs of the last k-step before the copy wait: half, or five eighths on
        // the W-only-prefetch kernels, whose copies of W land later (the gate/up
        // projections: 0.8% faster; half is best with both prefetches)
        constexpr int HALF = (SCHED & SCHED_PF_W_ONLY) ? NM * 5 / 8 : NM / 2;
        // The body is the same for every k-tile: near the end, the copies of
        // "k-tile t+STAGES-1" repeat the last k-tile into the free stage and
        // the reads of "k-tile t+1" land in registers that are not used again.
        auto tile_k = [&](int t, int st) {
            const int t_copy = min(t + STAGES - 1, nk - 1);
            const int st_copy = (st + STAGES - 1) % STAGES;
            const int st_next = (st + 1) % STAGES;
            // fragment-0 addresses of this tile's k-steps 1..KS-1 and of the
            // next tile's step 0 (each block's read adds an immediate offset)
            uint32_t ab[KS], bb[KS];
#pragma unroll
            for (int kk = 1; kk < KS; ++kk) {
                ab[kk] = a_off[kk] + st * STAGE_BYTES;
                bb[kk] = b_off[kk] + st * STAGE_BYTES;
            }
            const uint32_t ab_next = a_off[0] + st_next * STAGE_BYTES;
            const uint32_t bb_next = b_off[0] + st_next * STAGE_BYTES;
#pragma unroll
            for (int ks = 0; ks + 1 < KS; ++ks) {
                // ops of this step: NR reads, then copies ks*CPS .. ks*CPS+CPS-1
                // (SPREAD: reads and the remaining copies CA.. alternate)
                constexpr int Q = NR + CPS;
#pragma unroll
                for (int n = 0; n < NM; ++n) {
                    mf(ks & 1, n);
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int q = n * Q / NM; q < (n + 1) * Q / NM; ++q) {
                        if constexpr (SPREAD) {
                            // op q: a copy when q is odd and copies remain, else a read
                            const int nc = q < 2 * CPS ? (q + 1) / 2 : CPS;   // copies among ops < q+1
                            const bool is_copy = q < 2 * CPS ? (q & 1) : false;
                            const int ci = CA + ks * CPS + nc - 1;
                            if (is_copy) {
                                if (ci < L) dma_one(t_copy, st_copy, ci);
                            } else {
                                rd(ab[ks + 1], bb[ks + 1], (ks + 1) & 1, q - nc);
                            }
                        } else {
                            if (q < NR) rd(ab[ks + 1], bb[ks + 1], (ks + 1) & 1, q);
                            else if (ks * CPS + q - NR < L) dma_one(t_copy, st_copy, ks * CPS + q - NR);
                        }
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            if constexpr (PF_DIST > 0) prefetch(min(t + PF_DIST, nk - 1));
            constexpr int LB = (KS - 1) & 1;  // fragment buffer of the last step
            // last step, first half
#pragma unroll
            for (int n = 0; n < HALF; ++n) {
                mf(LB, n);
                __builtin_amdgcn_sched_barrier(0);
            }
            // k-tile t+1 landed (the copies of the STAGES-2 later ones and this
            // tile's prefetch loads stay in flight)
            wait_vm_lgkm<(STAGES - 2) * L + NPF>();
            barrier();
            // last step, second half, with step 0's fragments of k-tile t+1
            // (SPREAD: then the first CA copies of k-tile t+2 into this stage)
            constexpr int Q2 = NR + CA;
            const int t_copy2 = min(t + STAGES, nk - 1);
#pragma unroll
            for (int n = HALF; n < NM; ++n) {
                mf(LB, n);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int q = (n - HALF) * Q2 / (NM - HALF); q < (n - HALF + 1) * Q2 / (NM - HALF); ++q) {
                    if (q < NR) rd(ab_next, bb_next, 0, q);
                    else dma_one(t_copy2, st, q - NR);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        for (int kt = 0; kt < nk; ++kt) tile_k(kt, kt % STAGES);
        wait_vm_lgkm<0>();  // the trailing (repeated) copies
    }
    __syncthreads();  // no copies are in flight here: the stages are free

    // ---- epilogue: each 16-row half of a 32-row slice of a wave's tile goes
    // through LDS so that a lane owns 8 consecutive columns of a row (RoPE pairs
    // and gate/up pairs in one thread, 16-byte stores).  LDS (reusing the
    // stages): [staging slices of the NW waves][row scales BM][row partial
    // sums of squares WAVES_N x BM].
    const Epilogue& e = args.epi;
    constexpr int HR = 16;                        // rows staged at a time per wave
    constexpr int SROW = WTN + 4;                 // padded fp32 row of the staging slice
    static_assert((NW * HR * SROW + BM + WAVES_N * BM) * 4 <= STAGES * STAGE_ELEMS * 2,
                  "epilogue LDS fits in the stages");
    float* stile = (float*)smem + wave * (HR * SROW);
    float* sScale = (float*)smem + NW * HR * SROW;
    float* sPart = sScale + BM;
    if constexpr (SCALED) {
        if (tid < BM) sScale[tid] = row_scale;
        __syncthreads();
    }
    // Residual epilogues: a lane's 8 columns are the same in every slice, so
    // its gains are loaded once, and the residual rows of the next slice are
    // loaded before the current slice's stores.  Vector-memory operations
    // complete in order, so a load issued after a store waits for that store
    // too; issued this way, each slice waits for one load issued a slice
    // earlier instead of one round trip per chunk (70B O projection 3% and
    // 8B O 5% faster than loading each chunk's residual and gains in turn).
    constexpr int RCPR = WTN / 8;                       // 8-column chunks per row
    // (slices whose chunk count does not divide into lanes keep the plain flush)
    constexpr bool RES = (EPI == EPI_RESID || EPI == EPI_RESID_NORM) && 64 % RCPR == 0 &&
                         (HR * RCPR) % 64 == 0;
    constexpr int RIT = RES ? HR * RCPR / 64 : 1;       // chunks per lane per slice
    const int rch = lane % RCPR;
    const int rn = n0 + wn * WTN + rch * 8;
    float4 rcur[RIT][2], rnext[RIT][2];
    float rg[8];
    auto load_res = [&](int rbase, float4 (&r)[RIT][2]) {
#pragma unroll
        for (int k = 0; k < RIT; ++k) {
            const int m = min(m0 + rbase + lane / RCPR + k * (64 / RCPR), M - 1);
            const float* p = e.resid + (size_t)m * N + rn;
            r[k][0] = *(const float4*)p;
            r[k][1] = *(const float4*)(p + 4);
        }
    };
    if constexpr (RES) {
        if constexpr (EPI == EPI_RESID_NORM) {
            *(float4*)&rg[0] = *(const float4*)(e.gain + rn);
            *(float4*)&rg[4] = *(const float4*)(e.gain + rn + 4);
        }
        load_res(wm * WTM, rcur);
    }
    auto flush_res = [&](int rbase, int next_rbase) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        if (next_rbase >= 0) load_res(next_rbase, rnext);
#pragma unroll
        for (int k = 0; k < RIT; ++k) {
            const int row = lane / RCPR + k * (64 / RCPR);
            const int m = m0 + rbase + row;
            const float4 s0 = *(const float4*)&stile[row * SROW + rch * 8];
            const float4 s1 = *(const float4*)&stile[row * SROW + rch * 8 + 4];
            float v[8];
            v[0] = s0.x + rcur[k][0].x; v[1] = s0.y + rcur[k][0].y;
            v[2] = s0.z + rcur[k][0].z; v[3] = s0.w + rcur[k][0].w;
            v[4] = s1.x + rcur[k][1].x; v[5] = s1.y + rcur[k][1].y;
            v[6] = s1.z + rcur[k][1].z; v[7] = s1.w + rcur[k][1].w;
            float ss = 0.f;
            if (m < M) {
                const size_t idx = (size_t)m * N + rn;
                *(float4*)(e.out + idx) = make_float4(v[0], v[1], v[2], v[3]);
                *(float4*)(e.out + idx + 4) = make_float4(v[4], v[5], v[6], v[7]);
                if constexpr (EPI == EPI_RESID_NORM) {
                    float t[8];
#pragma unroll
                    for (int c = 0; c < 8; ++c) t[c] = v[c] * rg[c];
                    *(uint4*)((bf16_t*)e.a_out + idx) = pack8(t);
#pragma unroll
                    for (int c = 0; c < 8; ++c) ss += v[c] * v[c];
                }
            }
            if constexpr (EPI == EPI_RESID_NORM) {
#pragma unroll
                for (int off = 1; off < RCPR; off <<= 1) ss += __shfl_xor(ss, off, 64);
                if (rch == 0) sPart[wn * BM + rbase + row] = ss;
            }
        }
        if (next_rbase >= 0) {
#pragma unroll
            for (int k = 0; k < RIT; ++k) {
                rcur[k][0] = rnext[k][0];
                rcur[k][1] = rnext[k][1];
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };
    // the staged rows rbase .. rbase + HR - 1 of this wave's slice, from LDS to
    // the epilogue
    auto flush = [&](int rbase) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        if constexpr (EPI == EPI_SWIGLU) {
            constexpr int CPR = WTN / 16;         // (gate, up) chunk pairs per row
            for (int idx = lane; idx < HR * CPR; idx += 64) {
                const int row = idx / CPR, ch = idx % CPR;
                const int cg = (ch >> 2) * 64 + (ch & 3) * 8;   // gate columns in the slice
                const int m = m0 + rbase + row;
                float g[8], u[8];
                *(float4*)&g[0] = *(const float4*)&stile[row * SROW + cg];
                *(float4*)&g[4] = *(const float4*)&stile[row * SROW + cg + 4];
                *(float4*)&u[0] = *(const float4*)&stile[row * SROW + cg + 32];
                *(float4*)&u[4] = *(const float4*)&stile[row * SROW + cg + 36];
                const int f = ((n0 + wn * WTN + cg - (cg & 63)) >> 1) + (cg & 63);
                if (m < M) epi_swiglu8(e, m, f, N >> 1, g, u);
            }
        } else {
            constexpr int CPR = WTN / 8;          // 8-column chunks per row
            for (int idx = lane; idx < HR * CPR; idx += 64) {
                const int row = idx / CPR, ch = idx % CPR;
                const int m = m0 + rbase + row;
                const int n = n0 + wn * WTN + ch * 8;
                float v[8];
                *(float4*)&v[0] = *(const float4*)&stile[row * SROW + ch * 8];
                *(float4*)&v[4] = *(const float4*)&stile[row * SROW + ch * 8 + 4];
                if constexpr (EPI == EPI_QKV) {
                    if (m < M) epi_qkv8(e, m, n, v);
                } else if constexpr (EPI == EPI_LOGITS) {
                    if (m < M) epi_store8(e, m, n, N, v);
                } else {
                    float ss = 0.f;
                    if (m < M) {
                        epi_resid8(e, m, n, N, v);
                        if constexpr (EPI == EPI_RESID_NORM) ss = epi_norm_operand8(e, m, n, N, v);
                    }
                    if constexpr (EPI == EPI_RESID_NORM) {
                        // the CPR lanes of one row are consecutive: reduce over them
                        static_assert(CPR == 16 || CPR == 8, "row reduction width");
#pragma unroll
                        for (int off = 1; off < CPR; off <<= 1) ss += __shfl_xor(ss, off, 64);
                        if ((lane % CPR) == 0) sPart[wn * BM + rbase + row] = ss;
                    }
                }
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };
    if constexpr (M16) {
        // 16x16 blocks: register r of block (i, j) is row 16 i + 4 (lane / 16) + r,
        // column 16 j + lane % 16; a block row of 16 is one staging pass
        static_assert(HR == 16, "one 16-row block per pass");
#pragma unroll
        for (int i = 0; i < TMB; ++i) {
            const int rbase = wm * WTM + i * 16;
            float4 sc4 = make_float4(1.f, 1.f, 1.f, 1.f);
            if constexpr (SCALED) sc4 = *(const float4*)&sScale[rbase + 4 * (lane >> 4)];
            // unscaled epilogues still multiply by an (opaque) 1: staging the
            // accumulators by plain copies let the register allocator shuffle
            // them through the main loop (three AGPR moves per MFMA)
            else asm volatile("" : "+v"(sc4.x), "+v"(sc4.y), "+v"(sc4.z), "+v"(sc4.w));
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int rr = 4 * (lane >> 4) + r;
                const float sc = r == 0 ? sc4.x : r == 1 ? sc4.y : r == 2 ? sc4.z : sc4.w;
#pragma unroll
                for (int j = 0; j < TNB; ++j) stile[rr * SROW + j * 16 + (lane & 15)] = acc16[i][j][r] * sc;
            }
            if constexpr (RES) flush_res(rbase, i + 1 < TMB ? rbase + 16 : -1);
            else flush(rbase);
        }
    } else {
#pragma unroll
        for (int i = 0; i < TM; ++i) {
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int rbase = wm * WTM + i * 32 + half * HR;   // tile row of the staged rows
                // staged row rr of register r: 8 (r / 4) + 4 (lane / 32) + r % 4 - 16 half,
                // i.e. two runs of 4 consecutive rows whose scales are read at once
                float4 sc4[2] = {make_float4(1.f, 1.f, 1.f, 1.f), make_float4(1.f, 1.f, 1.f, 1.f)};
                if constexpr (SCALED) {
                    sc4[0] = *(const float4*)&sScale[rbase + 4 * (lane >> 5)];
                    sc4[1] = *(const float4*)&sScale[rbase + 8 + 4 * (lane >> 5)];
                }
#pragma unroll
                for (int r = 8 * half; r < 8 * half + 8; ++r) {
                    const int rr = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3) - half * HR;
                    const float4 s4 = sc4[(r >> 2) & 1];
                    const float sc = (r & 3) == 0 ? s4.x : (r & 3) == 1 ? s4.y : (r & 3) == 2 ? s4.z : s4.w;
#pragma unroll
                    for (int j = 0; j < TN; ++j)
                        stile[rr * SROW + j * 32 + (lane & 31)] = acc[i][j][r] * sc;
                }
                if constexpr (RES) flush_res(rbase, half == 0 ? rbase + HR : i + 1 < TM ? rbase + HR : -1);
                else flush(rbase);
            }
        }
    }

    if constexpr (EPI == EPI_RESID_NORM) {
        __syncthreads();
        for (int rl = tid; rl < BM; rl += 64 * NW) {
            const int m = m0 + rl;
            if (m < M) {
                float s = 0.f;
#pragma unroll
                for (int w = 0; w < WAVES_N; ++w) s += sPart[w * BM + rl];
                e.ssq_out[(size_t)(n0 / BN) * M + m] = s;
            }
        }
    }
}

// W [N, K] row-major -> 128 x 64 tiles, tile (N/128, K/64) row-major, each
// tile row-major (64 elements = 128 bytes per row): a pipeline stage of a
// projection then reads whole, contiguous 16 KB tiles.  One thread per 8
// elements.
__global__ void __launch_bounds__(256)
tile_weights_kernel(const bf16_t* __restrict__ src, bf16_t* __restrict__ dst, int N, int K) {
    const long idx = (long)blockIdx.x * 256 + threadIdx.x;  // 8-element unit
    const long units = (long)N * K / 8;
    if (idx >= units) return;
    const int n = (int)(idx / (K / 8));
    const int k = (int)(idx % (K / 8)) * 8;
    const size_t o = ((size_t)(n >> 7) * (K / 64) + (k >> 6)) * 8192 + (n & 127) * 64 + (k & 63);
    *(uint4*)(dst + o) = *(const uint4*)(src + (size_t)n * K + k);
}

struct TileCfg {
    int bm, bn, wm, wn, bk, stages, occ, sched;
};
// The host picks one per projection from its shape and epilogue (0, 1, 2, 4,
// 6, 7, 14, 16, 17, 18 on the shapes measured); the others stay for tuning and
// are covered by the parity tests like the rest.
constexpr TileCfg kTiles[] = {
    {256, 256, 4, 2, 64, 2, 2, 0},  // 8 waves (2 per SIMD), wave tile 64x128, BK 64, 128 KB LDS
    {256, 128, 2, 2, 32, 3, 2, 0},  // 4 waves, wave tile 128x64, 72 KB: 2 workgroups per CU
    {128, 128, 2, 2, 32, 4, 2, 0},  // 4 waves, wave tile 64x64, 64 KB: 2 workgroups per CU
    {256, 256, 2, 2, 64, 2, 1, 1},  // 4 waves (1 per SIMD), wave tile 128x128, interleaved, BK 64
    {256, 256, 2, 2, 64, 2, 1, 2},  // the same with the L2 prefetch
    {256, 128, 2, 2, 64, 3, 1, 0},  // 4 waves, BK 64, 3 stages (144 KB)
    {256, 192, 2, 2, 64, 2, 1, 1},  // interleaved, wave tile 128x96
    {256, 128, 2, 2, 64, 3, 1, 1},  // interleaved, wave tile 128x64, 3 stages
    {256, 256, 2, 2, 32, 4, 1, 1},  // interleaved 128x128, BK 32, 4 stages
    {256, 256, 2, 2, 64, 2, 1, 3},  // 3 on 16x16x32 MFMAs
    {256, 256, 2, 2, 64, 2, 1, 4},  // 4 on 16x16x32 MFMAs
    {256, 128, 2, 2, 64, 3, 1, 3},  // 7 on 16x16x32 MFMAs
    {256, 192, 2, 2, 64, 2, 1, 3},  // 6 on 16x16x32 MFMAs
    {256, 192, 2, 2, 64, 2, 1, 4},  // 12 with the L2 prefetch
    {256, 256, 2, 2, 64, 2, 1, 4 + 8},  // 10 with spread copies
    {256, 192, 2, 2, 64, 2, 1, 4 + 8},  // 13 with spread copies
    {256, 128, 2, 2, 64, 3, 1, 1 + 8},  // 7 with spread copies
    {256, 256, 2, 2, 64, 2, 1, 4 + 8 + 16},  // 14 prefetching W lines only
    {256, 192, 2, 2, 64, 2, 1, 4 + 8 + 16},  // 15 prefetching W lines only
};
constexpr int kNumTiles = sizeof(kTiles) / sizeof(kTiles[0]);

template <int BM, int BN, int WM, int WN, int BK, int ST, int OCC, int SCHED, int EPI>
hipError_t launch_one(const GemmArgs& a, hipStream_t s) {
    // a wave's column slice must hold whole (gate, up) 64-column pairs for
    // SwiGLU, and a power-of-two number of 8-column chunks (8 or 16) for the
    // norm-operand row reduction; other shapes reject those epilogues
    constexpr int WTN = BN / WN;
    if constexpr ((EPI == EPI_SWIGLU && WTN % 64 != 0) ||
                  (EPI == EPI_RESID_NORM && WTN != 64 && WTN != 128)) {
        return hipErrorInvalidValue;
    } else {
        const int tiles = ((a.M + BM - 1) / BM) * (((a.n_end ? a.n_end : a.N) - a.n_begin) / BN);
        hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WM, WN, BK, ST, OCC, EPI, SCHED>), dim3(tiles),
                           dim3(64 * WM * WN), 0, s, a);
        return hipGetLastError();
    }
}

template <int BM, int BN, int WM, int WN, int BK, int ST, int OCC, int SCHED = SCHED_PLAIN>
hipError_t launch_cfg(const GemmArgs& a, hipStream_t s) {
    switch (a.epi.kind) {
        case EPI_QKV: return launch_one<BM, BN, WM, WN, BK, ST, OCC, SCHED, EPI_QKV>(a, s);
        case EPI_SWIGLU: return launch_one<BM, BN, WM, WN, BK, ST, OCC, SCHED, EPI_SWIGLU>(a, s);
        case EPI_RESID: return launch_one<BM, BN, WM, WN, BK, ST, OCC, SCHED, EPI_RESID>(a, s);
        case EPI_RESID_NORM: return launch_one<BM, BN, WM, WN, BK, ST, OCC, SCHED, EPI_RESID_NORM>(a, s);
        case EPI_LOGITS: return launch_one<BM, BN, WM, WN, BK, ST, OCC, SCHED, EPI_LOGITS>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

int gemm_bf16_num_tile_cfgs() { return kNumTiles; }

bool gemm_bf16_offsets_fit(long M, long N, long K) {
    return M * K * 2 <= 0xffffffffL && N * K * 2 <= 0xffffffffL;
}

hipError_t tile_weights_launch(const void* src, void* dst, int N, int K, hipStream_t s) {
    if (N <= 0 || K <= 0 || N % 128 != 0 || K % 64 != 0 || src == dst) return hipErrorInvalidValue;
    const long units = (long)N * K / 8;
    hipLaunchKernelGGL(tile_weights_kernel, dim3((unsigned)((units + 255) / 256)), dim3(256), 0, s,
                       (const bf16_t*)src, (bf16_t*)dst, N, K);
    return hipGetLastError();
}

bool gemm_bf16_supports(int cfg, int M, int N, int K, int epi) {
    if (cfg < 0 || cfg >= kNumTiles) return false;
    const TileCfg t = kTiles[cfg];
    if (M <= 0 || N <= 0 || N % t.bn != 0 || K < t.bk || K % t.bk != 0) return false;
    // the interleaved schedules address A and W by 32-bit byte offsets
    if (t.sched != SCHED_PLAIN && !gemm_bf16_offsets_fit(M, N, K)) return false;
    const int wtn = t.bn / t.wn;
    if (epi == EPI_SWIGLU && wtn % 64 != 0) return false;
    if (epi == EPI_RESID_NORM && wtn != 64 && wtn != 128) return false;
    return true;
}

void gemm_bf16_tile(int cfg, int* bm, int* bn, int* threads) {
    *bm = kTiles[cfg].bm;
    *bn = kTiles[cfg].bn;
    *threads = 64 * kTiles[cfg].wm * kTiles[cfg].wn;
}

hipError_t gemm_bf16_launch(const GemmArgs& a, int cfg, hipStream_t s) {
    if (cfg < 0 || cfg >= kNumTiles) return hipErrorInvalidValue;
    if (!gemm_bf16_supports(cfg, a.M, a.N, a.K, a.epi.kind)) return hipErrorInvalidValue;
    const int n_end = a.n_end ? a.n_end : a.N;
    const int bn = kTiles[cfg].bn;
    if (a.n_begin < 0 || a.n_begin % bn != 0 || n_end % bn != 0 || n_end > a.N || a.n_begin >= n_end)
        return hipErrorInvalidValue;
    switch (cfg) {
        case 0: return launch_cfg<256, 256, 4, 2, 64, 2, 2>(a, s);
        case 1: return launch_cfg<256, 128, 2, 2, 32, 3, 2>(a, s);
        case 2: return launch_cfg<128, 128, 2, 2, 32, 4, 2>(a, s);
        case 3: return launch_cfg<256, 256, 2, 2, 64, 2, 1, SCHED_INTERLEAVE>(a, s);
        case 4: return launch_cfg<256, 256, 2, 2, 64, 2, 1, SCHED_INTERLEAVE_PF>(a, s);
        case 5: return launch_cfg<256, 128, 2, 2, 64, 3, 1>(a, s);
        case 6: return launch_cfg<256, 192, 2, 2, 64, 2, 1, SCHED_INTERLEAVE>(a, s);
        case 7: return launch_cfg<256, 128, 2, 2, 64, 3, 1, SCHED_INTERLEAVE>(a, s);
        case 8: return launch_cfg<256, 256, 2, 2, 32, 4, 1, SCHED_INTERLEAVE>(a, s);
        case 9: return launch_cfg<256, 256, 2, 2, 64, 2, 1, SCHED_I16>(a, s);
        case 10: return launch_cfg<256, 256, 2, 2, 64, 2, 1, SCHED_I16_PF>(a, s);
        case 11: return launch_cfg<256, 128, 2, 2, 64, 3, 1, SCHED_I16>(a, s);
        case 12: return launch_cfg<256, 192, 2, 2, 64, 2, 1, SCHED_I16>(a, s);
        case 13: return launch_cfg<256, 192, 2, 2, 64, 2, 1, SCHED_I16_PF>(a, s);
        case 14: return launch_cfg<256, 256, 2, 2, 64, 2, 1, SCHED_I16_PF + SCHED_SPREAD>(a, s);
        case 15: return launch_cfg<256, 192, 2, 2, 64, 2, 1, SCHED_I16_PF + SCHED_SPREAD>(a, s);
        case 16: return launch_cfg<256, 128, 2, 2, 64, 3, 1, SCHED_INTERLEAVE + SCHED_SPREAD>(a, s);
        case 17:
            return launch_cfg<256, 256, 2, 2, 64, 2, 1, SCHED_I16_PF + SCHED_SPREAD + SCHED_PF_W_ONLY>(a, s);
        default:
            return launch_cfg<256, 192, 2, 2, 64, 2, 1, SCHED_I16_PF + SCHED_SPREAD + SCHED_PF_W_ONLY>(a, s);
    }
}

}  // namespace llb
