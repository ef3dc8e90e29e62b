// Causal grouped-query attention, prefill, bf16 MFMA (head_dim 128).
//
// Computes, per query head h and query position p = pos0 + t, the softmax over
// keys n <= p of q.k_n / sqrt(hd) and sum_n softmax_n v_n ("How Llama 3.1
// Generates the Next Token": score q.k/sqrt(128), mask M = -inf for future
// positions; "Llama 3.1 70B", section "Grouped-Query Attention": a group of
// query heads shares one K/V head).
//
// Work split.  A query block is 32 consecutive positions of one sequence; one
// workgroup owns one KV head g and a PAIR of query blocks (i, nqb-1-i), so that
// every workgroup sees the same number of causal key tiles (the short block of
// the pair plus the long one).  Its waves are G heads x S key streams: wave
// (hl, s) computes query head g*G+hl and, in every pipeline stage of S
// consecutive 64-key tiles, the tile s of that stage.  With S = 2 the two
// streams of a head hold partial softmax states that are merged through LDS
// when a query block ends (the same merge rule as split-K decoding).
//
// Per 64-key tile a wave computes S^T = K . Q^T (64 keys x 32 queries) and
// O^T += V^T . P^T (128 dims x 32 queries) with v_mfma_f32_32x32x16_bf16, so a
// lane owns one query column: the softmax row statistics stay in the lane plus
// one exchange with lane ^ 32 (v_permlane32_swap).
//
// Data movement.  K and V tiles are copied global -> LDS by the DMA path
// (global_load_lds_dwordx4), NSTAGE stages ahead, in plain row-major [key][dim]
// form with a 16-byte chunk swizzle.  K fragments are ds_read_b128 of one key
// row; V^T fragments come from the same row-major V tile through
// ds_read_b64_tr_b16, which hands each lane four keys of one dim (within a group
// of 16 lanes, lane i receives element i%4 of the 8-byte blocks addressed by
// lanes i/4, 4+i/4, 8+i/4, 12+i/4).
//
// Softmax.  Scores stay in raw units s; the exponent is exp2(s*c - m*c) with
// c = log2(e)/sqrt(hd), one FMA and one v_exp_f32 per score.  The running
// offset m is only moved when a tile's maximum exceeds it by more than
// 2^LAZY_LOG2 in probability (checked for the whole wave), so the O^T rescale
// is skipped on most tiles; the final division by the running sum makes the
// result independent of the offset chosen.  The causal mask is applied only on
// tiles that reach past the block's first query position.
#include "common.cuh"
#include "kernels.h"

namespace llb {

namespace {

constexpr int AP_HD = 128;
constexpr int AP_BQ = 32;        // query positions per block
constexpr int AP_BKV = 64;       // keys per wave tile
constexpr int AP_TILE_BYTES = AP_BKV * AP_HD * 2;   // one K (or V) tile: 16 KB
constexpr float LAZY_LOG2 = 8.0f;
constexpr int AP_KD = 2;         // K fragments are read this many k-steps ahead of their MFMAs
constexpr int AP_VD = 1;         // V^T fragments this many 16-key steps ahead

typedef short v4i16 __attribute__((ext_vector_type(4)));

// ds_read_b64_tr_b16 at LDS byte address a (see the header comment for the lane
// layout); returned as two dwords.
LLB_DEV uint2 lds_read_tr16(uint32_t a) {
    const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4i16*)(uintptr_t)a);
    return __builtin_bit_cast(uint2, v);
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4v __attribute__((ext_vector_type(4)));

LLB_DEV uint4 lds_read_b128(uint32_t a) {
    const u32x4 v = *(const __attribute__((address_space(3))) u32x4*)(uintptr_t)a;
    return make_uint4(v.x, v.y, v.z, v.w);
}

// max / sum of a value with the one held by lane ^ 32
LLB_DEV float pair_max(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
LLB_DEV float pair_sum(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int G, int S, int NSTAGE>
__global__ void __launch_bounds__(64 * G * S)
attn_prefill_kernel(AttnArgs a) {
    constexpr int W = G * S;                          // waves per workgroup
    constexpr int STAGE_BYTES = S * AP_TILE_BYTES;    // K (or V) bytes per stage
    constexpr int BLK_PER_STAGE = STAGE_BYTES / 1024; // 1 KB DMA blocks (K or V)
    constexpr int D = 2 * BLK_PER_STAGE / W;          // DMA instructions per wave per stage
    static_assert((2 * BLK_PER_STAGE) % W == 0 && BLK_PER_STAGE % W == 0, "DMA split");
    static_assert(S == 1 || G * AP_TILE_BYTES <= 2 * STAGE_BYTES, "merge area");
    static_assert((NSTAGE - 2) * D < 64, "vmcnt range");

    // [K stage 0 .. NSTAGE-1][V stage 0 .. NSTAGE-1]
    __shared__ __attribute__((aligned(1024))) char smem[2 * NSTAGE * STAGE_BYTES];
    __shared__ float sML[S == 2 ? G * 2 * 64 : 1];

    const int T = a.T, pos0 = a.pos0;
    const int nqb = (T + AP_BQ - 1) / AP_BQ;
    const int npair = (nqb + 1) / 2;
    // Workgroup -> (sequence b, KV head g, query-block pair).  Workgroups are
    // dispatched round-robin over the 8 XCDs; when the (b, g) count allows,
    // every workgroup of one XCD works on the same (b, g), walking the pairs in
    // order, so the K/V rows that its ~32 concurrent workgroups stream stay in
    // that XCD's L2.
    int bg, pair;
    {
        const int id = blockIdx.x;
        const int nbg = a.n_kv * a.B;
        if (nbg % 8 == 0) {
            const int j = id / 8;
            bg = id % 8 + 8 * (j / npair);
            pair = j % npair;
        } else {
            bg = id / npair;
            pair = id % npair;
        }
    }
    const int g = bg % a.n_kv;
    const int b = bg / a.n_kv;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int hl = wave / S;
    const int sw = wave % S;
    const int h = g * G + hl;
    const int hf = lane >> 5;          // which 4-key half of each 8-key group
    const int l16 = lane & 15;

    // the two query blocks of this workgroup (one when the pair collapses)
    const int qblk0 = pair;
    const int qblk1 = nqb - 1 - pair;
    const int njobs = qblk1 > qblk0 ? 2 : 1;
    auto keys_of = [&](int qb) { return pos0 + min((qb + 1) * AP_BQ, T); };
    const int L0 = keys_of(qblk0);
    const int L1 = njobs == 2 ? keys_of(qblk1) : L0;
    const int nst0 = ((L0 + AP_BKV - 1) / AP_BKV + S - 1) / S;
    const int nst1 = njobs == 2 ? ((L1 + AP_BKV - 1) / AP_BKV + S - 1) / S : 0;
    const int total = nst0 + nst1;

    const size_t head_off = ((size_t)b * a.n_kv + g) * a.cap * AP_HD;
    const bf16_t* __restrict__ Kg = (const bf16_t*)a.k_cache + head_off;
    const bf16_t* __restrict__ Vg = (const bf16_t*)a.v_cache + head_off;
    const uint32_t k_lds = lds_offset(smem);
    const uint32_t v_lds = k_lds + NSTAGE * STAGE_BYTES;

    // ---- DMA of one stage: S tiles of K then S tiles of V -------------------
    // Block j of a region covers rows 4j..4j+3; lane -> (row 4j + lane/16, LDS
    // chunk lane%16).  K rows hold chunk c at c ^ (row & 15); V rows at
    // c ^ 4*(row & 3), the swizzles under which the fragment reads are free of
    // bank conflicts.
    auto issue = [&](int st, int buf) {
        const bool second = st >= nst0;
        const int key0 = (second ? st - nst0 : st) * (S * AP_BKV);
        const int last = (second ? L1 : L0) - 1;
#pragma unroll
        for (int i = 0; i < D; ++i) {
            const bool isK = i < D / 2;
            const int blk = (i * W + wave) % BLK_PER_STAGE;
            const int row = blk * 4 + (lane >> 4);
            const int c = isK ? (l16 ^ (row & 15)) : (l16 ^ (4 * (row & 3)));
            const int key = min(key0 + row, last);
            const bf16_t* src = (isK ? Kg : Vg) + (size_t)key * AP_HD + c * 8;
            dma16(src, (isK ? k_lds : v_lds) + buf * STAGE_BYTES + blk * 1024);
        }
    };

    // per-lane fragment addresses (relative to a tile's base)
    uint32_t kaddr[8];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
        kaddr[kk] = (lane & 31) * 256 + ((((2 * kk + hf) ^ l16) & 15) << 4);
    uint32_t vaddr[4];
    {
        const int j = l16 >> 2;  // key within the lane group's 4 rows
        const int m = l16 & 3;   // 8-byte dim block
        const int g1 = (lane >> 4) & 1;
#pragma unroll
        for (int os = 0; os < 4; ++os) {
            const int chunk = 4 * os + 2 * g1 + (m >> 1);
            vaddr[os] = (4 * hf + j) * 256 + ((chunk ^ (4 * j)) << 4) + 8 * (m & 1);
        }
    }

    const float c_log2 = 1.4426950408889634f / sqrtf((float)AP_HD);
    const float lazy_raw = LAZY_LOG2 / c_log2;

    // per-job state
    bf16x8 qf[8];
    f32x16 oacc[4];
    float m_run = 0.f, l_run = 0.f;
    int my_t = 0, my_pos = 0, q_first = 0, n_tiles = 0;

    auto begin_job = [&](int qb) {
        const int q0 = qb * AP_BQ;
        my_t = q0 + (lane & 31);
        my_pos = pos0 + my_t;
        q_first = pos0 + q0;
        n_tiles = (keys_of(qb) + AP_BKV - 1) / AP_BKV;
        const bf16_t* qrow =
            (const bf16_t*)a.q + (((size_t)b * a.n_heads + h) * T + my_t) * AP_HD + 8 * hf;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk)
            qf[kk] = as_bf16x8(my_t < T ? *(const uint4*)(qrow + 16 * kk) : make_uint4(0, 0, 0, 0));
        // Retire the query loads here, once per block: left pending, they would
        // make the compiler wait for every copy in flight before each tile.
        wait_vm<0>();
#pragma unroll
        for (int os = 0; os < 4; ++os)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[os][r] = 0.f;
        m_run = -1e30f;
        l_run = 0.f;
    };

    // one 64-key tile at LDS bases kb / vb; key0 = absolute key of its row 0
    auto tile = [&](uint32_t kb, uint32_t vb, int key0) {
        f32x16 s[2];
#pragma unroll
        for (int ms = 0; ms < 2; ++ms)
#pragma unroll
            for (int r = 0; r < 16; ++r) s[ms][r] = 0.f;
        // K fragments are read AP_KD k-steps ahead of the MFMAs that use them
        constexpr int KR = AP_KD + 1;
        uint4 kf[KR][2];
#pragma unroll
        for (int kk = 0; kk < AP_KD; ++kk) {
            kf[kk][0] = lds_read_b128(kb + kaddr[kk]);
            kf[kk][1] = lds_read_b128(kb + 32 * 256 + kaddr[kk]);
        }
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            if (kk + AP_KD < 8) {
                kf[(kk + AP_KD) % KR][0] = lds_read_b128(kb + kaddr[kk + AP_KD]);
                kf[(kk + AP_KD) % KR][1] = lds_read_b128(kb + 32 * 256 + kaddr[kk + AP_KD]);
            }
            __builtin_amdgcn_sched_barrier(0);
            s[0] = mfma32(as_bf16x8(kf[kk % KR][0]), qf[kk], s[0]);
            s[1] = mfma32(as_bf16x8(kf[kk % KR][1]), qf[kk], s[1]);
        }
        // V^T fragments of the first AP_VD 16-key steps, read while the softmax runs
        constexpr int VR = AP_VD + 1;
        uint2 vf[VR][4][2];
#pragma unroll
        for (int ks = 0; ks < AP_VD; ++ks)
#pragma unroll
            for (int os = 0; os < 4; ++os) {
                vf[ks][os][0] = lds_read_tr16(vb + ks * 16 * 256 + vaddr[os]);
                vf[ks][os][1] = lds_read_tr16(vb + ks * 16 * 256 + 8 * 256 + vaddr[os]);
            }
        if (key0 + AP_BKV - 1 > q_first) {  // tile reaches the diagonal
            const int lim = my_pos - key0 - 4 * hf;  // mask key offsets > lim
#pragma unroll
            for (int ms = 0; ms < 2; ++ms)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (ms * 32 + 8 * (r >> 2) + (r & 3) > lim) s[ms][r] = -INFINITY;
        }
        float mx = s[0][0];
#pragma unroll
        for (int ms = 0; ms < 2; ++ms)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[ms][r]);
        mx = pair_max(mx);
        if (__any(mx > m_run + lazy_raw)) {
            const float m_new = fmaxf(m_run, mx);
            const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * c_log2);
            m_run = m_new;
            l_run *= alpha;
#pragma unroll
            for (int os = 0; os < 4; ++os)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[os][r] *= alpha;
        }
        const float mc = -m_run * c_log2;
#pragma unroll
        for (int ms = 0; ms < 2; ++ms)
#pragma unroll
            for (int r = 0; r < 16; ++r) s[ms][r] = __builtin_amdgcn_exp2f(fmaf(s[ms][r], c_log2, mc));
        // O^T += V^T P^T over 4 steps of 16 keys.  MFMA k-index 0..7 of lane
        // half hf maps to keys 4hf+0..3 and 8+4hf+0..3 of the step, which is
        // where the S^T accumulator layout already holds them.  The running
        // sum adds the same bf16-rounded weights that enter the product, so
        // numerator and denominator see identical weights.
        const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            bf16x2_t pw[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                pw[e] = bf16x2_t{(__bf16)s[ks >> 1][8 * (ks & 1) + 2 * e],
                                 (__bf16)s[ks >> 1][8 * (ks & 1) + 2 * e + 1]};
                l_run = __builtin_amdgcn_fdot2_f32_bf16(pw[e], ones, l_run, false);
            }
            const bf16x8 pf = __builtin_bit_cast(bf16x8, pw);
            if (ks + AP_VD < 4) {
#pragma unroll
                for (int os = 0; os < 4; ++os) {
                    vf[(ks + AP_VD) % VR][os][0] = lds_read_tr16(vb + (ks + AP_VD) * 16 * 256 + vaddr[os]);
                    vf[(ks + AP_VD) % VR][os][1] =
                        lds_read_tr16(vb + (ks + AP_VD) * 16 * 256 + 8 * 256 + vaddr[os]);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int os = 0; os < 4; ++os) {
                const uint2 lo = vf[ks % VR][os][0], hi = vf[ks % VR][os][1];
                oacc[os] = mfma32(as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y)), pf, oacc[os]);
            }
        }
    };

    auto store_out = [&](float inv) {
        if (my_t < T) {
            bf16_t* orow = (bf16_t*)a.o + ((size_t)b * T + my_t) * ((size_t)a.n_heads * AP_HD) +
                           (size_t)h * AP_HD;
#pragma unroll
            for (int os = 0; os < 4; ++os)
#pragma unroll
                for (int rq = 0; rq < 4; ++rq) {
                    const int dim = os * 32 + 8 * rq + 4 * hf;
                    uint2 pk;
                    pk.x = pack_bf16x2(oacc[os][4 * rq + 0] * inv, oacc[os][4 * rq + 1] * inv);
                    pk.y = pack_bf16x2(oacc[os][4 * rq + 2] * inv, oacc[os][4 * rq + 3] * inv);
                    *(uint2*)(orow + dim) = pk;
                }
        }
    };

    // End of a query block.  buf: the stage buffer every wave has finished
    // reading (free for the merge of the two key streams).
    auto end_job = [&](int buf) {
        if constexpr (S == 1) {
            store_out(1.0f / pair_sum(l_run));
        } else {
            const uint32_t slot = (hl * AP_TILE_BYTES < STAGE_BYTES)
                                      ? k_lds + buf * STAGE_BYTES + hl * AP_TILE_BYTES
                                      : v_lds + buf * STAGE_BYTES + hl * AP_TILE_BYTES - STAGE_BYTES;
            wait_vm_lgkm<63>();
            barrier();
            if (sw == 1) {
#pragma unroll
                for (int os = 0; os < 4; ++os)
#pragma unroll
                    for (int rq = 0; rq < 4; ++rq) {
                        const f32x4v v = {oacc[os][4 * rq], oacc[os][4 * rq + 1],
                                          oacc[os][4 * rq + 2], oacc[os][4 * rq + 3]};
                        *(__attribute__((address_space(3))) f32x4v*)(uintptr_t)(
                            slot + ((os * 4 + rq) * 64 + lane) * 16) = v;
                    }
                sML[(hl * 2 + 0) * 64 + lane] = m_run;
                sML[(hl * 2 + 1) * 64 + lane] = l_run;
            }
            wait_vm_lgkm<63>();
            barrier();
            if (sw == 0) {
                const float m1 = sML[(hl * 2 + 0) * 64 + lane];
                const float l1 = sML[(hl * 2 + 1) * 64 + lane];
                const float m = fmaxf(m_run, m1);
                const float a0 = __builtin_amdgcn_exp2f((m_run - m) * c_log2);
                const float a1 = __builtin_amdgcn_exp2f((m1 - m) * c_log2);
#pragma unroll
                for (int os = 0; os < 4; ++os)
#pragma unroll
                    for (int rq = 0; rq < 4; ++rq) {
                        const f32x4v v = *(const __attribute__((address_space(3))) f32x4v*)(uintptr_t)(
                            slot + ((os * 4 + rq) * 64 + lane) * 16);
                        oacc[os][4 * rq + 0] = oacc[os][4 * rq + 0] * a0 + v.x * a1;
                        oacc[os][4 * rq + 1] = oacc[os][4 * rq + 1] * a0 + v.y * a1;
                        oacc[os][4 * rq + 2] = oacc[os][4 * rq + 2] * a0 + v.z * a1;
                        oacc[os][4 * rq + 3] = oacc[os][4 * rq + 3] * a0 + v.w * a1;
                    }
                store_out(1.0f / pair_sum(l_run * a0 + l1 * a1));
            }
        }
    };

    // ---- pipeline over the flat stage sequence of both query blocks ---------
    // step(st): wait for stage st, barrier (every wave is past stage st-1, so
    // its buffer is free), issue stage st+NSTAGE-1 into it, compute stage st.
    auto step = [&](int st, int buf) {
        if (st + NSTAGE - 2 < total) wait_vm_lgkm<(NSTAGE - 2) * D>();
        else wait_vm_lgkm<0>();
        barrier();
        const bool second = st >= nst0;
        const int ls = second ? st - nst0 : st;
        if (ls == 0) begin_job(second ? qblk1 : qblk0);
        if (st + NSTAGE - 1 < total) issue(st + NSTAGE - 1, (buf + NSTAGE - 1) % NSTAGE);
        const int t = ls * S + sw;
        if (t < n_tiles)
            tile(k_lds + buf * STAGE_BYTES + sw * AP_TILE_BYTES,
                 v_lds + buf * STAGE_BYTES + sw * AP_TILE_BYTES, t * AP_BKV);
        if (st == nst0 - 1 || st == total - 1) end_job(buf);
    };

#pragma unroll
    for (int st = 0; st < NSTAGE - 1; ++st)
        if (st < total) issue(st, st);
    for (int st0 = 0; st0 < total; st0 += NSTAGE) {
#pragma unroll
        for (int j = 0; j < NSTAGE; ++j)
            if (st0 + j < total) step(st0 + j, j);
    }
}

template <int G, int S, int NSTAGE>
hipError_t launch_g(const AttnArgs& a, hipStream_t s) {
    const int nqb = (a.T + AP_BQ - 1) / AP_BQ;
    hipLaunchKernelGGL((attn_prefill_kernel<G, S, NSTAGE>), dim3((nqb + 1) / 2 * a.n_kv * a.B),
                       dim3(64 * G * S), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t attn_prefill_bf16_launch(const AttnArgs& a, hipStream_t s) {
    if (a.hd != AP_HD || a.n_kv <= 0 || a.n_heads % a.n_kv != 0 || a.T <= 0 || a.B <= 0 ||
        a.pos0 < 0 || a.pos0 + a.T > a.cap || a.pos_b != nullptr)
        return hipErrorInvalidValue;
    switch (a.n_heads / a.n_kv) {
        case 1: return launch_g<1, 2, 2>(a, s);
        case 2: return launch_g<2, 2, 2>(a, s);
        case 4: return launch_g<4, 2, 2>(a, s);
        case 8: return launch_g<8, 1, 2>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace llb
