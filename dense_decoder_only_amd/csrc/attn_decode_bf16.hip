// Grouped-query attention for decode, bf16 (head_dim 128).
//
// One new query per sequence at position P attends to cache rows 0..P, i.e.
// L = P + 1 keys ("Llama 3 8B - Prepare Q, K, V", page header: decode reads
// L = P + 1 keys; the G query heads of a group share one cached K/V head,
// "Explanation").  The work is bandwidth-bound: every cached key and value is
// read once.
//
// Split-K: the L keys of each (sequence, KV head) are cut into chunks; one wave
// owns one chunk and streams it in 16-key steps.  Scores for all G heads of the
// group come from one 16x16x32 MFMA per 32 dims (K fragments are loaded from
// global memory straight into registers, heads padded to 16); the online
// softmax runs per head across the 16 keys; P.V runs on the vector ALU with
// each lane owning 8 output dims of one key slot.  Each chunk leaves an
// unnormalised (m, l, o) partial; a second kernel merges the chunks of a head in
// chunk order (log-sum-exp rescaling), so results do not depend on timing.
#include <algorithm>

#include "common.cuh"
#include "kernels.h"

namespace llb {

namespace {

constexpr int AD_TARGET_WAVES = 4096;
constexpr int AD_FUSED_MIN_UNITS = 128;  // (sequence, KV head) units for the one-workgroup-per-unit form

struct DecodePlan {
    int n_chunks;
    int chunk;  // keys per chunk, multiple of 16
};

DecodePlan plan_decode(int B, int n_kv, int n_keys) {
    const int units = B * n_kv;
    int n = (AD_TARGET_WAVES + units - 1) / units;
    const int max_n = (n_keys + 15) / 16;
    if (n > max_n) n = max_n;
    if (n < 1) n = 1;
    int ck = (n_keys + n - 1) / n;
    ck = (ck + 15) / 16 * 16;
    DecodePlan p;
    p.chunk = ck;
    p.n_chunks = (n_keys + ck - 1) / ck;
    return p;
}


// One wave's share of a decode attention unit (sequence b, KV head g): the
// 16-key steps starting at k_beg, k_beg + stride, ... below k_end, for the G
// query heads of the group.  Leaves the unnormalised partial state: m_run,
// l_run (every lane; base-2 units) and o[h][0..7] = sum_n p_n v_n[8*pc .. 8*pc+8]
// in lanes pc = lane < HD/8.
template <int HD, int G, int DEPTH>
__device__ __forceinline__ void decode_chunk(const AttnArgs& a, int b, int g, int k_beg, int stride, int k_end,
                                             float (&sP)[16][16], float (&sAl)[16], float (&o)[G][8],
                                             float& m_run, float& l_run) {
    constexpr int KST = HD / 32;        // 16x16x32 MFMA steps over head_dim
    constexpr int NC = HD / 8;          // 8-dim chunks (16 bytes) per row
    constexpr int KSL = 64 / NC;        // key slots per wave in the P.V phase
    constexpr int KPL = 16 / KSL;       // keys per slot per 16-key step
    static_assert(NC <= 64 && 16 % KSL == 0, "head_dim");
    const int lane = threadIdx.x & 63;
    const int bg = b * a.n_kv + g;
    const float scale_log2 = 1.4426950408889634f / sqrtf((float)HD);

    // Q fragments: B operand (column = head lane&15, dims 32kk + 8*(lane>>4) ..+8).
    // Every load below is unconditional (indices clamped into range, unused
    // values zeroed or masked afterwards): a load under a per-lane condition
    // becomes a branch, across which the compiler can only wait for all loads
    // in flight, which would serialise the prefetch.
    const int hq = lane & 15;
    bf16x8 qf[KST];
    uint4 qv[KST];
    {
        const bf16_t* qrow = (const bf16_t*)a.q + ((size_t)b * a.n_heads + g * G + min(hq, G - 1)) * HD;
#pragma unroll
        for (int kk = 0; kk < KST; ++kk) qv[kk] = *(const uint4*)(qrow + 32 * kk + 8 * (lane >> 4));
    }

    const size_t head_off = (size_t)bg * a.cap * HD;
    const bf16_t* __restrict__ Kg = (const bf16_t*)a.k_cache + head_off;
    const bf16_t* __restrict__ Vg = (const bf16_t*)a.v_cache + head_off;

    const int pc = lane % NC;   // P.V: dims 8*pc .. +8
    const int ps = lane / NC;   // P.V: key slot
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) o[h][e] = 0.f;
    m_run = -INFINITY;
    l_run = 0.f;

    // K and V of one 16-key step.  Keys at or past k_end read row k_end - 1
    // instead (a row already fetched: no extra HBM traffic); their scores are
    // masked to -inf, so their weights are 0 and their values add nothing.
    const int last = max(k_end - 1, 0);
    auto load_step = [&](int kt, uint4 (&kf)[KST], uint4 (&vf)[KPL]) {
        const int krow = min(kt + (lane & 15), last);
#pragma unroll
        for (int kk = 0; kk < KST; ++kk)
            kf[kk] = *(const uint4*)(Kg + (size_t)krow * HD + 32 * kk + 8 * (lane >> 4));
#pragma unroll
        for (int i = 0; i < KPL; ++i) {
            const int key = min(kt + ps * KPL + i, last);
            vf[i] = *(const uint4*)(Vg + (size_t)key * HD + 8 * pc);
        }
    };
    auto step = [&](int kt, const uint4 (&kf)[KST], const uint4 (&vf)[KPL]) {
        // ---- scores: D[key][head] = K . Q^T
        f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KST; ++kk) s = mfma16(as_bf16x8(kf[kk]), qf[kk], s);
        // lane -> head (lane & 15); reg r -> key kt + 4*(lane>>4) + r
        float mloc = -INFINITY;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int key = kt + 4 * (lane >> 4) + r;
            const float v = key < k_end ? s[r] * scale_log2 : -INFINITY;
            s[r] = v;
            mloc = fmaxf(mloc, v);
        }
        mloc = fmaxf(mloc, __shfl_xor(mloc, 16, 64));
        mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
        const float m_new = fmaxf(m_run, mloc);
        const float alpha = exp2f(m_run - m_new);
        float lsum = 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float p = exp2f(s[r] - m_new);
            s[r] = p;
            lsum += p;
        }
        lsum += __shfl_xor(lsum, 16, 64);
        lsum += __shfl_xor(lsum, 32, 64);
        l_run = l_run * alpha + lsum;
        m_run = m_new;
        // ---- publish p and alpha to the wave's LDS slice
#pragma unroll
        for (int r = 0; r < 4; ++r) sP[4 * (lane >> 4) + r][hq] = s[r];
        if (lane < 16) sAl[lane] = alpha;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // ---- P.V on the vector ALU
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float al = sAl[h];
#pragma unroll
            for (int e = 0; e < 8; ++e) o[h][e] *= al;
        }
#pragma unroll
        for (int i = 0; i < KPL; ++i) {
            float v[8];
            unpack_bf16x8(vf[i], v);
            const int kl = ps * KPL + i;
            // the G weights of key kl, read as whole float4 rows of sP
            float p[G < 4 ? 4 : G];
#pragma unroll
            for (int h4 = 0; h4 < (G + 3) / 4; ++h4)
                *(float4*)&p[4 * h4] = *(const float4*)&sP[kl][4 * h4];
#pragma unroll
            for (int h = 0; h < G; ++h)
#pragma unroll
                for (int e = 0; e < 8; ++e) o[h][e] += p[h] * v[e];
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };
    // DEPTH register buffers: the loads of the next DEPTH-1 steps are in flight
    // while a step is computed.  The same loads are issued on every path (steps
    // past the chunk re-read row k_end - 1), so the compiler's waits count
    // exactly the DEPTH-1 younger steps.
    uint4 kf[DEPTH][KST], vf[DEPTH][KPL];
#pragma unroll
    for (int d = 0; d + 1 < DEPTH; ++d) load_step(k_beg + stride * d, kf[d], vf[d]);
    // The query is consumed here, before the loop, so that no wait on it is
    // left inside the loop (heads past the group are zero columns).
#pragma unroll
    for (int kk = 0; kk < KST; ++kk) {
        asm volatile("" ::"v"(qv[kk].x), "v"(qv[kk].y), "v"(qv[kk].z), "v"(qv[kk].w));
        qf[kk] = as_bf16x8(hq < G ? qv[kk] : make_uint4(0, 0, 0, 0));
    }
    for (int kt = k_beg; kt < k_end; kt += stride * DEPTH) {
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) {
            const int kc = kt + stride * d;
            load_step(kc + stride * (DEPTH - 1), kf[(d + DEPTH - 1) % DEPTH], vf[(d + DEPTH - 1) % DEPTH]);
            if (kc < k_end) step(kc, kf[d], vf[d]);
        }
    }

    // reduce the key slots (lane bits above log2(NC))
#pragma unroll
    for (int off = NC; off < 64; off <<= 1)
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int e = 0; e < 8; ++e) o[h][e] += __shfl_xor(o[h][e], off, 64);

}

// Split over key chunks across workgroups (few units): one wave per chunk,
// partials to ws, merged by attn_decode_merge_kernel.
template <int HD, int G>
__global__ void __launch_bounds__(256)
attn_decode_kernel(AttnArgs a, int n_chunks, int chunk, float* __restrict__ part_o,
                   float* __restrict__ part_ml) {
    constexpr int NC = HD / 8;
    __shared__ __attribute__((aligned(16))) float sP[4][16][16];     // per wave: p[key][head]
    __shared__ float sAl[4][16];        // per wave: alpha[head]
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int wid = blockIdx.x * 4 + wave;
    if (wid >= a.B * a.n_kv * n_chunks) return;  // whole wave leaves; no block barriers below
    const int ci = wid % n_chunks;
    const int bg = wid / n_chunks;
    const int g = bg % a.n_kv;
    const int b = bg / a.n_kv;
    const int L = seq_start(a, b) + 1;
    const int k_beg = ci * chunk;
    const int k_end = min(L, k_beg + chunk);
    float o[G][8], m_run, l_run;
    decode_chunk<HD, G, 2>(a, b, g, k_beg, 16, k_end, sP[wave], sAl[wave], o, m_run, l_run);
    const int pc = lane % NC;
    const size_t base = ((size_t)b * a.n_heads + (size_t)g * G) * n_chunks + ci;
    if (lane < NC) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float* dst = part_o + (base + (size_t)h * n_chunks) * HD + 8 * pc;
            *(float4*)dst = make_float4(o[h][0], o[h][1], o[h][2], o[h][3]);
            *(float4*)(dst + 4) = make_float4(o[h][4], o[h][5], o[h][6], o[h][7]);
        }
    }
    if (lane < G) {
        part_ml[2 * (base + (size_t)lane * n_chunks) + 0] = m_run;
        part_ml[2 * (base + (size_t)lane * n_chunks) + 1] = l_run;
    }
}

// One workgroup attends over keys [k_lo, k_hi) of unit (sequence b, KV head g):
// its AD_FW waves take the 16-key steps in turn (wave w steps k_lo + 16 w,
// k_lo + 16 (w + AD_FW), ...: every wave streams from every part of the cache
// rows, so the waves progress evenly, measured, where contiguous chunks
// finished up to 1.7x apart) and their partial states are merged through LDS
// in wave order.  For each (head h of the group, dim j) this thread covers,
// emit(h, j, m, l, num) receives the merged state: running maximum m (base-2
// units), running sum l and unnormalised output num; the result is num / l.
constexpr int AD_FW = 8;

template <int HD, int G, typename Emit>
__device__ __forceinline__ void attend_unit(const AttnArgs& a, int b, int g, int k_lo, int k_hi, Emit&& emit) {
    constexpr int NC = HD / 8;
    __shared__ __attribute__((aligned(16))) float sP[AD_FW][16][16];
    __shared__ float sAl[AD_FW][16];
    __shared__ float sO[AD_FW][G][HD];
    __shared__ float sM[AD_FW][G], sL[AD_FW][G];
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    float o[G][8], m_run, l_run;
    decode_chunk<HD, G, (G <= 4 ? 3 : 2)>(a, b, g, k_lo + 16 * wave, 16 * AD_FW, k_hi, sP[wave], sAl[wave], o,
                                          m_run, l_run);
    if (lane < NC) {
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int e = 0; e < 8; ++e) sO[wave][h][8 * lane + e] = o[h][e];
    }
    if (lane < G) {
        sM[wave][lane] = m_run;
        sL[wave][lane] = l_run;
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < G * HD; idx += 64 * AD_FW) {
        const int h = idx / HD, j = idx % HD;
        float mmax = -INFINITY;
#pragma unroll
        for (int w = 0; w < AD_FW; ++w) mmax = fmaxf(mmax, sM[w][h]);
        float den = 0.f, num = 0.f;
#pragma unroll
        for (int w = 0; w < AD_FW; ++w) {
            const float wt = sL[w][h] > 0.f ? exp2f(sM[w][h] - mmax) : 0.f;  // empty waves add nothing
            den += wt * sL[w][h];
            num += wt * sO[w][h][j];
        }
        emit(h, j, mmax, den, num);
    }
}

// One workgroup per unit (sequence b, KV head g) when there are enough units to
// fill the GPU: the whole unit, keys 0..P_b, merged in the workgroup, so no
// partials leave it and no second kernel is needed.
template <int HD, int G>
__global__ void __launch_bounds__(64 * AD_FW)
attn_decode_fused_kernel(AttnArgs a) {
    const int g = blockIdx.x % a.n_kv;
    const int b = blockIdx.x / a.n_kv;
    const int L = seq_start(a, b) + 1;
    attend_unit<HD, G>(a, b, g, 0, L, [&](int h, int j, float, float den, float num) {
        ((bf16_t*)a.o)[((size_t)b * a.n_heads + (size_t)g * G + h) * HD + j] = f2bf(num / den);
    });
}

// One workgroup per (sequence, query head): merge the chunk partials in order.
template <int HD>
__global__ void __launch_bounds__(HD)
attn_decode_merge_kernel(AttnArgs a, int n_chunks, const float* __restrict__ part_o,
                         const float* __restrict__ part_ml) {
    const int bh = blockIdx.x;
    const int j = threadIdx.x;
    const float* ml = part_ml + (size_t)bh * n_chunks * 2;
    float mmax = -INFINITY;
#pragma unroll 8
    for (int c = 0; c < n_chunks; ++c) mmax = fmaxf(mmax, ml[2 * c]);
    float den = 0.f, num = 0.f;
#pragma unroll 8
    for (int c = 0; c < n_chunks; ++c) {
        const float w = exp2f(ml[2 * c] - mmax);
        den += w * ml[2 * c + 1];
        num += w * part_o[((size_t)bh * n_chunks + c) * HD + j];
    }
    ((bf16_t*)a.o)[(size_t)bh * HD + j] = f2bf(num / den);
}

template <int G>
hipError_t launch_g(const AttnArgs& a, const DecodePlan& p, float* part_o, float* part_ml,
                    hipStream_t s) {
    const int waves = a.B * a.n_kv * p.n_chunks;
    hipLaunchKernelGGL((attn_decode_kernel<128, G>), dim3((waves + 3) / 4), dim3(256), 0, s, a,
                       p.n_chunks, p.chunk, part_o, part_ml);
    return hipGetLastError();
}

template <int G>
hipError_t launch_fused(const AttnArgs& a, hipStream_t s) {
    hipLaunchKernelGGL((attn_decode_fused_kernel<128, G>), dim3(a.B * a.n_kv), dim3(64 * AD_FW), 0, s, a);
    return hipGetLastError();
}

}  // namespace

// Partials of the split form for any call reading at most n_keys keys: the
// chunk count of plan_decode is at most min(target chunks per unit, n_keys/16
// rounded up), a bound that grows with n_keys (the chunk count itself does not:
// 1001 keys over 256 units take 16 chunks, 1088 keys 14).
size_t attn_decode_ws_bytes(int B, int n_heads, int n_kv, int hd, int n_keys) {
    const int units = B * n_kv;
    const int n_target = (AD_TARGET_WAVES + units - 1) / units;
    const int chunks = std::max(1, std::min(n_target, (n_keys + 15) / 16));
    return (size_t)B * n_heads * chunks * (hd + 2) * sizeof(float);
}

hipError_t attn_decode_bf16_launch(const AttnArgs& a, float* ws, hipStream_t s) {
    if (a.hd != 128 || a.n_kv <= 0 || a.n_heads % a.n_kv != 0 || a.B <= 0 || a.pos0 < 0)
        return hipErrorInvalidValue;
    if (a.B * a.n_kv >= AD_FUSED_MIN_UNITS) {
        switch (a.n_heads / a.n_kv) {
            case 1: return launch_fused<1>(a, s);
            case 2: return launch_fused<2>(a, s);
            case 4: return launch_fused<4>(a, s);
            case 8: return launch_fused<8>(a, s);
            default: break;
        }
    }
    const int L = a.pos0 + 1;
    const DecodePlan p = plan_decode(a.B, a.n_kv, L);
    float* part_o = ws;
    float* part_ml = ws + (size_t)a.B * a.n_heads * p.n_chunks * a.hd;
    hipError_t err;
    switch (a.n_heads / a.n_kv) {
        case 1: err = launch_g<1>(a, p, part_o, part_ml, s); break;
        case 2: err = launch_g<2>(a, p, part_o, part_ml, s); break;
        case 4: err = launch_g<4>(a, p, part_o, part_ml, s); break;
        case 8: err = launch_g<8>(a, p, part_o, part_ml, s); break;
        case 16: err = launch_g<16>(a, p, part_o, part_ml, s); break;
        default: return hipErrorInvalidValue;
    }
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL((attn_decode_merge_kernel<128>), dim3(a.B * a.n_heads), dim3(128), 0, s, a,
                       p.n_chunks, part_o, part_ml);
    return hipGetLastError();
}

}  // namespace llb
