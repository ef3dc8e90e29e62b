// Causal grouped-query attention, prefill, bf16 MFMA (head_dim 128).
//
// Computes, per query head h and query position p = pos0 + t, the softmax over
// keys n <= p of q.k_n / sqrt(hd) and sum_n softmax_n v_n ("How Llama 3.1
// Generates the Next Token": score q.k/sqrt(128), mask M = -inf for future
// positions; "Llama 3.1 70B", section "Grouped-Query Attention": a group of
// query heads shares one K/V head).
//
// One workgroup = one KV head g, one block of 32 query positions, and all G
// query heads of the group (one wave per head).  Each 64-key K/V tile is staged
// once in LDS and used by the G waves, so K/V traffic is shared by the group
// instead of being repeated per query head.  Scores are computed transposed,
// S^T = K . Q^T, so that a lane owns one query column: the online-softmax max,
// sum and rescale stay inside the lane (plus one exchange with lane ^ 32).  The
// same transposed form O^T = V^T . P^T lets the probabilities feed the second
// MFMA straight from registers; V is staged transposed in LDS for that.
#include "common.cuh"
#include "kernels.h"

namespace llb {

namespace {

constexpr int AP_BQ = 32;    // query positions per workgroup
constexpr int AP_BKV = 64;   // keys per tile

template <int HD, int G>
__global__ void __launch_bounds__(64 * G)
attn_prefill_kernel(AttnArgs a) {
    constexpr int NT = 64 * G;
    constexpr int KCH = HD / 8;                      // 16-byte chunks per K row
    constexpr int KSTEPS = HD / 16;                  // MFMA k-steps over head_dim
    constexpr int OSUB = HD / 32;                    // O^T row blocks
    constexpr int K_PER_T = AP_BKV * KCH / NT;       // K chunks staged per thread
    constexpr int KPT = AP_BKV * HD / (8 * NT);      // keys per V unit (unit = KPT keys x 8 dims)
    static_assert(KCH == 16, "swizzles below assume 128-wide heads");
    static_assert(K_PER_T >= 1 && KPT >= 2 && KPT % 2 == 0, "thread count vs tile");

    __shared__ __attribute__((aligned(16))) bf16_t sK[2][AP_BKV * HD];
    __shared__ __attribute__((aligned(16))) bf16_t sVt[2][HD * AP_BKV];

    const int nqb = (a.T + AP_BQ - 1) / AP_BQ;
    const int qb = nqb - 1 - (int)blockIdx.x;  // longest rows first
    const int g = blockIdx.y;
    const int b = blockIdx.z;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int h = g * G + wave;
    const int q0 = qb * AP_BQ;
    const int my_t = q0 + (lane & 31);
    const int my_pos = a.pos0 + my_t;
    const int L = a.pos0 + min(q0 + AP_BQ, a.T);  // keys 0..L-1 are needed by this block
    const int ntiles = (L + AP_BKV - 1) / AP_BKV;

    // log2(e)/sqrt(hd): scores are kept in base-2 units so exp2 can be used.
    const float scale_log2 = 1.4426950408889634f / sqrtf((float)HD);

    bf16x8 qf[KSTEPS];
    {
        const bf16_t* qrow =
            (const bf16_t*)a.q + (((size_t)b * a.n_heads + h) * a.T + my_t) * HD + 8 * (lane >> 5);
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk)
            qf[kk] = as_bf16x8(my_t < a.T ? *(const uint4*)(qrow + 16 * kk) : make_uint4(0, 0, 0, 0));
    }

    const size_t head_off = ((size_t)b * a.n_kv + g) * a.cap * HD;
    const bf16_t* __restrict__ Kg = (const bf16_t*)a.k_cache + head_off;
    const bf16_t* __restrict__ Vg = (const bf16_t*)a.v_cache + head_off;

    uint4 rk[K_PER_T];
    uint4 rv[KPT];
    const int v_c = tid % KCH;   // dims 8*v_c .. +8
    const int v_kg = tid / KCH;  // keys KPT*v_kg .. +KPT

    auto load_tile = [&](int j) {
        const int kb = j * AP_BKV;
#pragma unroll
        for (int i = 0; i < K_PER_T; ++i) {
            const int idx = tid + i * NT;
            const int key = kb + idx / KCH;
            rk[i] = key < L ? *(const uint4*)(Kg + (size_t)key * HD + (idx % KCH) * 8)
                            : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const int key = kb + v_kg * KPT + i;
            rv[i] = key < L ? *(const uint4*)(Vg + (size_t)key * HD + v_c * 8) : make_uint4(0, 0, 0, 0);
        }
    };

    // V^T element (dim, key) lives at dim*64 + ((key/4 ^ f(dim)) * 4) + key%4 with
    // f(dim) = (dim / 2) & 15: the 32 lanes of a fragment read (8 bytes each, 32
    // consecutive dims, one key granule) then cover all 64 banks.
    auto vt_index = [](int dim, int key) {
        const int f = (dim >> 1) & 15;
        return dim * AP_BKV + ((((key >> 2) ^ f)) << 2) + (key & 3);
    };

    auto store_tile = [&](int buf) {
#pragma unroll
        for (int i = 0; i < K_PER_T; ++i) {
            const int idx = tid + i * NT;
            const int row = idx / KCH, c = idx % KCH;
            *(uint4*)&sK[buf][row * HD + ((c ^ (row & 15)) << 3)] = rk[i];
        }
        // transpose 8 dims x KPT keys into V^T rows, 2 keys (4 bytes) per store
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int dim = v_c * 8 + j;
#pragma unroll
            for (int i = 0; i < KPT; i += 2) {
                const uint32_t w0 = (&rv[i].x)[j >> 1];
                const uint32_t w1 = (&rv[i + 1].x)[j >> 1];
                const uint32_t e0 = (j & 1) ? (w0 >> 16) : (w0 & 0xffffu);
                const uint32_t e1 = (j & 1) ? (w1 >> 16) : (w1 & 0xffffu);
                *(uint32_t*)&sVt[buf][vt_index(dim, v_kg * KPT + i)] = e0 | (e1 << 16);
            }
        }
    };

    f32x16 oacc[OSUB];
#pragma unroll
    for (int os = 0; os < OSUB; ++os)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[os][r] = 0.f;
    float m_run = -INFINITY;
    float l_run = 0.f;

    auto compute = [&](int buf, int j) {
        const int kb = j * AP_BKV;
        // S^T (64 keys x 32 queries) = K . Q^T
        f32x16 s[2];
#pragma unroll
        for (int ms = 0; ms < 2; ++ms)
#pragma unroll
            for (int r = 0; r < 16; ++r) s[ms][r] = 0.f;
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk) {
            const int c = 2 * kk + (lane >> 5);
#pragma unroll
            for (int ms = 0; ms < 2; ++ms) {
                const int row = ms * 32 + (lane & 31);
                const bf16x8 kf =
                    as_bf16x8(*(const uint4*)&sK[buf][row * HD + ((c ^ (row & 15)) << 3)]);
                s[ms] = mfma32(kf, qf[kk], s[ms]);
            }
        }
        // causal mask, running max
        float mloc = -INFINITY;
#pragma unroll
        for (int ms = 0; ms < 2; ++ms)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = kb + ms * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                float v = s[ms][r] * scale_log2;
                if (key > my_pos) v = -INFINITY;
                s[ms][r] = v;
                mloc = fmaxf(mloc, v);
            }
        mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
        const float m_new = fmaxf(m_run, mloc);
        const float alpha = exp2f(m_run - m_new);
        float lsum = 0.f;
#pragma unroll
        for (int ms = 0; ms < 2; ++ms)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float p = exp2f(s[ms][r] - m_new);
                s[ms][r] = p;
                lsum += p;
            }
        l_run = l_run * alpha + lsum;
        m_run = m_new;
#pragma unroll
        for (int os = 0; os < OSUB; ++os)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[os][r] *= alpha;
        // O^T (hd x 32 queries) += V^T (hd x 64 keys) . P^T (64 keys x 32 queries)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            float pv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) pv[e] = s[ks >> 1][8 * (ks & 1) + e];
            const bf16x8 pf = to_bf16x8(pv);
            const int kb0 = (ks >> 1) * 32 + 16 * (ks & 1) + 4 * (lane >> 5);
#pragma unroll
            for (int os = 0; os < OSUB; ++os) {
                const int dim = os * 32 + (lane & 31);
                const uint2 lo = *(const uint2*)&sVt[buf][vt_index(dim, kb0)];
                const uint2 hi = *(const uint2*)&sVt[buf][vt_index(dim, kb0 + 8)];
                const bf16x8 vf = as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
                oacc[os] = mfma32(vf, pf, oacc[os]);
            }
        }
    };

    load_tile(0);
    store_tile(0);
    __syncthreads();
    for (int j = 0; j < ntiles; ++j) {
        const int cur = j & 1;
        if (j + 1 < ntiles) load_tile(j + 1);
        compute(cur, j);
        if (j + 1 < ntiles) store_tile(cur ^ 1);
        __syncthreads();
    }

    const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
    const float inv = 1.0f / l_tot;
    if (my_t < a.T) {
        bf16_t* orow = (bf16_t*)a.o + ((size_t)b * a.T + my_t) * ((size_t)a.n_heads * HD) +
                       (size_t)h * HD;
#pragma unroll
        for (int os = 0; os < OSUB; ++os)
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
                const int dim = os * 32 + 8 * rq + 4 * (lane >> 5);
                uint2 pk;
                pk.x = pack_bf16x2(oacc[os][4 * rq + 0] * inv, oacc[os][4 * rq + 1] * inv);
                pk.y = pack_bf16x2(oacc[os][4 * rq + 2] * inv, oacc[os][4 * rq + 3] * inv);
                *(uint2*)(orow + dim) = pk;
            }
    }
}

template <int G>
hipError_t launch_g(const AttnArgs& a, hipStream_t s) {
    const int nqb = (a.T + AP_BQ - 1) / AP_BQ;
    hipLaunchKernelGGL((attn_prefill_kernel<128, G>), dim3(nqb, a.n_kv, a.B), dim3(64 * G), 0, s,
                       a);
    return hipGetLastError();
}

}  // namespace

hipError_t attn_prefill_bf16_launch(const AttnArgs& a, hipStream_t s) {
    if (a.hd != 128 || a.n_kv <= 0 || a.n_heads % a.n_kv != 0 || a.T <= 0 || a.B <= 0)
        return hipErrorInvalidValue;
    switch (a.n_heads / a.n_kv) {
        case 1: return launch_g<1>(a, s);
        case 2: return launch_g<2>(a, s);
        case 4: return launch_g<4>(a, s);
        case 8: return launch_g<8>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace llb
