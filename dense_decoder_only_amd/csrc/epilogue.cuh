// Projection epilogues: what happens to one fp32 result C[m, n] of x.W^T.
//
//  EPI_QKV    RoPE on the Q and K columns (interleaved adjacent pairs rotated by
//             pos * omega_i, "How Llama 3.1 Generates the Next Token", section
//             "RoPE"), Q to the head-major query buffer, K and V to the cache row
//             of the token's position ("Llama 3 8B - Prepare Q, K, V",
//             "Explanation": keys and values are cached at n_kv_heads).
//  EPI_RESID  residual add in fp32 ("Llama 3.1 70B", section "Residual add").
//  EPI_RESID_NORM  the residual add, plus the next RMSNorm's bf16 operand h * g
//             and partial sums of h^2 ("Llama 3.1 70B", section "RMSNorm": one
//             fp32 reduction over the row's features).
//  EPI_SWIGLU SiLU(gate) * up, with gate and up in fp32 until the product
//             ("Llama 3.1 70B", section "SwiGLU MLP").
#pragma once

#include <type_traits>

#include "common.cuh"
#include "kernels.h"

namespace llb {

template <typename OT>
LLB_DEV void store_elem(void* base, size_t idx, float v) {
    if constexpr (sizeof(OT) == 4) {
        ((float*)base)[idx] = v;
    } else {
        ((bf16_t*)base)[idx] = f2bf(v);
    }
}

// v = C[m, n]; partner = C[m, n ^ 1] (the other member of the RoPE pair).
template <typename OT>
LLB_DEV void epi_qkv(const Epilogue& e, int m, int n, float v, float partner) {
    const int hd = e.hd;
    const int Hq = e.n_heads * hd;
    const int Hk = e.n_kv * hd;
    const int b = m / e.T;
    const int t = m - b * e.T;
    const int pos = seq_start(e, b) + t;
    const int j = n & (hd - 1);
    if (n < Hq + Hk) {
        const float2 cs = e.rope[(size_t)pos * (hd >> 1) + (j >> 1)];
        // even j: x'_j = x_j cos - x_{j+1} sin;  odd j: x'_j = x_{j-1} sin + x_j cos
        const float r = (j & 1) ? (partner * cs.y + v * cs.x) : (v * cs.x - partner * cs.y);
        if (n < Hq) {
            const int head = n / hd;
            store_elem<OT>(e.q_out, (((size_t)b * e.n_heads + head) * e.T + t) * hd + j, r);
        } else {
            const int head = (n - Hq) / hd;
            store_elem<OT>(e.k_cache, (((size_t)b * e.n_kv + head) * e.cap + pos) * hd + j, r);
        }
    } else {
        const int head = (n - Hq - Hk) / hd;
        store_elem<OT>(e.v_cache, (((size_t)b * e.n_kv + head) * e.cap + pos) * hd + j, v);
    }
}

LLB_DEV float epi_resid(const Epilogue& e, int m, int n, int N, float v) {
    const size_t idx = (size_t)m * N + n;
    const float h = e.resid[idx] + v;
    e.out[idx] = h;
    return h;
}

// Operand of the next RMSNorm: bf16(h * g), rounded once.
LLB_DEV void epi_norm_operand(const Epilogue& e, int m, int n, int N, float h) {
    ((bf16_t*)e.a_out)[(size_t)m * N + n] = f2bf(h * e.gain[n]);
}

// The same with the gain g = gain[n] loaded ahead: vector-memory operations
// complete in order, so a gain load issued after the residual store would wait
// for that store as well.
LLB_DEV void epi_norm_operand_g(const Epilogue& e, int m, int n, int N, float h, float g) {
    ((bf16_t*)e.a_out)[(size_t)m * N + n] = f2bf(h * g);
}

// gate = C[m, 64*grp + j], up = C[m, 64*grp + 32 + j]; feature f = 32*grp + j.
template <typename OT>
LLB_DEV void epi_swiglu(const Epilogue& e, int m, int f, int d_ff, float gate, float up) {
    if constexpr (std::is_same<OT, bf16_t>::value)
        store_elem<OT>(e.u_out, (size_t)m * d_ff + f, silu_bf16(gate) * up);
    else
        store_elem<OT>(e.u_out, (size_t)m * d_ff + f, silu_f(gate) * up);
}

// ---- 8-column forms: v[0..7] = C[m, n..n+7], n a multiple of 8 -------------

LLB_DEV uint4 pack8(const float* v) {
    return make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                      pack_bf16x2(v[6], v[7]));
}

// RoPE on 4 adjacent pairs (when the columns are Q or K), then one 16-byte store
// of 8 bf16 to the query buffer or the cache row.
LLB_DEV void epi_qkv8(const Epilogue& e, int m, int n, float* v) {
    const int hd = e.hd;
    const int Hq = e.n_heads * hd;
    const int Hk = e.n_kv * hd;
    const int b = m / e.T;
    const int t = m - b * e.T;
    const int pos = seq_start(e, b) + t;
    const int j = n & (hd - 1);
    bf16_t* dst;
    if (n < Hq + Hk) {
        const float4* cs4 = (const float4*)(e.rope + (size_t)pos * (hd >> 1) + (j >> 1));
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const float4 cs = cs4[p];  // (cos, sin) of pairs 2p and 2p+1
            const float x0 = v[4 * p], x1 = v[4 * p + 1], x2 = v[4 * p + 2], x3 = v[4 * p + 3];
            v[4 * p + 0] = x0 * cs.x - x1 * cs.y;
            v[4 * p + 1] = x0 * cs.y + x1 * cs.x;
            v[4 * p + 2] = x2 * cs.z - x3 * cs.w;
            v[4 * p + 3] = x2 * cs.w + x3 * cs.z;
        }
        if (n < Hq) {
            dst = (bf16_t*)e.q_out + (((size_t)b * e.n_heads + n / hd) * e.T + t) * hd + j;
        } else {
            dst = (bf16_t*)e.k_cache + (((size_t)b * e.n_kv + (n - Hq) / hd) * e.cap + pos) * hd + j;
        }
    } else {
        dst = (bf16_t*)e.v_cache + (((size_t)b * e.n_kv + (n - Hq - Hk) / hd) * e.cap + pos) * hd + j;
    }
    *(uint4*)dst = pack8(v);
}

// out = C (fp32 logits, two 16-byte stores).
LLB_DEV void epi_store8(const Epilogue& e, int m, int n, int N, const float* v) {
    const size_t idx = (size_t)m * N + n;
    *(float4*)(e.out + idx) = make_float4(v[0], v[1], v[2], v[3]);
    *(float4*)(e.out + idx + 4) = make_float4(v[4], v[5], v[6], v[7]);
}

// h = resid + C (fp32, two 16-byte loads and stores); returns h in v.
LLB_DEV void epi_resid8(const Epilogue& e, int m, int n, int N, float* v) {
    const size_t idx = (size_t)m * N + n;
    const float4 r0 = *(const float4*)(e.resid + idx);
    const float4 r1 = *(const float4*)(e.resid + idx + 4);
    v[0] += r0.x; v[1] += r0.y; v[2] += r0.z; v[3] += r0.w;
    v[4] += r1.x; v[5] += r1.y; v[6] += r1.z; v[7] += r1.w;
    *(float4*)(e.out + idx) = make_float4(v[0], v[1], v[2], v[3]);
    *(float4*)(e.out + idx + 4) = make_float4(v[4], v[5], v[6], v[7]);
}

// Gains of 8 columns n..n+7, loaded ahead of the residual stores (see
// epi_norm_operand_g), for epi_norm_operand8g.
LLB_DEV void epi_gain8(const Epilogue& e, int n, float* g) {
    *(float4*)&g[0] = *(const float4*)(e.gain + n);
    *(float4*)&g[4] = *(const float4*)(e.gain + n + 4);
}

// bf16(h * g) for 8 columns with the gains loaded ahead; returns the sum of h^2.
LLB_DEV float epi_norm_operand8g(const Epilogue& e, int m, int n, int N, const float* h, const float* g) {
    float t[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) t[k] = h[k] * g[k];
    *(uint4*)((bf16_t*)e.a_out + (size_t)m * N + n) = pack8(t);
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) s += h[k] * h[k];
    return s;
}

// bf16(h * g) for 8 columns; returns the sum of h^2 over them.
LLB_DEV float epi_norm_operand8(const Epilogue& e, int m, int n, int N, const float* h) {
    const float4 g0 = *(const float4*)(e.gain + n);
    const float4 g1 = *(const float4*)(e.gain + n + 4);
    const float t[8] = {h[0] * g0.x, h[1] * g0.y, h[2] * g0.z, h[3] * g0.w,
                        h[4] * g1.x, h[5] * g1.y, h[6] * g1.z, h[7] * g1.w};
    *(uint4*)((bf16_t*)e.a_out + (size_t)m * N + n) = pack8(t);
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) s += h[k] * h[k];
    return s;
}

// 8 features f..f+7: u = SiLU(gate) * up, one 16-byte store.
LLB_DEV void epi_swiglu8(const Epilogue& e, int m, int f, int d_ff, const float* gate,
                         const float* up) {
    float u[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) u[k] = silu_bf16(gate[k]) * up[k];
    *(uint4*)((bf16_t*)e.u_out + (size_t)m * d_ff + f) = pack8(u);
}

}  // namespace llb
