// Projection epilogues: what happens to one fp32 result C[m, n] of x.W^T.
//
//  EPI_QKV    RoPE on the Q and K columns (interleaved adjacent pairs rotated by
//             pos * omega_i, "How Llama 3.1 Generates the Next Token", section
//             "RoPE"), Q to the head-major query buffer, K and V to the cache row
//             of the token's position ("Llama 3 8B - Prepare Q, K, V",
//             "Explanation": keys and values are cached at n_kv_heads).
//  EPI_RESID  residual add in fp32 ("Llama 3.1 70B", section "Residual add").
//  EPI_SWIGLU SiLU(gate) * up, with gate and up in fp32 until the product
//             ("Llama 3.1 70B", section "SwiGLU MLP").
#pragma once

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
    const int pos = e.pos0 + t;
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

LLB_DEV void epi_resid(const Epilogue& e, int m, int n, int N, float v) {
    const size_t idx = (size_t)m * N + n;
    e.out[idx] = e.resid[idx] + v;
}

// gate = C[m, 64*grp + j], up = C[m, 64*grp + 32 + j]; feature f = 32*grp + j.
template <typename OT>
LLB_DEV void epi_swiglu(const Epilogue& e, int m, int f, int d_ff, float gate, float up) {
    store_elem<OT>(e.u_out, (size_t)m * d_ff + f, silu_f(gate) * up);
}

}  // namespace llb
