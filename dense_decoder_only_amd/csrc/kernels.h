// Internal interface between the host orchestrator (block.cpp) and the kernel
// translation units.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace llb {

enum EpiKind : int { EPI_QKV = 0, EPI_RESID = 1, EPI_SWIGLU = 2, EPI_RESID_NORM = 3, EPI_LOGITS = 4 };

// What a projection does with its fp32 result C[m, n] (after the row's inverse
// RMS is applied when the A operand was normalised).
struct Epilogue {
    int kind;
    // EPI_QKV: columns [0, n_heads*hd) are Q, then K, then V (each head hd wide).
    // Q and K are rotated (interleaved pairs, rope[pos][i] = (cos, sin)); Q goes to
    // q_out [B, n_heads, T, hd], K/V to cache rows pos = pos0 + t of [B, n_kv, cap, hd].
    void* q_out;
    void* k_cache;
    void* v_cache;
    const float2* rope;
    int T, pos0, cap, n_heads, n_kv, hd;
    // Per-sequence start positions [B] (device; decode with T = 1), or null:
    // every sequence starts at pos0.
    const int* pos_b;
    // EPI_RESID: out[m, n] = resid[m, n] + C[m, n]   (fp32, [M, N] row-major)
    const float* resid;
    float* out;
    // EPI_RESID_NORM: as EPI_RESID, and also the next RMSNorm's operand
    // a_out[m, n] = bf16(out[m, n] * gain[n]) and the partial sum of out^2 over the
    // tile's columns, one partial per column tile: ssq_out[tile_n * M + m] from
    // the prefill GEMM, ssq_out[tile_n * MT + m] from the decode kernels.
    const float* gain;
    void* a_out;
    float* ssq_out;
    // EPI_SWIGLU: columns come in 64-wide groups [gate 32 | up 32]; feature
    // f = group*32 + j gets u[m, f] = SiLU(C_gate) * C_up, u is [M, N/2].
    void* u_out;
    // EPI_LOGITS: out[m, n] = C[m, n] (fp32 [M, N]; C carries the row's 1/rms
    // like EPI_QKV and EPI_SWIGLU).  Uses `out`.
};

// C = A . W^T.  W: [N, K], fp32 row-major or bf16 in the tiled layout below.
// bf16 path: A is bf16 [M, K].  For EPI_QKV and EPI_SWIGLU, A holds v * g of an
// RMSNorm (v the residual stream, g its gain) and the row's inverse RMS
// 1/sqrt(sum/K + eps), sum over the ssq_count partials of ssq_in (laid out as
// the producing kernel wrote them: [p][M] prefill, [p][MT] decode), scales C
// before the epilogue.
// fp32 path: A is fp32 [M, K]; when `norm`, the kernel forms the RMSNorm itself
// (A * gain, row inverse RMS over K).
struct GemmArgs {
    const void* A;
    const float* gain;
    const void* W;
    int M, N, K;
    int norm;
    float eps;
    const float* ssq_in;
    int ssq_count;
    Epilogue epi;
    // Output columns [n_begin, n_end) of this launch (prefill GEMM only; both
    // multiples of the tile's BN; n_end = 0 means N).  N still sets the strides.
    int n_begin, n_end;
};

// Start position of sequence b (see Epilogue::pos_b).
template <typename Args>
__device__ __forceinline__ int seq_start(const Args& e, int b) {
    return e.pos_b ? e.pos_b[b] : e.pos0;
}

// ---- bf16 MFMA projections -----------------------------------------------
// Large-M projection (prefill): LDS-staged bf16 MFMA tiles.
hipError_t gemm_bf16_launch(const GemmArgs& a, int tile_cfg, hipStream_t s);
// Tile configurations available to gemm_bf16_launch: returns BM, BN, threads.
// Whether tile configuration cfg can run C[M, N] = A[M, K] W^T with epilogue
// kind epi (BN divides N, BK divides K, the per-wave column slice holds the
// epilogue's column groups; the interleaved configurations also need
// gemm_bf16_offsets_fit).
bool gemm_bf16_supports(int cfg, int M, int N, int K, int epi);
// Whether every byte offset into A [M, K] and W [N, K] (bf16) fits 32 bits.
bool gemm_bf16_offsets_fit(long M, long N, long K);
void gemm_bf16_tile(int tile_cfg, int* bm, int* bn, int* threads);
int gemm_bf16_num_tile_cfgs();
// The bf16 projections read W in 128-row x 64-column tiles: element (n, k) of
// W [N, K] at ((n/128) * (K/64) + k/64) * 8192 + (n%128) * 64 + k%64.  Converts a
// row-major W (N % 128 == 0, K % 64 == 0) into that layout (src != dst).
hipError_t tile_weights_launch(const void* src, void* dst, int N, int K, hipStream_t s);

// Small-M projection (decode, M <= 64): weight-streaming split-K over 128-row
// column tiles.  ws: gemv_bf16_ws_bytes(M, N, splits) bytes of fp32 partials.
// With several splits a second kernel sums the partials in split order and
// applies the epilogue.  EPI_RESID_NORM writes one partial sum of squares per
// column tile (gemv_bf16_ssq_parts(N) of them).  The decode kernels lay partial
// sums of squares out as [P][MT], partial p of row m at ssq[p * MT + m] with
// MT = 32 (M <= 32) or 64; a one-partial operand is the plain [M] row.
size_t gemv_bf16_ws_bytes(int M, int N, int splits);
int gemv_bf16_ssq_parts(int N);
int gemv_bf16_splits(int M, int N, int K);
hipError_t gemv_bf16_launch(const GemmArgs& a, int splits, float* ws, hipStream_t s);
// Narrow weight streaming (decode, M <= 64): one workgroup per rw (16 or 32) W
// rows over all of K, its four waves splitting K and summing in LDS; epilogues
// EPI_QKV, EPI_RESID, EPI_RESID_NORM in the same kernel (no partials in HBM).
// EPI_RESID_NORM writes N / rw partial sums of squares.  Needs N % 128 == 0 (the
// tiled weight layout) and K a multiple of 64 with K >= 256.
bool gemv_narrow_supports(int M, int N, int K, int epi, int rw);
// The QKV projection with the attention RMSNorm formed inside the narrow kernel
// (args.norm = 1: A is fp32 x [M, K] and args.gain its gain; no ssq_in): at
// most 32 token rows and one workgroup per CU (N / rw <= num_cus).
bool gemv_narrow_norm_supports(int M, int N, int K, int rw, int num_cus);
hipError_t gemv_narrow_launch(const GemmArgs& a, int rw, int num_cus, hipStream_t s);

// RMSNorm operand: a[m, :] = bf16(x[m, :] * g), ssq[m] = sum_j x[m, j]^2 (fp32).
hipError_t norm_rows_launch(const float* x, const float* g, void* a, float* ssq, int M, int d,
                            hipStream_t s);

// ---- fp32 projections (SIMT) ----------------------------------------------
hipError_t gemm_f32_launch(const GemmArgs& a, hipStream_t s);

// ---- attention --------------------------------------------------------------
struct AttnArgs {
    const void* q;        // prefill: [B, n_heads, T, hd]; decode: [B, n_heads, hd]
    const void* k_cache;  // [B, n_kv, cap, hd]
    const void* v_cache;
    void* o;              // [B, T, n_heads*hd]
    int B, T, pos0, cap, n_heads, n_kv, hd;
    // Per-sequence start positions [B] (device), or null: all start at pos0.  With
    // them, pos0 is their maximum (it sizes the work split).
    const int* pos_b;
};
hipError_t attn_prefill_bf16_launch(const AttnArgs& a, hipStream_t s);
// Split-K decode attention + merge.  ws: attn_decode_ws_bytes(...) bytes.
size_t attn_decode_ws_bytes(int B, int n_heads, int n_kv, int hd, int n_keys);
hipError_t attn_decode_bf16_launch(const AttnArgs& a, float* ws, hipStream_t s);
// Plain fp32 attention (prefill or decode, any T).
hipError_t attn_f32_launch(const AttnArgs& a, hipStream_t s);

// ---- cache helpers ---------------------------------------------------------
// ---- model: token embedding and the LM head's rows ---------------------------
// x[m, :] = fp32(E[tok[m], :]) for the bf16 table E [vocab, d] (ids outside the
// vocabulary give NaN rows); tok: device [M].
hipError_t embed_launch(const int* tok, const void* E, float* x, int M, int d, int vocab, hipStream_t s);
// dst[b, :] = src[b*T + T - 1, :], fp32 rows of d.
hipError_t last_rows_launch(const float* src, float* dst, int B, int T, int d, hipStream_t s);

// dst[0..n) = src[0..n) (src on the host), through kernel arguments: ordered on
// stream s like the kernels, and src may be reused as soon as this returns.
hipError_t store_ints_launch(int* dst, const int* src, int n, hipStream_t s);
// ---- measurement probes (probes.hip) -----------------------------------------
// Stream `bytes` (a multiple of 16) from src with n_wg workgroups of 256 lanes;
// sink gets one word per workgroup.
hipError_t probe_read_launch(const void* src, size_t bytes, uint32_t* sink, int n_wg, hipStream_t s);
// dst[0..bytes) = src[0..bytes), the same access pattern.
hipError_t probe_copy_launch(void* dst, const void* src, size_t bytes, int n_wg, hipStream_t s);
// n_wg workgroups of 4 waves, each wave iters x 8 independent 16x16x32 bf16 MFMAs;
// sink gets one float per wave (4 n_wg).
hipError_t probe_mfma_launch(float* sink, int n_wg, int iters, hipStream_t s);

hipError_t kv_append_launch(void* kc, void* vc, const void* kn, const void* vn, int B, int n_kv,
                            int cap, int pos0, int n_new, int hd, int elem_bytes, hipStream_t s);

}  // namespace llb
