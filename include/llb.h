/*
 * llb.h -- C ABI of a Llama-3/3.1 dense decoder block on MI355X (gfx950).
 *
 * One block computes, per token (pre-norm residual block, "Llama 3.1 70B"
 * LLM diagram tool, section "Transformer layer"):
 *
 *     h = x + Wo . Attn(RMSNorm(x; g1))
 *     y = h + Wdown . (SiLU(Wgate . RMSNorm(h; g2)) * (Wup . RMSNorm(h; g2)))
 *
 * where Attn is causal grouped-query attention with interleaved-pair RoPE over a
 * KV cache kept at n_kv_heads ("Llama 3 8B - Prepare Q, K, V", atlas.klimoza.dev:
 * header shapes and "Explanation"; "How Llama 3.1 Generates the Next Token",
 * section "RoPE").
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Pointers named x, y, k_cache, v_cache, q, o, ws, k_new, v_new are DEVICE
 *    pointers owned by the caller.  llb_config and llb_weights are host structs;
 *    the pointers inside llb_weights are device pointers.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Every
 *    call except create/destroy only enqueues work on it and returns without
 *    synchronising.
 *  - Weights use nn.Linear's [out, in] row-major layout ("Llama 3 8B - Prepare
 *    Q, K, V", layers.py excerpt: F.linear computes x A^T, so the weight is
 *    stored transposed).  Their element type, the gains' and the KV cache's is
 *    llb_config.wdtype (fp32 or bf16).  The residual stream x, h, y is always fp32.
 *  - Activations are row-major: x, y are [B, T, d_model] fp32, contiguous.
 *  - Caches are [B, n_kv_heads, cache_cap, head_dim] in wdtype; row p of a
 *    sequence holds position p; cached keys are stored after RoPE.
 *  - Errors: every argument check runs on the host before any launch.  A bad
 *    argument returns LLB_E_INVALID, an unsupported shape LLB_E_UNSUPPORTED, a
 *    position range beyond cache_cap or max_positions LLB_E_CAPACITY, a HIP
 *    runtime failure LLB_E_HIP, a failed allocation LLB_E_NOMEM.  Nothing is
 *    enqueued when a check fails.  llb_last_error() returns a thread-local
 *    message for the last non-OK status of the calling thread.  Nothing throws.
 *  - Determinism: identical inputs give bitwise-identical outputs (no float
 *    atomics; split reductions are summed in a fixed order).
 *  - A handle is immutable after create; calls on different streams are safe
 *    when their caches and workspaces are distinct.
 */
#ifndef LLB_H
#define LLB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    LLB_OK = 0,
    LLB_E_INVALID = -1,
    LLB_E_UNSUPPORTED = -2,
    LLB_E_CAPACITY = -3,
    LLB_E_HIP = -4,
    LLB_E_NOMEM = -5
} llb_status;

typedef enum { LLB_F32 = 0, LLB_BF16 = 1 } llb_dtype;

/* Block hyper-parameters, named as on the pages ("Llama 3 8B - Prepare Q, K,
 * V", sku_list excerpt: dim, n_heads, n_kv_heads, norm_eps, rope_theta,
 * use_scaled_rope).  Requirements: n_heads % n_kv_heads == 0,
 * n_heads / n_kv_heads <= 16, head_dim in {64, 128}, d_model and d_ff multiples
 * of 64, max_positions >= 1.  bf16 blocks additionally need head_dim == 128,
 * n_heads / n_kv_heads in {1, 2, 4, 8} (the query-head groups the attention
 * kernels hold), d_model and d_ff multiples of 256 and an even n_heads
 * (LLB_E_UNSUPPORTED otherwise, from create, before anything is allocated). */
typedef struct {
    int32_t d_model;          /* residual width d */
    int32_t n_heads;          /* query heads */
    int32_t n_kv_heads;       /* key/value heads (GQA groups) */
    int32_t head_dim;         /* per-head width */
    int32_t d_ff;             /* SwiGLU hidden width */
    float   eps;              /* RMSNorm epsilon, inside the square root (1e-5) */
    float   rope_theta;       /* RoPE base (500000) */
    int32_t rope_scaling;     /* 0: plain schedule; 1: llama3 long-context scaling */
    float   rs_factor;        /* llama3 scaling: slow-down factor of low frequencies (8) */
    float   rs_low_freq_factor;   /* (1) */
    float   rs_high_freq_factor;  /* (4) */
    int32_t rs_orig_max_pos;  /* original context length (8192) */
    int32_t max_positions;    /* RoPE table length: every position used must be < this */
    int32_t wdtype;           /* llb_dtype of weights, gains and KV cache */
} llb_config;

/* Device pointers to the caller's weights, [out, in] row-major, wdtype.
 * attn_norm, ffn_norm: [d_model].  wq: [n_heads*head_dim, d_model].
 * wk, wv: [n_kv_heads*head_dim, d_model].  wo: [d_model, n_heads*head_dim].
 * w_gate, w_up: [d_ff, d_model].  w_down: [d_model, d_ff]. */
typedef struct {
    const void *attn_norm, *wq, *wk, *wv, *wo, *ffn_norm, *w_gate, *w_up, *w_down;
} llb_weights;

typedef struct llb_block llb_block;

/* Creates a block: copies and repacks the weights into library-owned device
 * memory, builds the RoPE cos/sin table for positions [0, max_positions)
 * ("Llama 3 8B - Prepare Q, K, V", model.py precompute_freqs_cis: float32
 * inverse frequencies and float32 position*frequency products; llama3 scaling
 * per "How Llama 3.1 Generates the Next Token", section "RoPE"), and
 * synchronises `stream`.  The caller may free its weight tensors afterwards.
 * Uses the current HIP device. */
llb_status llb_block_create(const llb_config* cfg, const llb_weights* w, void* stream,
                            llb_block** out);

/* Frees the library-owned memory of a handle.  Waits for the device first.
 * NULL is accepted.  The library keeps a set of its live handles and checks
 * every handle argument against it before reading through it: a handle that
 * was already destroyed, or any other pointer that create did not return,
 * gives LLB_E_INVALID without being dereferenced (a new handle may later be
 * created at the address of a destroyed one; that address is then live again). */
llb_status llb_block_destroy(llb_block* blk);

/* Bytes of device workspace that llb_block_prefill (B sequences of T tokens)
 * and, when T == 1, llb_block_decode need.  0 on a bad handle or size. */
size_t llb_block_workspace_bytes(const llb_block* blk, int32_t B, int32_t T);

/* Test and inspection hook: byte offsets, within the workspace of a call over
 * B sequences of T new tokens (a decode call when decode != 0, which needs
 * T == 1), of the intermediate results that call leaves there once it has run:
 *   offsets[0]  rotated queries Q [B, n_heads, T, head_dim] (wdtype), the output
 *               of the QKV projection's RoPE ("How Llama 3.1 Generates the Next
 *               Token", section "RoPE");
 *   offsets[1]  attention output O [B*T, n_heads*head_dim] (wdtype), heads as
 *               contiguous column slices ("Llama 3.1 70B", "Grouped-Query
 *               Attention");
 *   offsets[2]  h = x + O Wo^T [B*T, d_model] fp32 ("Llama 3.1 70B", "Residual add");
 *   offsets[3]  u = SiLU(gate) * up [B*T, d_ff] (wdtype) ("Llama 3.1 70B",
 *               "SwiGLU MLP").
 * The same call on another stream may overwrite them; they are valid until the
 * next call that uses the workspace. */
llb_status llb_block_workspace_layout(const llb_block* blk, int32_t B, int32_t T, int32_t decode,
                                      size_t* offsets);

/* Prefill: T new tokens per sequence at positions 0..T-1 over an empty cache
 * ("Llama 3.1 70B", "Transformer layer" and "Grouped-Query Attention": causal
 * attention, each query sees itself and earlier positions).  Writes the
 * rotated keys and the values of the T tokens to cache rows 0..T-1 and
 * y = block(x).  x, y: [B, T, d_model] fp32 (y may alias x).
 * Needs T <= cache_cap and T <= max_positions. */
llb_status llb_block_prefill(llb_block* blk, const float* x, float* y, int32_t B, int32_t T,
                             void* k_cache, void* v_cache, int32_t cache_cap,
                             void* ws, size_t ws_bytes, void* stream);

/* Chunked prefill: T new tokens per sequence at positions
 * start_pos..start_pos+T-1 against a cache whose rows 0..start_pos-1 already
 * hold earlier tokens ("Llama 3 8B - Prepare Q, K, V": the model's forward
 * takes the tokens and a start position and slices the rotation table from
 * it).  Query t attends to cache rows 0..start_pos+t.  Writes the rotated keys
 * and the values of the T tokens to cache rows start_pos..start_pos+T-1 and
 * y = block(x).  x, y: [B, T, d_model] fp32 (y may alias x).  start_pos = 0 is
 * llb_block_prefill.  Workspace: llb_block_workspace_bytes(blk, B, T).
 * Needs start_pos >= 0 and start_pos + T <= cache_cap, <= max_positions. */
llb_status llb_block_prefill_at(llb_block* blk, const float* x, float* y, int32_t B, int32_t T,
                                int32_t start_pos, void* k_cache, void* v_cache,
                                int32_t cache_cap, void* ws, size_t ws_bytes, void* stream);

/* Decode: one new token per sequence at position start_pos = P, attending to
 * cache rows 0..P-1 plus its own key, L = P + 1 keys ("Llama 3 8B - Prepare Q,
 * K, V", header: decode reads L = P + 1 keys).  Writes cache row P and
 * y = block(x).  x, y: [B, 1, d_model] fp32 (y may alias x).
 * Needs P + 1 <= cache_cap and P < max_positions. */
llb_status llb_block_decode(llb_block* blk, const float* x, float* y, int32_t B, int32_t start_pos,
                            void* k_cache, void* v_cache, int32_t cache_cap,
                            void* ws, size_t ws_bytes, void* stream);

/* Ragged decode: as llb_block_decode, but sequence b's new token sits at its
 * own position start_pos[b] and attends to its cache rows 0..start_pos[b]
 * (L_b = start_pos[b] + 1 keys; the pages give one start position per call, a
 * batch of different lengths is this library's extension).  start_pos is a
 * HOST array of B entries, read during the call (it reaches the device in
 * kernel arguments, so the caller may reuse it once the call returns).  Writes cache row
 * start_pos[b] of sequence b.  Workspace: llb_block_workspace_bytes(blk, B, 1).
 * Needs every start_pos[b] >= 0, start_pos[b] + 1 <= cache_cap and
 * start_pos[b] < max_positions; a violation fails before anything is queued. */
llb_status llb_block_decode_ragged(llb_block* blk, const float* x, float* y, int32_t B,
                                   const int32_t* start_pos, void* k_cache, void* v_cache,
                                   int32_t cache_cap, void* ws, size_t ws_bytes, void* stream);

/* For callers that cannot allocate device memory, nor hand the library a
 * workspace: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  The same decode as llb_block_decode (the same kernels and
 * results, bit for bit), with its workspace taken from a static scratch array
 * of 64 MiB that the library holds on each GPU it runs on until the process
 * ends.  It allocates nothing: no hipMalloc, hipFree or allocating library
 * routine, and it records no timing events (llb_block_set_stage_timing does not
 * apply).  The caller still passes x, y and the caches.  A call whose workspace
 * (llb_block_workspace_bytes(blk, B, 1) at its P) exceeds 64 MiB fails with
 * LLB_E_CAPACITY before anything is queued; for the 8B and 70B shapes it holds
 * B up to 64 at any P the RoPE table allows.  The array keeps the last call's
 * contents; no part of it has to start at zero (each call writes everything it
 * reads).  Every call on one GPU shares that GPU's array: calls that overlap in
 * time on one GPU (on different streams, or from different threads) race and
 * must be ordered by the caller.  LLB_E_HIP if the array's device address could
 * not be looked up when the block was created. */
llb_status llb_block_decode_noalloc(llb_block* blk, const float* x, float* y, int32_t B, int32_t start_pos,
                                    void* k_cache, void* v_cache, int32_t cache_cap, void* stream);

/* Copies k_new, v_new [B, n_kv_heads, n_new, head_dim] (wdtype) into cache
 * rows start_pos..start_pos+n_new-1 of every sequence and KV head: the cache
 * update of "Llama 3 8B - Prepare Q, K, V" ("Explanation" and the model.py
 * excerpt: the keys and values of the positions being processed are stored in
 * the cache at their positions, at n_kv_heads, keys already rotated), for
 * keys and values computed elsewhere (for example to seed a cache).  Needs
 * start_pos + n_new <= cache_cap; a bad size fails before anything is queued. */
llb_status llb_kv_append(const llb_block* blk, void* k_cache, void* v_cache, int32_t B,
                         int32_t cache_cap, int32_t start_pos, int32_t n_new,
                         const void* k_new, const void* v_new, void* stream);

/* Attention alone, on the block's head layout and dtype (unit-level access to
 * the kernels used inside prefill/decode).
 * llb_attention_prefill: q [B, n_heads, T, head_dim] holds rotated queries at
 *   positions start_pos..start_pos+T-1; keys/values are cache rows
 *   0..start_pos+T-1; query t sees keys <= start_pos+t ("How Llama 3.1
 *   Generates the Next Token", block notation: mask M is -inf for future
 *   positions; score q.k/sqrt(head_dim)).  o: [B, T, n_heads*head_dim].
 * llb_attention_decode: q [B, n_heads, head_dim], one query per sequence at
 *   position start_pos reading keys 0..start_pos; o: [B, n_heads*head_dim];
 *   needs ws of llb_attention_workspace_bytes(blk, B, start_pos + 1) bytes.
 * Query head h reads KV head h / (n_heads / n_kv_heads).  All in wdtype. */
llb_status llb_attention_prefill(const llb_block* blk, const void* q, const void* k_cache,
                                 const void* v_cache, void* o, int32_t B, int32_t T,
                                 int32_t start_pos, int32_t cache_cap, void* stream);
llb_status llb_attention_decode(const llb_block* blk, const void* q, const void* k_cache,
                                const void* v_cache, void* o, int32_t B, int32_t start_pos,
                                int32_t cache_cap, void* ws, size_t ws_bytes, void* stream);
size_t llb_attention_workspace_bytes(const llb_block* blk, int32_t B, int32_t n_keys);
/* llb_attention_decode_ragged: as llb_attention_decode, but query b sits at its
 * own position start_pos[b] (a HOST array of B entries, read during the call)
 * and reads keys 0..start_pos[b] of its sequence (L_b = start_pos[b] + 1 keys,
 * "Llama 3 8B - Prepare Q, K, V", header; per-sequence lengths are this
 * library's extension).  The same attention llb_block_decode_ragged runs.
 * ws: llb_attention_workspace_bytes(blk, B, max_b start_pos[b] + 1) bytes. */
llb_status llb_attention_decode_ragged(const llb_block* blk, const void* q, const void* k_cache,
                                       const void* v_cache, void* o, int32_t B, const int32_t* start_pos,
                                       int32_t cache_cap, void* ws, size_t ws_bytes, void* stream);

/* Measurement hook for benchmarking tools.  While enabled, every
 * llb_block_prefill / llb_block_decode call on `blk` records HIP events on its
 * stream before and after each of its five stages, in this order: QKV
 * projection (with RMSNorm, RoPE and the cache write), attention, output
 * projection (+ residual), gate/up projection (with RMSNorm and SiLU.up), down
 * projection (+ residual).  llb_block_stage_times waits for the recorded
 * events, writes the summed milliseconds of each stage to ms[0..4] and the
 * number of recorded calls to *n_calls, and clears the record.  Disabled by
 * default; enabling it costs one event record per stage boundary. */
llb_status llb_block_set_stage_timing(llb_block* blk, int32_t enable);
llb_status llb_block_stage_times(llb_block* blk, float* ms, int32_t* n_calls);

/* ---- Model: embedding, n_layers blocks, final RMSNorm, LM head ------------
 * "Llama 3.1 70B" (sections on the token embedding, the stack of transformer
 * layers and the LM head) and "How Llama 3.1 Generates the Next Token" (the
 * unembedding: a final RMSNorm, then one linear map from d_model to the
 * vocabulary, untied from the embedding).  bf16 weights only.
 *
 * llb_model_create: cfg as for llb_block_create (every layer has that shape);
 *   embed and lm_head are [vocab, d_model] bf16 device matrices, final_norm [d]
 *   bf16, layers an array of n_layers weight sets.  Everything is copied (the
 *   caller may free its tensors afterwards).  vocab must be a multiple of 128
 *   (LLB_E_UNSUPPORTED otherwise).  Uses the current device; synchronises.
 * llb_model_forward: tokens [B, T] int32 device ids at positions
 *   start_pos..start_pos+T-1 of every sequence; k_caches / v_caches are HOST
 *   arrays of n_layers device pointers, each a cache as in llb_block_prefill.
 *   T = 1 decodes (one token at position start_pos, reading L = start_pos + 1
 *   keys per layer), T > 1 prefills a chunk.  logits: fp32, [B, T, vocab], or
 *   [B, vocab] for the last position of each sequence when last_only != 0.  An
 *   id outside [0, vocab) gives NaN hidden states and logits to its sequence
 *   (through attention the NaN reaches the sequence's other positions of this
 *   call and the cache rows it writes), never to other sequences; the table is
 *   never read out of range.  Needs start_pos + T <= cache_cap and
 *   <= max_positions; the workspace is llb_model_workspace_bytes(m, B, T,
 *   last_only) bytes.  Enqueues on `stream`. */
typedef struct llb_model llb_model;
llb_status llb_model_create(const llb_config* cfg, int32_t n_layers, int32_t vocab, const void* embed,
                            const llb_weights* layers, const void* final_norm, const void* lm_head,
                            void* stream, llb_model** out);
llb_status llb_model_destroy(llb_model* m);
size_t llb_model_workspace_bytes(const llb_model* m, int32_t B, int32_t T, int32_t last_only);
llb_status llb_model_forward(llb_model* m, const int32_t* tokens, int32_t B, int32_t T, int32_t start_pos,
                             void* const* k_caches, void* const* v_caches, int32_t cache_cap,
                             int32_t last_only, float* logits, void* ws, size_t ws_bytes, void* stream);

/* Tuning and test hooks for the bf16 prefill projections.  The library holds
 * a fixed table of GEMM tile configurations (workgroup tile BM x BN, waves,
 * k-depth, pipeline stages, schedule); by default each projection picks one
 * from M, N and K.  llb_gemm_tile_info writes configuration `cfg`'s tile rows
 * and columns to *bm and *bn (LLB_E_INVALID if cfg is outside
 * [0, llb_gemm_num_tiles())).  llb_block_set_tiles fixes the configuration of
 * the QKV, output, gate/up and down projections of later calls on `blk` that
 * run them as GEMMs: prefill calls, and decode calls over more than 64
 * sequences (smaller decode batches use the weight-streaming kernels); fp32
 * blocks ignore it.  -1 restores the automatic choice; values outside
 * [-1, count) give LLB_E_INVALID and change nothing.  A call whose
 * configuration for some projection has a BN that does not divide that
 * projection's N, or a per-wave column slice that cannot hold its fused
 * epilogue, or (the interleaved configurations, which address their operands
 * by 32-bit byte offsets) an operand of 4 GiB or more, fails with
 * LLB_E_UNSUPPORTED before any work is queued.  The automatic choice falls
 * back to the plain configurations for such operands. */
int32_t llb_gemm_num_tiles(void);
llb_status llb_gemm_tile_info(int32_t cfg, int32_t* bm, int32_t* bn);
llb_status llb_block_set_tiles(llb_block* blk, int32_t qkv, int32_t o, int32_t gate_up, int32_t down);

/* Tuning and test hook for the bf16 decode projections (llb_block_decode,
 * llb_block_decode_ragged and the model's decode over at most 64 sequences).
 * Each projection streams its weights through one of two kernels:
 *   0  = split-K, 128 weight rows per workgroup, weights and token rows staged
 *        through LDS by DMA; with K split over workgroups a second kernel sums
 *        the fp32 partials in split order;
 *   16, 32 = narrow: that many weight rows per workgroup over the whole of K
 *        (its four waves split K and sum in LDS; one kernel); QKV, O and down
 *        only (the gate/up pairs need 64-row groups).
 * -1 restores the automatic choice.  Every choice computes the same products;
 * results differ only in summation order (parity with the oracle holds for
 * each).  Values outside those sets give LLB_E_INVALID and change nothing; a
 * later decode call whose choice does not fit a projection's shape fails with
 * LLB_E_UNSUPPORTED before any work is queued. */
llb_status llb_block_set_decode_kernels(llb_block* blk, int32_t qkv, int32_t o, int32_t gate_up,
                                        int32_t down);

/* ---- Measurement probes ---------------------------------------------------
 * Not part of the block: instruments that measure, on the GPU in use, the two
 * rates the block's kernels are bound by, so that roofline fractions can be
 * given against measured peaks as well as nominal ones.  Each enqueues one
 * kernel on `stream` (current device) and is timed by the caller.
 * llb_probe_hbm_read: streams `bytes` (a positive multiple of 16) from src with
 *   16-byte loads over n_workgroups workgroups of 256 lanes; sink (device) gets
 *   one uint32 per workgroup.  Bytes moved: `bytes`.
 * llb_probe_hbm_copy: copies `bytes` from src to dst (non-overlapping) with the
 *   same pattern.  Bytes moved: 2 * `bytes`.
 * llb_probe_mfma_bf16: n_workgroups workgroups of 4 waves; each wave issues
 *   iters x 8 independent 16x16x32 bf16 MFMAs on pseudo-random operands; sink
 *   (device) gets 4 * n_workgroups floats.  FLOPs: n_workgroups * 4 * iters * 8
 *   * 16384.
 * A bad argument gives LLB_E_INVALID before anything is queued. */
llb_status llb_probe_hbm_read(const void* src, size_t bytes, int32_t n_workgroups, void* sink, void* stream);
llb_status llb_probe_hbm_copy(void* dst, const void* src, size_t bytes, int32_t n_workgroups, void* stream);
llb_status llb_probe_mfma_bf16(int32_t n_workgroups, int32_t iters, void* sink, void* stream);

/* Thread-local text describing the last non-OK status ("" if none). */
const char* llb_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* LLB_H */
