// Host side of the block library: argument validation, weight repacking, the
// RoPE table, workspace planning and the kernel sequence of one block call.
// Public interface: include/llb.h.
#include "llb.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <algorithm>
#include <cstring>
#include <mutex>
#include <string>
#include <unordered_set>
#include <vector>

#include "kernels.h"

// The no-allocation entry point's scratch (see scratch_setup below).
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

thread_local std::string g_err;

constexpr uint64_t kMagic = 0x4b434f4c42424c4cull;  // "LLBBLOCK"

// Live handles.  Every entry point looks a handle up here before reading
// through it, so a pointer that was never returned by a create call, or whose
// destroy has already run, is rejected without being dereferenced.
struct Registry {
    std::mutex mu;
    std::unordered_set<const void*> blocks, models;
};
Registry& registry() {
    static Registry r;
    return r;
}
void register_live(std::unordered_set<const void*> Registry::*set, const void* h) {
    Registry& r = registry();
    std::lock_guard<std::mutex> lk(r.mu);
    (r.*set).insert(h);
}
bool is_live(std::unordered_set<const void*> Registry::*set, const void* h) {
    Registry& r = registry();
    std::lock_guard<std::mutex> lk(r.mu);
    return (r.*set).count(h) != 0;
}
// Removes h; false when it was not live.
bool unregister_live(std::unordered_set<const void*> Registry::*set, const void* h) {
    Registry& r = registry();
    std::lock_guard<std::mutex> lk(r.mu);
    return (r.*set).erase(h) == 1;
}

llb_status fail(llb_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
llb_status fail(llb_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return st;
}

llb_status hip_fail(hipError_t e, const char* what) {
    return fail(LLB_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

size_t align_up(size_t v) { return (v + 255) & ~size_t(255); }

// ---- static scratch of llb_block_decode_noalloc -------------------------------
// Device memory for callers that cannot allocate: one copy of this array per GPU
// the library runs on, held until the process ends.  Host code never uses the
// array's name as an address (on the host it is only a stand-in for the device
// symbol): llb_block_create looks up each device's copy once, with that device
// current, and the entry point passes that address to the kernels.
constexpr int kMaxDevices = 64;
struct ScratchTable {
    std::mutex mu;
    bool looked_up[kMaxDevices] = {};
    void* ptr[kMaxDevices] = {};
    hipError_t err[kMaxDevices] = {};
};
ScratchTable& scratch_table() {
    static ScratchTable t;
    return t;
}

// Looks up the current device's copy of `scratch` (once per device).
void scratch_setup(int device) {
    if (device < 0 || device >= kMaxDevices) return;
    ScratchTable& t = scratch_table();
    std::lock_guard<std::mutex> lk(t.mu);
    if (t.looked_up[device]) return;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    t.looked_up[device] = true;
    t.err[device] = e;
    t.ptr[device] = e == hipSuccess ? p : nullptr;
}

// The device address of `device`'s scratch copy, or null (with the lookup's error).
void* scratch_ptr(int device, hipError_t* err) {
    *err = hipErrorInvalidDevice;
    if (device < 0 || device >= kMaxDevices) return nullptr;
    ScratchTable& t = scratch_table();
    std::lock_guard<std::mutex> lk(t.mu);
    if (!t.looked_up[device]) return nullptr;
    *err = t.err[device];
    return t.ptr[device];
}

constexpr double kPi = 3.14159265358979323846;

}  // namespace

struct llb_block {
    uint64_t magic;
    llb_config cfg;
    int es;          // bytes per weight / cache element
    int device;
    // Projection weights [N, K] (bf16: in the 128 x 64 tiled layout of
    // tile_weights_launch; fp32: row-major).
    void* wqkv;      // [(n_heads + 2 n_kv) hd, d]: Q rows, then K, then V
    void* wo;        // [d, n_heads hd]
    void* wgu;       // [2 d_ff, d]: 64-row groups [gate 32 rows | up 32 rows]
    void* wdown;     // [d, d_ff]
    float* g1;       // attention RMSNorm gain, fp32 [d]
    float* g2;       // FFN RMSNorm gain, fp32 [d]
    float2* rope;    // [max_positions][hd/2] (cos, sin)
    int tile_qkv, tile_o, tile_gu, tile_down;  // bf16 prefill tile choice per projection (-1 = pick by M)
    int dec_qkv, dec_o, dec_gu, dec_down;  // decode kernel per projection (llb_block_set_decode_kernels)
    int num_cus;                     // compute units of the device
    int timing;                      // record stage events on every call
    std::vector<hipEvent_t> events;  // 6 per recorded call
    size_t events_used;
};

namespace {

bool handle_ok(const llb_block* b) {
    return b != nullptr && is_live(&Registry::blocks, b) && b->magic == kMagic;
}

llb_status check_config(const llb_config* c) {
    if (!c) return fail(LLB_E_INVALID, "config is NULL");
    if (c->d_model <= 0 || c->n_heads <= 0 || c->n_kv_heads <= 0 || c->head_dim <= 0 || c->d_ff <= 0)
        return fail(LLB_E_INVALID, "dimensions must be positive");
    if (c->n_heads % c->n_kv_heads != 0)
        return fail(LLB_E_INVALID, "n_heads (%d) is not a multiple of n_kv_heads (%d)", c->n_heads,
                    c->n_kv_heads);
    if (!(c->eps >= 0.0f) || !std::isfinite(c->eps)) return fail(LLB_E_INVALID, "eps must be >= 0");
    if (!(c->rope_theta > 1.0f) || !std::isfinite(c->rope_theta))
        return fail(LLB_E_INVALID, "rope_theta must be > 1");
    if (c->max_positions <= 0) return fail(LLB_E_INVALID, "max_positions must be positive");
    if (c->wdtype != LLB_F32 && c->wdtype != LLB_BF16) return fail(LLB_E_INVALID, "unknown wdtype");
    if (c->rope_scaling != 0 && c->rope_scaling != 1) return fail(LLB_E_INVALID, "rope_scaling must be 0 or 1");
    if (c->rope_scaling == 1) {
        if (!(c->rs_factor > 0.0f) || !(c->rs_low_freq_factor > 0.0f) ||
            !(c->rs_high_freq_factor > c->rs_low_freq_factor) || c->rs_orig_max_pos <= 0)
            return fail(LLB_E_INVALID, "llama3 scaling needs factor > 0, 0 < low < high, orig > 0");
    }
    const int G = c->n_heads / c->n_kv_heads;
    if (G > 16) return fail(LLB_E_UNSUPPORTED, "n_heads / n_kv_heads = %d > 16", G);
    if (c->head_dim != 64 && c->head_dim != 128)
        return fail(LLB_E_UNSUPPORTED, "head_dim %d not in {64, 128}", c->head_dim);
    if (c->d_model % 64 != 0 || c->d_ff % 64 != 0)
        return fail(LLB_E_UNSUPPORTED, "d_model and d_ff must be multiples of 64");
    if (c->wdtype == LLB_BF16) {
        if (c->head_dim != 128) return fail(LLB_E_UNSUPPORTED, "bf16 blocks need head_dim 128");
        // the bf16 attention kernels hold a query-head group of 1, 2, 4 or 8 per KV head
        if (G != 1 && G != 2 && G != 4 && G != 8)
            return fail(LLB_E_UNSUPPORTED, "bf16 blocks need n_heads / n_kv_heads in {1, 2, 4, 8} (got %d)", G);
        if (c->d_model % 256 != 0 || c->d_ff % 256 != 0 || c->n_heads % 2 != 0)
            return fail(LLB_E_UNSUPPORTED,
                        "bf16 blocks need d_model, d_ff multiples of 256 and even n_heads");
    }
    return LLB_OK;
}

// RoPE table: omega_i = 1/theta^(2i/hd) as float32 (power in double rounded to
// float, then a float reciprocal), optional llama3 band scaling in double
// rounded to float, angle = float(pos) * omega_i in float, cos/sin of that
// angle in double rounded to float.
std::vector<float2> build_rope_table(const llb_config& c) {
    const int half = c.head_dim / 2;
    std::vector<float> inv(half);
    for (int i = 0; i < half; ++i) {
        const float p = (float)std::pow((double)c.rope_theta, 2.0 * i / c.head_dim);
        inv[i] = 1.0f / p;
    }
    if (c.rope_scaling == 1) {
        const double factor = c.rs_factor, lo = c.rs_low_freq_factor, hi = c.rs_high_freq_factor;
        const double orig = c.rs_orig_max_pos;
        const double low_wavelen = orig / lo, high_wavelen = orig / hi;
        for (int i = 0; i < half; ++i) {
            const double w = inv[i];
            const double wavelen = 2.0 * kPi / w;
            double nw;
            if (wavelen < high_wavelen) {
                nw = w;
            } else if (wavelen > low_wavelen) {
                nw = w / factor;
            } else {
                const double s = (orig / wavelen - lo) / (hi - lo);
                nw = (1.0 - s) * w / factor + s * w;
            }
            inv[i] = (float)nw;
        }
    }
    std::vector<float2> t((size_t)c.max_positions * half);
    for (int p = 0; p < c.max_positions; ++p) {
        const float fp = (float)p;
        for (int i = 0; i < half; ++i) {
            volatile float ang = fp * inv[i];  // one float multiply, no contraction
            const double a = (double)ang;
            t[(size_t)p * half + i] = make_float2((float)std::cos(a), (float)std::sin(a));
        }
    }
    return t;
}

void free_block(llb_block* b) {
    if (!b) return;
    void* ptrs[] = {b->wqkv, b->wo, b->wgu, b->wdown, b->g1, b->g2, b->rope};
    for (void* p : ptrs)
        if (p) (void)hipFree(p);
    for (hipEvent_t ev : b->events) (void)hipEventDestroy(ev);
    b->events.clear();
}

// Next stage-boundary event of a recorded call (the pool grows on demand).
hipError_t stage_event(llb_block* b, hipStream_t s) {
    if (!b->timing) return hipSuccess;
    if (b->events_used == b->events.size()) {
        hipEvent_t ev;
        hipError_t e = hipEventCreate(&ev);
        if (e != hipSuccess) return e;
        b->events.push_back(ev);
    }
    return hipEventRecord(b->events[b->events_used++], s);
}

struct WsPlan {
    size_t q = 0, o = 0, h = 0, u = 0, a1 = 0, a2 = 0, ssq1 = 0, ssq2 = 0, pos = 0, scratch = 0, total = 0;
    size_t scratch_bytes = 0;
};

// Workspace layout for one call: Q_r, O, h, u, the two RMSNorm operands (bf16
// x*g1 and h*g2) with their row sums of squares, then a scratch area (split-K
// partials of the decode projections, decode-attention partials).
WsPlan plan_ws(const llb_block* b, int B, int T, bool decode, int n_keys) {
    const llb_config& c = b->cfg;
    const size_t es = b->es;
    const size_t M = (size_t)B * T;
    WsPlan p;
    size_t off = 0;
    p.q = off; off += align_up((size_t)B * c.n_heads * T * c.head_dim * es);
    p.o = off; off += align_up(M * c.n_heads * c.head_dim * es);
    p.h = off; off += align_up(M * c.d_model * sizeof(float));
    p.u = off; off += align_up(M * c.d_ff * es);
    if (c.wdtype == LLB_BF16) {
        p.a1 = off; off += align_up(M * c.d_model * 2);
        p.a2 = off; off += align_up(M * c.d_model * 2);
        // row sums of squares of x: one, or the partials a previous block's down
        // projection wrote (one per output column tile, token rows padded to 64)
        p.ssq1 = off; off += align_up(std::max<size_t>(M, 64) * (size_t)(c.d_model / 16) * sizeof(float));
        // partial sums of h^2: one per output column tile of the O projection
        // (16 columns at the narrowest, token rows padded to 64 in decode)
        p.ssq2 = off; off += align_up(std::max<size_t>(M, 64) * (size_t)(c.d_model / 16) * sizeof(float));
    }
    size_t part = 0;
    if (decode && c.wdtype == LLB_BF16) {
        const int d = c.d_model, hq = c.n_heads * c.head_dim;
        const int nqkv = (c.n_heads + 2 * c.n_kv_heads) * c.head_dim;
        if (B <= 64) {
            const int shapes[4][2] = {{nqkv, d}, {d, hq}, {2 * c.d_ff, d}, {d, c.d_ff}};
            for (auto& s : shapes) {
                const int sp = llb::gemv_bf16_splits(B, s[0], s[1]);
                const size_t need = llb::gemv_bf16_ws_bytes(B, s[0], sp);
                if (need > part) part = need;
            }
        }
        const size_t att = llb::attn_decode_ws_bytes(B, c.n_heads, c.n_kv_heads, c.head_dim, n_keys);
        if (att > part) part = att;
    }
    if (decode) {  // per-sequence start positions of a ragged decode call
        p.pos = off;
        off += align_up((size_t)B * sizeof(int32_t));
    }
    p.scratch = off;
    p.scratch_bytes = part;
    off += align_up(part);
    p.total = off;
    return p;
}

// Picks the prefill tile configuration (see gemm_bf16.hip) of C[M,N] = A[M,K] W^T
// with epilogue kind epi, from measurements of the whole block on MI355X
// (steady clocks):
//  - long inputs (M >= 4096): 256x256 tiles; for the normalised-operand
//    projections (QKV, gate/up), the output projection with the next norm's
//    operand (70B: 1.87 against 2.03 ms on the 8-wave kernel) and long K (the
//    down projection) the interleaved kernel on 16x16x32 MFMAs with the L2
//    prefetch and spread copies, for the others the interleaved 32x32x16
//    kernel with the prefetch at large N and the 8-wave kernel otherwise; the
//    gate/up projection, whose band of A panels stays in the last-level cache
//    over 14 column blocks, prefetches W lines only (70B gate/up -2%; the
//    down projection, whose A streams from HBM, is 5% slower that way), and
//    so does the output projection with the next norm's operand (70B O
//    -1.6%);
//  - 256x192 tiles when they fill whole rounds of the 256 compute units (the
//    QKV projection on the 16x16x32 spread-copy kernel prefetching W lines
//    only, the whole A being cache-resident at these sizes (8B QKV -4%);
//    others on the interleaved 32x32x16 kernel);
//  - 256x256 tiles once they fill at least 160 compute units (gate/up on the
//    16x16x32 spread-copy kernel prefetching W lines only, 8B gate/up -3%;
//    the rest on the 8-wave kernel);
//  - 256x128 tiles (interleaved, BK 64, 3 stages; spread copies for the
//    residual epilogues, the down and output projections: 8B O -3%) from 192
//    tiles up when K is a multiple of 64; two 256x128 or 128x128 workgroups
//    per CU below that;
//  - operands past 4 GiB (beyond the interleaved kernels' 32-bit offsets): the
//    plain 8-wave or 256x128 / 128x128 kernels.
int pick_tile(int M, int N, int K, int epi) {
    const int pm = (M + 255) / 256;
    const bool scaled = epi == llb::EPI_QKV || epi == llb::EPI_SWIGLU;
    if (!llb::gemm_bf16_offsets_fit(M, N, K))  // beyond the interleaved schedules' reach
        return N % 256 == 0 ? 0 : N % 128 != 0 ? -1 : M > 128 ? 1 : 2;
    if (N % 256 == 0 && M >= 4096)
        return (epi == llb::EPI_SWIGLU || epi == llb::EPI_RESID_NORM) ? 17
               : (scaled || K >= 16384) ? 14 : N >= 32768 ? 4 : 0;
    if (N % 128 != 0) return -1;
    if (N % 192 == 0 && K % 64 == 0 && ((long)pm * (N / 192)) % 256 == 0) return epi == llb::EPI_QKV ? 18 : 6;
    if (N % 256 == 0 && (long)pm * (N / 256) >= 160) return epi == llb::EPI_SWIGLU ? 17 : 0;
    const long t128 = (long)pm * (N / 128);
    if (t128 >= 192 && K % 64 == 0) return (epi == llb::EPI_RESID || epi == llb::EPI_RESID_NORM) ? 16 : 7;
    return M > 128 ? 1 : 2;
}

int tile_for(const llb_block* b, int override_cfg, int M, int N, int K, int epi) {
    (void)b;
    return override_cfg >= 0 ? override_cfg : pick_tile(M, N, K, epi);
}

// The 256x128 interleaved configuration (spread copies) that takes over a
// projection's last, partly filled round of 256-wide tiles.
constexpr int kTailCfg = 16;

// First output column of the tail of C[M, N] = A W^T under configuration cfg:
// when 256-wide tiles fill r >= 1 whole rounds of the compute units and leave
// the next round at most half full, the columns of the whole rounds keep cfg
// and the rest run as 256x128 tiles, which fill that last round twice as
// densely at half the length per tile.  0 = no split.
int tail_split(const llb_block* b, int cfg, const llb::GemmArgs& a) {
    int bm, bn, nt;
    llb::gemm_bf16_tile(cfg, &bm, &bn, &nt);
    int tbm, tbn;
    llb::gemm_bf16_tile(kTailCfg, &tbm, &tbn, &nt);
    if (bn != 256 || bm != tbm || a.epi.kind == llb::EPI_RESID_NORM ||
        !llb::gemm_bf16_supports(kTailCfg, a.M, a.N, a.K, a.epi.kind))
        return 0;
    const long pm = (a.M + bm - 1) / bm;
    const long tiles = pm * (a.N / bn);
    const long rounds = tiles / b->num_cus, rem = tiles % b->num_cus;
    if (rounds < 1 || rem == 0 || rem > b->num_cus / 2 || (rounds * b->num_cus) % pm != 0) return 0;
    return (int)(rounds * b->num_cus / pm) * bn;
}

// Most partial sums of squares the gate/up weight-streaming kernel gathers per
// row (16 loads of 4 rows per thread).
int max_ssq_parts(int M) { return M <= 32 ? 512 : 256; }

// Decode (M <= 64) kernel of a projection C[M, N] = A W^T with epilogue epi:
// the number of weight rows per workgroup of the narrow kernel (16 or 32), or
// 0 for the 128-row split-K kernel.  Automatic choice (measured on MI355X, 8B and 70B
// decode): the narrow kernel re-reads every token row per workgroup, so it
// only pays where that operand is small, at most 32 token rows and K <= 4096
// (the 8B QKV and O projections): 32 weight rows when that still occupies 3/4
// of the CUs, else 16.  Everything else streams 128-row tiles with split-K.
// An O projection (EPI_RESID_NORM) keeps its N / rows partial sums of squares
// within what the gate/up kernel gathers.  `forced` >= 0 is the caller's
// choice; -1 is returned when it does not fit.
int decode_rows(const llb_block* b, int forced, int M, int N, int K, int epi) {
    auto fits = [&](int rw) {
        return llb::gemv_narrow_supports(M, N, K, epi, rw) &&
               (epi != llb::EPI_RESID_NORM || N / rw <= max_ssq_parts(M));
    };
    if (forced == 0) return 0;
    if (forced > 0) return fits(forced) ? forced : -1;
    if (N / 128 >= 192 || M > 32 || K > 4096) return 0;
    if (fits(32) && 4 * (N / 32) >= 3 * b->num_cus) return 32;
    if (fits(16)) return 16;
    return 0;
}

llb_status run_proj(const llb_block* b, const llb::GemmArgs& a, bool small_m, float* part,
                    int tile, bool auto_tile, hipStream_t s, const char* what, int rows = 0) {
    hipError_t e;
    if (b->cfg.wdtype == LLB_F32) {
        e = llb::gemm_f32_launch(a, s);
    } else if (small_m && rows > 0) {
        e = llb::gemv_narrow_launch(a, rows, b->num_cus, s);
    } else if (small_m) {
        const int sp = llb::gemv_bf16_splits(a.M, a.N, a.K);
        e = llb::gemv_bf16_launch(a, sp, part, s);
    } else {
        if (tile < 0) return fail(LLB_E_UNSUPPORTED, "%s: no tile fits N=%d", what, a.N);
        const int split = auto_tile ? tail_split(b, tile, a) : 0;
        if (split > 0) {
            llb::GemmArgs head = a, tail = a;
            head.n_begin = 0;
            head.n_end = split;
            tail.n_begin = split;
            tail.n_end = a.N;
            e = llb::gemm_bf16_launch(head, tile, s);
            if (e == hipSuccess) e = llb::gemm_bf16_launch(tail, kTailCfg, s);
        } else {
            e = llb::gemm_bf16_launch(a, tile, s);
        }
    }
    if (e != hipSuccess) return hip_fail(e, what);
    return LLB_OK;
}

// Blocks run back to back (a model) hand the attention RMSNorm of the next
// block to the down projection of this one: its epilogue writes, besides
// y = h + down, the next block's operand bf16(y * g1') and partial sums of y^2
// into the workspace's a1 / ssq1, which the next call (same workspace) uses
// instead of running the norm kernel.
struct NormChain {
    int in_parts;          // > 0: a1 / ssq1 already hold this block's operand and that many partials
    const float* out_gain; // non-null: also write the next block's operand with this gain
    int out_parts;         // set by run_block: partials written (0: the next block normalises itself)
};

// Most row-sum partials the decode QKV kernels gather (4 float4 loads per thread).
int qkv_max_parts(int M) { return 4 * (M <= 32 ? 32 : 16); }

// The kernel sequence of one block call over M = B*T tokens at positions
// pos0..pos0+T-1 ("Llama 3.1 70B", section "Transformer layer"):
//   h = x + Wo . Attn(RMSNorm(x)),  y = h + Wdown . SwiGLU(RMSNorm(h)).
// pos_host: per-sequence start positions (host, B entries; T = 1), or null:
// every sequence starts at pos0.  With them, pos0 is their maximum.
// check_only: run every argument check and return before anything is queued.
// events: record the stage-timing events when the handle has timing enabled
// (false: never, so that the call creates no events).
llb_status run_block(llb_block* b, const float* x, float* y, int B, int T, int pos0, void* kc,
                     void* vc, int cap, void* ws, size_t ws_bytes, hipStream_t s, bool decode,
                     const int32_t* pos_host = nullptr, NormChain* chain = nullptr,
                     bool check_only = false, bool events = true) {
    const llb_config& c = b->cfg;
    const int L = pos0 + T;
    const WsPlan p = plan_ws(b, B, T, decode, L);
    if (ws_bytes < p.total)
        return fail(LLB_E_INVALID, "workspace too small: %zu < %zu bytes", ws_bytes, p.total);
    char* w = (char*)ws;
    void* q = w + p.q;
    void* o = w + p.o;
    float* h = (float*)(w + p.h);
    void* u = w + p.u;
    void* a1 = w + p.a1;
    void* a2 = w + p.a2;
    float* ssq1 = (float*)(w + p.ssq1);
    float* ssq2 = (float*)(w + p.ssq2);
    float* part = (float*)(w + p.scratch);
    const int M = B * T;
    const int d = c.d_model, hd = c.head_dim;
    const bool bf16 = c.wdtype == LLB_BF16;
    const bool small_m = decode && M <= 64;
    const int nqkv = (c.n_heads + 2 * c.n_kv_heads) * hd;
    const int tile_qkv = tile_for(b, b->tile_qkv, M, nqkv, d, llb::EPI_QKV);
    const int tile_o = tile_for(b, b->tile_o, M, d, c.n_heads * hd, llb::EPI_RESID_NORM);
    const int tile_gu = tile_for(b, b->tile_gu, M, 2 * c.d_ff, d, llb::EPI_SWIGLU);
    const int tile_down = tile_for(b, b->tile_down, M, d, c.d_ff, llb::EPI_RESID);
    const int hq = c.n_heads * hd;
    const int rows_qkv = small_m ? decode_rows(b, b->dec_qkv, M, nqkv, d, llb::EPI_QKV) : 0;
    const int rows_o = small_m ? decode_rows(b, b->dec_o, M, d, hq, llb::EPI_RESID_NORM) : 0;
    const int rows_down = small_m ? decode_rows(b, b->dec_down, M, d, c.d_ff, llb::EPI_RESID) : 0;
    const int rows_gu = small_m ? decode_rows(b, b->dec_gu, M, 2 * c.d_ff, d, llb::EPI_SWIGLU) : 0;
    if (bf16 && small_m && (rows_qkv < 0 || rows_o < 0 || rows_gu < 0 || rows_down < 0))
        return fail(LLB_E_UNSUPPORTED, "decode kernel choice (%d, %d, %d, %d) does not fit this block",
                    b->dec_qkv, b->dec_o, b->dec_gu, b->dec_down);
    if (bf16 && !small_m) {
        // every projection's tile fits before anything is queued
        const struct { int cfg, N, K, epi; const char* what; } chk[] = {
            {tile_qkv, nqkv, d, llb::EPI_QKV, "qkv projection"},
            {tile_o, d, c.n_heads * hd, llb::EPI_RESID_NORM, "output projection"},
            {tile_gu, 2 * c.d_ff, d, llb::EPI_SWIGLU, "gate/up projection"},
            {tile_down, d, c.d_ff, llb::EPI_RESID, "down projection"}};
        for (const auto& k : chk)
            if (!llb::gemm_bf16_supports(k.cfg, M, k.N, k.K, k.epi))
                return fail(LLB_E_UNSUPPORTED, "%s: tile configuration %d does not fit N=%d K=%d", k.what,
                            k.cfg, k.N, k.K);
    }

    if (check_only) return LLB_OK;
    // stage-timing events (none when the caller asked for a call that creates nothing)
    auto mark = [&]() -> hipError_t { return events ? stage_event(b, s) : hipSuccess; };

    const int* pos_b = nullptr;
    if (pos_host) {
        // the positions travel to the workspace in kernel arguments, ahead of the
        // kernels that read them
        pos_b = (const int*)(w + p.pos);
        const hipError_t ce = llb::store_ints_launch((int*)pos_b, pos_host, B, s);
        if (ce != hipSuccess) return hip_fail(ce, "start positions");
    }

    llb::Epilogue e{};
    e.rope = b->rope;
    e.T = T; e.pos0 = pos0; e.cap = cap; e.n_heads = c.n_heads; e.n_kv = c.n_kv_heads; e.hd = hd;
    e.pos_b = pos_b;

    hipError_t te = mark();
    if (te != hipSuccess) return hip_fail(te, "stage timing");

    // 1. RMSNorm(x) . Wqkv^T, RoPE, Q -> workspace, K/V -> cache rows pos0..pos0+T-1
    llb::GemmArgs a{};
    a.W = b->wqkv; a.M = M; a.N = nqkv; a.K = d; a.eps = c.eps;
    if (bf16 && chain && chain->in_parts > 0) {
        // the previous block's down projection wrote the operand and the partials
        a.A = a1; a.ssq_in = ssq1; a.ssq_count = chain->in_parts;
    } else if (bf16 && rows_qkv > 0 && llb::gemv_narrow_norm_supports(M, nqkv, d, rows_qkv, b->num_cus)) {
        // the narrow decode kernel forms the RMSNorm itself from x and g1
        a.A = x; a.gain = b->g1; a.norm = 1;
    } else if (bf16) {
        hipError_t ne = llb::norm_rows_launch(x, b->g1, a1, ssq1, M, d, s);
        if (ne != hipSuccess) return hip_fail(ne, "attention RMSNorm");
        a.A = a1; a.ssq_in = ssq1; a.ssq_count = 1;
    } else {
        a.A = x; a.gain = b->g1; a.norm = 1;
    }
    a.epi = e; a.epi.kind = llb::EPI_QKV; a.epi.q_out = q; a.epi.k_cache = kc; a.epi.v_cache = vc;
    llb_status st = run_proj(b, a, small_m, part, tile_qkv, b->tile_qkv < 0, s, "qkv projection", rows_qkv);
    if (st != LLB_OK) return st;
    if ((te = mark()) != hipSuccess) return hip_fail(te, "stage timing");

    // 2. attention over cache rows 0..pos0+t
    llb::AttnArgs at{};
    at.q = q; at.k_cache = kc; at.v_cache = vc; at.o = o; at.B = B; at.T = T; at.pos0 = pos0;
    at.cap = cap; at.n_heads = c.n_heads; at.n_kv = c.n_kv_heads; at.hd = hd;
    at.pos_b = pos_b;
    hipError_t he;
    if (!bf16) he = llb::attn_f32_launch(at, s);
    else if (decode) he = llb::attn_decode_bf16_launch(at, part, s);
    else he = llb::attn_prefill_bf16_launch(at, s);
    if (he != hipSuccess) return hip_fail(he, "attention");
    if ((te = mark()) != hipSuccess) return hip_fail(te, "stage timing");

    // 3. h = x + O . Wo^T   (bf16: also the FFN RMSNorm's operand and row sums of h^2)
    a = llb::GemmArgs{};
    a.A = o; a.W = b->wo; a.M = M; a.N = d; a.K = c.n_heads * hd; a.eps = c.eps;
    a.epi = e; a.epi.resid = x; a.epi.out = h;
    int ssq2_count = 1;
    if (bf16) {
        a.epi.kind = llb::EPI_RESID_NORM; a.epi.gain = b->g2; a.epi.a_out = a2; a.epi.ssq_out = ssq2;
        if (!small_m) {
            if (tile_o < 0) return fail(LLB_E_UNSUPPORTED, "output projection: no tile fits N=%d", d);
            int bm, bn, nt;
            llb::gemm_bf16_tile(tile_o, &bm, &bn, &nt);
            ssq2_count = d / bn;
        } else {
            // one partial per column tile of the decode kernel
            ssq2_count = rows_o > 0 ? d / rows_o : llb::gemv_bf16_ssq_parts(d);
        }
    } else {
        a.epi.kind = llb::EPI_RESID;
    }
    st = run_proj(b, a, small_m, part, tile_o, b->tile_o < 0, s, "output projection", rows_o);
    if (st != LLB_OK) return st;
    if ((te = mark()) != hipSuccess) return hip_fail(te, "stage timing");

    // 4. u = SiLU(RMSNorm(h) . Wgate^T) * (RMSNorm(h) . Wup^T)
    a = llb::GemmArgs{};
    a.W = b->wgu; a.M = M; a.N = 2 * c.d_ff; a.K = d; a.eps = c.eps;
    if (bf16) {
        a.A = a2; a.ssq_in = ssq2; a.ssq_count = ssq2_count;
    } else {
        a.A = h; a.gain = b->g2; a.norm = 1;
    }
    a.epi = e; a.epi.kind = llb::EPI_SWIGLU; a.epi.u_out = u;
    st = run_proj(b, a, small_m, part, tile_gu, b->tile_gu < 0, s, "gate/up projection", rows_gu);
    if (st != LLB_OK) return st;
    if ((te = mark()) != hipSuccess) return hip_fail(te, "stage timing");

    // 5. y = h + u . Wdown^T
    a = llb::GemmArgs{};
    a.A = u; a.W = b->wdown; a.M = M; a.N = d; a.K = c.d_ff; a.eps = c.eps;
    a.epi = e; a.epi.kind = llb::EPI_RESID; a.epi.resid = h; a.epi.out = y;
    int out_parts = 0;
    if (bf16 && chain && chain->out_gain) {
        // the next block's RMSNorm operand too, when the down projection's
        // kernel has that epilogue and the next QKV kernel can gather the partials
        if (small_m) {
            const int parts = rows_down > 0 ? d / rows_down : llb::gemv_bf16_ssq_parts(d);
            if (parts <= qkv_max_parts(M)) out_parts = parts;
        } else if (llb::gemm_bf16_supports(tile_down, M, d, c.d_ff, llb::EPI_RESID_NORM)) {
            int bm, bn, nt;
            llb::gemm_bf16_tile(tile_down, &bm, &bn, &nt);
            out_parts = d / bn;
        }
        if (out_parts > 0) {
            a.epi.kind = llb::EPI_RESID_NORM;
            a.epi.gain = chain->out_gain; a.epi.a_out = a1; a.epi.ssq_out = ssq1;
        }
    }
    st = run_proj(b, a, small_m, part, tile_down, b->tile_down < 0, s, "down projection", rows_down);
    if (st != LLB_OK) return st;
    if (chain) chain->out_parts = out_parts;
    if ((te = mark()) != hipSuccess) return hip_fail(te, "stage timing");
    return LLB_OK;
}

// fp32 copy of a gain vector of d elements (es bytes each, on the device).
hipError_t widen_gain(const void* src, float* dst, size_t d, size_t es, hipStream_t s) {
    std::vector<unsigned char> raw(d * es);
    std::vector<float> f(d);
    hipError_t e = hipMemcpyAsync(raw.data(), src, d * es, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return e;
    for (size_t i = 0; i < d; ++i) {
        if (es == 4) {
            std::memcpy(&f[i], &raw[4 * i], 4);
        } else {
            uint16_t hbits;
            std::memcpy(&hbits, &raw[2 * i], 2);
            const uint32_t u = (uint32_t)hbits << 16;
            std::memcpy(&f[i], &u, 4);
        }
    }
    e = hipMemcpyAsync(dst, f.data(), d * 4, hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    return e;
}

}  // namespace

extern "C" {

const char* llb_last_error(void) { return g_err.c_str(); }

llb_status llb_block_create(const llb_config* cfg, const llb_weights* w, void* stream,
                            llb_block** out) {
    if (!out) return fail(LLB_E_INVALID, "out is NULL");
    *out = nullptr;
    llb_status st = check_config(cfg);
    if (st != LLB_OK) return st;
    if (!w || !w->attn_norm || !w->wq || !w->wk || !w->wv || !w->wo || !w->ffn_norm || !w->w_gate ||
        !w->w_up || !w->w_down)
        return fail(LLB_E_INVALID, "a weight pointer is NULL");
    const llb_config& c = *cfg;
    hipStream_t s = (hipStream_t)stream;

    llb_block* b = new (std::nothrow) llb_block();
    if (!b) return fail(LLB_E_NOMEM, "host allocation failed");
    b->cfg = c;
    b->es = c.wdtype == LLB_BF16 ? 2 : 4;
    b->tile_qkv = b->tile_o = b->tile_gu = b->tile_down = -1;
    b->dec_qkv = b->dec_o = b->dec_gu = b->dec_down = -1;
    b->timing = 0;
    b->events_used = 0;
    hipError_t e = hipGetDevice(&b->device);
    if (e != hipSuccess) { delete b; return hip_fail(e, "hipGetDevice"); }
    e = hipDeviceGetAttribute(&b->num_cus, hipDeviceAttributeMultiprocessorCount, b->device);
    if (e != hipSuccess || b->num_cus <= 0) {
        delete b;
        return hip_fail(e != hipSuccess ? e : hipErrorInvalidDevice, "compute unit count");
    }
    // the no-allocation entry point's scratch on this device (its own error is
    // kept and reported by that entry point)
    scratch_setup(b->device);

    const size_t es = b->es, d = c.d_model, hd = c.head_dim, dff = c.d_ff;
    const size_t nq = (size_t)c.n_heads * hd, nkv = (size_t)c.n_kv_heads * hd;
    struct { void** p; size_t n; } allocs[] = {
        {&b->wqkv, (nq + 2 * nkv) * d * es}, {&b->wo, d * nq * es}, {&b->wgu, 2 * dff * d * es},
        {&b->wdown, d * dff * es},          {(void**)&b->g1, d * 4}, {(void**)&b->g2, d * 4},
        {(void**)&b->rope, (size_t)c.max_positions * (hd / 2) * sizeof(float2)}};
    for (auto& a : allocs) {
        e = hipMalloc(a.p, a.n);
        if (e != hipSuccess) {
            free_block(b);
            delete b;
            return fail(LLB_E_NOMEM, "hipMalloc(%zu) failed: %s", a.n, hipGetErrorString(e));
        }
    }

    auto cpy = [&](void* dst, const void* src, size_t n) {
        if (e == hipSuccess) e = hipMemcpyAsync(dst, src, n, hipMemcpyDeviceToDevice, s);
    };
    cpy(b->wqkv, w->wq, nq * d * es);
    cpy((char*)b->wqkv + nq * d * es, w->wk, nkv * d * es);
    cpy((char*)b->wqkv + (nq + nkv) * d * es, w->wv, nkv * d * es);
    cpy(b->wo, w->wo, d * nq * es);
    cpy(b->wdown, w->w_down, d * dff * es);
    // gate/up interleave: 32-row groups of gate and up alternate
    if (e == hipSuccess)
        e = hipMemcpy2DAsync(b->wgu, 64 * d * es, w->w_gate, 32 * d * es, 32 * d * es, dff / 32,
                             hipMemcpyDeviceToDevice, s);
    if (e == hipSuccess)
        e = hipMemcpy2DAsync((char*)b->wgu + 32 * d * es, 64 * d * es, w->w_up, 32 * d * es,
                             32 * d * es, dff / 32, hipMemcpyDeviceToDevice, s);
    // bf16 weights go into the projections' 128 x 64 tiled layout (contiguous
    // 16 KB tiles: whole DRAM pages per pipeline stage)
    if (e == hipSuccess && c.wdtype == LLB_BF16) {
        struct { void* p; size_t n, k; } mats[] = {
            {b->wqkv, nq + 2 * nkv, d}, {b->wo, d, nq}, {b->wgu, 2 * dff, d}, {b->wdown, d, dff}};
        size_t most = 0;
        for (auto& m : mats) most = std::max(most, m.n * m.k * es);
        void* tmp = nullptr;
        e = hipMalloc(&tmp, most);
        for (auto& m : mats) {
            if (e != hipSuccess) break;
            e = hipMemcpyAsync(tmp, m.p, m.n * m.k * es, hipMemcpyDeviceToDevice, s);
            if (e == hipSuccess) e = llb::tile_weights_launch(tmp, m.p, (int)m.n, (int)m.k, s);
        }
        if (e == hipSuccess) e = hipStreamSynchronize(s);
        if (tmp) {
            const hipError_t fe = hipFree(tmp);
            if (e == hipSuccess) e = fe;
        }
    }
    // gains: widen to fp32 on the host (bf16 -> fp32 is exact)
    std::vector<unsigned char> graw(d * es);
    std::vector<float> gf(d);
    const void* gsrc[2] = {w->attn_norm, w->ffn_norm};
    float* gdst[2] = {b->g1, b->g2};
    for (int k = 0; k < 2 && e == hipSuccess; ++k) {
        e = hipMemcpyAsync(graw.data(), gsrc[k], d * es, hipMemcpyDeviceToHost, s);
        if (e == hipSuccess) e = hipStreamSynchronize(s);
        if (e != hipSuccess) break;
        for (size_t i = 0; i < d; ++i) {
            if (es == 4) {
                std::memcpy(&gf[i], &graw[4 * i], 4);
            } else {
                uint16_t hbits;
                std::memcpy(&hbits, &graw[2 * i], 2);
                uint32_t u = (uint32_t)hbits << 16;
                std::memcpy(&gf[i], &u, 4);
            }
        }
        e = hipMemcpyAsync(gdst[k], gf.data(), d * 4, hipMemcpyHostToDevice, s);
        if (e == hipSuccess) e = hipStreamSynchronize(s);
    }
    if (e == hipSuccess) {
        std::vector<float2> rope = build_rope_table(c);
        e = hipMemcpyAsync(b->rope, rope.data(), rope.size() * sizeof(float2),
                           hipMemcpyHostToDevice, s);
        if (e == hipSuccess) e = hipStreamSynchronize(s);
    }
    if (e != hipSuccess) {
        free_block(b);
        delete b;
        return hip_fail(e, "weight upload");
    }
    b->magic = kMagic;
    register_live(&Registry::blocks, b);
    *out = b;
    return LLB_OK;
}

llb_status llb_block_destroy(llb_block* b) {
    if (!b) return LLB_OK;
    if (!unregister_live(&Registry::blocks, b)) return fail(LLB_E_INVALID, "not a live block handle");
    (void)hipDeviceSynchronize();
    free_block(b);
    b->magic = 0;
    delete b;
    return LLB_OK;
}

size_t llb_block_workspace_bytes(const llb_block* b, int32_t B, int32_t T) {
    if (!handle_ok(b) || B <= 0 || T <= 0) return 0;
    size_t n = plan_ws(b, B, T, false, T).total;
    if (T == 1) {
        const size_t dn = plan_ws(b, B, 1, true, b->cfg.max_positions).total;
        if (dn > n) n = dn;
    }
    return n;
}

llb_status llb_block_workspace_layout(const llb_block* b, int32_t B, int32_t T, int32_t decode,
                                      size_t* offsets) {
    if (!handle_ok(b)) return fail(LLB_E_INVALID, "not a live block handle");
    if (!offsets) return fail(LLB_E_INVALID, "offsets is NULL");
    if (B <= 0 || T <= 0 || (decode && T != 1)) return fail(LLB_E_INVALID, "bad sizes");
    const WsPlan p = plan_ws(b, B, T, decode != 0, T);
    offsets[0] = p.q;
    offsets[1] = p.o;
    offsets[2] = p.h;
    offsets[3] = p.u;
    return LLB_OK;
}

static llb_status check_call(const llb_block* b, const void* x, const void* y, int B, int T,
                             const void* kc, const void* vc, int cap, const void* ws) {
    if (!handle_ok(b)) return fail(LLB_E_INVALID, "not a live block handle");
    if (!x || !y || !kc || !vc || !ws) return fail(LLB_E_INVALID, "a buffer pointer is NULL");
    if (B <= 0 || T <= 0) return fail(LLB_E_INVALID, "B and T must be positive");
    if (cap <= 0) return fail(LLB_E_INVALID, "cache_cap must be positive");
    return LLB_OK;
}

llb_status llb_block_prefill(llb_block* b, const float* x, float* y, int32_t B, int32_t T,
                             void* k_cache, void* v_cache, int32_t cache_cap, void* ws,
                             size_t ws_bytes, void* stream) {
    llb_status st = check_call(b, x, y, B, T, k_cache, v_cache, cache_cap, ws);
    if (st != LLB_OK) return st;
    if (T > cache_cap) return fail(LLB_E_CAPACITY, "T=%d exceeds cache_cap=%d", T, cache_cap);
    if (T > b->cfg.max_positions)
        return fail(LLB_E_CAPACITY, "T=%d exceeds max_positions=%d", T, b->cfg.max_positions);
    return run_block(b, x, y, B, T, 0, k_cache, v_cache, cache_cap, ws, ws_bytes,
                     (hipStream_t)stream, false);
}

llb_status llb_block_prefill_at(llb_block* b, const float* x, float* y, int32_t B, int32_t T,
                                int32_t start_pos, void* k_cache, void* v_cache, int32_t cache_cap,
                                void* ws, size_t ws_bytes, void* stream) {
    llb_status st = check_call(b, x, y, B, T, k_cache, v_cache, cache_cap, ws);
    if (st != LLB_OK) return st;
    if (start_pos < 0) return fail(LLB_E_INVALID, "start_pos must be >= 0");
    if ((long)start_pos + T > cache_cap)
        return fail(LLB_E_CAPACITY, "start_pos+T=%ld exceeds cache_cap=%d", (long)start_pos + T, cache_cap);
    if ((long)start_pos + T > b->cfg.max_positions)
        return fail(LLB_E_CAPACITY, "start_pos+T=%ld exceeds max_positions=%d", (long)start_pos + T,
                    b->cfg.max_positions);
    return run_block(b, x, y, B, T, start_pos, k_cache, v_cache, cache_cap, ws, ws_bytes,
                     (hipStream_t)stream, false);
}

llb_status llb_block_decode(llb_block* b, const float* x, float* y, int32_t B, int32_t start_pos,
                            void* k_cache, void* v_cache, int32_t cache_cap, void* ws,
                            size_t ws_bytes, void* stream) {
    llb_status st = check_call(b, x, y, B, 1, k_cache, v_cache, cache_cap, ws);
    if (st != LLB_OK) return st;
    if (start_pos < 0) return fail(LLB_E_INVALID, "start_pos must be >= 0");
    if (start_pos + 1 > cache_cap)
        return fail(LLB_E_CAPACITY, "start_pos+1=%d exceeds cache_cap=%d", start_pos + 1, cache_cap);
    if (start_pos >= b->cfg.max_positions)
        return fail(LLB_E_CAPACITY, "start_pos=%d >= max_positions=%d", start_pos,
                    b->cfg.max_positions);
    return run_block(b, x, y, B, 1, start_pos, k_cache, v_cache, cache_cap, ws, ws_bytes,
                     (hipStream_t)stream, true);
}

llb_status llb_block_decode_ragged(llb_block* b, const float* x, float* y, int32_t B,
                                   const int32_t* start_pos, void* k_cache, void* v_cache,
                                   int32_t cache_cap, void* ws, size_t ws_bytes, void* stream) {
    llb_status st = check_call(b, x, y, B, 1, k_cache, v_cache, cache_cap, ws);
    if (st != LLB_OK) return st;
    if (!start_pos) return fail(LLB_E_INVALID, "start_pos is NULL");
    int max_pos = 0;
    for (int i = 0; i < B; ++i) {
        const int p = start_pos[i];
        if (p < 0) return fail(LLB_E_INVALID, "start_pos[%d]=%d must be >= 0", i, p);
        if (p + 1 > cache_cap)
            return fail(LLB_E_CAPACITY, "start_pos[%d]+1=%d exceeds cache_cap=%d", i, p + 1, cache_cap);
        if (p >= b->cfg.max_positions)
            return fail(LLB_E_CAPACITY, "start_pos[%d]=%d >= max_positions=%d", i, p, b->cfg.max_positions);
        max_pos = std::max(max_pos, p);
    }
    return run_block(b, x, y, B, 1, max_pos, k_cache, v_cache, cache_cap, ws, ws_bytes,
                     (hipStream_t)stream, true, start_pos);
}

llb_status llb_block_decode_noalloc(llb_block* b, const float* x, float* y, int32_t B, int32_t start_pos,
                                    void* k_cache, void* v_cache, int32_t cache_cap, void* stream) {
    if (!handle_ok(b)) return fail(LLB_E_INVALID, "not a live block handle");
    if (!x || !y || !k_cache || !v_cache) return fail(LLB_E_INVALID, "a buffer pointer is NULL");
    if (B <= 0) return fail(LLB_E_INVALID, "B must be positive");
    if (cache_cap <= 0) return fail(LLB_E_INVALID, "cache_cap must be positive");
    if (start_pos < 0) return fail(LLB_E_INVALID, "start_pos must be >= 0");
    if (start_pos + 1 > cache_cap)
        return fail(LLB_E_CAPACITY, "start_pos+1=%d exceeds cache_cap=%d", start_pos + 1, cache_cap);
    if (start_pos >= b->cfg.max_positions)
        return fail(LLB_E_CAPACITY, "start_pos=%d >= max_positions=%d", start_pos, b->cfg.max_positions);
    const size_t need = plan_ws(b, B, 1, true, start_pos + 1).total;
    if (need > kScratchBytes)
        return fail(LLB_E_CAPACITY,
                    "this call needs %zu bytes of scratch; the static scratch holds %zu (use "
                    "llb_block_decode with a workspace of llb_block_workspace_bytes bytes)",
                    need, kScratchBytes);
    hipError_t se;
    void* ws = scratch_ptr(b->device, &se);
    if (!ws) return hip_fail(se, "static scratch lookup");
    return run_block(b, x, y, B, 1, start_pos, k_cache, v_cache, cache_cap, ws, kScratchBytes,
                     (hipStream_t)stream, true, nullptr, nullptr, false, /*events=*/false);
}

llb_status llb_kv_append(const llb_block* b, void* k_cache, void* v_cache, int32_t B,
                         int32_t cache_cap, int32_t start_pos, int32_t n_new, const void* k_new,
                         const void* v_new, void* stream) {
    if (!handle_ok(b)) return fail(LLB_E_INVALID, "not a live block handle");
    if (!k_cache || !v_cache || !k_new || !v_new) return fail(LLB_E_INVALID, "a buffer pointer is NULL");
    if (B <= 0 || n_new < 0 || start_pos < 0 || cache_cap <= 0)
        return fail(LLB_E_INVALID, "bad sizes");
    if ((long)start_pos + n_new > cache_cap)
        return fail(LLB_E_CAPACITY, "start_pos+n_new=%ld exceeds cache_cap=%d",
                    (long)start_pos + n_new, cache_cap);
    hipError_t e = llb::kv_append_launch(k_cache, v_cache, k_new, v_new, B, b->cfg.n_kv_heads,
                                         cache_cap, start_pos, n_new, b->cfg.head_dim, b->es,
                                         (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "kv_append");
    return LLB_OK;
}

llb_status llb_attention_prefill(const llb_block* b, const void* q, const void* k_cache,
                                 const void* v_cache, void* o, int32_t B, int32_t T,
                                 int32_t start_pos, int32_t cache_cap, void* stream) {
    if (!handle_ok(b)) return fail(LLB_E_INVALID, "not a live block handle");
    if (!q || !k_cache || !v_cache || !o) return fail(LLB_E_INVALID, "a buffer pointer is NULL");
    if (B <= 0 || T <= 0 || start_pos < 0 || cache_cap <= 0) return fail(LLB_E_INVALID, "bad sizes");
    if ((long)start_pos + T > cache_cap)
        return fail(LLB_E_CAPACITY, "start_pos+T exceeds cache_cap");
    const llb_config& c = b->cfg;
    llb::AttnArgs at{};
    at.q = q; at.k_cache = k_cache; at.v_cache = v_cache; at.o = o; at.B = B; at.T = T;
    at.pos0 = start_pos; at.cap = cache_cap; at.n_heads = c.n_heads; at.n_kv = c.n_kv_heads;
    at.hd = c.head_dim;
    hipError_t e = c.wdtype == LLB_F32 ? llb::attn_f32_launch(at, (hipStream_t)stream)
                                       : llb::attn_prefill_bf16_launch(at, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "attention prefill");
    return LLB_OK;
}

size_t llb_attention_workspace_bytes(const llb_block* b, int32_t B, int32_t n_keys) {
    if (!handle_ok(b) || B <= 0 || n_keys <= 0) return 0;
    const llb_config& c = b->cfg;
    // partials of the split form, then B start positions
    const size_t pos = align_up((size_t)B * sizeof(int32_t));
    if (c.wdtype == LLB_F32) return 256 + pos;
    return align_up(llb::attn_decode_ws_bytes(B, c.n_heads, c.n_kv_heads, c.head_dim, n_keys)) + pos;
}

llb_status llb_attention_decode(const llb_block* b, const void* q, const void* k_cache,
                                const void* v_cache, void* o, int32_t B, int32_t start_pos,
                                int32_t cache_cap, void* ws, size_t ws_bytes, void* stream) {
    if (!handle_ok(b)) return fail(LLB_E_INVALID, "not a live block handle");
    if (!q || !k_cache || !v_cache || !o || !ws) return fail(LLB_E_INVALID, "a buffer pointer is NULL");
    if (B <= 0 || start_pos < 0 || cache_cap <= 0) return fail(LLB_E_INVALID, "bad sizes");
    if (start_pos + 1 > cache_cap) return fail(LLB_E_CAPACITY, "start_pos+1 exceeds cache_cap");
    const size_t need = llb_attention_workspace_bytes(b, B, start_pos + 1);
    if (ws_bytes < need) return fail(LLB_E_INVALID, "workspace too small: %zu < %zu", ws_bytes, need);
    const llb_config& c = b->cfg;
    llb::AttnArgs at{};
    at.q = q; at.k_cache = k_cache; at.v_cache = v_cache; at.o = o; at.B = B; at.T = 1;
    at.pos0 = start_pos; at.cap = cache_cap; at.n_heads = c.n_heads; at.n_kv = c.n_kv_heads;
    at.hd = c.head_dim;
    hipError_t e = c.wdtype == LLB_F32
                       ? llb::attn_f32_launch(at, (hipStream_t)stream)
                       : llb::attn_decode_bf16_launch(at, (float*)ws, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "attention decode");
    return LLB_OK;
}

llb_status llb_probe_hbm_read(const void* src, size_t bytes, int32_t n_workgroups, void* sink, void* stream) {
    if (!src || !sink) return fail(LLB_E_INVALID, "a buffer pointer is NULL");
    if (bytes == 0 || bytes % 16 != 0 || n_workgroups <= 0)
        return fail(LLB_E_INVALID, "bytes must be a positive multiple of 16 and n_workgroups positive");
    const hipError_t e = llb::probe_read_launch(src, bytes, (uint32_t*)sink, n_workgroups, (hipStream_t)stream);
    return e == hipSuccess ? LLB_OK : hip_fail(e, "read probe");
}

llb_status llb_probe_hbm_copy(void* dst, const void* src, size_t bytes, int32_t n_workgroups, void* stream) {
    if (!src || !dst) return fail(LLB_E_INVALID, "a buffer pointer is NULL");
    if (bytes == 0 || bytes % 16 != 0 || n_workgroups <= 0)
        return fail(LLB_E_INVALID, "bytes must be a positive multiple of 16 and n_workgroups positive");
    const hipError_t e = llb::probe_copy_launch(dst, src, bytes, n_workgroups, (hipStream_t)stream);
    return e == hipSuccess ? LLB_OK : hip_fail(e, "copy probe");
}

llb_status llb_probe_mfma_bf16(int32_t n_workgroups, int32_t iters, void* sink, void* stream) {
    if (!sink) return fail(LLB_E_INVALID, "sink is NULL");
    if (n_workgroups <= 0 || iters <= 0) return fail(LLB_E_INVALID, "n_workgroups and iters must be positive");
    const hipError_t e = llb::probe_mfma_launch((float*)sink, n_workgroups, iters, (hipStream_t)stream);
    return e == hipSuccess ? LLB_OK : hip_fail(e, "MFMA probe");
}

llb_status llb_attention_decode_ragged(const llb_block* b, const void* q, const void* k_cache,
                                       const void* v_cache, void* o, int32_t B, const int32_t* start_pos,
                                       int32_t cache_cap, void* ws, size_t ws_bytes, void* stream) {
    if (!handle_ok(b)) return fail(LLB_E_INVALID, "not a live block handle");
    if (!q || !k_cache || !v_cache || !o || !ws || !start_pos)
        return fail(LLB_E_INVALID, "a buffer pointer is NULL");
    if (B <= 0 || cache_cap <= 0) return fail(LLB_E_INVALID, "bad sizes");
    int max_pos = 0;
    for (int i = 0; i < B; ++i) {
        if (start_pos[i] < 0) return fail(LLB_E_INVALID, "start_pos[%d]=%d must be >= 0", i, start_pos[i]);
        if (start_pos[i] + 1 > cache_cap)
            return fail(LLB_E_CAPACITY, "start_pos[%d]+1=%d exceeds cache_cap=%d", i, start_pos[i] + 1, cache_cap);
        max_pos = std::max(max_pos, start_pos[i]);
    }
    const size_t need = llb_attention_workspace_bytes(b, B, max_pos + 1);
    if (ws_bytes < need) return fail(LLB_E_INVALID, "workspace too small: %zu < %zu", ws_bytes, need);
    const llb_config& c = b->cfg;
    hipStream_t s = (hipStream_t)stream;
    llb::AttnArgs at{};
    at.q = q; at.k_cache = k_cache; at.v_cache = v_cache; at.o = o; at.B = B; at.T = 1;
    at.pos0 = max_pos; at.cap = cache_cap; at.n_heads = c.n_heads; at.n_kv = c.n_kv_heads;
    at.hd = c.head_dim;
    // the positions travel to the end of the workspace in kernel arguments
    int* pos_dev = (int*)((char*)ws + need - align_up((size_t)B * sizeof(int32_t)));
    hipError_t e = llb::store_ints_launch(pos_dev, start_pos, B, s);
    if (e != hipSuccess) return hip_fail(e, "start positions");
    at.pos_b = pos_dev;
    e = c.wdtype == LLB_F32 ? llb::attn_f32_launch(at, s) : llb::attn_decode_bf16_launch(at, (float*)ws, s);
    if (e != hipSuccess) return hip_fail(e, "attention decode");
    return LLB_OK;
}

int32_t llb_gemm_num_tiles(void) { return llb::gemm_bf16_num_tile_cfgs(); }

llb_status llb_gemm_tile_info(int32_t cfg, int32_t* bm, int32_t* bn) {
    if (cfg < 0 || cfg >= llb::gemm_bf16_num_tile_cfgs()) return fail(LLB_E_INVALID, "no tile configuration %d", cfg);
    if (!bm || !bn) return fail(LLB_E_INVALID, "output pointer is NULL");
    int m, n, t;
    llb::gemm_bf16_tile(cfg, &m, &n, &t);
    *bm = m;
    *bn = n;
    return LLB_OK;
}

llb_status llb_block_set_tiles(llb_block* b, int32_t qkv, int32_t o, int32_t gate_up, int32_t down) {
    if (!handle_ok(b)) return fail(LLB_E_INVALID, "not a live block handle");
    const int n = llb::gemm_bf16_num_tile_cfgs();
    for (int32_t v : {qkv, o, gate_up, down})
        if (v < -1 || v >= n) return fail(LLB_E_INVALID, "tile configuration %d outside [-1, %d)", v, n);
    b->tile_qkv = qkv;
    b->tile_o = o;
    b->tile_gu = gate_up;
    b->tile_down = down;
    return LLB_OK;
}

llb_status llb_block_set_decode_kernels(llb_block* b, int32_t qkv, int32_t o, int32_t gate_up,
                                        int32_t down) {
    if (!handle_ok(b)) return fail(LLB_E_INVALID, "not a live block handle");
    for (int32_t v : {qkv, o, down})
        if (v != -1 && v != 0 && v != 16 && v != 32)
            return fail(LLB_E_INVALID, "decode kernel choice %d not in {-1, 0, 16, 32}", v);
    if (gate_up != -1 && gate_up != 0)
        return fail(LLB_E_INVALID, "gate/up decode kernel choice %d not in {-1, 0}", gate_up);
    b->dec_qkv = qkv;
    b->dec_o = o;
    b->dec_gu = gate_up;
    b->dec_down = down;
    return LLB_OK;
}

llb_status llb_block_set_stage_timing(llb_block* b, int32_t enable) {
    if (!handle_ok(b)) return fail(LLB_E_INVALID, "not a live block handle");
    b->timing = enable ? 1 : 0;
    return LLB_OK;
}

llb_status llb_block_stage_times(llb_block* b, float* ms, int32_t* n_calls) {
    if (!handle_ok(b)) return fail(LLB_E_INVALID, "not a live block handle");
    if (!ms || !n_calls) return fail(LLB_E_INVALID, "output pointer is NULL");
    for (int i = 0; i < 5; ++i) ms[i] = 0.f;
    const size_t calls = b->events_used / 6;
    if (calls > 0) {
        hipError_t e = hipEventSynchronize(b->events[b->events_used - 1]);
        if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
        for (size_t c = 0; c < calls; ++c)
            for (int i = 0; i < 5; ++i) {
                float t = 0.f;
                e = hipEventElapsedTime(&t, b->events[6 * c + i], b->events[6 * c + i + 1]);
                if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
                ms[i] += t;
            }
    }
    *n_calls = (int32_t)calls;
    b->events_used = 0;
    return LLB_OK;
}


// ---- model: embedding, n_layers blocks, final RMSNorm, LM head ---------------

struct llb_model {
    uint32_t magic;
    llb_config cfg;
    int n_layers, vocab;
    std::vector<llb_block*> layers;
    void* embed;   // [vocab, d] bf16, row-major
    float* gain;   // [d] fp32
    void* head;    // [vocab, d] bf16, 128 x 64 tiled layout
};

static constexpr uint32_t kModelMagic = 0x4c4c4d44u;

static bool model_ok(const llb_model* m) {
    return m != nullptr && is_live(&Registry::models, m) && m->magic == kModelMagic;
}

static void free_model(llb_model* m) {
    for (llb_block* b : m->layers) llb_block_destroy(b);
    m->layers.clear();
    if (m->embed) (void)hipFree(m->embed);
    if (m->gain) (void)hipFree(m->gain);
    if (m->head) (void)hipFree(m->head);
    m->embed = m->head = nullptr;
    m->gain = nullptr;
}

llb_status llb_model_create(const llb_config* cfg, int32_t n_layers, int32_t vocab, const void* embed,
                            const llb_weights* layers, const void* final_norm, const void* lm_head,
                            void* stream, llb_model** out) {
    if (!out) return fail(LLB_E_INVALID, "out is NULL");
    *out = nullptr;
    llb_status st = check_config(cfg);
    if (st != LLB_OK) return st;
    if (cfg->wdtype != LLB_BF16) return fail(LLB_E_UNSUPPORTED, "models need bf16 weights");
    if (n_layers < 0) return fail(LLB_E_INVALID, "n_layers must be >= 0");
    if (vocab <= 0 || vocab % 128 != 0) return fail(LLB_E_UNSUPPORTED, "vocab %d must be a positive multiple of 128", vocab);
    if (!embed || !final_norm || !lm_head || (n_layers > 0 && !layers))
        return fail(LLB_E_INVALID, "a weight pointer is NULL");
    hipStream_t s = (hipStream_t)stream;
    llb_model* m = new (std::nothrow) llb_model();
    if (!m) return fail(LLB_E_NOMEM, "host allocation failed");
    m->cfg = *cfg;
    m->n_layers = n_layers;
    m->vocab = vocab;
    for (int l = 0; l < n_layers; ++l) {
        llb_block* b = nullptr;
        st = llb_block_create(cfg, &layers[l], stream, &b);
        if (st != LLB_OK) {
            free_model(m);
            delete m;
            return st;
        }
        m->layers.push_back(b);
    }
    const size_t d = cfg->d_model, V = vocab, mat = V * d * 2;
    hipError_t e = hipMalloc(&m->embed, mat);
    if (e == hipSuccess) e = hipMalloc(&m->head, mat);
    if (e == hipSuccess) e = hipMalloc((void**)&m->gain, d * 4);
    if (e != hipSuccess) {
        free_model(m);
        delete m;
        return fail(LLB_E_NOMEM, "hipMalloc of the embedding / head failed: %s", hipGetErrorString(e));
    }
    e = hipMemcpyAsync(m->embed, embed, mat, hipMemcpyDeviceToDevice, s);
    if (e == hipSuccess) e = llb::tile_weights_launch(lm_head, m->head, (int)V, (int)d, s);
    if (e == hipSuccess) e = widen_gain(final_norm, m->gain, d, 2, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) {
        free_model(m);
        delete m;
        return hip_fail(e, "model weight upload");
    }
    m->magic = kModelMagic;
    register_live(&Registry::models, m);
    *out = m;
    return LLB_OK;
}

llb_status llb_model_destroy(llb_model* m) {
    if (!m) return LLB_OK;
    if (!unregister_live(&Registry::models, m)) return fail(LLB_E_INVALID, "not a live model handle");
    (void)hipDeviceSynchronize();
    free_model(m);
    m->magic = 0;
    delete m;
    return LLB_OK;
}

namespace {
struct ModelWs {
    size_t x = 0, blk = 0, blk_bytes = 0, xl = 0, a = 0, ssq = 0, scratch = 0, scratch_bytes = 0, total = 0;
};
ModelWs plan_model_ws(const llb_model* m, int B, int T, bool last_only) {
    ModelWs p;
    const size_t d = m->cfg.d_model;
    const int M = B * T, R = (last_only && T > 1) ? B : M;
    size_t off = 0;
    p.x = off; off += align_up((size_t)M * d * 4);
    p.blk_bytes = m->n_layers > 0 ? llb_block_workspace_bytes(m->layers[0], B, T) : 0;
    p.blk = off; off += align_up(p.blk_bytes);
    if (R != M) { p.xl = off; off += align_up((size_t)R * d * 4); }
    p.a = off; off += align_up((size_t)R * d * 2);
    p.ssq = off; off += align_up((size_t)R * 4);
    if (R <= 64) {
        const int sp = llb::gemv_bf16_splits(R, m->vocab, (int)d);
        p.scratch_bytes = llb::gemv_bf16_ws_bytes(R, m->vocab, sp);
    }
    p.scratch = off; off += align_up(p.scratch_bytes);
    p.total = off;
    return p;
}
}  // namespace

size_t llb_model_workspace_bytes(const llb_model* m, int32_t B, int32_t T, int32_t last_only) {
    if (!model_ok(m) || B <= 0 || T <= 0) return 0;
    return plan_model_ws(m, B, T, last_only != 0).total;
}

llb_status llb_model_forward(llb_model* m, const int32_t* tokens, int32_t B, int32_t T, int32_t start_pos,
                             void* const* k_caches, void* const* v_caches, int32_t cache_cap,
                             int32_t last_only, float* logits, void* ws, size_t ws_bytes, void* stream) {
    if (!model_ok(m)) return fail(LLB_E_INVALID, "not a live model handle");
    if (!tokens || !logits || !ws) return fail(LLB_E_INVALID, "a buffer pointer is NULL");
    if (B <= 0 || T <= 0) return fail(LLB_E_INVALID, "B and T must be positive");
    if (start_pos < 0) return fail(LLB_E_INVALID, "start_pos must be >= 0");
    if (m->n_layers > 0) {
        if (!k_caches || !v_caches) return fail(LLB_E_INVALID, "cache arrays are NULL");
        for (int l = 0; l < m->n_layers; ++l)
            if (!k_caches[l] || !v_caches[l]) return fail(LLB_E_INVALID, "cache of layer %d is NULL", l);
        if ((long)start_pos + T > cache_cap)
            return fail(LLB_E_CAPACITY, "start_pos+T=%ld exceeds cache_cap=%d", (long)start_pos + T, cache_cap);
        if ((long)start_pos + T > m->cfg.max_positions)
            return fail(LLB_E_CAPACITY, "start_pos+T=%ld exceeds max_positions=%d", (long)start_pos + T,
                        m->cfg.max_positions);
    }
    const bool lo = last_only != 0;
    const ModelWs p = plan_model_ws(m, B, T, lo);
    if (ws_bytes < p.total) return fail(LLB_E_INVALID, "workspace too small: %zu < %zu bytes", ws_bytes, p.total);
    const int d = m->cfg.d_model, M = B * T;
    const int R = (lo && T > 1) ? B : M;  // rows the LM head scores
    // the head's kernel choice, checked before anything is queued
    const int head_tile = R <= 64 ? -1 : pick_tile(R, m->vocab, d, llb::EPI_LOGITS);
    if (R > 64 && !llb::gemm_bf16_supports(head_tile, R, m->vocab, d, llb::EPI_LOGITS))
        return fail(LLB_E_UNSUPPORTED, "LM head: no tile fits vocab=%d", m->vocab);
    hipStream_t s = (hipStream_t)stream;
    char* w = (char*)ws;
    float* x = (float*)(w + p.x);
    if (m->n_layers > 0) {
        NormChain ch{0, m->n_layers > 1 ? m->layers[1]->g1 : nullptr, 0};
        const llb_status st = run_block(m->layers[0], x, x, B, T, start_pos, k_caches[0], v_caches[0],
                                        cache_cap, w + p.blk, p.blk_bytes, s, T == 1, nullptr, &ch, true);
        if (st != LLB_OK) return st;
    }
    hipError_t e = llb::embed_launch(tokens, m->embed, x, M, d, m->vocab, s);
    if (e != hipSuccess) return hip_fail(e, "embedding");
    // the blocks, in place on x, each handing the next one its attention RMSNorm
    // (positions and buffers were checked above; every layer has the shape and
    // kernel choices of layer 0, whose call is checked before anything is queued)
    int parts = 0;
    for (int l = 0; l < m->n_layers; ++l) {
        NormChain ch{parts, l + 1 < m->n_layers ? m->layers[l + 1]->g1 : nullptr, 0};
        const llb_status st = run_block(m->layers[l], x, x, B, T, start_pos, k_caches[l], v_caches[l],
                                        cache_cap, w + p.blk, p.blk_bytes, s, T == 1, nullptr, &ch);
        if (st != LLB_OK) return st;
        parts = ch.out_parts;
    }
    const float* src = x;
    if (R != M) {
        e = llb::last_rows_launch(x, (float*)(w + p.xl), B, T, d, s);
        if (e != hipSuccess) return hip_fail(e, "last rows");
        src = (const float*)(w + p.xl);
    }
    // final RMSNorm operand (bf16 x * g and fp32 sum of squares), then the head
    // with the row's 1/rms in its epilogue
    void* a = w + p.a;
    float* ssq = (float*)(w + p.ssq);
    e = llb::norm_rows_launch(src, m->gain, a, ssq, R, d, s);
    if (e != hipSuccess) return hip_fail(e, "final RMSNorm");
    llb::GemmArgs g{};
    g.A = a; g.W = m->head; g.M = R; g.N = m->vocab; g.K = d; g.eps = m->cfg.eps;
    g.ssq_in = ssq; g.ssq_count = 1;
    g.epi.kind = llb::EPI_LOGITS; g.epi.out = logits;
    if (R <= 64) {
        e = llb::gemv_bf16_launch(g, llb::gemv_bf16_splits(R, m->vocab, d), (float*)(w + p.scratch), s);
    } else {
        e = llb::gemm_bf16_launch(g, head_tile, s);
    }
    if (e != hipSuccess) return hip_fail(e, "LM head");
    return LLB_OK;
}

}  // extern "C"
