"""Benchmark of the Llama-3 block library on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--warmup-seconds S] [--no-cpu-baseline] [--no-others]

One step is one llb_block_prefill call of the Llama-3.1-70B block on B=1 x
T=16384 tokens with llama3-scaled RoPE (RMSNorm + QKV + RoPE + cache write,
causal GQA attention, O projection + residual, RMSNorm + gate/up + SiLU.up,
down projection + residual), inputs resident in HBM: the largest of the
workloads that fit one GPU.  Prints ONE JSON line.  Besides the headline
number it reports:
  * roofline: the dominant kernel of the step (the gate/up projection), its
    algorithmic FLOPs per launch over its average launch time, measured with
    HIP events on the launch stream over the timed region, against the nominal
    bf16 MFMA peak and against the peak measured on this GPU in the same run;
  * measured_peaks: HBM read and copy rates and the bf16 MFMA rate of this GPU,
    from the library's probe kernels;
  * step_ms_p10 / p50 / p90: the distribution of single-step times;
  * cpu_baseline: the fp64 CPU oracle timed on the host on a bounded sample of
    the same workload (its first 1024 tokens: by causality exactly a 1024-token
    prefill of the same block);
  * workloads: the 8B prefill (B=1, T=2048), 8B decode (B=32, P=1000), 70B
    decode (B=64, P=4096), 8B ragged decode (B=32, start positions spread over
    0..2000) and 8B chunked prefill (B=1, T=2048 at start 2048), each timed the
    same way (decode with two weight and cache sets used alternately, so that
    the 256 MB last-level cache cannot hold the working set between steps),
    each with per-stage times, step percentiles and a roofline block for its
    own dominant kernel;
  * model_workloads: the whole Llama-3.1-8B model (embedding, 32 blocks, final
    RMSNorm, LM head over 128256 ids) on 32-sequence decode (P=1000) and on a
    2048-token prefill (last-position logits).
Inputs are seeded synthetic tensors with the workload's shapes and
distributions; nothing is read from disk.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "Llama-3 block tok/s; decode HBM GB/s and prefill MFMA TFLOP/s vs peak"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
HEADLINE = "70b_bf16_prefill"
OTHERS = ("8b_bf16_prefill", "8b_bf16_decode", "70b_bf16_decode", "8b_bf16_ragged_decode",
          "8b_bf16_chunked_prefill")

# The kernel(s) of each stage, by mode (bf16 blocks; the launch shapes the
# library picks for the workloads above).
STAGE_KERNELS = {
    "prefill": {
        "qkv": "gemm_bf16_kernel (QKV projection: RMSNorm row scale, RoPE, cache write)",
        "attention": "attn_prefill_kernel (causal GQA flash attention)",
        "o_proj": "gemm_bf16_kernel (O projection + residual + FFN RMSNorm operand)",
        "gate_up": "gemm_bf16_kernel (gate/up projection with RMSNorm row scale and SiLU.up)",
        "down": "gemm_bf16_kernel (down projection + residual)",
    },
    "decode": {
        "qkv": "gemv_narrow_kernel / gemv_bf16_kernel (QKV weight streaming, RoPE, cache write)",
        "attention": "attn_decode_fused_kernel (one workgroup per sequence and KV head)",
        "o_proj": "gemv_narrow_kernel / gemv_bf16_kernel (O weight streaming + residual)",
        "gate_up": "gemv_bf16_kernel (gate/up weight streaming, SiLU.up)",
        "down": "gemv_bf16_kernel + gemv_reduce_kernel (down weight streaming, split-K, residual)",
    },
}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ------------------------------------------------------------- algorithmic work
def stage_flops(wl):
    """Algorithmic FLOPs per stage: 2 per multiply-add of each projection; attention
    4*hd*n_heads per visible (query, key) pair (Q.K and P.V), causal pairs only."""
    import workloads
    s = wl.shape
    M = wl.B * wl.T
    d, hd, f = s.d_model, s.head_dim, s.d_ff
    if wl.mode == "prefill":
        pairs = wl.B * (wl.T * wl.P + wl.T * (wl.T + 1) // 2)
    elif wl.ragged:
        pairs = sum(p + 1 for p in workloads.ragged_positions(wl))
    else:
        pairs = wl.B * (wl.P + 1)
    return {
        "qkv": 2 * M * d * (s.n_heads + 2 * s.n_kv_heads) * hd,
        "attention": 4 * hd * s.n_heads * pairs,
        "o_proj": 2 * M * s.n_heads * hd * d,
        "gate_up": 2 * M * d * 2 * f,
        "down": 2 * M * f * d,
    }


def stage_bytes(wl):
    """Algorithmic HBM bytes per stage: each weight once, norm gains, KV rows read
    (P cached rows) and written (new rows), x read and y written."""
    import workloads
    s = wl.shape
    es = 2 if s.dtype == "bf16" else 4
    M = wl.B * wl.T
    d, hd, f = s.d_model, s.head_dim, s.d_ff
    kv_row = s.n_kv_heads * hd * es
    return {
        "qkv": (s.n_heads + 2 * s.n_kv_heads) * hd * d * es + d * es + M * d * 4 + 2 * M * kv_row,
        "attention": 2 * kv_row * (sum(workloads.ragged_positions(wl)) if wl.ragged else wl.B * wl.P),
        "o_proj": d * s.n_heads * hd * es,
        "gate_up": 2 * f * d * es + d * es,
        "down": d * f * es + M * d * 4,
    }


# ------------------------------------------------------------- measured peaks
def measure_peaks():
    """HBM read / copy rates and the bf16 MFMA rate of this GPU, from the
    library's probe kernels, each after a warm-up of at least 0.3 s of the same
    kernel (the clocks settle under load)."""
    import torch
    from dense_decoder_only_amd import llb

    cus = torch.cuda.get_device_properties(0).multi_processor_count
    stream = torch.cuda.current_stream()
    out = {"compute_units": cus}

    def timed(fn, reps, warm_s=0.3):
        t_end = time.perf_counter() + warm_s
        while time.perf_counter() < t_end:
            fn()
            torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        ev[0].record(stream)
        for i in range(reps):
            fn()
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        ts = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(reps))
        return ts[len(ts) // 2]

    # The best of a few launch shapes is the peak: the rate this GPU sustains.
    nbytes = 1 << 30     # 1 GiB: four times the last-level cache
    src = torch.empty(nbytes // 4, dtype=torch.int32, device="cuda").random_()
    dst = torch.empty_like(src)
    sink = torch.empty(16 * cus, dtype=torch.int32, device="cuda")
    read, copy = {}, {}
    for per_cu in (4, 8, 16):
        n_wg = per_cu * cus
        ms = timed(lambda: llb.llb_probe_hbm_read(src, sink, n_wg), 20)
        read[n_wg] = round(nbytes / (ms * 1e-3) / 1e9, 1)
        ms = timed(lambda: llb.llb_probe_hbm_copy(dst, src, n_wg), 20)
        copy[n_wg] = round(2 * nbytes / (ms * 1e-3) / 1e9, 1)
    out["hbm_read_gbs"] = max(read.values())
    out["hbm_copy_gbs"] = max(copy.values())
    out["hbm_read_gbs_by_workgroups"] = read
    out["hbm_copy_gbs_by_workgroups"] = copy
    del src, dst, sink
    iters = 20000
    mfma = {}
    for per_cu in (1, 2):
        mwg = per_cu * cus
        msink = torch.empty(4 * mwg, dtype=torch.float32, device="cuda")
        ms = timed(lambda: llb.llb_probe_mfma_bf16(mwg, iters, msink), 10, warm_s=0.5)
        mfma[mwg] = round(mwg * 4 * iters * 8 * 16384 / (ms * 1e-3) / 1e12, 1)
    out["mfma_bf16_tflops"] = max(mfma.values())
    out["mfma_bf16_tflops_by_workgroups"] = mfma
    out["method"] = ("HBM: median of 20 launches streaming 1 GiB (contiguous share per workgroup, 16-byte loads, "
                     "4, 8 and 16 workgroups per CU; copy counts read + write), best shape; MFMA: median of 10 "
                     f"launches of 1 or 2 workgroups per CU, 4 waves each, {iters} x 8 independent 16x16x32 bf16 "
                     "MFMAs per wave on pseudo-random operands, best shape")
    torch.cuda.empty_cache()
    return out


# ------------------------------------------------------------- GPU timing
def _warm(step, warmup, warm_seconds, sync_every=4):
    import torch
    t_warm = time.perf_counter()
    n_warm = 0
    while n_warm < warmup or time.perf_counter() - t_warm < warm_seconds:
        step(n_warm)
        n_warm += 1
        if n_warm % sync_every == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return n_warm


def _timed_loops(step, steps, stream):
    """(mean ms over one loop of `steps` back-to-back steps, list of per-step ms
    from a second loop with an event between consecutive steps)."""
    import torch
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(steps):
        step(i)
    t1.record(stream)
    torch.cuda.synchronize()
    total = t0.elapsed_time(t1)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record(stream)
    for i in range(steps):
        step(i)
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    return total / steps, per


def time_workload(name, steps, warmup, sets=1, warm_seconds=0.5, tiles=None, decode_kernels=None):
    import torch
    import workloads
    from dense_decoder_only_amd import llb

    wl = workloads.get(name)
    shp = wl.shape
    dev = "cuda"
    cap = workloads.cache_capacity(workloads.max_start(wl) + wl.T)
    log(f"{name}: building {sets} weight/cache set(s) on the GPU")
    blocks, caches = [], []
    w, gen = workloads.make_weights(shp, wl.seed, device=dev)
    x = workloads.make_x(wl.B, wl.T, shp.d_model, gen, device=dev)
    for i in range(sets):
        blocks.append(llb.llb_block_create(llb.make_config(shp, cap), w))
        if tiles is not None:
            llb.llb_block_set_tiles(blocks[-1], *tiles)
        if decode_kernels is not None:
            llb.llb_block_set_decode_kernels(blocks[-1], *decode_kernels)
        kc, vc = workloads.make_cache(shp, wl.B, workloads.max_start(wl), cap, gen, device=dev)
        caches.append((kc, vc))
    del w
    y = torch.empty_like(x)
    ws = llb.workspace(blocks[0], wl.B, wl.T)
    positions = workloads.ragged_positions(wl) if wl.ragged else None
    torch.cuda.synchronize()

    def step(i):
        blk = blocks[i % sets]
        kc, vc = caches[i % sets]
        if wl.mode == "prefill" and wl.P > 0:
            llb.llb_block_prefill_at(blk, x, y, wl.B, wl.T, wl.P, kc, vc, cap, ws)
        elif wl.mode == "prefill":
            llb.llb_block_prefill(blk, x, y, wl.B, wl.T, kc, vc, cap, ws)
        elif wl.ragged:
            llb.llb_block_decode_ragged(blk, x, y, wl.B, positions, kc, vc, cap, ws)
        else:
            llb.llb_block_decode(blk, x, y, wl.B, wl.P, kc, vc, cap, ws)

    # At least `warmup` steps and at least `warm_seconds` of back-to-back work:
    # the GPU's clocks take a few hundred milliseconds of load to settle.
    n_warm = _warm(step, warmup, warm_seconds)
    log(f"{name}: {n_warm} warm-up steps")
    stream = torch.cuda.current_stream()
    # The whole-call time comes from a loop without the per-stage events (each
    # event record adds a few microseconds between kernels); a second loop gives
    # single-step times, a third (with the stage events) the per-stage split.
    mean_ms, step_ms = _timed_loops(step, steps, stream)
    for b in blocks:
        llb.llb_block_set_stage_timing(b, True)
        llb.llb_block_stage_times(b)           # clear
    torch.cuda.synchronize()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    stage_ms = {k: 0.0 for k in llb.STAGES}
    calls = 0
    for b in blocks:
        ms, n = llb.llb_block_stage_times(b)
        llb.llb_block_set_stage_timing(b, False)
        for k in stage_ms:
            stage_ms[k] += ms[k]
        calls += n
    for b in blocks:
        llb.llb_block_destroy(b)
    del caches, x, y, ws
    torch.cuda.empty_cache()
    per_call = {k: v / calls for k, v in stage_ms.items()}
    return wl, mean_ms, step_ms, per_call


def time_model(name, steps, warmup, warm_seconds=0.5):
    """Times one whole-model forward per step (embedding, every block, final norm,
    LM head; last-position logits for a prefill).  Returns (workload, ms/step,
    per-step ms, algorithmic bytes, algorithmic FLOPs)."""
    import torch
    import workloads
    from dense_decoder_only_amd import llb

    wl = workloads.get(name)
    shp = wl.shape
    cap = workloads.cache_capacity(wl.P + wl.T)
    log(f"{name}: building the {wl.layers}-layer model on the GPU")
    params, gen = workloads.make_model_weights(shp, wl.layers, wl.vocab, wl.seed, device="cuda")
    model = llb.llb_model_create(llb.make_config(shp, cap), params["layers"], wl.vocab, params["embed"],
                                 params["final_norm"], params["lm_head"])
    del params
    torch.cuda.empty_cache()
    kcs, vcs = [], []
    for _ in range(wl.layers):
        k, v = workloads.make_cache(shp, wl.B, wl.P, cap, gen, device="cuda")
        kcs.append(k)
        vcs.append(v)
    tok = workloads.make_tokens(wl.B, wl.T, wl.vocab, gen, device="cuda")
    last_only = wl.mode == "prefill"
    logits = torch.empty((wl.B, wl.vocab), dtype=torch.float32, device="cuda")
    ws = llb.model_workspace(model, wl.B, wl.T, last_only)

    def step(i):
        llb.llb_model_forward(model, tok, wl.B, wl.T, wl.P, kcs, vcs, cap, last_only, logits, ws)

    _warm(step, warmup, warm_seconds, sync_every=1)
    mean_ms, step_ms = _timed_loops(step, steps, torch.cuda.current_stream())
    llb.llb_model_destroy(model)
    del kcs, vcs, ws, logits
    torch.cuda.empty_cache()
    by = stage_bytes(wl)
    fl = stage_flops(wl)
    es = 2
    head_rows = wl.B
    total_bytes = wl.layers * sum(by.values()) + wl.vocab * shp.d_model * es + head_rows * wl.vocab * 4
    total_flops = wl.layers * sum(fl.values()) + 2 * head_rows * wl.vocab * shp.d_model
    return wl, mean_ms, step_ms, total_bytes, total_flops


def _pct(vals, q):
    s = sorted(vals)
    if not s:
        return None
    k = (len(s) - 1) * q
    lo = int(k)
    hi = min(lo + 1, len(s) - 1)
    return s[lo] + (s[hi] - s[lo]) * (k - lo)


def traffic_from_profile(key):
    """HBM bytes per launch measured with rocprofv3 FETCH_SIZE/WRITE_SIZE for the
    current kernel source, if such a record exists (profiles/traffic.json)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get(key)
    except Exception:
        return None
    if not rec:
        return None
    import hashlib
    for src in rec["sources"]:
        h = hashlib.sha256(open(os.path.join(ROOT, "dense_decoder_only_amd", "csrc", src), "rb").read())
        if h.hexdigest()[:16] != rec["source_sha"].get(src):
            return None
    return rec["bytes_per_call"]


def roofline(wl, stage_ms, peaks):
    """Roofline block of the workload's dominant kernel (its longest stage)."""
    fl = stage_flops(wl)
    by = stage_bytes(wl)
    dom = max(stage_ms, key=lambda k: stage_ms[k])
    t = stage_ms[dom] * 1e-3
    if wl.mode == "prefill":
        achieved = fl[dom] / t / 1e12
        r = {"bound": "mfma", "stage": dom, "kernel": STAGE_KERNELS["prefill"][dom],
             "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
             "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "flops_per_call": fl[dom]}
        if peaks:
            r["measured_peak"] = peaks["mfma_bf16_tflops"]
            r["frac_measured_peak"] = round(achieved / peaks["mfma_bf16_tflops"], 4)
    else:
        achieved = by[dom] / t / 1e9
        r = {"bound": "hbm", "stage": dom, "kernel": STAGE_KERNELS["decode"][dom],
             "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
             "frac": round(achieved / PEAK_HBM_GBS, 4), "bytes_per_call": by[dom]}
        if peaks:
            r["measured_peak"] = peaks["hbm_read_gbs"]
            r["frac_measured_peak"] = round(achieved / peaks["hbm_read_gbs"], 4)
    r["avg_call_ms"] = round(stage_ms[dom], 5)
    r["timing"] = "HIP events on the launch stream around the stage, averaged over the timed steps"
    r["traffic"] = traffic_from_profile(f"{wl.name}:{dom}")
    return r


def summarize(wl, ms, step_ms, stage_ms, peaks):
    fl = stage_flops(wl)
    by = stage_bytes(wl)
    tok = wl.B * wl.T
    out = {
        "tokens_per_s": tok / (ms * 1e-3),
        "ms_per_step": ms,
        "step_ms_p10": round(_pct(step_ms, 0.1), 5),
        "step_ms_p50": round(_pct(step_ms, 0.5), 5),
        "step_ms_p90": round(_pct(step_ms, 0.9), 5),
        "stages_ms": {k: round(v, 5) for k, v in stage_ms.items()},
    }
    if wl.mode == "prefill":
        total = sum(fl.values())
        out["tflops"] = total / (ms * 1e-3) / 1e12
        out["frac_bf16_peak"] = out["tflops"] / PEAK_BF16_TFLOPS
        if peaks:
            out["frac_bf16_measured_peak"] = out["tflops"] / peaks["mfma_bf16_tflops"]
        out["algorithmic_flops"] = total
        out["stage_tflops"] = {k: round(fl[k] / (stage_ms[k] * 1e-3) / 1e12, 2) for k in fl}
    else:
        total = sum(by.values())
        out["hbm_gbs"] = total / (ms * 1e-3) / 1e9
        out["frac_hbm_peak"] = out["hbm_gbs"] / PEAK_HBM_GBS
        if peaks:
            out["frac_hbm_measured_peak"] = out["hbm_gbs"] / peaks["hbm_read_gbs"]
        out["algorithmic_bytes"] = total
        out["stage_gbs"] = {k: round(by[k] / (stage_ms[k] * 1e-3) / 1e9, 1) for k in by}
    out["roofline"] = roofline(wl, stage_ms, peaks)
    return out


# ------------------------------------------------------------- CPU oracle baseline
CPU_SAMPLE_TOKENS = 1024


def cpu_baseline(name):
    """The fp64 numpy oracle on a bounded sample of the workload: its first
    CPU_SAMPLE_TOKENS tokens of each sequence (prefill) or the whole call
    (decode), repeated until at least 10 s have passed."""
    import threadpoolctl
    import oracle
    import workloads

    wl = workloads.get(name)
    log(f"cpu baseline: generating {name} inputs on the host")
    inp = workloads.make_inputs(wl)
    T = min(wl.T, CPU_SAMPLE_TOKENS) if wl.mode == "prefill" else wl.T
    x = inp["x"][:, :T].contiguous()
    info = threadpoolctl.threadpool_info()
    threads = max([i.get("num_threads", 1) for i in info if i.get("user_api") == "blas"] or [1])
    avail = len(os.sched_getaffinity(0))
    log(f"cpu baseline: oracle on {threads} BLAS threads ({avail} cores available)")
    runs = 0
    t0 = time.perf_counter()
    while runs == 0 or (time.perf_counter() - t0 < 10.0 and runs < 50):
        oracle.block_forward(wl.shape, inp["weights"], x, inp["k_cache"], inp["v_cache"], wl.P)
        runs += 1
    dt = (time.perf_counter() - t0) / runs
    what = (f"the first {T} of the {wl.T} tokens (causality makes them exactly a {T}-token prefill)"
            if T < wl.T else "the whole call")
    return {"value": wl.B * T / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "cores_available": avail,
            "sample": f"{runs} oracle block forward(s) of {name} over {what}, B={wl.B}, float64 numpy on "
                      f"{threads} BLAS threads, {dt:.2f} s wall each, {dt * runs:.1f} s in all"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--warmup-seconds", type=float, default=0.5,
                    help="keep warming up until this much time has passed (clocks settle under load)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-others", action="store_true")
    ap.add_argument("--no-peaks", action="store_true", help="skip the probe kernels (measured peaks)")
    ap.add_argument("--only", default=None, help="time only this workload (diagnostics)")
    ap.add_argument("--decode-kernels", default=None, metavar="Q,O,GU,D",
                    help="decode kernel of the QKV, O, gate/up and down projections (-1 automatic, "
                         "0 split-K, 16/32 narrow rows); with --only")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (calibrates the "
                         "HBM byte counters FETCH_SIZE / WRITE_SIZE against a known size)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the block runs on one "
              "device and no multi-GPU path exists", file=sys.stderr)
        sys.exit(2)

    import torch
    assert torch.cuda.is_available(), "no GPU"
    torch.cuda.set_device(0)

    if args.copy_probe:
        n = args.copy_probe * (1 << 20) // 4
        a = torch.ones(n, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n * 4, "launches": 3}), flush=True)
        return

    peaks = None
    if not args.no_peaks and args.only is None:
        log("measuring HBM and MFMA peaks with the probe kernels")
        peaks = measure_peaks()
        log(f"peaks: {peaks}")

    name = args.only or HEADLINE
    drows = tuple(int(v) for v in args.decode_kernels.split(",")) if args.decode_kernels else None
    steps = args.steps
    wl, ms, step_ms, st = time_workload(name, steps, args.warmup, sets=2 if "decode" in name else 1,
                                        warm_seconds=args.warmup_seconds, decode_kernels=drows)
    head = summarize(wl, ms, step_ms, st, peaks)
    log(f"{name}: {ms:.3f} ms/step, {head['tokens_per_s']:.0f} tok/s")

    result = {
        "metric": METRIC,
        "value": round(head["tokens_per_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "step_ms_p10": head["step_ms_p10"],
        "step_ms_p90": head["step_ms_p90"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": name, "B": wl.B, "T": wl.T, "P": wl.P, "d_model": wl.shape.d_model,
                   "n_heads": wl.shape.n_heads, "n_kv_heads": wl.shape.n_kv_heads,
                   "head_dim": wl.shape.head_dim, "d_ff": wl.shape.d_ff,
                   "rope_scaling": "llama3" if wl.shape.rope_scaling else "none",
                   "parallelism": "none (1 GPU)"},
        "roofline": head["roofline"],
        "measured_peaks": peaks,
        "headline_detail": head,
    }

    if not args.no_others and args.only is None:
        others = {}
        for other in OTHERS:
            sets = 2 if "decode" in other else 1
            owl, oms, ostep, ost = time_workload(other, args.steps, max(2, args.warmup // 2), sets=sets,
                                                 warm_seconds=args.warmup_seconds)
            others[other] = summarize(owl, oms, ostep, ost, peaks)
            log(f"{other}: {oms:.3f} ms/step")
        result["other_workloads"] = others

        models = {}
        for mname in ("8b_bf16_model_decode", "8b_bf16_model_prefill"):
            mwl, mms, mstep, mby, mfl = time_model(mname, 10, 2, warm_seconds=args.warmup_seconds)
            tok = mwl.B * mwl.T
            entry = {"tokens_per_s": tok / (mms * 1e-3), "ms_per_step": mms, "layers": mwl.layers,
                     "vocab": mwl.vocab, "step_ms_p10": round(_pct(mstep, 0.1), 4),
                     "step_ms_p90": round(_pct(mstep, 0.9), 4)}
            if mwl.mode == "decode":
                entry["hbm_gbs"] = mby / (mms * 1e-3) / 1e9
                entry["frac_hbm_peak"] = entry["hbm_gbs"] / PEAK_HBM_GBS
            else:
                entry["tflops"] = mfl / (mms * 1e-3) / 1e12
                entry["frac_bf16_peak"] = entry["tflops"] / PEAK_BF16_TFLOPS
            models[mname] = entry
            log(f"{mname}: {mms:.3f} ms/step")
        result["model_workloads"] = models

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(name)
    else:
        result["cpu_baseline"] = None

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
