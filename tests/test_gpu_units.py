"""Unit parity of every stage of a block call, at the workload sizes, in the
launch configuration bench.py times.

A block call leaves its intermediate results in the workspace (Q, the attention
output O, h and u; offsets from llb_block_workspace_layout) and its keys and
values in the cache.  Each stage is checked against the oracle's own steps fed
the GPU's inputs to that stage, so every kernel is held to its own rounding
instead of to the whole block's accumulated error (which, measured against the
branch it belongs to, reaches ~0.1 in prefill and would hide a one-key mask
error):

  QKV    Q, K, V = RoPE(r1 * (bf16(x * g1) W^T)), r1 = 1/sqrt(mean(x^2) + eps)
         ("Llama 3.1 70B", "RMSNorm"; "How Llama 3.1 Generates the Next Token",
         "RoPE"): bf16 outputs, against the GPU's Q and its cache rows;
  attn   softmax(Q K^T / sqrt(hd)) V over keys 0..position, on the GPU's Q and
         cache ("How Llama 3.1 Generates the Next Token", block notation): bf16;
  O      h = x + O Wo^T on the GPU's O ("Llama 3.1 70B", "Residual add"): fp32;
  FFN    u = SiLU(r2 * (bf16(h * g2) Wg^T)) * (r2 * (bf16(h * g2) Wu^T)) on the
         GPU's h ("Llama 3.1 70B", "SwiGLU MLP"): bf16;
  down   y = h + u Wd^T on the GPU's h and u: fp32.

bf16(.) is the operand's single rounding (round to nearest even), which the
test forms on the CPU the way the kernels do (an fp32 product, then bf16).
Bars: bf16 outputs per element |gpu - ref| <= 2^-8 |ref| (+ 2^-8 sum_n p_n |v_n|
for attention, whose weights are rounded before P.V in prefill) + 1e-3 rms(ref);
fp32 outputs max|gpu - ref| / rms(ref) <= 1e-4 (fp32 accumulation over K up to
28672 products; a wrong term or index is O(1)).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from dense_decoder_only_amd import llb
from gpu_util import GpuBlock, bf16_err, note, rel_err

pytestmark = pytest.mark.gpu

C_BF16 = 1e-3      # bf16 outputs: 1e-3 rms(ref) besides the half-ulp term
BAR_F32 = 1e-4     # fp32 outputs: max|gpu - ref| / rms(ref)

# sampled rows of the 70B 16K prefill (first, last, tile and round edges)
C5_ROWS = [0, 1, 31, 32, 255, 256, 4095, 4096, 8191, 8192, 12345, 16351, 16352, 16383]
# sampled rows of the 8B chunked prefill (positions 2048 + t)
CHUNK_ROWS = [0, 1, 63, 64, 1000, 2046, 2047]


def _region(ws, off, dtype, shape):
    n = int(np.prod(shape)) * torch.tensor([], dtype=dtype).element_size()
    return ws[off:off + n].view(dtype).view(*shape)


def _scaling(shp):
    if not shp.rope_scaling:
        return None
    return dict(factor=shp.rs_factor, low_freq_factor=shp.rs_low_freq_factor,
                high_freq_factor=shp.rs_high_freq_factor, orig_max_pos=shp.rs_orig_max_pos)


def _operand(v, gain):
    """The bf16 operand of an RMSNorm, v * g rounded once, widened to fp64."""
    op = (v.float() * gain.float()).to(torch.bfloat16)
    return oracle.to64(op)


def _inv_rms(v, eps):
    """The RMSNorm row scale 1 / sqrt(mean(v^2) + eps), fp64."""
    v = oracle.to64(v)
    return 1.0 / np.sqrt(np.mean(v * v, axis=-1, keepdims=True) + eps)


def _run(wl, inp):
    """One block call of workload wl on the GPU; returns CPU copies of y, the
    caches and the workspace's Q, O, h and u."""
    cap = inp["cap"]
    shp = wl.shape
    gb = GpuBlock(shp, inp["weights"], max_positions=cap)
    try:
        kd, vd = inp["k_cache"].cuda(), inp["v_cache"].cuda()
        x = inp["x"].cuda()
        decode = wl.mode == "decode"
        ws = gb.workspace(wl.B, wl.T)
        y = torch.empty_like(x)
        note(f"units {wl.name}: GPU call B={wl.B} T={wl.T} P={wl.P}")
        if wl.ragged:
            llb.llb_block_decode_ragged(gb.blk, x, y, wl.B, workloads.ragged_positions(wl), kd, vd, cap, ws)
        elif decode:
            llb.llb_block_decode(gb.blk, x, y, wl.B, wl.P, kd, vd, cap, ws)
        else:
            llb.llb_block_prefill_at(gb.blk, x, y, wl.B, wl.T, wl.P, kd, vd, cap, ws)
        torch.cuda.synchronize()
        lay = llb.llb_block_workspace_layout(gb.blk, wl.B, wl.T, decode)
        M, H, hd = wl.B * wl.T, shp.n_heads, shp.head_dim
        out = {
            "y": y.cpu(), "k": kd.cpu(), "v": vd.cpu(),
            "q": _region(ws, lay["q"], torch.bfloat16, (wl.B, H, wl.T, hd)).cpu(),
            "o": _region(ws, lay["o"], torch.bfloat16, (wl.B, wl.T, H * hd)).cpu(),
            "h": _region(ws, lay["h"], torch.float32, (wl.B, wl.T, shp.d_model)).cpu(),
            "u": _region(ws, lay["u"], torch.bfloat16, (wl.B, wl.T, shp.d_ff)).cpu(),
        }
        assert M == wl.B * wl.T
    finally:
        gb.close()
    return out


def _check_units(wl, inp, g, rows):
    shp = wl.shape
    W = {k: oracle.to64(v) for k, v in inp["weights"].items()}
    H, Hkv, hd, eps = shp.n_heads, shp.n_kv_heads, shp.head_dim, shp.eps
    n = len(rows)
    starts = workloads.ragged_positions(wl) if wl.ragged else [wl.P] * wl.B
    x = inp["x"][:, rows]                                       # [B, n, d] fp32
    errs = {}

    # ---- QKV projection: RMSNorm operand, RoPE, Q to the workspace, K/V to the cache
    a = _operand(x, inp["weights"]["attn_norm"]) * _inv_rms(x, eps)
    e_q = e_k = e_v = 0.0
    for b in range(wl.B):
        pos = starts[b] + np.asarray(rows)
        cos, sin = oracle.rope_cos_sin(pos, hd, shp.rope_theta, _scaling(shp))
        q_ref = oracle.apply_rope((a[b] @ W["wq"].T).reshape(n, H, hd).transpose(1, 0, 2), cos, sin)
        k_ref = oracle.apply_rope((a[b] @ W["wk"].T).reshape(n, Hkv, hd).transpose(1, 0, 2), cos, sin)
        v_ref = (a[b] @ W["wv"].T).reshape(n, Hkv, hd).transpose(1, 0, 2)
        e_q = max(e_q, bf16_err(g["q"][b][:, rows], q_ref, c=C_BF16))
        pt = torch.as_tensor(pos)
        e_k = max(e_k, bf16_err(g["k"][b][:, pt], k_ref, c=C_BF16))
        e_v = max(e_v, bf16_err(g["v"][b][:, pt], v_ref, c=C_BF16))
    errs.update(q=e_q, k=e_k, v=e_v)

    # ---- attention on the GPU's Q and cache rows 0..position
    e_o = 0.0
    for b in range(wl.B):
        pos = starts[b] + np.asarray(rows)
        L = int(pos.max()) + 1
        qb = g["q"][b][:, rows]
        kb, vb = g["k"][b][:, :L], g["v"][b][:, :L]
        o_ref = oracle.attention(qb, kb, vb, pos, n_keys=L).transpose(1, 0, 2).reshape(n, H * hd)
        mag = oracle.attention(qb, kb, vb.abs(), pos, n_keys=L).transpose(1, 0, 2).reshape(n, H * hd)
        e_o = max(e_o, bf16_err(g["o"][b][rows], o_ref, c=C_BF16, mag=mag))
    errs["attn"] = e_o

    # ---- output projection + residual on the GPU's O
    o = oracle.to64(g["o"][:, rows])
    h_ref = oracle.to64(x) + o @ W["wo"].T
    h = g["h"][:, rows]
    errs["h"] = rel_err(h, h_ref)

    # ---- FFN RMSNorm, gate/up and SiLU * up on the GPU's h
    a2 = _operand(h, inp["weights"]["ffn_norm"]) * _inv_rms(h, eps)
    u_ref = oracle.silu(a2 @ W["w_gate"].T) * (a2 @ W["w_up"].T)
    errs["u"] = bf16_err(g["u"][:, rows], u_ref, c=C_BF16)

    # ---- down projection + residual on the GPU's h and u
    y_ref = oracle.to64(h) + oracle.to64(g["u"][:, rows]) @ W["w_down"].T
    errs["y"] = rel_err(g["y"][:, rows], y_ref)
    return errs


@pytest.mark.parametrize("name", ["8b_bf16_prefill", "8b_bf16_decode", "70b_bf16_decode",
                                  "8b_bf16_ragged_decode", "8b_bf16_chunked_prefill", "70b_bf16_prefill"])
def test_stage_parity_at_workload_size(name):
    wl = workloads.get(name)
    note(f"units {name}: generating inputs")
    cap = workloads.cache_capacity(workloads.max_start(wl) + wl.T)
    inp = workloads.make_inputs(wl, cap=cap)
    g = _run(wl, inp)
    if wl.T > 4096:
        rows = C5_ROWS
    elif wl.P > 0 and wl.mode == "prefill":
        rows = CHUNK_ROWS
    else:
        rows = list(range(wl.T))
    note(f"units {name}: oracle stages on {len(rows)} row(s) per sequence")
    errs = _check_units(wl, inp, g, rows)
    note("units " + name + ": " + "  ".join(f"{k} {v:.3g}" for k, v in errs.items()))
    for k in ("q", "k", "v", "attn", "u"):
        assert errs[k] <= 1.0, (k, errs[k])
    for k in ("h", "y"):
        assert errs[k] <= BAR_F32, (k, errs[k])
    # the cache rows before the call are untouched
    if not wl.ragged:
        assert torch.equal(g["k"][:, :, :wl.P], inp["k_cache"][:, :, :wl.P])
        assert torch.equal(g["v"][:, :, :wl.P], inp["v_cache"][:, :, :wl.P])
    assert math.isfinite(errs["y"])
