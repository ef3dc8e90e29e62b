"""Plain fp64 CPU oracle of one Llama-3/3.1 dense pre-norm decoder block.

TEST INFRASTRUCTURE ONLY.  Imported by tests/, __graft_entry__.smoke() and
bench.py's cpu_baseline leg; never by the product path.  It shares no code
with the HIP library (no kernels, headers, tables or helpers).

Everything is evaluated in float64 from the given inputs (bf16 inputs are
widened exactly).  Nothing is rounded to bf16: the oracle is the definition
of what the block computes, not an emulation of the GPU's roundings.  The
one place where the pages fix a lower precision is the RoPE angle: Meta's
`precompute_freqs_cis` (quoted on "Llama 3 8B - Prepare Q, K, V",
atlas.klimoza.dev, model.py excerpt) forms the inverse frequencies and the
position-times-frequency product in float32, so `rope_angles` does the same
and only then evaluates cos/sin in float64.

Sources (page title, section):
  [P1] "Llama 3.1 70B", ainfra.dev LLM diagram tool: sections "Transformer
       layer", "RMSNorm", "Grouped-Query Attention", "Residual add",
       "SwiGLU MLP".
  [P2] "Inside a Transformer Block: FFN, the Residual Stream, and
       Normalization", blog.truongducdung.dev: section 05 (RMSNorm) and
       section 06 (parameter counts, count_params output).
  [P3] "How Llama 3.1 Generates the Next Token", ashwinnarayan.com: block
       diagram notation, "What's RMSNorm?", "What's the SWIGLU block?",
       "RoPE" (rotation formula, angle schedule, long-context adjustment).
  [P4] "Llama 3 8B - Prepare Q, K, V", atlas.klimoza.dev: header shapes,
       "Parameters" table, model.py excerpts (precompute_freqs_cis,
       apply_rotary_emb, forward(tokens, start_pos)), layers.py excerpts
       (weights stored [out, in], F.linear computes x A^T).

Readings where the pages are silent:
  * llama3 frequency scaling: the pages only say that the fastest rotations
    are kept, the slowest are slowed by the factor (8) and an intermediate
    band is blended.  Reading: wavelength lambda = 2*pi/omega; keep omega if
    lambda < orig/high_freq_factor; use omega/factor if lambda >
    orig/low_freq_factor; otherwise blend linearly in orig/lambda.  This
    blend shape is "parity unpinned" by the pages (only its end points and
    monotonicity are pinned).
  * decode mask: a query at absolute position m sees keys 0..m (the cache
    holds positions 0..m-1 and the new key is m).
  * GQA: query head h reads KV head floor(h / (n_heads / n_kv_heads)).
"""
from __future__ import annotations

import math
from typing import Dict, Optional, Sequence

import numpy as np

__all__ = [
    "to64", "expected_weight_shapes", "block_param_counts", "rmsnorm", "rope_inv_freq",
    "rope_angles", "rope_cos_sin", "apply_rope", "attention", "silu", "swiglu", "block_forward",
]


def to64(a) -> np.ndarray:
    """Widen a numpy array or a CPU torch tensor (fp32 or bf16) to float64."""
    if hasattr(a, "detach"):  # torch tensor; bf16 has no numpy dtype
        a = a.detach()
        if str(a.dtype) == "torch.bfloat16":
            a = a.float()
        a = a.cpu().numpy()
    return np.asarray(a, dtype=np.float64)


# --------------------------------------------------------------------------
# shapes and parameter counts
# --------------------------------------------------------------------------
def expected_weight_shapes(d_model: int, n_heads: int, n_kv_heads: int, head_dim: int,
                           d_ff: int) -> Dict[str, tuple]:
    """Weight shapes in nn.Linear's [out, in] layout ([P4] layers.py: the weight is
    allocated transposed because F.linear computes x A^T).  Q has n_heads*head_dim
    outputs, K and V n_kv_heads*head_dim ([P4] "Parameters" table); the SwiGLU
    gate/up map d -> d_ff and down d_ff -> d ([P1] "SwiGLU MLP"); two RMSNorm gains
    of width d ([P1] "Transformer layer")."""
    return {
        "attn_norm": (d_model,),
        "wq": (n_heads * head_dim, d_model),
        "wk": (n_kv_heads * head_dim, d_model),
        "wv": (n_kv_heads * head_dim, d_model),
        "wo": (d_model, n_heads * head_dim),
        "ffn_norm": (d_model,),
        "w_gate": (d_ff, d_model),
        "w_up": (d_ff, d_model),
        "w_down": (d_model, d_ff),
    }


def block_param_counts(d_model, n_heads, n_kv_heads, head_dim, d_ff) -> Dict[str, int]:
    """Parameter counts of one block from its weight shapes ([P4] "Parameters";
    [P2] section 06 block total, which includes the two RMSNorm gains)."""
    sh = expected_weight_shapes(d_model, n_heads, n_kv_heads, head_dim, d_ff)
    n = {k: int(np.prod(v)) for k, v in sh.items()}
    qkv = n["wq"] + n["wk"] + n["wv"]
    ffn = n["w_gate"] + n["w_up"] + n["w_down"]
    return {"qkv": qkv, "attn": qkv + n["wo"], "ffn": ffn, "block": sum(n.values()),
            **{"n_" + k: v for k, v in n.items()}}


# --------------------------------------------------------------------------
# RMSNorm
# --------------------------------------------------------------------------
def rmsnorm(x, g, eps: float) -> np.ndarray:
    """RMSNorm over the last axis: x / sqrt(mean(x^2) + eps) * g.

    [P1] "RMSNorm": y = x / sqrt(mean(x^2) + eps) * g, eps inside the square root,
    per token over its d features.  [P3] "What's RMSNorm?": same formula, no mean
    subtraction, one learned multiplier per coordinate.
    """
    x = to64(x)
    g = to64(g)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * g


# --------------------------------------------------------------------------
# RoPE
# --------------------------------------------------------------------------
def rope_inv_freq(head_dim: int, theta: float, scaling: Optional[dict] = None) -> np.ndarray:
    """Per-pair rotation speeds omega_i, i = 0..head_dim/2-1, as float32 values.

    Base schedule omega_i = theta^(-2i/head_dim) ([P3] "RoPE", "Why use different
    rotation speeds?"), formed as in [P4] precompute_freqs_cis: the power and the
    reciprocal are float32 quantities.  Here the power is evaluated in float64 and
    rounded to float32, then 1/that is rounded to float32.

    `scaling` (llama3 long-context adjustment, [P3] "RoPE": fastest rotations kept,
    slowest slowed by the factor, an intermediate band blended) is a dict with keys
    factor, low_freq_factor, high_freq_factor, orig_max_pos; the blend follows the
    reading in this module's docstring and is evaluated in float64, rounded to
    float32.
    """
    half = head_dim // 2
    out = np.empty(half, dtype=np.float64)
    for i in range(half):
        p = np.float32(float(theta) ** (2.0 * i / head_dim))
        w = np.float32(np.float32(1.0) / p)
        out[i] = float(w)
    if scaling:
        factor = float(scaling["factor"])
        lo = float(scaling["low_freq_factor"])
        hi = float(scaling["high_freq_factor"])
        orig = float(scaling["orig_max_pos"])
        low_wavelen = orig / lo
        high_wavelen = orig / hi
        for i in range(half):
            w = out[i]
            wavelen = 2.0 * math.pi / w
            if wavelen < high_wavelen:
                nw = w
            elif wavelen > low_wavelen:
                nw = w / factor
            else:
                s = (orig / wavelen - lo) / (hi - lo)
                nw = (1.0 - s) * w / factor + s * w
            out[i] = float(np.float32(nw))
    return out


def rope_angles(positions: Sequence[int], inv_freq: np.ndarray) -> np.ndarray:
    """phi[m, i] = m * omega_i, with both factors and the product in float32, as
    [P4] precompute_freqs_cis does (arange(..., float32), torch.outer).  Positions
    count from 0 ([P3] "RoPE": at position zero no rotation is applied)."""
    m = np.asarray(positions, dtype=np.float32)[:, None]
    w = np.asarray(inv_freq, dtype=np.float32)[None, :]
    return (m * w).astype(np.float64)


def rope_cos_sin(positions, head_dim, theta, scaling=None):
    phi = rope_angles(positions, rope_inv_freq(head_dim, theta, scaling))
    return np.cos(phi), np.sin(phi)


def apply_rope(x, cos, sin) -> np.ndarray:
    """Rotate adjacent pairs (x_2i, x_2i+1) by phi ([P3] "RoPE", "What exactly are we
    rotating?": x'_2i = x_2i cos - x_2i+1 sin, x'_2i+1 = x_2i sin + x_2i+1 cos; pairs
    are adjacent coordinates as in [P4] apply_rotary_emb's reshape(..., -1, 2)).

    x: [..., T, hd]; cos, sin: [T, hd/2] broadcast over the leading axes.
    """
    x = to64(x)
    xe = x[..., 0::2]
    xo = x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = xe * cos - xo * sin
    out[..., 1::2] = xe * sin + xo * cos
    return out


# --------------------------------------------------------------------------
# attention
# --------------------------------------------------------------------------
def attention(q, k, v, q_pos, n_keys: Optional[int] = None) -> np.ndarray:
    """Causal grouped-query attention for one sequence.

    q: [H, Tq, hd] (rotated queries), k, v: [Hkv, L, hd] (rotated keys, values) for
    key positions 0..L-1; q_pos[t] is the absolute position of query t.  Query t
    sees keys n <= q_pos[t] ([P3] block notation: M is 0 for allowed positions and
    -inf for future ones).  Score s = q.k / sqrt(hd) ([P3] "Where does position
    enter the computation?"), softmax over keys, o = sum_n p_n v_n.  Query head h
    uses KV head floor(h / (H/Hkv)) ([P3] g(i) = ceil(i/4) with 1-based heads;
    [P1] "Grouped-Query Attention": each group of query heads shares one K/V head,
    repeat_kv after the cache read).
    """
    q = to64(q)
    k = to64(k)
    v = to64(v)
    H, Tq, hd = q.shape
    Hkv, L, _ = k.shape
    if n_keys is not None:
        L = n_keys
        k = k[:, :L]
        v = v[:, :L]
    G = H // Hkv
    q_pos = np.asarray(q_pos, dtype=np.int64)
    mask = np.arange(L)[None, :] <= q_pos[:, None]          # [Tq, L]
    scale = 1.0 / math.sqrt(hd)
    out = np.empty((H, Tq, hd), dtype=np.float64)
    for h in range(H):
        g = h // G
        s = (q[h] @ k[g].T) * scale
        s = np.where(mask, s, -np.inf)
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=1, keepdims=True)
        out[h] = p @ v[g]
    return out


# --------------------------------------------------------------------------
# SwiGLU
# --------------------------------------------------------------------------
def silu(z) -> np.ndarray:
    """SiLU(a) = a * sigma(a), sigma(a) = 1 / (1 + e^-a) ([P3] "What's the SWIGLU
    block?")."""
    z = to64(z)
    return z / (1.0 + np.exp(-z))


def swiglu(a, w_gate, w_up, w_down) -> np.ndarray:
    """W_down (SiLU(W_gate a) * (W_up a)), weights in [out, in] layout, no biases
    ([P1] "SwiGLU MLP"; [P3] m = [SiLU(z W1) (.) (z W3)] W2)."""
    a = to64(a)
    gate = a @ to64(w_gate).T
    up = a @ to64(w_up).T
    return (silu(gate) * up) @ to64(w_down).T


# --------------------------------------------------------------------------
# the block
# --------------------------------------------------------------------------
def block_forward(cfg, w, x, k_cache, v_cache, start_pos: int = 0,
                  rows: Optional[Sequence[int]] = None, return_parts: bool = False):
    """One pre-norm decoder block: h = x + Attn(RMSNorm1(x)); y = h + SwiGLU(RMSNorm2(h)).

    [P1] "Transformer layer" (DecoderLayer.forward), [P3] block outline.  The T new
    tokens of each sequence sit at absolute positions start_pos..start_pos+T-1
    ([P4] forward(tokens, start_pos) slices the rotation table at
    [start_pos : start_pos + T]).  Their rotated keys and values are written to the
    cache at those rows ([P4] "Explanation": keys and values are cached at n_kv_heads
    and repeated across the group only after the cache read), then every query
    attends to cache rows 0..its own position.  Prefill is start_pos = 0 over an
    empty cache; decode is T = 1 at start_pos = P, reading L = P + 1 keys ([P4]
    header).

    cfg: object with d_model, n_heads, n_kv_heads, head_dim, d_ff, eps, rope_theta,
         rope_scaling (bool) and rs_* fields.
    w:   dict attn_norm, wq, wk, wv, wo, ffn_norm, w_gate, w_up, w_down ([out, in]).
    x:   [B, T, d].   k_cache, v_cache: [B, n_kv, cap, hd] (rows < start_pos used).
    rows: optional subset of token indices t whose outputs are computed; keys and
         values are still formed for every token.  Valid because a causal block's
         row t depends on tokens 0..t only.
    Returns y [B, T or len(rows), d], and the new cache rows k_new, v_new
    [B, n_kv, T, hd] (K rotated, V not).
    """
    d, H, Hkv, hd = cfg.d_model, cfg.n_heads, cfg.n_kv_heads, cfg.head_dim
    sh = expected_weight_shapes(d, H, Hkv, hd, cfg.d_ff)
    W = {}
    for name, shape in sh.items():
        W[name] = to64(w[name])
        if W[name].shape != shape:
            raise ValueError(f"{name}: shape {W[name].shape} != {shape}")
    x = to64(x)
    B, T, _ = x.shape
    kc = to64(k_cache)
    vc = to64(v_cache)
    scaling = None
    if cfg.rope_scaling:
        scaling = dict(factor=cfg.rs_factor, low_freq_factor=cfg.rs_low_freq_factor,
                       high_freq_factor=cfg.rs_high_freq_factor, orig_max_pos=cfg.rs_orig_max_pos)
    pos = np.arange(start_pos, start_pos + T)
    cos, sin = rope_cos_sin(pos, hd, cfg.rope_theta, scaling)
    sel = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64)

    n = len(sel)
    a = rmsnorm(x, W["attn_norm"], cfg.eps)                              # [B, T, d]
    k_new = (a @ W["wk"].T).reshape(B, T, Hkv, hd).transpose(0, 2, 1, 3)  # [B, Hkv, T, hd]
    v_new = (a @ W["wv"].T).reshape(B, T, Hkv, hd).transpose(0, 2, 1, 3)
    k_new = apply_rope(k_new, cos, sin)
    q = (a[:, sel] @ W["wq"].T).reshape(B, n, H, hd).transpose(0, 2, 1, 3)  # [B, H, n, hd]
    q = apply_rope(q, cos[sel], sin[sel])
    L = start_pos + T
    o = np.empty((B, n, H * hd), dtype=np.float64)
    for b in range(B):
        keys = np.concatenate([kc[b, :, :start_pos], k_new[b]], axis=1)   # [Hkv, L, hd]
        vals = np.concatenate([vc[b, :, :start_pos], v_new[b]], axis=1)
        ob = attention(q[b], keys, vals, pos[sel], n_keys=L)              # [H, n, hd]
        o[b] = ob.transpose(1, 0, 2).reshape(n, H * hd)
    h = x[:, sel] + o @ W["wo"].T
    a2 = rmsnorm(h, W["ffn_norm"], cfg.eps)
    y = h + swiglu(a2, W["w_gate"], W["w_up"], W["w_down"])
    if return_parts:
        return y, k_new, v_new, {"q": q, "o": o, "h": h}
    return y, k_new, v_new
