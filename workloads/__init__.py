"""Seeded synthetic workloads for the Llama-3 decoder block.

This module holds shapes, seeds and random draws only; it contains none of
the block's arithmetic.  Both the HIP path's tests/bench and the CPU oracle
take their inputs from here, so the two sides see identical tensors while
sharing no code that computes anything.

Shapes follow the pages:
  * "Llama 3.1 70B" (ainfra.dev LLM diagram tool), sections "Grouped-Query
    Attention" and "SwiGLU MLP": d=8192, 64 query / 8 KV heads, head_dim 128,
    d_ff 28672, llama3 RoPE scaling to 128K.
  * "Llama 3 8B - Prepare Q, K, V" (atlas.klimoza.dev), header and the
    sku_list excerpt: d=4096, 32 / 8 heads, eps 1e-5, rope_theta 500000,
    decode at P = 1000 cached positions.
  * "Inside a Transformer Block" (blog.truongducdung.dev) section 06: d_ff
    14336 for the 8B model.

Value distributions (readings of the workload descriptions):
  * weights ~ N(0, 1/d_in) -- variance 1/d_in, i.e. std d_in**-0.5, where d_in
    is the input width of that matrix (d for Wq/Wk/Wv/Wgate/Wup, n_heads*hd
    for Wo, d_ff for Wdown);
  * RMSNorm gains ~ 1 + N(0, 0.1) -- variance 0.1;
  * x ~ N(0, 1) in fp32;
  * decode caches ~ N(0, 1), taken as already-rotated keys and values.
For bf16 configurations every weight, gain and cache value is rounded to
bf16 once at generation; x stays fp32 (the residual stream is fp32).
Draw order per seed: g1, wq, wk, wv, wo, g2, w_gate, w_up, w_down, x,
k_cache, v_cache.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import torch

__all__ = ["BlockShape", "Workload", "CONFIGS", "WEIGHT_NAMES", "make_weights",
           "make_x", "make_cache", "make_inputs", "cache_capacity", "get"]

WEIGHT_NAMES = ("attn_norm", "wq", "wk", "wv", "wo", "ffn_norm", "w_gate", "w_up", "w_down")


@dataclasses.dataclass(frozen=True)
class BlockShape:
    d_model: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    d_ff: int
    eps: float = 1e-5
    rope_theta: float = 500000.0
    rope_scaling: bool = False          # llama3 long-context frequency scaling
    rs_factor: float = 8.0
    rs_low_freq_factor: float = 1.0
    rs_high_freq_factor: float = 4.0
    rs_orig_max_pos: int = 8192
    dtype: str = "bf16"                 # weights, gains, KV cache: "bf16" or "f32"

    @property
    def group(self) -> int:
        return self.n_heads // self.n_kv_heads

    @property
    def qkv_out(self) -> int:
        return (self.n_heads + 2 * self.n_kv_heads) * self.head_dim

    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    def weight_shapes(self) -> Dict[str, tuple]:
        d, hd, f = self.d_model, self.head_dim, self.d_ff
        return {
            "attn_norm": (d,),
            "wq": (self.n_heads * hd, d),
            "wk": (self.n_kv_heads * hd, d),
            "wv": (self.n_kv_heads * hd, d),
            "wo": (d, self.n_heads * hd),
            "ffn_norm": (d,),
            "w_gate": (f, d),
            "w_up": (f, d),
            "w_down": (d, f),
        }


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    shape: BlockShape
    mode: str          # "prefill" or "decode"
    B: int
    T: int = 1         # new tokens per sequence (1 for decode)
    P: int = 0         # cached positions before the call (start position)
    seed: int = 0
    ragged: bool = False  # decode: sequence b starts at ragged_positions(self)[b] (mean P)
    layers: int = 0       # > 0: a whole model of this many blocks with embedding and LM head
    vocab: int = 0

    @property
    def tokens(self) -> int:
        return self.B * self.T


TINY = BlockShape(d_model=512, n_heads=8, n_kv_heads=2, head_dim=64, d_ff=1408, dtype="f32")
LLAMA31_8B = BlockShape(d_model=4096, n_heads=32, n_kv_heads=8, head_dim=128, d_ff=14336)
LLAMA31_70B = BlockShape(d_model=8192, n_heads=64, n_kv_heads=8, head_dim=128, d_ff=28672,
                         rope_scaling=True)

CONFIGS: Dict[str, Workload] = {
    "tiny_f32_prefill": Workload("tiny_f32_prefill", TINY, "prefill", B=1, T=64, seed=1),
    "8b_bf16_prefill": Workload("8b_bf16_prefill", LLAMA31_8B, "prefill", B=1, T=2048, seed=2),
    "8b_bf16_decode": Workload("8b_bf16_decode", LLAMA31_8B, "decode", B=32, T=1, P=1000, seed=3),
    "70b_bf16_decode": Workload("70b_bf16_decode", LLAMA31_70B, "decode", B=64, T=1, P=4096, seed=4),
    "70b_bf16_prefill": Workload("70b_bf16_prefill", LLAMA31_70B, "prefill", B=1, T=16384, seed=5),
    # the whole Llama-3.1-8B stack: embedding, 32 blocks, final norm, LM head over
    # 128256 ids (logits of the last position for the prefill)
    "8b_bf16_model_decode": Workload("8b_bf16_model_decode", LLAMA31_8B, "decode", B=32, T=1, P=1000, seed=8,
                                     layers=32, vocab=128256),
    "8b_bf16_model_prefill": Workload("8b_bf16_model_prefill", LLAMA31_8B, "prefill", B=1, T=2048, seed=9,
                                      layers=32, vocab=128256),
    # 32 sequences of different lengths, evenly spread over 0..2P (mean P = 1000)
    "8b_bf16_ragged_decode": Workload("8b_bf16_ragged_decode", LLAMA31_8B, "decode", B=32, T=1, P=1000,
                                      seed=7, ragged=True),
    # second 2048-token chunk of a 4096-token prompt: positions 2048..4095 over a
    # 2048-row cache prefix
    "8b_bf16_chunked_prefill": Workload("8b_bf16_chunked_prefill", LLAMA31_8B, "prefill", B=1, T=2048,
                                        P=2048, seed=6),
}


def get(name: str) -> Workload:
    return CONFIGS[name]


def cache_capacity(positions: int) -> int:
    """Cache rows to allocate for `positions` rows: rounded up to 64."""
    return max(64, (positions + 63) // 64 * 64)


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _randn(shape, gen, device, std=1.0, mean=0.0, out_dtype=torch.float32):
    t = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    if mean != 0.0:
        t.add_(mean)
    return t.to(out_dtype)


def make_weights(shape: BlockShape, seed: int, device="cpu", gen: Optional[torch.Generator] = None):
    """Weights in nn.Linear layout [out, in], dtype per shape.dtype.

    Returns (weights dict, generator) so that later draws continue the stream.
    """
    gen = gen if gen is not None else _gen(seed, device)
    wd = shape.torch_dtype()
    d, hd = shape.d_model, shape.head_dim
    sh = shape.weight_shapes()
    w = {}
    w["attn_norm"] = _randn(sh["attn_norm"], gen, device, std=0.1 ** 0.5, mean=1.0, out_dtype=wd)
    w["wq"] = _randn(sh["wq"], gen, device, std=d ** -0.5, out_dtype=wd)
    w["wk"] = _randn(sh["wk"], gen, device, std=d ** -0.5, out_dtype=wd)
    w["wv"] = _randn(sh["wv"], gen, device, std=d ** -0.5, out_dtype=wd)
    w["wo"] = _randn(sh["wo"], gen, device, std=(shape.n_heads * hd) ** -0.5, out_dtype=wd)
    w["ffn_norm"] = _randn(sh["ffn_norm"], gen, device, std=0.1 ** 0.5, mean=1.0, out_dtype=wd)
    w["w_gate"] = _randn(sh["w_gate"], gen, device, std=d ** -0.5, out_dtype=wd)
    w["w_up"] = _randn(sh["w_up"], gen, device, std=d ** -0.5, out_dtype=wd)
    w["w_down"] = _randn(sh["w_down"], gen, device, std=shape.d_ff ** -0.5, out_dtype=wd)
    return w, gen


def make_model_weights(shape: BlockShape, n_layers: int, vocab: int, seed: int, device="cpu"):
    """A model's weights: the embedding table [vocab, d] ~ N(0, 1) (the trunk then
    starts at unit RMS, like the block inputs), n_layers block weight sets
    (make_weights, drawn in layer order), the final gain 1 + N(0, 0.1) and the LM
    head [vocab, d] ~ N(0, 1/d).  Returns (params, generator)."""
    gen = _gen(seed, device)
    wd = shape.torch_dtype()
    d = shape.d_model
    params = {"embed": _randn((vocab, d), gen, device, out_dtype=wd)}
    params["layers"] = [make_weights(shape, seed, device, gen=gen)[0] for _ in range(n_layers)]
    params["final_norm"] = _randn((d,), gen, device, std=0.1 ** 0.5, mean=1.0, out_dtype=wd)
    params["lm_head"] = _randn((vocab, d), gen, device, std=d ** -0.5, out_dtype=wd)
    return params, gen


def make_tokens(B: int, T: int, vocab: int, gen: torch.Generator, device="cpu") -> torch.Tensor:
    """Token ids, uniform over the vocabulary, int32 [B, T]."""
    return torch.randint(0, vocab, (B, T), generator=gen, device=device, dtype=torch.int64).to(torch.int32)


def make_x(B: int, T: int, d: int, gen: torch.Generator, device="cpu") -> torch.Tensor:
    """Residual-stream input x ~ N(0, 1), fp32, [B, T, d]."""
    return _randn((B, T, d), gen, device)


def ragged_positions(wl: Workload):
    """Start positions of a ragged decode workload: sequence b at
    round((2b + 1) P / B), evenly spread over 0..2P (mean P)."""
    return [int(round((2 * b + 1) * wl.P / wl.B)) for b in range(wl.B)]


def max_start(wl: Workload) -> int:
    return max(ragged_positions(wl)) if wl.ragged else wl.P


def make_cache(shape: BlockShape, B: int, P: int, cap: int, gen: torch.Generator, device="cpu",
               fill=0.0):
    """K and V caches [B, n_kv, cap, hd]; rows 0..P-1 ~ N(0,1), rows P.. = `fill`."""
    wd = shape.torch_dtype()
    kc = torch.full((B, shape.n_kv_heads, cap, shape.head_dim), fill, dtype=wd, device=device)
    vc = torch.full_like(kc, fill)
    if P > 0:
        kc[:, :, :P] = _randn((B, shape.n_kv_heads, P, shape.head_dim), gen, device, out_dtype=wd)
        vc[:, :, :P] = _randn((B, shape.n_kv_heads, P, shape.head_dim), gen, device, out_dtype=wd)
    return kc, vc


def make_inputs(wl: Workload, device="cpu", cap: Optional[int] = None):
    """All inputs of one workload: weights, x, caches (with capacity `cap`)."""
    w, gen = make_weights(wl.shape, wl.seed, device)
    x = make_x(wl.B, wl.T, wl.shape.d_model, gen, device)
    if cap is None:
        cap = cache_capacity(max_start(wl) + wl.T)
    kc, vc = make_cache(wl.shape, wl.B, max_start(wl), cap, gen, device)
    return {"weights": w, "x": x, "k_cache": kc, "v_cache": vc, "cap": cap}
