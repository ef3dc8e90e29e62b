"""Python binding of the C ABI in include/llb.h (argument marshalling only).

Every function has the name of its C counterpart and forwards to it through
ctypes; all compute runs in the HIP library.  Tensors are torch CUDA (ROCm)
tensors; their data pointers and torch's current stream are handed over as
plain pointers.  If the library is not built, loading fails loudly: there is
no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "_lib", "libllb.so")

LLB_OK = 0
LLB_E_INVALID = -1
LLB_E_UNSUPPORTED = -2
LLB_E_CAPACITY = -3
LLB_E_HIP = -4
LLB_E_NOMEM = -5
LLB_F32 = 0
LLB_BF16 = 1

STATUS_NAMES = {0: "LLB_OK", -1: "LLB_E_INVALID", -2: "LLB_E_UNSUPPORTED", -3: "LLB_E_CAPACITY",
                -4: "LLB_E_HIP", -5: "LLB_E_NOMEM"}

EXPORTED = ("llb_block_create", "llb_block_destroy", "llb_block_workspace_bytes",
            "llb_block_prefill", "llb_block_prefill_at", "llb_block_decode", "llb_block_decode_ragged", "llb_kv_append", "llb_attention_prefill",
            "llb_attention_decode", "llb_attention_decode_ragged", "llb_attention_workspace_bytes", "llb_block_set_stage_timing",
            "llb_block_stage_times", "llb_gemm_num_tiles", "llb_gemm_tile_info", "llb_block_set_tiles", "llb_block_set_decode_kernels",
            "llb_model_create", "llb_model_destroy", "llb_model_workspace_bytes", "llb_model_forward",
            "llb_block_workspace_layout", "llb_block_decode_noalloc", "llb_probe_hbm_read",
            "llb_probe_hbm_copy", "llb_probe_mfma_bf16", "llb_last_error")

STAGES = ("qkv", "attention", "o_proj", "gate_up", "down")


class llb_config(ctypes.Structure):
    _fields_ = [
        ("d_model", ctypes.c_int32), ("n_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("d_ff", ctypes.c_int32), ("eps", ctypes.c_float),
        ("rope_theta", ctypes.c_float), ("rope_scaling", ctypes.c_int32),
        ("rs_factor", ctypes.c_float), ("rs_low_freq_factor", ctypes.c_float),
        ("rs_high_freq_factor", ctypes.c_float), ("rs_orig_max_pos", ctypes.c_int32),
        ("max_positions", ctypes.c_int32), ("wdtype", ctypes.c_int32),
    ]


class llb_weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("attn_norm", "wq", "wk", "wv", "wo", "ffn_norm", "w_gate", "w_up", "w_down")]


class LlbError(RuntimeError):
    def __init__(self, status: int, what: str, msg: str):
        super().__init__(f"{what}: {STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


_lib = None


def load_library(path: str = LIB_PATH):
    """Loads libllb.so once; raises if it is missing (no CPU fallback exists)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"HIP block library not built: {path} is missing "
                           "(run `python -m dense_decoder_only_amd.build`)")
    lib = ctypes.CDLL(path)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    lib.llb_block_create.argtypes = [ctypes.POINTER(llb_config), ctypes.POINTER(llb_weights), vp,
                                     ctypes.POINTER(vp)]
    lib.llb_block_create.restype = ctypes.c_int
    lib.llb_block_destroy.argtypes = [vp]
    lib.llb_block_destroy.restype = ctypes.c_int
    lib.llb_block_workspace_bytes.argtypes = [vp, i32, i32]
    lib.llb_block_workspace_bytes.restype = sz
    lib.llb_block_prefill.argtypes = [vp, vp, vp, i32, i32, vp, vp, i32, vp, sz, vp]
    lib.llb_block_prefill.restype = ctypes.c_int
    lib.llb_block_prefill_at.argtypes = [vp, vp, vp, i32, i32, i32, vp, vp, i32, vp, sz, vp]
    lib.llb_block_prefill_at.restype = ctypes.c_int
    lib.llb_block_decode.argtypes = [vp, vp, vp, i32, i32, vp, vp, i32, vp, sz, vp]
    lib.llb_block_decode_ragged.argtypes = [vp, vp, vp, i32, ctypes.POINTER(i32), vp, vp, i32, vp, sz, vp]
    lib.llb_block_decode_ragged.restype = ctypes.c_int
    lib.llb_block_decode.restype = ctypes.c_int
    lib.llb_kv_append.argtypes = [vp, vp, vp, i32, i32, i32, i32, vp, vp, vp]
    lib.llb_kv_append.restype = ctypes.c_int
    lib.llb_attention_prefill.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, vp]
    lib.llb_attention_prefill.restype = ctypes.c_int
    lib.llb_attention_decode.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, vp, sz, vp]
    lib.llb_attention_decode.restype = ctypes.c_int
    lib.llb_attention_decode_ragged.argtypes = [vp, vp, vp, vp, vp, i32, ctypes.POINTER(i32), i32, vp, sz, vp]
    lib.llb_attention_decode_ragged.restype = ctypes.c_int
    lib.llb_attention_workspace_bytes.argtypes = [vp, i32, i32]
    lib.llb_attention_workspace_bytes.restype = sz
    lib.llb_block_set_stage_timing.argtypes = [vp, i32]
    lib.llb_block_set_stage_timing.restype = ctypes.c_int
    lib.llb_block_stage_times.argtypes = [vp, ctypes.POINTER(ctypes.c_float), ctypes.POINTER(i32)]
    lib.llb_block_stage_times.restype = ctypes.c_int
    lib.llb_gemm_num_tiles.argtypes = []
    lib.llb_gemm_num_tiles.restype = i32
    lib.llb_gemm_tile_info.argtypes = [i32, ctypes.POINTER(i32), ctypes.POINTER(i32)]
    lib.llb_gemm_tile_info.restype = ctypes.c_int
    lib.llb_block_set_tiles.argtypes = [vp, i32, i32, i32, i32]
    lib.llb_block_set_tiles.restype = ctypes.c_int
    lib.llb_block_set_decode_kernels.argtypes = [vp, i32, i32, i32, i32]
    lib.llb_block_set_decode_kernels.restype = ctypes.c_int
    lib.llb_model_create.argtypes = [ctypes.POINTER(llb_config), i32, i32, vp, ctypes.POINTER(llb_weights), vp, vp,
                                     vp, ctypes.POINTER(vp)]
    lib.llb_model_create.restype = ctypes.c_int
    lib.llb_model_destroy.argtypes = [vp]
    lib.llb_model_destroy.restype = ctypes.c_int
    lib.llb_model_workspace_bytes.argtypes = [vp, i32, i32, i32]
    lib.llb_model_workspace_bytes.restype = sz
    lib.llb_model_forward.argtypes = [vp, vp, i32, i32, i32, ctypes.POINTER(vp), ctypes.POINTER(vp), i32, i32, vp,
                                      vp, sz, vp]
    lib.llb_model_forward.restype = ctypes.c_int
    lib.llb_block_decode_noalloc.argtypes = [vp, vp, vp, i32, i32, vp, vp, i32, vp]
    lib.llb_block_decode_noalloc.restype = ctypes.c_int
    lib.llb_block_workspace_layout.argtypes = [vp, i32, i32, i32, ctypes.POINTER(sz)]
    lib.llb_block_workspace_layout.restype = ctypes.c_int
    lib.llb_probe_hbm_read.argtypes = [vp, sz, i32, vp, vp]
    lib.llb_probe_hbm_read.restype = ctypes.c_int
    lib.llb_probe_hbm_copy.argtypes = [vp, vp, sz, i32, vp]
    lib.llb_probe_hbm_copy.restype = ctypes.c_int
    lib.llb_probe_mfma_bf16.argtypes = [i32, i32, vp, vp]
    lib.llb_probe_mfma_bf16.restype = ctypes.c_int
    lib.llb_last_error.argtypes = []
    lib.llb_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def llb_last_error() -> str:
    return load_library().llb_last_error().decode()


def _check(status: int, what: str):
    if status != LLB_OK:
        raise LlbError(status, what, llb_last_error())


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to the block library must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def make_config(shape, max_positions: int) -> llb_config:
    """llb_config from an object with the block's hyper-parameters (d_model,
    n_heads, n_kv_heads, head_dim, d_ff, eps, rope_theta, rope_scaling, rs_*,
    dtype 'bf16' | 'f32')."""
    return llb_config(
        d_model=shape.d_model, n_heads=shape.n_heads, n_kv_heads=shape.n_kv_heads,
        head_dim=shape.head_dim, d_ff=shape.d_ff, eps=shape.eps, rope_theta=shape.rope_theta,
        rope_scaling=1 if shape.rope_scaling else 0, rs_factor=shape.rs_factor,
        rs_low_freq_factor=shape.rs_low_freq_factor, rs_high_freq_factor=shape.rs_high_freq_factor,
        rs_orig_max_pos=shape.rs_orig_max_pos, max_positions=max_positions,
        wdtype=LLB_BF16 if shape.dtype == "bf16" else LLB_F32)


class Block:
    """A created block handle (llb_block*).  Destroy with llb_block_destroy."""

    def __init__(self, handle: int, cfg: llb_config):
        self.handle = ctypes.c_void_p(handle)
        self.cfg = cfg

    @property
    def ptr(self):
        return self.handle


def llb_block_create(cfg: llb_config, weights: Dict[str, torch.Tensor], stream=None) -> Block:
    lib = load_library()
    w = llb_weights(**{k: weights[k].data_ptr() for k in
                       ("attn_norm", "wq", "wk", "wv", "wo", "ffn_norm", "w_gate", "w_up", "w_down")})
    for k, t in weights.items():
        if not t.is_contiguous():
            raise ValueError(f"weight {k} must be contiguous")
    out = ctypes.c_void_p()
    _check(lib.llb_block_create(ctypes.byref(cfg), ctypes.byref(w), _stream(stream), ctypes.byref(out)),
           "llb_block_create")
    return Block(out.value, cfg)


def llb_block_destroy(blk: Block) -> None:
    _check(load_library().llb_block_destroy(blk.handle), "llb_block_destroy")
    blk.handle = ctypes.c_void_p(0)


def llb_block_workspace_bytes(blk: Block, B: int, T: int) -> int:
    return int(load_library().llb_block_workspace_bytes(blk.handle, B, T))


def llb_block_prefill(blk: Block, x, y, B, T, k_cache, v_cache, cache_cap, ws, stream=None):
    _check(load_library().llb_block_prefill(blk.handle, _ptr(x), _ptr(y), B, T, _ptr(k_cache),
                                            _ptr(v_cache), cache_cap, _ptr(ws), ws.numel() * ws.element_size(),
                                            _stream(stream)), "llb_block_prefill")


def llb_block_prefill_at(blk: Block, x, y, B, T, start_pos, k_cache, v_cache, cache_cap, ws, stream=None):
    _check(load_library().llb_block_prefill_at(blk.handle, _ptr(x), _ptr(y), B, T, start_pos, _ptr(k_cache),
                                               _ptr(v_cache), cache_cap, _ptr(ws), ws.numel() * ws.element_size(),
                                               _stream(stream)), "llb_block_prefill_at")


def llb_block_decode(blk: Block, x, y, B, start_pos, k_cache, v_cache, cache_cap, ws, stream=None):
    _check(load_library().llb_block_decode(blk.handle, _ptr(x), _ptr(y), B, start_pos, _ptr(k_cache),
                                           _ptr(v_cache), cache_cap, _ptr(ws), ws.numel() * ws.element_size(),
                                           _stream(stream)), "llb_block_decode")


def llb_block_decode_noalloc(blk: Block, x, y, B, start_pos, k_cache, v_cache, cache_cap, stream=None):
    """llb_block_decode on the library's static scratch: no workspace argument."""
    _check(load_library().llb_block_decode_noalloc(blk.handle, _ptr(x), _ptr(y), B, start_pos, _ptr(k_cache),
                                                   _ptr(v_cache), cache_cap, _stream(stream)),
           "llb_block_decode_noalloc")


def llb_block_decode_ragged(blk: Block, x, y, B, start_pos, k_cache, v_cache, cache_cap, ws, stream=None):
    """start_pos: B host integers (a list or a CPU tensor), one position per sequence."""
    if len(start_pos) != B:
        raise ValueError("start_pos must have B entries")
    pos = (ctypes.c_int32 * B)(*[int(p) for p in start_pos])
    _check(load_library().llb_block_decode_ragged(blk.handle, _ptr(x), _ptr(y), B, pos, _ptr(k_cache),
                                                  _ptr(v_cache), cache_cap, _ptr(ws),
                                                  ws.numel() * ws.element_size(), _stream(stream)),
           "llb_block_decode_ragged")


def llb_kv_append(blk: Block, k_cache, v_cache, B, cache_cap, start_pos, n_new, k_new, v_new,
                  stream=None):
    _check(load_library().llb_kv_append(blk.handle, _ptr(k_cache), _ptr(v_cache), B, cache_cap,
                                        start_pos, n_new, _ptr(k_new), _ptr(v_new), _stream(stream)),
           "llb_kv_append")


def llb_attention_prefill(blk: Block, q, k_cache, v_cache, o, B, T, start_pos, cache_cap, stream=None):
    _check(load_library().llb_attention_prefill(blk.handle, _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                                _ptr(o), B, T, start_pos, cache_cap, _stream(stream)),
           "llb_attention_prefill")


def llb_attention_workspace_bytes(blk: Block, B: int, n_keys: int) -> int:
    return int(load_library().llb_attention_workspace_bytes(blk.handle, B, n_keys))


def llb_attention_decode(blk: Block, q, k_cache, v_cache, o, B, start_pos, cache_cap, ws, stream=None):
    _check(load_library().llb_attention_decode(blk.handle, _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                               _ptr(o), B, start_pos, cache_cap, _ptr(ws),
                                               ws.numel() * ws.element_size(), _stream(stream)),
           "llb_attention_decode")


def llb_attention_decode_ragged(blk: Block, q, k_cache, v_cache, o, B, start_pos, cache_cap, ws, stream=None):
    """start_pos: B host integers, one position per sequence."""
    if len(start_pos) != B:
        raise ValueError("start_pos must have B entries")
    pos = (ctypes.c_int32 * B)(*[int(p) for p in start_pos])
    _check(load_library().llb_attention_decode_ragged(blk.handle, _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(o),
                                                      B, pos, cache_cap, _ptr(ws), ws.numel() * ws.element_size(),
                                                      _stream(stream)), "llb_attention_decode_ragged")


class Model:
    """A created model handle (llb_model*).  Destroy with llb_model_destroy."""

    def __init__(self, handle: int, cfg: llb_config, n_layers: int, vocab: int):
        self.handle = ctypes.c_void_p(handle)
        self.cfg = cfg
        self.n_layers = n_layers
        self.vocab = vocab


_BLOCK_KEYS = ("attn_norm", "wq", "wk", "wv", "wo", "ffn_norm", "w_gate", "w_up", "w_down")


def llb_model_create(cfg: llb_config, layers, vocab: int, embed: torch.Tensor, final_norm: torch.Tensor,
                     lm_head: torch.Tensor, stream=None) -> Model:
    """layers: a list of per-layer weight dicts (device tensors, as for llb_block_create)."""
    for t in [embed, final_norm, lm_head] + [w[k] for w in layers for k in _BLOCK_KEYS]:
        if not t.is_contiguous():
            raise ValueError("model weights must be contiguous")
    arr = (llb_weights * max(1, len(layers)))()
    for i, w in enumerate(layers):
        arr[i] = llb_weights(**{k: w[k].data_ptr() for k in _BLOCK_KEYS})
    out = ctypes.c_void_p()
    _check(load_library().llb_model_create(ctypes.byref(cfg), len(layers), vocab, _ptr(embed), arr, _ptr(final_norm),
                                           _ptr(lm_head), _stream(stream), ctypes.byref(out)), "llb_model_create")
    return Model(out.value, cfg, len(layers), vocab)


def llb_model_destroy(m: Model) -> None:
    _check(load_library().llb_model_destroy(m.handle), "llb_model_destroy")
    m.handle = ctypes.c_void_p(0)


def llb_model_workspace_bytes(m: Model, B: int, T: int, last_only: bool) -> int:
    return int(load_library().llb_model_workspace_bytes(m.handle, B, T, 1 if last_only else 0))


def model_workspace(m: Model, B: int, T: int, last_only: bool, device="cuda") -> torch.Tensor:
    n = llb_model_workspace_bytes(m, B, T, last_only)
    if n == 0:
        raise ValueError("llb_model_workspace_bytes returned 0 (bad handle or sizes)")
    return torch.empty(n, dtype=torch.uint8, device=device)


def llb_model_forward(m: Model, tokens, B, T, start_pos, k_caches, v_caches, cache_cap, last_only, logits, ws,
                      stream=None):
    """tokens: int32 device tensor [B, T]; k_caches / v_caches: lists of n_layers device tensors."""
    if tokens.dtype != torch.int32:
        raise ValueError("tokens must be int32")
    if len(k_caches) != m.n_layers or len(v_caches) != m.n_layers:
        raise ValueError("one K and one V cache per layer")
    n = max(1, m.n_layers)
    kc = (ctypes.c_void_p * n)(*[c.data_ptr() for c in k_caches])
    vc = (ctypes.c_void_p * n)(*[c.data_ptr() for c in v_caches])
    _check(load_library().llb_model_forward(m.handle, _ptr(tokens), B, T, start_pos, kc, vc, cache_cap,
                                            1 if last_only else 0, _ptr(logits), _ptr(ws),
                                            ws.numel() * ws.element_size(), _stream(stream)), "llb_model_forward")


def llb_probe_hbm_read(src, sink, n_workgroups: int, stream=None) -> None:
    """Streams src (a contiguous device tensor) once; sink: n_workgroups uint32 words."""
    _check(load_library().llb_probe_hbm_read(_ptr(src), src.numel() * src.element_size(), n_workgroups,
                                             _ptr(sink), _stream(stream)), "llb_probe_hbm_read")


def llb_probe_hbm_copy(dst, src, n_workgroups: int, stream=None) -> None:
    _check(load_library().llb_probe_hbm_copy(_ptr(dst), _ptr(src), src.numel() * src.element_size(),
                                             n_workgroups, _stream(stream)), "llb_probe_hbm_copy")


def llb_probe_mfma_bf16(n_workgroups: int, iters: int, sink, stream=None) -> None:
    """sink: 4 * n_workgroups floats."""
    _check(load_library().llb_probe_mfma_bf16(n_workgroups, iters, _ptr(sink), _stream(stream)),
           "llb_probe_mfma_bf16")


def llb_gemm_num_tiles() -> int:
    return int(load_library().llb_gemm_num_tiles())


def llb_gemm_tile_info(cfg: int):
    """(BM, BN) of prefill tile configuration `cfg`."""
    bm, bn = ctypes.c_int32(), ctypes.c_int32()
    _check(load_library().llb_gemm_tile_info(cfg, ctypes.byref(bm), ctypes.byref(bn)), "llb_gemm_tile_info")
    return int(bm.value), int(bn.value)


def llb_block_set_tiles(blk: Block, qkv: int = -1, o: int = -1, gate_up: int = -1, down: int = -1) -> None:
    _check(load_library().llb_block_set_tiles(blk.handle, qkv, o, gate_up, down), "llb_block_set_tiles")


def llb_block_set_decode_kernels(blk: Block, qkv: int = -1, o: int = -1, gate_up: int = -1, down: int = -1) -> None:
    _check(load_library().llb_block_set_decode_kernels(blk.handle, qkv, o, gate_up, down),
           "llb_block_set_decode_kernels")


def llb_block_set_stage_timing(blk: Block, enable: bool) -> None:
    _check(load_library().llb_block_set_stage_timing(blk.handle, 1 if enable else 0),
           "llb_block_set_stage_timing")


def llb_block_stage_times(blk: Block):
    """(summed milliseconds per stage as a dict, number of recorded calls)."""
    ms = (ctypes.c_float * 5)()
    n = ctypes.c_int32()
    _check(load_library().llb_block_stage_times(blk.handle, ms, ctypes.byref(n)), "llb_block_stage_times")
    return dict(zip(STAGES, [float(v) for v in ms])), int(n.value)


WS_REGIONS = ("q", "o", "h", "u")


def llb_block_workspace_layout(blk: Block, B: int, T: int, decode: bool) -> Dict[str, int]:
    """Byte offsets of the intermediate results Q, O, h, u in a call's workspace."""
    offs = (ctypes.c_size_t * 4)()
    _check(load_library().llb_block_workspace_layout(blk.handle, B, T, 1 if decode else 0, offs),
           "llb_block_workspace_layout")
    return dict(zip(WS_REGIONS, [int(v) for v in offs]))


def workspace(blk: Block, B: int, T: int, device="cuda") -> torch.Tensor:
    """A uint8 device tensor of llb_block_workspace_bytes(B, T) bytes."""
    n = llb_block_workspace_bytes(blk, B, T)
    if n == 0:
        raise ValueError("llb_block_workspace_bytes returned 0 (bad handle or sizes)")
    return torch.empty(n, dtype=torch.uint8, device=device)
