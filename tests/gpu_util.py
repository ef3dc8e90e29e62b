"""Helpers for the GPU tests: upload seeded inputs, run the block through the C
ABI, and the parity metric max|gpu - oracle| / rms(oracle)."""
from __future__ import annotations

import dataclasses
import sys

import numpy as np
import torch

import oracle
import workloads
from dense_decoder_only_amd import llb

DEV = "cuda"


def note(msg: str):
    print(f"[gpu-test] {msg}", flush=True)
    sys.stdout.flush()


def rel_err(gpu, ref) -> float:
    g = oracle.to64(gpu)
    r = oracle.to64(ref)
    assert g.shape == r.shape, (g.shape, r.shape)
    rms = float(np.sqrt(np.mean(r * r)))
    return float(np.max(np.abs(g - r))) / rms


def bf16_err(gpu, ref, c=1e-2, mag=None) -> float:
    """Parity of a bf16-stored output, per element:
        |g_i - r_i| / (2^-8 |r_i| + 2^-8 mag_i + c rms(r));  <= 1 passes.

    2^-8 |r_i| is half a bf16 ulp of the stored value (8 significant bits), the
    rounding every bf16 output carries.  mag_i (optional) is the magnitude sum
    of the terms that were rounded to bf16 before being combined, e.g. the
    attention output over |v| (sum_n p_n |v_n|) when the weights p_n are rounded
    (2^-9 each) before P.V; 2^-8 mag_i allows two such roundings.  c rms(r)
    bounds the rest (errors from many rounded operands, random in sign)."""
    g = oracle.to64(gpu)
    r = oracle.to64(ref)
    assert g.shape == r.shape, (g.shape, r.shape)
    rms = float(np.sqrt(np.mean(r * r)))
    den = 2.0 ** -8 * np.abs(r) + c * rms
    if mag is not None:
        den = den + 2.0 ** -8 * oracle.to64(mag)
    return float(np.max(np.abs(g - r) / den))


def shape(**kw) -> workloads.BlockShape:
    return workloads.BlockShape(**kw)


def upload_weights(w):
    return {k: v.to(DEV).contiguous() for k, v in w.items()}


class GpuBlock:
    """A block created on the GPU from CPU weights, with its own workspace."""

    def __init__(self, shp: workloads.BlockShape, w_cpu, max_positions: int):
        self.shape = shp
        self.w_gpu = upload_weights(w_cpu)
        self.cfg = llb.make_config(shp, max_positions)
        self.blk = llb.llb_block_create(self.cfg, self.w_gpu)
        self.ws = {}

    def workspace(self, B, T):
        key = (B, T)
        if key not in self.ws:
            self.ws[key] = llb.workspace(self.blk, B, T)
        return self.ws[key]

    def prefill(self, x, kc, vc):
        B, T, _ = x.shape
        y = torch.empty_like(x)
        llb.llb_block_prefill(self.blk, x, y, B, T, kc, vc, kc.shape[2], self.workspace(B, T))
        return y

    def prefill_at(self, x, kc, vc, P):
        B, T, _ = x.shape
        y = torch.empty_like(x)
        llb.llb_block_prefill_at(self.blk, x, y, B, T, P, kc, vc, kc.shape[2], self.workspace(B, T))
        return y

    def decode(self, x, kc, vc, P):
        B = x.shape[0]
        y = torch.empty_like(x)
        llb.llb_block_decode(self.blk, x, y, B, P, kc, vc, kc.shape[2], self.workspace(B, 1))
        return y

    def close(self):
        if self.blk is not None and self.blk.handle.value:
            llb.llb_block_destroy(self.blk)
        self.blk = None


def gen_inputs(shp, seed, B, T, P, cap, fill=0.0):
    w, gen = workloads.make_weights(shp, seed)
    x = workloads.make_x(B, T, shp.d_model, gen)
    kc, vc = workloads.make_cache(shp, B, P, cap, gen, fill=fill)
    return w, x, kc, vc
