"""The block's calls launch kernels only (no allocation, no memset, no host
synchronisation), so a caller may capture them into a HIP graph.  Each test
captures one call, replays it several times with eager calls and host
synchronisations in between, and checks every replay against the eager call
bit for bit (outputs and the cache rows the call writes)."""
from __future__ import annotations

import pytest
import torch

import workloads
from gpu_util import GpuBlock, gen_inputs, note, shape

pytestmark = pytest.mark.gpu

SHP = dict(d_model=512, n_heads=8, n_kv_heads=2, head_dim=128, d_ff=768)


def _replays_match(call, outs, clear, n_replays=3):
    """call(stream) enqueues the work; outs: tensors it writes; clear() zeroes
    what the call writes (and does not read first).  Eager result, then graph
    replays with eager work between them, each compared bit for bit."""
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        call(s)
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call(torch.cuda.current_stream())
    torch.cuda.synchronize()
    for r in range(n_replays):
        clear()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, ref):
            assert torch.equal(o, e), f"replay {r} differs from the eager call"
        with torch.cuda.stream(s):
            call(s)  # eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("B,P", [(4, 100), (40, 300), (64, 200)])
def test_decode_replays_in_a_graph(B, P):
    from dense_decoder_only_amd import llb
    shp = shape(**SHP)
    cap = workloads.cache_capacity(P + 1)
    w, x, kc, vc = gen_inputs(shp, 41 + B, B, 1, P, cap)
    note(f"graph replay: decode B={B} P={P}")
    gb = GpuBlock(shp, w, max_positions=cap)
    try:
        xd, kd, vd = x.cuda(), kc.cuda(), vc.cuda()
        y = torch.empty_like(xd)
        ws = gb.workspace(B, 1)
        def clear():
            y.zero_()
            kd[:, :, P].zero_()
            vd[:, :, P].zero_()
        _replays_match(lambda st: llb.llb_block_decode(gb.blk, xd, y, B, P, kd, vd, cap, ws, stream=st),
                       [y, kd, vd], clear)
    finally:
        gb.close()


def test_ragged_decode_replays_in_a_graph():
    from dense_decoder_only_amd import llb
    shp = shape(**SHP)
    B, P = 6, 150
    pos = [0, 17, 150, 63, 99, 150]
    cap = workloads.cache_capacity(P + 1)
    w, x, kc, vc = gen_inputs(shp, 47, B, 1, P, cap)
    note("graph replay: ragged decode")
    gb = GpuBlock(shp, w, max_positions=cap)
    try:
        xd, kd, vd = x.cuda(), kc.cuda(), vc.cuda()
        y = torch.empty_like(xd)
        ws = gb.workspace(B, 1)
        def clear():
            y.zero_()
            for b, p in enumerate(pos):
                kd[b, :, p].zero_()
                vd[b, :, p].zero_()
        _replays_match(lambda st: llb.llb_block_decode_ragged(gb.blk, xd, y, B, pos, kd, vd, cap, ws, stream=st),
                       [y, kd, vd], clear)
    finally:
        gb.close()


def test_prefill_replays_in_a_graph():
    from dense_decoder_only_amd import llb
    shp = shape(**SHP)
    B, T = 2, 96
    cap = workloads.cache_capacity(T)
    w, x, kc, vc = gen_inputs(shp, 43, B, T, 0, cap)
    note("graph replay: prefill")
    gb = GpuBlock(shp, w, max_positions=cap)
    try:
        xd, kd, vd = x.cuda(), kc.cuda(), vc.cuda()
        y = torch.empty_like(xd)
        ws = gb.workspace(B, T)
        def clear():
            y.zero_()
            kd[:, :, :T].zero_()
            vd[:, :, :T].zero_()
        _replays_match(lambda st: llb.llb_block_prefill(gb.blk, xd, y, B, T, kd, vd, cap, ws, stream=st),
                       [y, kd, vd], clear)
    finally:
        gb.close()
