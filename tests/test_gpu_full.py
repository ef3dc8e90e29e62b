"""Block parity at the full workload sizes, in the launch configuration that
bench.py times (same entry points, shapes and dtypes).

  * 8B prefill (B=1, T=2048), 8B chunked prefill (B=1, T=2048 at start 2048) and
    8B decode (B=32, P=1000): every output row.
  * 70B decode (B=64, P=4096, llama3-scaled RoPE): every output row.
  * 8B ragged decode (B=32, start positions spread over 0..2000): every row, each
    against the oracle on its own sequence.
  * 70B long prefill (B=1, T=16384): keys/values for all 16384 tokens are checked
    against the oracle; y on a fixed set of sampled rows (first, last, tile edges),
    which the oracle computes one by one (a causal block's row t depends only on
    tokens 0..t).
Bar on y: max|gpu - oracle| / rms(oracle) <= 2e-2; on the written bf16 cache rows, per
element |gpu - oracle| <= 2^-8 |oracle| + 1e-2 rms(oracle) (bf16 storage plus operand rounding).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import GpuBlock, bf16_err, note, rel_err

pytestmark = pytest.mark.gpu

C5_ROWS = [0, 1, 31, 32, 63, 64, 255, 256, 1000, 4095, 4096, 8191, 8192, 12345, 16320, 16351,
           16352, 16382, 16383]


def _inputs(wl):
    cap = workloads.cache_capacity(workloads.max_start(wl) + wl.T)
    return workloads.make_inputs(wl, cap=cap)


@pytest.mark.parametrize("name", ["8b_bf16_prefill", "70b_bf16_prefill", "8b_bf16_chunked_prefill"])
def test_full_prefill(name):
    wl = workloads.get(name)
    note(f"full {name}: generating inputs")
    inp = _inputs(wl)
    cap = inp["cap"]
    gb = GpuBlock(wl.shape, inp["weights"], max_positions=cap)
    try:
        kd, vd = inp["k_cache"].cuda(), inp["v_cache"].cuda()
        note(f"full {name}: GPU prefill B={wl.B} T={wl.T} at start {wl.P}")
        y = gb.prefill_at(inp["x"].cuda(), kd, vd, wl.P) if wl.P else gb.prefill(inp["x"].cuda(), kd, vd)
        torch.cuda.synchronize()
        y, kd, vd = y.cpu(), kd.cpu(), vd.cpu()
    finally:
        gb.close()
    rows = C5_ROWS if wl.T > 4096 else None
    note(f"full {name}: oracle (rows={'sampled' if rows else 'all'})")
    y_ref, k_ref, v_ref = oracle.block_forward(wl.shape, inp["weights"], inp["x"], inp["k_cache"],
                                               inp["v_cache"], wl.P, rows=rows)
    if rows is not None:
        y = y[:, rows]
    e_y = rel_err(y, y_ref)
    e_k = bf16_err(kd[:, :, wl.P:wl.P + wl.T], k_ref)
    e_v = bf16_err(vd[:, :, wl.P:wl.P + wl.T], v_ref)
    assert torch.equal(kd[:, :, :wl.P], inp["k_cache"][:, :, :wl.P])
    note(f"full {name}: y {e_y:.3e} k {e_k:.3f} v {e_v:.3f}")
    assert e_y <= 2e-2
    assert e_k <= 1.0 and e_v <= 1.0


@pytest.mark.parametrize("name", ["8b_bf16_decode", "70b_bf16_decode"])
def test_full_decode(name):
    wl = workloads.get(name)
    note(f"full {name}: generating inputs")
    inp = _inputs(wl)
    cap = inp["cap"]
    gb = GpuBlock(wl.shape, inp["weights"], max_positions=cap)
    try:
        kd, vd = inp["k_cache"].cuda(), inp["v_cache"].cuda()
        note(f"full {name}: GPU decode B={wl.B} P={wl.P}")
        y = gb.decode(inp["x"].cuda(), kd, vd, wl.P)
        torch.cuda.synchronize()
        y, kd, vd = y.cpu(), kd.cpu(), vd.cpu()
    finally:
        gb.close()
    note(f"full {name}: oracle")
    y_ref, k_ref, v_ref = oracle.block_forward(wl.shape, inp["weights"], inp["x"], inp["k_cache"],
                                               inp["v_cache"], wl.P)
    e_y = rel_err(y, y_ref)
    e_k = bf16_err(kd[:, :, wl.P:wl.P + 1], k_ref)
    e_v = bf16_err(vd[:, :, wl.P:wl.P + 1], v_ref)
    note(f"full {name}: y {e_y:.3e} k {e_k:.3f} v {e_v:.3f}")
    assert e_y <= 2e-2
    assert e_k <= 1.0 and e_v <= 1.0
    assert torch.equal(kd[:, :, :wl.P], inp["k_cache"][:, :, :wl.P])


def test_full_ragged_decode():
    """8B ragged decode (B=32, start positions spread over 0..2000): every row
    against the oracle run on its own sequence at its own position."""
    from dense_decoder_only_amd import llb
    wl = workloads.get("8b_bf16_ragged_decode")
    pos = workloads.ragged_positions(wl)
    note("full 8b_bf16_ragged_decode: generating inputs")
    inp = _inputs(wl)
    cap = inp["cap"]
    gb = GpuBlock(wl.shape, inp["weights"], max_positions=cap)
    try:
        kd, vd = inp["k_cache"].cuda(), inp["v_cache"].cuda()
        y = torch.empty(wl.B, 1, wl.shape.d_model, device="cuda")
        note(f"full 8b_bf16_ragged_decode: GPU decode B={wl.B} positions {min(pos)}..{max(pos)}")
        llb.llb_block_decode_ragged(gb.blk, inp["x"].cuda(), y, wl.B, pos, kd, vd, cap, gb.workspace(wl.B, 1))
        torch.cuda.synchronize()
        y, kd, vd = y.cpu(), kd.cpu(), vd.cpu()
    finally:
        gb.close()
    note("full 8b_bf16_ragged_decode: oracle per sequence")
    e_y = e_k = 0.0
    for b, p in enumerate(pos):
        sl = slice(b, b + 1)
        y_ref, k_ref, v_ref = oracle.block_forward(wl.shape, inp["weights"], inp["x"][sl], inp["k_cache"][sl],
                                                   inp["v_cache"][sl], p)
        e_y = max(e_y, rel_err(y[sl], y_ref))
        e_k = max(e_k, bf16_err(kd[sl, :, p:p + 1], k_ref), bf16_err(vd[sl, :, p:p + 1], v_ref))
    note(f"full 8b_bf16_ragged_decode: worst y {e_y:.3e} worst k/v {e_k:.3f}")
    assert e_y <= 2e-2 and e_k <= 1.0
