"""llb_block_decode_noalloc (the decode on the library's static scratch) against
llb_block_decode (the same decode on a caller's workspace), through the C ABI.

Both run the same kernels on the same inputs, so y and the written cache rows
must agree bit for bit.  Two calls in a row on one block, the second with a
smaller batch and position, show that the scratch's previous contents do not
leak into a later call; a call beyond the scratch's size is refused before
anything is queued.  Inputs are drawn on the GPU (this compares two GPU paths;
the decode itself is held to the oracle by the other tests).
"""
import pytest
import torch

import workloads
from dense_decoder_only_amd import llb

pytestmark = pytest.mark.gpu


def _note(msg):
    print(f"[gpu-test] {msg}", flush=True)


@pytest.mark.parametrize("name,calls", [
    ("8b", [(32, 1000), (8, 300)]),
    ("70b", [(64, 4096), (16, 129)]),
])
def test_noalloc_decode_matches_workspace_decode(name, calls):
    shp = workloads.LLAMA31_8B if name == "8b" else workloads.LLAMA31_70B
    w, gen = workloads.make_weights(shp, 31, device="cuda")
    cap = workloads.cache_capacity(max(P for _, P in calls) + 1)
    blk = llb.llb_block_create(llb.make_config(shp, cap), w)
    try:
        del w
        for B, P in calls:
            _note(f"noalloc {name} decode B={B} P={P}")
            x = workloads.make_x(B, 1, shp.d_model, gen, device="cuda")
            kc, vc = workloads.make_cache(shp, B, P, cap, gen, device="cuda")
            kc2, vc2 = kc.clone(), vc.clone()
            y1 = torch.full_like(x, float("nan"))
            y2 = torch.full_like(x, float("nan"))
            ws = llb.workspace(blk, B, 1)
            llb.llb_block_decode(blk, x, y1, B, P, kc, vc, cap, ws)
            llb.llb_block_decode_noalloc(blk, x, y2, B, P, kc2, vc2, cap)
            torch.cuda.synchronize()
            assert torch.isfinite(y1).all()
            assert torch.equal(y1, y2)
            assert torch.equal(kc, kc2) and torch.equal(vc, vc2)
            del ws
    finally:
        llb.llb_block_destroy(blk)


def test_noalloc_decode_refuses_calls_beyond_its_scratch():
    """The 8B block over 1024 sequences needs about 80 MB of workspace, more
    than the 64 MiB scratch: LLB_E_CAPACITY, and nothing is written."""
    shp = workloads.LLAMA31_8B
    w, gen = workloads.make_weights(shp, 32, device="cuda")
    cap = 64
    blk = llb.llb_block_create(llb.make_config(shp, cap), w)
    try:
        B, P = 1024, 10
        assert llb.llb_block_workspace_bytes(blk, B, 1) > (64 << 20)
        x = workloads.make_x(B, 1, shp.d_model, gen, device="cuda")
        kc, vc = workloads.make_cache(shp, B, P, cap, gen, device="cuda")
        k0 = kc.clone()
        y = torch.full_like(x, 7.0)
        _note("noalloc refusal B=1024")
        with pytest.raises(llb.LlbError) as ei:
            llb.llb_block_decode_noalloc(blk, x, y, B, P, kc, vc, cap)
        assert ei.value.status == llb.LLB_E_CAPACITY
        assert "static scratch" in str(ei.value)
        torch.cuda.synchronize()
        assert torch.all(y == 7.0) and torch.equal(kc, k0)
        # a call that fits still runs on the same block afterwards
        B2 = 4
        x2 = workloads.make_x(B2, 1, shp.d_model, gen, device="cuda")
        kc2, vc2 = workloads.make_cache(shp, B2, P, cap, gen, device="cuda")
        y2 = torch.empty_like(x2)
        llb.llb_block_decode_noalloc(blk, x2, y2, B2, P, kc2, vc2, cap)
        torch.cuda.synchronize()
        assert torch.isfinite(y2).all()
    finally:
        llb.llb_block_destroy(blk)
