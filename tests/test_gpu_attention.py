"""Unit parity of the attention kernels (llb_attention_prefill / _decode) on
seeded bf16 queries, keys and values, against the oracle's fp64 attention fed
the same bf16 values.

Bar, per element: |gpu - oracle| <= 2^-8 |o| + 2^-8 sum_n p_n |v_n| + 1e-3 rms(o).
The output is stored in bf16 (half an ulp is 2^-8 of the value).  The prefill
kernel also rounds each softmax weight to bf16 before the P.V product (2^-9
relative per weight); with few visible keys these roundings do not average out
and reach 2^-9 sum_n p_n |v_n|, which the oracle gives as its attention over |v|.

Structured cases catch what random inputs hide: a dominant key must be
returned exactly, zero scores must give the plain mean of the visible values
(a dropped first key or an extra key moves it by one part in L), and rows
beyond the last visible key hold a large sentinel.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from dense_decoder_only_amd import llb
from gpu_util import bf16_err, note, rel_err, shape

pytestmark = pytest.mark.gpu

SENTINEL = 4096.0


def _block(G, Hkv=2, max_positions=8192):
    shp = shape(d_model=256, n_heads=G * Hkv, n_kv_heads=Hkv, head_dim=128, d_ff=256)
    w, _ = workloads.make_weights(shp, 0)
    w = {k: v.cuda() for k, v in w.items()}
    cfg = llb.make_config(shp, max_positions)
    return shp, llb.llb_block_create(cfg, w), w


def _rand(shape_, gen, scale=1.0):
    return (torch.randn(shape_, generator=gen) * scale).to(torch.bfloat16)


def _oracle_prefill(q, kc, vc, pos0, T):
    B = q.shape[0]
    out = []
    for b in range(B):
        o = oracle.attention(q[b], kc[b], vc[b], np.arange(pos0, pos0 + T), n_keys=pos0 + T)
        out.append(o.transpose(1, 0, 2).reshape(T, -1))
    return np.stack(out)


@pytest.mark.parametrize("G,B,T,pos0", [
    (4, 1, 1, 0), (4, 2, 31, 0), (4, 1, 64, 0), (4, 2, 100, 0), (4, 1, 300, 0),
    (8, 1, 130, 0), (1, 2, 70, 0), (2, 1, 65, 0),
    (4, 2, 50, 17), (8, 1, 33, 64), (4, 1, 1, 500),
    (4, 1, 1000, 0), (8, 1, 513, 37), (4, 2, 257, 300), (2, 1, 400, 5), (1, 1, 200, 3),
])
def test_attention_prefill_random(G, B, T, pos0):
    shp, blk, _ = _block(G)
    try:
        H, Hkv, hd = shp.n_heads, shp.n_kv_heads, 128
        cap = workloads.cache_capacity(pos0 + T)
        gen = torch.Generator().manual_seed(1000 + T + pos0 + G)
        q = _rand((B, H, T, hd), gen)
        kc = torch.full((B, Hkv, cap, hd), SENTINEL, dtype=torch.bfloat16)
        vc = kc.clone()
        kc[:, :, :pos0 + T] = _rand((B, Hkv, pos0 + T, hd), gen, 0.6)
        vc[:, :, :pos0 + T] = _rand((B, Hkv, pos0 + T, hd), gen)
        note(f"attn prefill G={G} B={B} T={T} pos0={pos0}")
        o = torch.empty(B, T, H * hd, dtype=torch.bfloat16, device="cuda")
        llb.llb_attention_prefill(blk, q.cuda(), kc.cuda(), vc.cuda(), o, B, T, pos0, cap)
        ref = _oracle_prefill(q, kc, vc, pos0, T)
        mag = _oracle_prefill(q, kc, vc.abs(), pos0, T)
        e = bf16_err(o.cpu(), ref, c=1e-3, mag=mag)
        note(f"  bf16 err {e:.3f} (max/rms {rel_err(o.cpu(), ref):.2e})")
        assert e <= 1.0
    finally:
        llb.llb_block_destroy(blk)


@pytest.mark.parametrize("G", [4, 8])
@pytest.mark.parametrize("shift,pos0,T", [(0, 0, 127), (1, 0, 127), (0, 200, 100), (1, 200, 100),
                                           (1, 0, 64), (1, 31, 33)])
def test_attention_prefill_structured_mask(shift, pos0, T, G):
    """Key n is 4 * e_(n mod 128); the query at position p is c * e_((p + shift) mod 128)
    with a score of 30 for a matching key and 0 otherwise.  shift=0: the query's
    own key dominates (dropping the diagonal from the mask would show); shift=1:
    the next, future key would dominate if the mask leaked it.  Softmax weights
    are exactly 1 or ~e^-30, so only the bf16 output rounding remains."""
    shp, blk, _ = _block(G)
    try:
        B, H, Hkv, hd = 1, shp.n_heads, 2, 128
        cap = workloads.cache_capacity(pos0 + T)
        gen = torch.Generator().manual_seed(77 + pos0 + T)
        kc = torch.zeros(B, Hkv, cap, hd, dtype=torch.bfloat16)
        for n in range(pos0 + T):
            kc[:, :, n, n % 128] = 4.0
        vc = _rand((B, Hkv, cap, hd), gen)
        q = torch.zeros(B, H, T, hd, dtype=torch.bfloat16)
        for t in range(T):
            q[:, :, t, (pos0 + t + shift) % 128] = 30.0 * math.sqrt(hd) / 4.0
        note(f"attn prefill structured G={G} shift={shift} pos0={pos0} T={T}")
        o = torch.empty(B, T, H * hd, dtype=torch.bfloat16, device="cuda")
        llb.llb_attention_prefill(blk, q.cuda(), kc.cuda(), vc.cuda(), o, B, T, pos0, cap)
        ref = _oracle_prefill(q, kc, vc, pos0, T)
        e = bf16_err(o.cpu(), ref, c=1e-3)
        note(f"  bf16 err {e:.3f}")
        assert e <= 1.0
    finally:
        llb.llb_block_destroy(blk)


@pytest.mark.parametrize("G", [4, 8])
def test_attention_prefill_growing_scores(G):
    """Scores rise along the keys (score of key n for the query at p is
    0.05 n + noise), so the softmax offset keeps moving up tile after tile:
    a running maximum that is not raised far enough, or a rescale that is
    applied to the wrong rows, shows as a relative error far above bf16."""
    shp, blk, _ = _block(G)
    try:
        B, H, Hkv, hd = 1, shp.n_heads, 2, 128
        T, pos0 = 900, 0
        cap = workloads.cache_capacity(pos0 + T)
        gen = torch.Generator().manual_seed(91)
        kc = _rand((B, Hkv, cap, hd), gen, 0.05)
        kc[:, :, :, 0] = (torch.arange(cap, dtype=torch.float32) * 0.05 / 4.0).to(torch.bfloat16)
        vc = _rand((B, Hkv, cap, hd), gen)
        q = _rand((B, H, T, hd), gen, 0.05)
        q[..., 0] = 4.0 * math.sqrt(hd)
        note("attn prefill growing scores")
        o = torch.empty(B, T, H * hd, dtype=torch.bfloat16, device="cuda")
        llb.llb_attention_prefill(blk, q.cuda(), kc.cuda(), vc.cuda(), o, B, T, pos0, cap)
        ref = _oracle_prefill(q, kc, vc, pos0, T)
        mag = _oracle_prefill(q, kc, vc.abs(), pos0, T)
        e = bf16_err(o.cpu(), ref, c=1e-3, mag=mag)
        note(f"  bf16 err {e:.3f} (max/rms {rel_err(o.cpu(), ref):.2e})")
        assert e <= 1.0
    finally:
        llb.llb_block_destroy(blk)


def _run_decode(blk, shp, q, kc, vc, P):
    B = q.shape[0]
    H, hd = shp.n_heads, 128
    cap = kc.shape[2]
    ws = torch.empty(llb.llb_attention_workspace_bytes(blk, B, P + 1), dtype=torch.uint8, device="cuda")
    o = torch.empty(B, H * hd, dtype=torch.bfloat16, device="cuda")
    llb.llb_attention_decode(blk, q.cuda(), kc.cuda(), vc.cuda(), o, B, P, cap, ws)
    return o.cpu()


def _oracle_decode(q, kc, vc, P):
    out = []
    for b in range(q.shape[0]):
        o = oracle.attention(q[b][:, None, :], kc[b], vc[b], [P], n_keys=P + 1)
        out.append(o[:, 0, :].reshape(-1))
    return np.stack(out)


@pytest.mark.parametrize("G,B,P,Hkv", [
    (4, 1, 0, 2), (4, 3, 1, 2), (4, 2, 14, 2), (4, 2, 15, 2), (4, 2, 16, 2), (4, 32, 1000, 2),
    (8, 2, 4096, 2), (1, 2, 200, 2), (2, 3, 77, 2), (8, 64, 129, 2), (8, 1, 16383, 2),
    # >= 128 (sequence, KV head) units: one workgroup per unit, chunks merged in LDS
    (4, 64, 300, 2), (2, 64, 17, 2), (1, 128, 40, 2),
    # the 8B and 70B decode shapes: 8 KV heads, 256 and 512 units, L = P + 1 keys
    (4, 32, 1000, 8), (8, 64, 4096, 8),
    # the same kernel at the first fused unit count and at ragged key counts
    (4, 16, 999, 8), (8, 16, 4095, 8), (8, 64, 0, 8), (4, 32, 1, 8),
])
def test_attention_decode_random(G, B, P, Hkv):
    shp, blk, _ = _block(G, Hkv, max_positions=16384)
    try:
        H, hd = shp.n_heads, 128
        cap = workloads.cache_capacity(P + 1)
        gen = torch.Generator().manual_seed(2000 + P + G + B)
        q = _rand((B, H, hd), gen)
        kc = torch.full((B, Hkv, cap, hd), SENTINEL, dtype=torch.bfloat16)
        vc = kc.clone()
        kc[:, :, :P + 1] = _rand((B, Hkv, P + 1, hd), gen, 0.6)
        vc[:, :, :P + 1] = _rand((B, Hkv, P + 1, hd), gen)
        note(f"attn decode G={G} B={B} P={P} Hkv={Hkv} ({B * Hkv} units)")
        o = _run_decode(blk, shp, q, kc, vc, P)
        ref = _oracle_decode(q, kc, vc, P)
        mag = _oracle_decode(q, kc, vc.abs(), P)
        e = bf16_err(o, ref, c=1e-3, mag=mag)
        note(f"  bf16 err {e:.3f} (max/rms {rel_err(o, ref):.2e})")
        assert e <= 1.0
    finally:
        llb.llb_block_destroy(blk)


# (G, B, Hkv): 4 units (the split-over-workgroups form), 256 units of 4 heads and
# 128 units of 8 heads (one workgroup per unit, the form the 8B and 70B decode run)
UNIT_SHAPES = [(4, 2, 2), (4, 32, 8), (8, 16, 8)]


@pytest.mark.parametrize("G,B,Hkv", UNIT_SHAPES)
@pytest.mark.parametrize("P", [1, 63, 1000, 4096])
def test_attention_decode_uniform_scores_give_mean_of_all_keys(P, G, B, Hkv):
    """q = 0: every visible key has score 0, so o = mean of the P + 1 values.
    V row 0 carries a large marker: dropping key 0 (or reading one key more)
    changes o[0] by about marker / (P + 1)."""
    shp, blk, _ = _block(G, Hkv)
    try:
        H, hd = shp.n_heads, 128
        cap = workloads.cache_capacity(P + 2)
        q = torch.zeros(B, H, hd, dtype=torch.bfloat16)
        kc = torch.zeros(B, Hkv, cap, hd, dtype=torch.bfloat16)
        vc = torch.zeros(B, Hkv, cap, hd, dtype=torch.bfloat16)
        vc[:, :, 0, 0] = 256.0          # first key's marker
        vc[:, :, P, 1] = 256.0          # own (newest) key's marker
        vc[:, :, P + 1, 2] = 256.0      # one past the end: must not be read
        vc[:, :, P + 2:, 3] = 256.0     # every row after that
        note(f"attn decode uniform P={P} G={G} B={B} Hkv={Hkv} ({B * Hkv} units)")
        o = _run_decode(blk, shp, q, kc, vc, P).float().view(B, H, hd)
        expect = 256.0 / (P + 1)
        assert torch.allclose(o[:, :, 0], torch.full_like(o[:, :, 0], expect), rtol=8e-3)
        assert torch.allclose(o[:, :, 1], torch.full_like(o[:, :, 1], expect), rtol=8e-3)
        assert torch.all(o[:, :, 2] == 0)
        assert torch.all(o[:, :, 3] == 0)
        assert torch.all(o[:, :, 4:] == 0)
    finally:
        llb.llb_block_destroy(blk)


@pytest.mark.parametrize("mode,G,B,Hkv,P", [
    ("prefill", 4, 1, 2, 700), ("decode", 4, 1, 2, 700),
    # one workgroup per (sequence, KV head): 256 units of 4 heads, 512 of 8
    ("decode", 4, 32, 8, 1000), ("decode", 8, 64, 8, 4096), ("prefill", 8, 2, 8, 700),
])
def test_attention_dominant_key_is_selected(mode, G, B, Hkv, P):
    """One key aligned with the query and 30 units of score above the rest: the
    output is that key's value row, to bf16 precision.  The dominant key sits at
    a different row in each sequence, the last one at row P (the newest key)."""
    shp, blk, _ = _block(G, Hkv)
    try:
        H, hd = shp.n_heads, 128
        T = 1 if mode == "decode" else 40
        pos0 = P if mode == "decode" else P - T + 1
        cap = workloads.cache_capacity(P + 1)
        gen = torch.Generator().manual_seed(3 + B + P)
        # the dominant row of sequence b: spread over 0..pos0 (the first query's
        # own position in prefill), the last sequence at the newest visible row
        stars = [(123 + 37 * b) % (pos0 + 1) for b in range(B)]
        stars[-1] = pos0
        kc = _rand((B, Hkv, cap, hd), gen, 0.05)
        vc = _rand((B, Hkv, cap, hd), gen)
        for b, star in enumerate(stars):
            kc[b, :, star, :] = 0
            kc[b, :, star, 0] = 4.0
        q = torch.zeros(B, H, T, hd, dtype=torch.bfloat16)
        q[..., 0] = 30.0 * math.sqrt(hd) / 4.0   # q.k_star / sqrt(hd) = 30
        note(f"attn dominant key {mode} G={G} B={B} Hkv={Hkv} P={P} ({B * Hkv} units)")
        if mode == "decode":
            o = _run_decode(blk, shp, q[:, :, 0], kc, vc, P).float().view(B, H, hd)
            o = o[:, :, None, :]
        else:
            out = torch.empty(B, T, H * hd, dtype=torch.bfloat16, device="cuda")
            llb.llb_attention_prefill(blk, q.cuda(), kc.cuda(), vc.cuda(), out, B, T, pos0, cap)
            o = out.cpu().float().view(B, T, H, hd).permute(0, 2, 1, 3)
        # ref[b, h] = value row stars[b] of KV head h // G
        ref = vc[torch.arange(B)[:, None], (torch.arange(H) // G)[None, :],
                 torch.tensor(stars)[:, None]].float()
        assert torch.allclose(o, ref[:, :, None, :].expand_as(o), atol=2e-2, rtol=1e-2)
    finally:
        llb.llb_block_destroy(blk)


def test_kv_append_is_exact():
    shp, blk, _ = _block(4)
    try:
        B, Hkv, hd, cap = 3, 2, 128, 96
        gen = torch.Generator().manual_seed(9)
        kc = _rand((B, Hkv, cap, hd), gen).cuda()
        vc = _rand((B, Hkv, cap, hd), gen).cuda()
        k0, v0 = kc.cpu(), vc.cpu()
        kn = _rand((B, Hkv, 20, hd), gen)
        vn = _rand((B, Hkv, 20, hd), gen)
        note("kv_append")
        llb.llb_kv_append(blk, kc, vc, B, cap, 40, 20, kn.cuda(), vn.cuda())
        k1, v1 = kc.cpu(), vc.cpu()
        k0[:, :, 40:60] = kn
        v0[:, :, 40:60] = vn
        assert torch.equal(k1, k0) and torch.equal(v1, v0)
        with pytest.raises(llb.LlbError) as ei:
            llb.llb_kv_append(blk, kc, vc, B, cap, 90, 20, kn.cuda(), vn.cuda())
        assert ei.value.status == llb.LLB_E_CAPACITY
    finally:
        llb.llb_block_destroy(blk)


def test_capacity_and_workspace_errors():
    shp, blk, _ = _block(4, max_positions=100)
    try:
        B, T = 1, 64
        x = torch.zeros(B, T, 256, device="cuda")
        y = torch.empty_like(x)
        kc = torch.zeros(B, 2, 64, 128, dtype=torch.bfloat16, device="cuda")
        vc = torch.zeros_like(kc)
        ws = llb.workspace(blk, B, T)
        note("error paths")
        with pytest.raises(llb.LlbError) as ei:      # T > cap
            llb.llb_block_prefill(blk, x, y, B, T, kc[:, :, :32].contiguous(), vc[:, :, :32].contiguous(), 32, ws)
        assert ei.value.status == llb.LLB_E_CAPACITY
        with pytest.raises(llb.LlbError) as ei:      # workspace too small
            llb.llb_block_prefill(blk, x, y, B, T, kc, vc, 64, ws[: ws.numel() // 2])
        assert ei.value.status == llb.LLB_E_INVALID
        x1 = x[:, :1].contiguous()
        ws1 = llb.workspace(blk, B, 1)
        with pytest.raises(llb.LlbError) as ei:      # P + 1 > cap
            llb.llb_block_decode(blk, x1, x1.clone(), B, 64, kc, vc, 64, ws1)
        assert ei.value.status == llb.LLB_E_CAPACITY
        big = torch.zeros(B, 2, 256, 128, dtype=torch.bfloat16, device="cuda")
        with pytest.raises(llb.LlbError) as ei:      # beyond the RoPE table
            llb.llb_block_decode(blk, x1, x1.clone(), B, 150, big, big.clone(), 256, ws1)
        assert ei.value.status == llb.LLB_E_CAPACITY
    finally:
        llb.llb_block_destroy(blk)


def test_double_destroy_is_rejected():
    """A destroyed handle leaves the library's set of live handles: destroying
    it again, or calling through it, gives LLB_E_INVALID and reads nothing."""
    import ctypes
    shp, blk, _ = _block(4)
    raw = ctypes.c_void_p(blk.handle.value)
    llb.llb_block_destroy(blk)
    lib = llb.load_library()
    assert lib.llb_block_destroy(raw) == llb.LLB_E_INVALID
    assert "live" in llb.llb_last_error()
    assert lib.llb_block_workspace_bytes(raw, 1, 1) == 0
    with pytest.raises(llb.LlbError) as ei:
        llb.llb_block_set_tiles(llb.Block(raw.value, None))
    assert ei.value.status == llb.LLB_E_INVALID
    # a model handle likewise
    params, _ = workloads.make_model_weights(shp, 1, 128, 5)
    dev = [{k: v.cuda() for k, v in params["layers"][0].items()}]
    m = llb.llb_model_create(llb.make_config(shp, 64), dev, 128, params["embed"].cuda(),
                             params["final_norm"].cuda(), params["lm_head"].cuda())
    mraw = ctypes.c_void_p(m.handle.value)
    llb.llb_model_destroy(m)
    assert lib.llb_model_destroy(mraw) == llb.LLB_E_INVALID
    assert lib.llb_model_workspace_bytes(mraw, 1, 1, 0) == 0


def _run_decode_ragged(blk, shp, q, kc, vc, pos):
    B = q.shape[0]
    H, hd = shp.n_heads, 128
    cap = kc.shape[2]
    ws = torch.empty(llb.llb_attention_workspace_bytes(blk, B, max(pos) + 1), dtype=torch.uint8, device="cuda")
    o = torch.empty(B, H * hd, dtype=torch.bfloat16, device="cuda")
    llb.llb_attention_decode_ragged(blk, q.cuda(), kc.cuda(), vc.cuda(), o, B, pos, cap, ws)
    return o.cpu()


def _spread_positions(B, P):
    """round((2b + 1) P / B): evenly spread over 0..2P (the ragged decode workload's rule)."""
    return [int(round((2 * b + 1) * P / B)) for b in range(B)]


@pytest.mark.parametrize("G,B,Hkv,kind", [
    (4, 32, 8, "spread1000"),    # the 8B ragged decode: 31..1969, long sequences cut into pieces
    (8, 64, 8, "random4096"),    # 70B heads, positions 0..4096 at random
    (4, 40, 4, "one_long"),      # 160 units, one sequence 20x the others
    (4, 3, 2, "random300"),      # 6 units: the split-over-workgroups form with per-sequence lengths
    (2, 64, 2, "equal"),         # equal lengths: balanced already, one workgroup per unit
])
def test_attention_decode_ragged(G, B, Hkv, kind):
    """Query b at its own position P_b reads keys 0..P_b of its sequence: every
    query against the oracle on its own sequence; cache rows past P_b hold a
    large sentinel that must never be read."""
    gen = torch.Generator().manual_seed(5000 + B + G)
    if kind == "spread1000":
        pos = _spread_positions(B, 1000)
    elif kind == "random4096":
        pos = torch.randint(0, 4097, (B,), generator=gen).tolist()
        pos[0], pos[1], pos[-1] = 0, 4096, 17
    elif kind == "one_long":
        pos = [100] * B
        pos[7] = 2047
    elif kind == "random300":
        pos = [0, 300, 123]
    else:
        pos = [500] * B
    shp, blk, _ = _block(G, Hkv, max_positions=8192)
    try:
        H, hd = shp.n_heads, 128
        cap = workloads.cache_capacity(max(pos) + 2)
        q = _rand((B, H, hd), gen)
        kc = torch.full((B, Hkv, cap, hd), SENTINEL, dtype=torch.bfloat16)
        vc = kc.clone()
        for b, p in enumerate(pos):
            kc[b, :, :p + 1] = _rand((Hkv, p + 1, hd), gen, 0.6)
            vc[b, :, :p + 1] = _rand((Hkv, p + 1, hd), gen)
        note(f"attn decode ragged {kind} G={G} B={B} Hkv={Hkv} positions {min(pos)}..{max(pos)}")
        o = _run_decode_ragged(blk, shp, q, kc, vc, pos)
        worst = 0.0
        for b, p in enumerate(pos):
            ref = oracle.attention(q[b][:, None, :], kc[b], vc[b], [p], n_keys=p + 1)[:, 0, :].reshape(-1)
            mag = oracle.attention(q[b][:, None, :], kc[b], vc[b].abs(), [p], n_keys=p + 1)[:, 0, :].reshape(-1)
            worst = max(worst, bf16_err(o[b], ref, c=1e-3, mag=mag))
        note(f"  worst bf16 err {worst:.3f}")
        assert worst <= 1.0
    finally:
        llb.llb_block_destroy(blk)


@pytest.mark.parametrize("G,B,Hkv", [(4, 32, 8), (8, 64, 8), (4, 3, 2)])
def test_attention_decode_ragged_uniform_scores_give_mean_of_own_keys(G, B, Hkv):
    """q = 0, so query b's output is the mean of its P_b + 1 values.  V carries
    markers on key 0, on key P_b (the newest) and on key P_b + 1 (one past the
    end, never read), so a piece boundary that drops or repeats a key, or a
    piece that reads into the next, moves the result by about marker / (P_b + 1)."""
    pos = _spread_positions(B, 1000) if B >= 32 else [0, 999, 257]
    shp, blk, _ = _block(G, Hkv)
    try:
        H, hd = shp.n_heads, 128
        cap = workloads.cache_capacity(max(pos) + 2)
        q = torch.zeros(B, H, hd, dtype=torch.bfloat16)
        kc = torch.zeros(B, Hkv, cap, hd, dtype=torch.bfloat16)
        vc = torch.zeros(B, Hkv, cap, hd, dtype=torch.bfloat16)
        for b, p in enumerate(pos):
            vc[b, :, 0, 0] = 256.0
            vc[b, :, p, 1] = 256.0
            vc[b, :, p + 1:, 2] = 256.0
        note(f"attn decode ragged uniform G={G} B={B} Hkv={Hkv}")
        o = _run_decode_ragged(blk, shp, q, kc, vc, pos).float().view(B, H, hd)
        for b, p in enumerate(pos):
            expect = torch.full_like(o[b, :, 0], 256.0 / (p + 1))
            if p == 0:
                expect = torch.full_like(o[b, :, 0], 256.0)   # key 0 is the newest: both markers
            assert torch.allclose(o[b, :, 0], expect, rtol=8e-3), (b, p)
            assert torch.allclose(o[b, :, 1], torch.full_like(o[b, :, 1], 256.0 / (p + 1)), rtol=8e-3), (b, p)
            assert torch.all(o[b, :, 2] == 0), (b, p)
            assert torch.all(o[b, :, 3:] == 0), (b, p)
    finally:
        llb.llb_block_destroy(blk)
