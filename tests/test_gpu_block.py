"""GPU parity of the block (prefill and decode) against the fp64 CPU oracle,
through the C ABI.

Bars (max|gpu - oracle| / rms(oracle)):
  * fp32 blocks: 1e-5 on y and on the cache rows written.
  * bf16 blocks: 2e-2 on y.  The cache rows (rotated K, V) are stored in bf16:
    per element |gpu - oracle| <= 2^-8 |oracle| (half an ulp of the stored value)
    + 1e-2 rms(oracle) (the 2^-9 rounding of the normalised bf16 operand, carried
    through the dot product).
Rows beyond the valid cache range hold a large sentinel, so any read past the
last key shows up as a parity failure.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import GpuBlock, bf16_err, gen_inputs, note, rel_err, shape

pytestmark = pytest.mark.gpu

SENTINEL = 512.0


def _run_prefill(shp, seed, B, T, cap=None, rows=None):
    cap = cap or workloads.cache_capacity(T)
    w, x, kc, vc = gen_inputs(shp, seed, B, T, 0, cap, fill=SENTINEL)
    note(f"prefill {shp.dtype} d={shp.d_model} H={shp.n_heads}/{shp.n_kv_heads} B={B} T={T} cap={cap}")
    gb = GpuBlock(shp, w, max_positions=cap)
    try:
        kd, vd, xd = kc.cuda(), vc.cuda(), x.cuda()
        y = gb.prefill(xd, kd, vd)
        torch.cuda.synchronize()
        y, kd, vd = y.cpu(), kd.cpu(), vd.cpu()
    finally:
        gb.close()
    y_ref, k_ref, v_ref = oracle.block_forward(shp, w, x, kc, vc, 0, rows=rows)
    if rows is not None:
        y = y[:, rows]
    return y, kd, vd, y_ref, k_ref, v_ref


@pytest.mark.parametrize("name", ["tiny_f32_prefill"])
def test_tiny_f32_prefill(name):
    wl = workloads.get(name)
    y, kd, vd, y_ref, k_ref, v_ref = _run_prefill(wl.shape, wl.seed, wl.B, wl.T)
    T = wl.T
    e_y = rel_err(y, y_ref)
    e_k = rel_err(kd[:, :, :T], k_ref)
    e_v = rel_err(vd[:, :, :T], v_ref)
    note(f"{name}: y {e_y:.2e}  k {e_k:.2e}  v {e_v:.2e}")
    assert e_y <= 1e-5 and e_k <= 1e-5 and e_v <= 1e-5
    assert torch.all(kd[:, :, T:] == SENTINEL) and torch.all(vd[:, :, T:] == SENTINEL)


@pytest.mark.parametrize("B,P", [(1, 0), (3, 37), (2, 130)])
def test_tiny_f32_decode(B, P):
    shp = workloads.get("tiny_f32_prefill").shape
    cap = workloads.cache_capacity(P + 1)
    w, x, kc, vc = gen_inputs(shp, 100 + P, B, 1, P, cap, fill=SENTINEL)
    note(f"decode f32 B={B} P={P}")
    gb = GpuBlock(shp, w, max_positions=cap)
    try:
        kd, vd = kc.cuda(), vc.cuda()
        y = gb.decode(x.cuda(), kd, vd, P).cpu()
        kd, vd = kd.cpu(), vd.cpu()
    finally:
        gb.close()
    y_ref, k_ref, v_ref = oracle.block_forward(shp, w, x, kc, vc, P)
    e_y = rel_err(y, y_ref)
    e_k = rel_err(kd[:, :, P:P + 1], k_ref)
    note(f"  y {e_y:.2e} k {e_k:.2e}")
    assert e_y <= 1e-5 and e_k <= 1e-5
    assert torch.equal(kd[:, :, :P], kc[:, :, :P])            # older rows untouched
    assert torch.all(kd[:, :, P + 1:] == SENTINEL)


BF16_SMALL = [
    # (d, H, Hkv, d_ff, B, T, scaled)
    (512, 8, 2, 768, 2, 100, False),     # group of 4, ragged T
    (1024, 16, 2, 1024, 1, 77, True),    # group of 8, llama3-scaled RoPE
    (512, 4, 4, 512, 1, 33, False),      # MHA
    (768, 4, 2, 1280, 3, 64, False),     # group of 2, d not a multiple of 512
    (512, 8, 2, 768, 1, 300, False),     # several query/key tiles, many row tiles
    (512, 8, 2, 768, 2, 2100, False),    # M = 4200: the 256x256 projection tiles, ragged M
    (256, 4, 2, 5120, 1, 1000, False),   # gate/up on the interleaved 4-wave kernel, ragged M, K = 256
    (2048, 16, 4, 512, 1, 3000, False),  # o and down on 256x128 BK-64 tiles, ragged M
    (512, 8, 2, 5120, 1, 2048, False),   # gate/up: 1.25 rounds of 256x256 tiles, the tail on 256x128
]


@pytest.mark.parametrize("d,H,Hkv,dff,B,T,scaled", BF16_SMALL)
def test_bf16_prefill_small(d, H, Hkv, dff, B, T, scaled):
    shp = shape(d_model=d, n_heads=H, n_kv_heads=Hkv, head_dim=128, d_ff=dff, rope_scaling=scaled)
    y, kd, vd, y_ref, k_ref, v_ref = _run_prefill(shp, 7 + T, B, T)
    e_y = rel_err(y, y_ref)
    e_k = bf16_err(kd[:, :, :T], k_ref)
    e_v = bf16_err(vd[:, :, :T], v_ref)
    note(f"  y {e_y:.2e}  k {e_k:.3f}  v {e_v:.3f}")
    assert e_y <= 2e-2
    assert e_k <= 1.0 and e_v <= 1.0
    assert torch.all(kd[:, :, T:].float() == SENTINEL)


# Every prefill GEMM tile configuration on every projection whose N its BN
# divides: d = 1536 and 2 d_ff = 1536 are multiples of 768 = lcm(128, 192, 256),
# QKV N = 24 heads x 128 = 3072 as well; M = 300 leaves a ragged second row tile.
TILE_SHAPE = dict(d_model=1536, n_heads=16, n_kv_heads=4, head_dim=128, d_ff=768)


def _tile_count():
    """Entries of the library's prefill tile table (0 when it is not built)."""
    try:
        from dense_decoder_only_amd import llb
        return llb.llb_gemm_num_tiles()
    except Exception:
        return 0


@pytest.mark.parametrize("cfg", range(_tile_count()))
def test_bf16_prefill_every_tile_config(cfg):
    from dense_decoder_only_amd import llb
    bm, bn = llb.llb_gemm_tile_info(cfg)
    shp = shape(**TILE_SHAPE, rope_scaling=False)
    B, T = 1, 300
    cap = workloads.cache_capacity(T)
    w, x, kc, vc = gen_inputs(shp, 900 + cfg, B, T, 0, cap, fill=SENTINEL)
    y_ref, k_ref, v_ref = oracle.block_forward(shp, w, x, kc, vc, 0)
    nqkv = (shp.n_heads + 2 * shp.n_kv_heads) * shp.head_dim
    Ns = {"qkv": nqkv, "o": shp.d_model, "gate_up": 2 * shp.d_ff, "down": shp.d_model}
    gb = GpuBlock(shp, w, max_positions=cap)
    ran = []
    try:
        for proj, N in Ns.items():
            llb.llb_block_set_tiles(gb.blk, **{proj: cfg})
            note(f"tile config {cfg} ({bm}x{bn}) on the {proj} projection (N={N})")
            kd, vd = kc.cuda(), vc.cuda()
            try:
                y = gb.prefill(x.cuda(), kd, vd)
                torch.cuda.synchronize()
            except llb.LlbError as err:
                # refused before any work: BN does not divide N, or the per-wave
                # slice cannot hold a fused epilogue (SwiGLU pairs, norm sums)
                assert err.status == llb.LLB_E_UNSUPPORTED, str(err)
                assert N % bn != 0 or proj in ("o", "gate_up"), str(err)
                note(f"  refused: {err}")
                continue
            finally:
                llb.llb_block_set_tiles(gb.blk)
            assert N % bn == 0
            y, kd, vd = y.cpu(), kd.cpu(), vd.cpu()
            e_y = rel_err(y, y_ref)
            e_k = bf16_err(kd[:, :, :T], k_ref)
            e_v = bf16_err(vd[:, :, :T], v_ref)
            note(f"  y {e_y:.2e}  k {e_k:.3f}  v {e_v:.3f}")
            assert e_y <= 2e-2 and e_k <= 1.0 and e_v <= 1.0
            assert torch.all(kd[:, :, T:].float() == SENTINEL)
            ran.append(proj)
    finally:
        gb.close()
    assert ran, "no projection accepted the configuration"


# Grids whose column-panel count is a multiple of 8 while the row-panel count is
# not a multiple of 8 (nor 16 or 32) take the prefill GEMM's column-interleaved
# tile order (XCD x on the column panels n = x mod 8, groups of 8 row panels, the
# last group short): d = d_ff = 2048 gives 8 or 16 column panels for the O, down
# and gate/up projections, T = 300 and 2100 give 2 and 9 row panels.  (The 70B
# and 8B full-size tests take the 16 x 16, 32 x 8 and 8 x 32 block orders.)
@pytest.mark.parametrize("T", [300, 2100])
def test_bf16_prefill_column_interleaved_tile_order(T):
    shp = shape(d_model=2048, n_heads=16, n_kv_heads=4, head_dim=128, d_ff=2048, rope_scaling=False)
    y, kd, vd, y_ref, k_ref, v_ref = _run_prefill(shp, 321 + T, 1, T)
    e_y = rel_err(y, y_ref)
    e_k = bf16_err(kd[:, :, :T], k_ref)
    e_v = bf16_err(vd[:, :, :T], v_ref)
    note(f"  y {e_y:.2e}  k {e_k:.3f}  v {e_v:.3f}")
    assert e_y <= 2e-2 and e_k <= 1.0 and e_v <= 1.0
    assert torch.all(kd[:, :, T:].float() == SENTINEL)


# Long inputs (M >= 4096 rows) take the 256 x 256 kernels that prefetch W lines
# only for the gate/up and output projections, and A and W lines for QKV and
# the long-K down projection (K = d_ff = 16384); T = 4100 leaves a 4-row last
# row panel on all four, and 17 row panels
# that no block tile order divides.  y is compared on sampled rows (the causal
# block makes each row's output depend only on the rows before it), including
# the last panel's; K and V on every row.
def test_bf16_prefill_long_ragged_rows():
    shp = shape(d_model=1024, n_heads=8, n_kv_heads=2, head_dim=128, d_ff=16384, rope_scaling=True)
    T = 4100
    rows = [0, 1, 255, 256, 2047, 2048, 4095, 4096, 4097, 4099]
    y, kd, vd, y_ref, k_ref, v_ref = _run_prefill(shp, 4100, 1, T, rows=rows)
    e_y = rel_err(y, y_ref)
    e_k = bf16_err(kd[:, :, :T], k_ref)
    e_v = bf16_err(vd[:, :, :T], v_ref)
    note(f"  y {e_y:.2e}  k {e_k:.3f}  v {e_v:.3f}")
    assert e_y <= 2e-2 and e_k <= 1.0 and e_v <= 1.0
    assert torch.all(kd[:, :, T:].float() == SENTINEL)


def test_tile_override_rejects_bad_values():
    from dense_decoder_only_amd import llb
    shp = shape(**TILE_SHAPE, rope_scaling=False)
    w, _, _, _ = gen_inputs(shp, 5, 1, 1, 0, 16)
    gb = GpuBlock(shp, w, max_positions=16)
    try:
        n = llb.llb_gemm_num_tiles()
        for bad in (-2, n):
            with pytest.raises(llb.LlbError) as ei:
                llb.llb_block_set_tiles(gb.blk, qkv=bad)
            assert ei.value.status == llb.LLB_E_INVALID
        with pytest.raises(llb.LlbError):
            llb.llb_gemm_tile_info(n)
    finally:
        gb.close()


@pytest.mark.parametrize("B,P,G", [(5, 300, 4), (40, 64, 4), (64, 300, 4), (70, 20, 4), (2, 1000, 8), (1, 0, 4)])
def test_bf16_decode_small(B, P, G):
    Hkv = 2
    shp = shape(d_model=512, n_heads=G * Hkv, n_kv_heads=Hkv, head_dim=128, d_ff=768,
                rope_scaling=(G == 8))
    cap = workloads.cache_capacity(P + 1)
    w, x, kc, vc = gen_inputs(shp, 11 + P, B, 1, P, cap, fill=SENTINEL)
    note(f"decode bf16 B={B} P={P} G={G}")
    gb = GpuBlock(shp, w, max_positions=cap)
    try:
        kd, vd = kc.cuda(), vc.cuda()
        y = gb.decode(x.cuda(), kd, vd, P).cpu()
        kd = kd.cpu()
    finally:
        gb.close()
    y_ref, k_ref, _ = oracle.block_forward(shp, w, x, kc, vc, P)
    e_y = rel_err(y, y_ref)
    e_k = bf16_err(kd[:, :, P:P + 1], k_ref)
    note(f"  y {e_y:.2e} k {e_k:.3f}")
    assert e_y <= 2e-2 and e_k <= 1.0
    assert torch.equal(kd[:, :, :P], kc[:, :, :P])
    assert torch.all(kd[:, :, P + 1:].float() == SENTINEL)


@pytest.mark.parametrize("B", [5, 40])
@pytest.mark.parametrize("kernels", [(0, 0, 0, 0), (16, 16, 0, 16), (32, 32, -1, 32), (16, 32, 0, 0)])
@pytest.mark.parametrize("d,dff", [(512, 768), (1024, 2816)])
def test_bf16_decode_kernel_choices(B, kernels, d, dff):
    """Every decode projection kernel against the oracle: the split-K kernel
    (128 weight rows per workgroup, partials summed by a second kernel) and the
    narrow kernel (16 or 32 weight rows per workgroup over all of K), for the
    QKV (RoPE, cache write), O (residual, next RMSNorm's operand and partial
    sums of squares, which the gate/up kernel gathers) and down projections;
    B = 40 holds 64 token rows per tile."""
    from dense_decoder_only_amd import llb
    shp = shape(d_model=d, n_heads=8, n_kv_heads=2, head_dim=128, d_ff=dff)
    P = 150
    cap = workloads.cache_capacity(P + 1)
    w, x, kc, vc = gen_inputs(shp, 23 + B + d, B, 1, P, cap)
    note(f"decode kernels {kernels} B={B} d={d} d_ff={dff}")
    gb = GpuBlock(shp, w, max_positions=cap)
    try:
        llb.llb_block_set_decode_kernels(gb.blk, *kernels)
        kd, vd = kc.cuda(), vc.cuda()
        y = gb.decode(x.cuda(), kd, vd, P).cpu()
        kd, vd = kd.cpu(), vd.cpu()
    finally:
        gb.close()
    y_ref, k_ref, v_ref = oracle.block_forward(shp, w, x, kc, vc, P)
    e_y = rel_err(y, y_ref)
    e_k = bf16_err(kd[:, :, P:P + 1], k_ref)
    e_v = bf16_err(vd[:, :, P:P + 1], v_ref)
    note(f"  y {e_y:.2e} k {e_k:.3f} v {e_v:.3f}")
    assert e_y <= 2e-2 and e_k <= 1.0 and e_v <= 1.0


def test_decode_kernels_rejects_bad_values():
    from dense_decoder_only_amd import llb
    shp = shape(d_model=512, n_heads=8, n_kv_heads=2, head_dim=128, d_ff=768)
    w, _, _, _ = gen_inputs(shp, 3, 1, 1, 0, 64)
    gb = GpuBlock(shp, w, max_positions=64)
    try:
        for bad in ((8, -1, -1, -1), (-1, 64, -1, -1), (-1, -1, -1, -2), (-1, -1, 16, -1), (1, -1, -1, -1)):
            with pytest.raises(llb.LlbError):
                llb.llb_block_set_decode_kernels(gb.blk, *bad)
        llb.llb_block_set_decode_kernels(gb.blk)
    finally:
        gb.close()


def _ragged_positions(B, P_max, seed):
    g = torch.Generator().manual_seed(seed)
    pos = torch.randint(0, P_max + 1, (B,), generator=g).tolist()
    pos[0] = 0                     # an empty prefix
    pos[-1] = P_max                # the longest sequence
    return pos


@pytest.mark.parametrize("B,P_max,Hkv,G,dtype", [
    (5, 300, 2, 4, "bf16"),     # split-over-workgroups attention, weight-streaming projections
    (40, 200, 4, 4, "bf16"),    # one workgroup per (sequence, KV head)
    (70, 150, 2, 8, "bf16"),    # M = 70: the projections run as GEMM tiles
    (6, 90, 2, 4, "f32"),
])
def test_ragged_decode(B, P_max, Hkv, G, dtype):
    """Every sequence decodes one token at its own position: y row b against the
    oracle run on sequence b alone at start position P_b; only cache row P_b of
    sequence b changes (rows past it hold the sentinel and must stay unread)."""
    from dense_decoder_only_amd import llb
    shp = shape(d_model=512, n_heads=G * Hkv, n_kv_heads=Hkv, head_dim=128 if dtype == "bf16" else 64,
                d_ff=768, rope_scaling=(G == 8), dtype=dtype)
    pos = _ragged_positions(B, P_max, 7 + B)
    cap = workloads.cache_capacity(P_max + 1)
    w, x, kc, vc = gen_inputs(shp, 13 + B, B, 1, P_max, cap, fill=SENTINEL)
    for b, p in enumerate(pos):                       # rows >= P_b: sentinel
        kc[b, :, p:] = SENTINEL
        vc[b, :, p:] = SENTINEL
    note(f"ragged decode {dtype} B={B} positions {min(pos)}..{max(pos)}")
    gb = GpuBlock(shp, w, max_positions=cap)
    try:
        kd, vd = kc.cuda(), vc.cuda()
        y = torch.empty(B, 1, shp.d_model, device="cuda")
        llb.llb_block_decode_ragged(gb.blk, x.cuda(), y, B, pos, kd, vd, cap, gb.workspace(B, 1))
        y, kd, vd = y.cpu(), kd.cpu(), vd.cpu()
    finally:
        gb.close()
    bar = 2e-2 if dtype == "bf16" else 1e-5
    worst_y, worst_k = 0.0, 0.0
    for b, p in enumerate(pos):
        y_ref, k_ref, v_ref = oracle.block_forward(shp, w, x[b:b + 1], kc[b:b + 1], vc[b:b + 1], p)
        worst_y = max(worst_y, rel_err(y[b:b + 1], y_ref))
        if dtype == "bf16":
            worst_k = max(worst_k, bf16_err(kd[b:b + 1, :, p:p + 1], k_ref), bf16_err(vd[b:b + 1, :, p:p + 1], v_ref))
        else:
            worst_k = max(worst_k, rel_err(kd[b:b + 1, :, p:p + 1], k_ref))
        assert torch.equal(kd[b, :, :p], kc[b, :, :p]) and torch.equal(vd[b, :, :p], vc[b, :, :p])
        assert torch.all(kd[b, :, p + 1:].float() == SENTINEL)
    note(f"  worst y {worst_y:.2e}  worst k/v {worst_k:.3f}")
    assert worst_y <= bar
    assert worst_k <= (1.0 if dtype == "bf16" else 1e-5)


def test_ragged_decode_with_equal_positions_is_decode():
    from dense_decoder_only_amd import llb
    shp = shape(d_model=512, n_heads=8, n_kv_heads=2, head_dim=128, d_ff=768)
    B, P = 9, 77
    cap = workloads.cache_capacity(P + 1)
    w, x, kc, vc = gen_inputs(shp, 17, B, 1, P, cap)
    gb = GpuBlock(shp, w, max_positions=cap)
    try:
        k1, v1, k2, v2 = kc.cuda(), vc.cuda(), kc.cuda(), vc.cuda()
        y1 = gb.decode(x.cuda(), k1, v1, P)
        y2 = torch.empty_like(y1)
        llb.llb_block_decode_ragged(gb.blk, x.cuda(), y2, B, [P] * B, k2, v2, cap, gb.workspace(B, 1))
        torch.cuda.synchronize()
        assert torch.equal(y1, y2) and torch.equal(k1, k2) and torch.equal(v1, v2)
    finally:
        gb.close()


def test_ragged_decode_rejects_bad_positions():
    from dense_decoder_only_amd import llb
    shp = shape(d_model=512, n_heads=8, n_kv_heads=2, head_dim=128, d_ff=768)
    B, cap = 3, 64
    w, x, kc, vc = gen_inputs(shp, 19, B, 1, 10, cap)
    gb = GpuBlock(shp, w, max_positions=cap)
    try:
        kd, vd = kc.cuda(), vc.cuda()
        y = torch.empty(B, 1, shp.d_model, device="cuda")
        for pos, status in (([0, -1, 3], llb.LLB_E_INVALID), ([0, 64, 3], llb.LLB_E_CAPACITY)):
            with pytest.raises(llb.LlbError) as ei:
                llb.llb_block_decode_ragged(gb.blk, x.cuda(), y, B, pos, kd, vd, cap, gb.workspace(B, 1))
            assert ei.value.status == status
        with pytest.raises(ValueError):
            llb.llb_block_decode_ragged(gb.blk, x.cuda(), y, B, [1, 2], kd, vd, cap, gb.workspace(B, 1))
        torch.cuda.synchronize()
        assert torch.equal(kd.cpu(), kc)
    finally:
        gb.close()


def test_bf16_prefill_then_decode_matches_longer_prefill():
    """GPU prefill(T) fills the cache; GPU decode at P = T must equal row T of the
    oracle's prefill(T + 1) (the oracle never sees GPU data)."""
    shp = shape(d_model=512, n_heads=8, n_kv_heads=2, head_dim=128, d_ff=768)
    B, T = 3, 45
    cap = workloads.cache_capacity(T + 1)
    w, x, kc, vc = gen_inputs(shp, 21, B, T + 1, 0, cap, fill=SENTINEL)
    note("prefill -> decode continuation")
    gb = GpuBlock(shp, w, max_positions=cap)
    try:
        kd, vd, xd = kc.cuda(), vc.cuda(), x.cuda()
        gb.prefill(xd[:, :T].contiguous(), kd, vd)
        y = gb.decode(xd[:, T:].contiguous(), kd, vd, T).cpu()
    finally:
        gb.close()
    y_ref, _, _ = oracle.block_forward(shp, w, x, kc, vc, 0)
    e = rel_err(y[:, 0], y_ref[:, T])
    note(f"  y {e:.2e}")
    assert e <= 2e-2


@pytest.mark.parametrize("B,P,T,G,scaled", [
    (2, 300, 100, 4, False),    # chunk shorter than the prefix
    (1, 37, 513, 4, False),     # several query tiles, key tiles straddle the prefix end
    (1, 1000, 257, 8, True),    # group of 8, llama3-scaled RoPE at positions past 1000
    (2, 500, 1100, 4, False),   # M = 2200: the 256x256 projection tiles, ragged
])
def test_bf16_chunked_prefill(B, P, T, G, scaled):
    """T tokens at positions P..P+T-1 against a random cache prefix: y and the new
    cache rows against the oracle; rows below P untouched, rows from P+T on keep
    the sentinel."""
    Hkv = 2
    shp = shape(d_model=512, n_heads=G * Hkv, n_kv_heads=Hkv, head_dim=128, d_ff=768,
                rope_scaling=scaled)
    cap = workloads.cache_capacity(P + T)
    w, x, kc, vc = gen_inputs(shp, 31 + P + T, B, T, P, cap, fill=SENTINEL)
    note(f"chunked prefill bf16 B={B} P={P} T={T} G={G}")
    gb = GpuBlock(shp, w, max_positions=cap)
    try:
        kd, vd = kc.cuda(), vc.cuda()
        y = gb.prefill_at(x.cuda(), kd, vd, P).cpu()
        kd, vd = kd.cpu(), vd.cpu()
    finally:
        gb.close()
    y_ref, k_ref, v_ref = oracle.block_forward(shp, w, x, kc, vc, P)
    e_y = rel_err(y, y_ref)
    e_k = bf16_err(kd[:, :, P:P + T], k_ref)
    e_v = bf16_err(vd[:, :, P:P + T], v_ref)
    note(f"  y {e_y:.2e}  k {e_k:.3f}  v {e_v:.3f}")
    assert e_y <= 2e-2 and e_k <= 1.0 and e_v <= 1.0
    assert torch.equal(kd[:, :, :P], kc[:, :, :P]) and torch.equal(vd[:, :, :P], vc[:, :, :P])
    assert torch.all(kd[:, :, P + T:].float() == SENTINEL)


def test_f32_chunked_prefill():
    wl = workloads.get("tiny_f32_prefill")
    shp = wl.shape
    B, P, T = 2, 40, 24
    cap = workloads.cache_capacity(P + T)
    w, x, kc, vc = gen_inputs(shp, 77, B, T, P, cap, fill=SENTINEL)
    note(f"chunked prefill f32 B={B} P={P} T={T}")
    gb = GpuBlock(shp, w, max_positions=cap)
    try:
        kd, vd = kc.cuda(), vc.cuda()
        y = gb.prefill_at(x.cuda(), kd, vd, P).cpu()
        kd, vd = kd.cpu(), vd.cpu()
    finally:
        gb.close()
    y_ref, k_ref, v_ref = oracle.block_forward(shp, w, x, kc, vc, P)
    e_y, e_k, e_v = rel_err(y, y_ref), rel_err(kd[:, :, P:P + T], k_ref), rel_err(vd[:, :, P:P + T], v_ref)
    note(f"  y {e_y:.2e}  k {e_k:.2e}  v {e_v:.2e}")
    assert e_y <= 1e-5 and e_k <= 1e-5 and e_v <= 1e-5
    assert torch.equal(kd[:, :, :P], kc[:, :, :P])
    assert torch.all(kd[:, :, P + T:] == SENTINEL)


def test_bf16_prefill_in_chunks_matches_one_prefill():
    """GPU prefill of the first T1 tokens, then a GPU chunk of T2 at start T1: the
    chunk's outputs equal rows T1.. of the oracle's single prefill of T1 + T2."""
    shp = shape(d_model=512, n_heads=8, n_kv_heads=2, head_dim=128, d_ff=768)
    B, T1, T2 = 2, 300, 200
    cap = workloads.cache_capacity(T1 + T2)
    w, x, kc, vc = gen_inputs(shp, 41, B, T1 + T2, 0, cap, fill=SENTINEL)
    note("prefill -> chunked prefill continuation")
    gb = GpuBlock(shp, w, max_positions=cap)
    try:
        kd, vd, xd = kc.cuda(), vc.cuda(), x.cuda()
        gb.prefill(xd[:, :T1].contiguous(), kd, vd)
        y = gb.prefill_at(xd[:, T1:].contiguous(), kd, vd, T1).cpu()
    finally:
        gb.close()
    y_ref, _, _ = oracle.block_forward(shp, w, x, kc, vc, 0, rows=list(range(T1, T1 + T2)))
    e = rel_err(y, y_ref)
    note(f"  y {e:.2e}")
    assert e <= 2e-2


def test_chunked_prefill_rejects_bad_positions():
    from dense_decoder_only_amd import llb
    shp = shape(d_model=512, n_heads=8, n_kv_heads=2, head_dim=128, d_ff=768)
    cap = 64
    w, x, kc, vc = gen_inputs(shp, 3, 1, 16, 0, cap)
    gb = GpuBlock(shp, w, max_positions=cap)
    try:
        kd, vd, xd = kc.cuda(), vc.cuda(), x.cuda()
        for P, status in ((-1, llb.LLB_E_INVALID), (cap - 15, llb.LLB_E_CAPACITY)):
            with pytest.raises(llb.LlbError) as ei:
                gb.prefill_at(xd, kd, vd, P)
            assert ei.value.status == status
        torch.cuda.synchronize()
        assert torch.equal(kd.cpu(), kc)                      # nothing was written
    finally:
        gb.close()


def test_decode_workspace_query_covers_every_position():
    """llb_block_workspace_bytes(B, 1) covers a decode at any start position
    below max_positions: the split attention's chunk count is not monotone in
    the key count (here 1001 keys need more chunks than 1088), so the query
    must return a bound, not the size at max_positions.  A workspace of exactly
    the advertised size decodes at P = 1000, 1087 and 0."""
    from dense_decoder_only_amd import llb
    shp = shape(d_model=512, n_heads=8, n_kv_heads=2, head_dim=128, d_ff=768)
    B, cap = 64, 1088
    w, x, kc, vc = gen_inputs(shp, 31, B, 1, cap - 1, cap)
    note("decode workspace bound")
    gb = GpuBlock(shp, w, max_positions=cap)
    try:
        n = llb.llb_block_workspace_bytes(gb.blk, B, 1)
        ws = torch.empty(n, dtype=torch.uint8, device="cuda")
        xd = x.cuda()
        for P in (1000, cap - 1, 0):
            kd, vd = kc.cuda(), vc.cuda()
            y = torch.empty_like(xd)
            llb.llb_block_decode(gb.blk, xd, y, B, P, kd, vd, cap, ws)
            if P == 1000:
                y_ref, _, _ = oracle.block_forward(shp, w, x, kc, vc, P)
                assert rel_err(y.cpu(), y_ref) <= 2e-2
        torch.cuda.synchronize()
    finally:
        gb.close()


def test_empty_inputs_are_rejected_before_any_launch():
    """B = 0 or T = 0 (an empty batch) is an argument error on every entry point,
    reported before anything is queued: the cache is untouched and the
    workspace size query answers 0."""
    from dense_decoder_only_amd import llb
    shp = shape(d_model=512, n_heads=8, n_kv_heads=2, head_dim=128, d_ff=768)
    cap = 64
    w, x, kc, vc = gen_inputs(shp, 4, 2, 8, 8, cap)
    gb = GpuBlock(shp, w, max_positions=cap)
    try:
        kd, vd, xd = kc.cuda(), vc.cuda(), x.cuda()
        y = torch.empty_like(xd)
        ws = gb.workspace(2, 8)
        assert llb.llb_block_workspace_bytes(gb.blk, 0, 8) == 0
        assert llb.llb_block_workspace_bytes(gb.blk, 2, 0) == 0
        calls = [
            lambda: llb.llb_block_prefill(gb.blk, xd, y, 0, 8, kd, vd, cap, ws),
            lambda: llb.llb_block_prefill(gb.blk, xd, y, 2, 0, kd, vd, cap, ws),
            lambda: llb.llb_block_prefill_at(gb.blk, xd, y, 2, 0, 8, kd, vd, cap, ws),
            lambda: llb.llb_block_decode(gb.blk, xd, y, 0, 8, kd, vd, cap, ws),
            lambda: llb.llb_block_decode_ragged(gb.blk, xd, y, 0, [], kd, vd, cap, ws),
        ]
        for call in calls:
            with pytest.raises(llb.LlbError) as ei:
                call()
            assert ei.value.status == llb.LLB_E_INVALID
        torch.cuda.synchronize()
        assert torch.equal(kd.cpu(), kc) and torch.equal(vd.cpu(), vc)
    finally:
        gb.close()


def test_bf16_prefill_is_deterministic():
    shp = shape(d_model=512, n_heads=8, n_kv_heads=2, head_dim=128, d_ff=768)
    B, T = 2, 130
    cap = workloads.cache_capacity(T)
    w, x, kc, vc = gen_inputs(shp, 5, B, T, 0, cap)
    note("determinism")
    gb = GpuBlock(shp, w, max_positions=cap)
    try:
        outs = []
        for _ in range(3):
            kd, vd = kc.cuda(), vc.cuda()
            outs.append((gb.prefill(x.cuda(), kd, vd).cpu(), kd.cpu()))
        for y, k in outs[1:]:
            assert torch.equal(y, outs[0][0]) and torch.equal(k, outs[0][1])
        # decode path too
        kd, vd = kc.cuda(), vc.cuda()
        gb.prefill(x.cuda(), kd, vd)
        d1 = gb.decode(x[:, :1].cuda(), kd.clone(), vd.clone(), T - 1).cpu()
        d2 = gb.decode(x[:, :1].cuda(), kd.clone(), vd.clone(), T - 1).cpu()
        assert torch.equal(d1, d2)
    finally:
        gb.close()


@pytest.mark.parametrize("kern", [-1, 0])
def test_bf16_decode_split_k_with_dirty_workspace(kern):
    """The decode projections sum split-K partials in a fixed order: in LDS
    (narrow kernel) or through the workspace (split-K kernels).  A workspace full of stale bytes, and calls back to back on one
    workspace, give bit-identical results to a zeroed one."""
    shp = shape(d_model=512, n_heads=8, n_kv_heads=2, head_dim=128, d_ff=768)
    B, P = 7, 77
    cap = workloads.cache_capacity(P + 1)
    w, x, kc, vc = gen_inputs(shp, 17, B, 1, P, cap)
    note("decode split-K counters")
    gb = GpuBlock(shp, w, max_positions=cap)
    try:
        from dense_decoder_only_amd import llb
        llb.llb_block_set_decode_kernels(gb.blk, kern, kern, kern, kern)
        ws = gb.workspace(B, 1)
        outs = []
        for fill in (0, 0xFF, 0x01, None, None):
            if fill is not None:
                ws.fill_(fill)
            kd, vd = kc.cuda(), vc.cuda()
            y = torch.empty(B, 1, shp.d_model, device="cuda")
            llb.llb_block_decode(gb.blk, x.cuda(), y, B, P, kd, vd, cap, ws)
            outs.append((y.cpu(), kd.cpu()))
        for y, k in outs[1:]:
            assert torch.equal(y, outs[0][0]) and torch.equal(k, outs[0][1])
        y_ref, _, _ = oracle.block_forward(shp, w, x, kc, vc, P)
        assert rel_err(outs[0][0], y_ref) <= 2e-2
    finally:
        gb.close()


def test_y_may_alias_x():
    shp = shape(d_model=512, n_heads=8, n_kv_heads=2, head_dim=128, d_ff=768)
    B, T = 1, 40
    cap = workloads.cache_capacity(T)
    w, x, kc, vc = gen_inputs(shp, 6, B, T, 0, cap)
    note("in-place x += block(x)")
    gb = GpuBlock(shp, w, max_positions=cap)
    try:
        from dense_decoder_only_amd import llb
        xd = x.cuda()
        y_sep = gb.prefill(xd, kc.cuda(), vc.cuda()).cpu()
        llb.llb_block_prefill(gb.blk, xd, xd, B, T, kc.cuda(), vc.cuda(), cap, gb.workspace(B, T))
        assert torch.equal(xd.cpu(), y_sep)
    finally:
        gb.close()
