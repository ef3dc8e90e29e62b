"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test ties one oracle function to a printed value (tests/golden), a closed
form, an invariant, a special case that reduces to a library routine, or brute
force on tiny inputs.  They are chosen so that a plausible slip (eps outside the
square root, a rotate-half pairing, a flipped rotation sign, a modulo GQA map,
an off-by-one causal mask, swapped gate/up roles, a transposed weight) fails at
least one of them.
"""
import json
import math
import os
import types

import numpy as np
import pytest
import torch

import oracle
import workloads

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_values.json")))


def _cfg(**kw):
    base = dict(d_model=64, n_heads=4, n_kv_heads=2, head_dim=16, d_ff=96, eps=1e-5,
                rope_theta=500000.0, rope_scaling=False, rs_factor=8.0, rs_low_freq_factor=1.0,
                rs_high_freq_factor=4.0, rs_orig_max_pos=8192)
    base.update(kw)
    return types.SimpleNamespace(**base)


def _rand_weights(cfg, rng, scale=1.0):
    sh = oracle.expected_weight_shapes(cfg.d_model, cfg.n_heads, cfg.n_kv_heads, cfg.head_dim, cfg.d_ff)
    w = {}
    for k, s in sh.items():
        if k.endswith("norm"):
            w[k] = 1.0 + 0.3 * rng.standard_normal(s)
        else:
            w[k] = scale * rng.standard_normal(s) / math.sqrt(s[1])
    return w


# ----------------------------------------------------------------- parameter counts
def test_qkv_params_8b_page_table():
    g = GOLD["qkv_params_8b"]
    n = oracle.block_param_counts(**g["shape"])
    assert n["n_wq"] == g["value"]["wq"]
    assert n["n_wk"] == g["value"]["wk"]
    assert n["n_wv"] == g["value"]["wv"]
    assert n["qkv"] == g["value"]["total"]
    assert n["qkv"] * 32 == g["value"]["times_32_blocks"]


def test_block_params_8b_and_ffn_share():
    g = GOLD["block_params_8b"]
    n = oracle.block_param_counts(**g["shape"])
    assert n["block"] == g["value"]["block"]
    assert round(100.0 * n["ffn"] / n["block"], 1) == g["value"]["ffn_share_pct_1dp"]


def test_block_params_qwen_with_bias():
    # a second architecture (4 KV heads, d=3584) exercises the K/V widths; the page's
    # count includes Q/K/V biases, which this block does not have, so add them here.
    g = GOLD["block_params_qwen25_7b"]
    s = g["shape"]
    n = oracle.block_param_counts(**s)
    bias = s["n_heads"] * s["head_dim"] + 2 * s["n_kv_heads"] * s["head_dim"]
    assert n["block"] + bias == g["value"]["block"]
    assert round(100.0 * n["ffn"] / (n["block"] + bias), 1) == g["value"]["ffn_share_pct_1dp"]


def test_workload_generators_match_oracle_shapes():
    for wl in workloads.CONFIGS.values():
        s = wl.shape
        assert s.weight_shapes() == oracle.expected_weight_shapes(
            s.d_model, s.n_heads, s.n_kv_heads, s.head_dim, s.d_ff)
    c = workloads.get("8b_bf16_decode")
    assert c.P + 1 == GOLD["decode_keys_read"]["L"]


# ----------------------------------------------------------------- RMSNorm
def test_rmsnorm_page_example():
    g = GOLD["rmsnorm_example"]
    for x, rms in zip(g["inputs"], g["rms_2dp"]):
        x = np.array(x, dtype=np.float64)
        assert round(float(np.sqrt(np.mean(x * x))), 2) == pytest.approx(rms)
        out = oracle.rmsnorm(x, np.ones(3), eps=0.0)
        assert np.round(out, 2).tolist() == g["output_2dp"]


def test_rmsnorm_unit_rms_closed_form_and_eps_inside_sqrt():
    rng = np.random.default_rng(0)
    for scale in (1e-4, 1e-3, 1.0, 30.0):
        x = scale * rng.standard_normal((5, 256))
        out = oracle.rmsnorm(x, np.ones(256), eps=1e-5)
        ms = np.mean(x * x, axis=-1)
        expect = np.sqrt(ms / (ms + 1e-5))
        np.testing.assert_allclose(np.sqrt(np.mean(out * out, axis=-1)), expect, rtol=1e-12)


def test_rmsnorm_gain_is_per_feature_and_scale_invariant():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((3, 32))
    g = rng.standard_normal(32)
    a = oracle.rmsnorm(x, g, 0.0)
    b = oracle.rmsnorm(10.0 * x, g, 0.0)
    np.testing.assert_allclose(a, b, rtol=1e-12)
    base = oracle.rmsnorm(x, np.ones(32), 0.0)
    np.testing.assert_allclose(a, base * g[None, :], rtol=1e-12)


# ----------------------------------------------------------------- RoPE
def test_rope_rotate_90_degrees():
    g = GOLD["rope_rotate_90"]
    x = np.array([[g["input"]]], dtype=np.float64)          # [1, 1, 2]
    phi = math.radians(g["angle_deg"])
    out = oracle.apply_rope(x, np.array([[math.cos(phi)]]), np.array([[math.sin(phi)]]))
    np.testing.assert_allclose(out[0, 0], g["output"], atol=1e-15)


def test_rope_relative_position_example():
    g = GOLD["rope_relative_example"]
    w = np.array([math.radians(g["omega_deg_per_position"])])

    def rot(pos):
        phi = oracle.rope_angles([pos], w)
        return oracle.apply_rope(np.array([[g["pair"]]], dtype=float), np.cos(phi), np.sin(phi))[0, 0]

    q, k = rot(g["q_pos"]), rot(g["k_pos"])
    ang_q = math.degrees(math.atan2(q[1], q[0])) % 360
    ang_k = math.degrees(math.atan2(k[1], k[0])) % 360
    assert ang_q == pytest.approx(g["angles_deg"][0], abs=1e-4)
    assert ang_k == pytest.approx(g["angles_deg"][1], abs=1e-4)
    assert abs(float(q @ k)) < 1e-6
    assert abs(float(rot(g["shifted_q_pos"]) @ rot(g["shifted_k_pos"]))) < 1e-6
    # moving only the key changes the dot product
    assert abs(float(q @ rot(g["k_pos"] + 1))) > 0.4


def test_rope_schedule_closed_form():
    g = GOLD["rope_first_pair_speed"]
    w = oracle.rope_inv_freq(g["head_dim"], g["theta"])
    assert len(w) == g["pairs"]
    assert w[0] == g["omega_0_rad_per_position"]
    i = np.arange(64)
    np.testing.assert_allclose(w, 500000.0 ** (-2.0 * i / 128), rtol=2e-7)
    assert np.all(np.diff(w) < 0)


def test_rope_pairs_are_adjacent_and_norm_preserving():
    hd = 16
    rng = np.random.default_rng(2)
    cos, sin = oracle.rope_cos_sin(np.arange(7), hd, 10000.0)
    for j in range(hd):
        e = np.zeros((1, 7, hd))
        e[0, :, j] = 1.0
        out = oracle.apply_rope(e, cos, sin)
        pair = {j, j ^ 1}
        nz = {c for c in range(hd) if np.any(np.abs(out[0, 1:, c]) > 1e-12)}
        assert nz == pair, (j, nz)
    x = rng.standard_normal((3, 7, hd))
    out = oracle.apply_rope(x, cos, sin)
    np.testing.assert_allclose(out[:, 0], x[:, 0], atol=1e-15)            # position 0: identity
    np.testing.assert_allclose((out[..., 0::2] ** 2 + out[..., 1::2] ** 2),
                               (x[..., 0::2] ** 2 + x[..., 1::2] ** 2), rtol=1e-12)


def test_rope_relative_identity_and_sign():
    # q_m . k_n depends only on n - m (exact angles so that the identity is exact)
    hd = 8
    rng = np.random.default_rng(3)
    w = np.array([1.0, 0.3, 0.05, 0.001])
    q = rng.standard_normal(hd)
    k = rng.standard_normal(hd)

    def rot(v, m):
        phi = m * w[None, :]
        return oracle.apply_rope(v[None, None, :], np.cos(phi), np.sin(phi))[0, 0]

    d1 = rot(q, 5) @ rot(k, 2)
    d2 = rot(q, 105) @ rot(k, 102)
    assert d1 == pytest.approx(d2, rel=1e-12, abs=1e-12)
    # counter-clockwise convention: rotating by +phi then by -phi gives back x
    phi = np.array([[0.7]])
    y = oracle.apply_rope(np.array([[[0.3, -1.2]]]), np.cos(phi), np.sin(phi))
    z = oracle.apply_rope(y, np.cos(-phi), np.sin(-phi))
    np.testing.assert_allclose(z[0, 0], [0.3, -1.2], atol=1e-15)
    assert y[0, 0, 1] == pytest.approx(0.3 * math.sin(0.7) - 1.2 * math.cos(0.7))


def test_rope_angles_use_float32_product():
    w = oracle.rope_inv_freq(128, 500000.0)
    phi = oracle.rope_angles([16383], w)
    expect = (np.float32(16383) * w.astype(np.float32)).astype(np.float64)
    assert np.array_equal(phi[0], expect)


def test_llama3_scaling_regimes():
    base = oracle.rope_inv_freq(128, 500000.0)
    sc = dict(factor=8.0, low_freq_factor=1.0, high_freq_factor=4.0, orig_max_pos=8192)
    w = oracle.rope_inv_freq(128, 500000.0, sc)
    lam = 2 * math.pi / base
    keep = lam < 8192 / 4
    slow = lam > 8192 / 1
    blend = ~keep & ~slow
    assert keep.sum() == 29 and slow.sum() == 29 and blend.sum() == 6
    assert np.array_equal(np.nonzero(keep)[0], np.arange(29))
    assert np.array_equal(w[keep], base[keep])
    assert np.array_equal(w[slow], base[slow] / 8.0)
    assert np.all(w[blend] < base[blend]) and np.all(w[blend] > base[blend] / 8.0)
    assert np.all(np.diff(w) < 0)


@pytest.mark.parametrize("i", [10, 30, 50])
def test_llama3_blend_is_continuous_at_both_thresholds(i):
    """The pages fix the two outer regimes (fastest rotations kept, slowest slowed
    by the factor) but not the blend between them; whatever the blend, it must
    meet each outer regime where the band begins and ends.  orig_max_pos is set
    so that pair i's wavelength sits a relative delta inside the band: just
    above orig/high the oracle's speed must approach omega_i, just below
    orig/low it must approach omega_i / factor, both to within O(delta).  A
    blend with its ends swapped, or one that jumps at either threshold, fails."""
    base = oracle.rope_inv_freq(128, 500000.0)
    lam = 2 * math.pi / base[i]
    for delta in (1e-3, 1e-5):
        near_high = dict(factor=8.0, low_freq_factor=1.0, high_freq_factor=4.0,
                         orig_max_pos=4.0 * lam / (1.0 + delta))      # lam = orig/4 * (1 + delta)
        w = oracle.rope_inv_freq(128, 500000.0, near_high)[i]
        assert abs(w / base[i] - 1.0) <= 2.0 * delta + 1e-6
        assert w < base[i]                                             # inside the band: slowed a little
        near_low = dict(factor=8.0, low_freq_factor=1.0, high_freq_factor=4.0,
                        orig_max_pos=lam / (1.0 - delta))             # lam = orig * (1 - delta)
        w = oracle.rope_inv_freq(128, 500000.0, near_low)[i]
        assert abs(w / (base[i] / 8.0) - 1.0) <= 3.0 * delta + 1e-6
        assert w > base[i] / 8.0
    # just outside the band on either side: exactly the outer regimes
    out_high = dict(factor=8.0, low_freq_factor=1.0, high_freq_factor=4.0, orig_max_pos=4.0 * lam * 1.001)
    assert oracle.rope_inv_freq(128, 500000.0, out_high)[i] == base[i]
    out_low = dict(factor=8.0, low_freq_factor=1.0, high_freq_factor=4.0, orig_max_pos=lam * 0.999)
    assert oracle.rope_inv_freq(128, 500000.0, out_low)[i] == np.float32(base[i] / 8.0)


def test_llama3_blend_is_monotone_across_the_band():
    """Sweeping orig_max_pos moves pair i's wavelength through the whole band;
    the scaled speed must fall monotonically from omega_i to omega_i / factor
    (a blend in the wrong direction, or non-monotone in the band, fails)."""
    base = oracle.rope_inv_freq(128, 500000.0)
    i = 31
    lam = 2 * math.pi / base[i]
    ws = []
    for orig in np.linspace(lam * 1.0001, 4.0 * lam * 0.9999, 200):
        sc = dict(factor=8.0, low_freq_factor=1.0, high_freq_factor=4.0, orig_max_pos=float(orig))
        ws.append(oracle.rope_inv_freq(128, 500000.0, sc)[i])
    ws = np.array(ws)
    # orig grows: the pair moves from the slow end (omega/8) to the fast end (omega)
    assert np.all(np.diff(ws) >= 0)
    assert ws[0] < base[i] / 8.0 * 1.001 and ws[-1] > base[i] * 0.999


# ----------------------------------------------------------------- attention
def _rand_qkv(rng, H=4, Hkv=2, T=9, hd=8):
    return (rng.standard_normal((H, T, hd)), rng.standard_normal((Hkv, T, hd)),
            rng.standard_normal((Hkv, T, hd)))


def test_attention_single_key_returns_v_exactly():
    rng = np.random.default_rng(4)
    q, k, v = _rand_qkv(rng, T=1)
    o = oracle.attention(q, k, v, [0])
    for h in range(4):
        assert np.array_equal(o[h, 0], v[h // 2, 0])


def test_attention_gqa_equals_mha_with_repeat_kv():
    rng = np.random.default_rng(5)
    q, k, v = _rand_qkv(rng, H=8, Hkv=2, T=11)
    o = oracle.attention(q, k, v, np.arange(11))
    o_mha = oracle.attention(q, np.repeat(k, 4, axis=0), np.repeat(v, 4, axis=0), np.arange(11))
    np.testing.assert_allclose(o, o_mha, rtol=0, atol=0)
    # a modulo head map would pair head 1 with kv head 1; contiguous groups pair it with 0
    o_head1 = oracle.attention(q[1:2], k[0:1], v[0:1], np.arange(11))
    np.testing.assert_allclose(o[1], o_head1[0], rtol=0, atol=0)


def test_attention_matches_torch_sdpa_causal():
    rng = np.random.default_rng(6)
    q, k, v = _rand_qkv(rng, H=6, Hkv=3, T=13, hd=16)
    o = oracle.attention(q, k, v, np.arange(13))
    tq = torch.from_numpy(q)[None]
    tk = torch.from_numpy(np.repeat(k, 2, axis=0))[None]
    tv = torch.from_numpy(np.repeat(v, 2, axis=0))[None]
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True)[0].numpy()
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-12)


def test_attention_causal_invariance_and_uniform_weights():
    rng = np.random.default_rng(7)
    q, k, v = _rand_qkv(rng, T=10)
    full = oracle.attention(q, k, v, np.arange(10))
    part = oracle.attention(q[:, :6], k[:, :6], v[:, :6], np.arange(6))
    np.testing.assert_allclose(full[:, :6], part, rtol=1e-14, atol=1e-14)
    o = oracle.attention(np.zeros_like(q), k, v, np.arange(10))
    for m in range(10):
        np.testing.assert_allclose(o[0, m], v[0, :m + 1].mean(axis=0), rtol=1e-13, atol=1e-14)


def test_attention_decode_sees_all_cached_keys_plus_own():
    # one query at position P reads L = P + 1 keys; with equal scores the output is
    # the mean of all P + 1 values, so a dropped first key or an extra key shows.
    rng = np.random.default_rng(8)
    P = 20
    k = np.zeros((1, P + 1, 8))
    v = rng.standard_normal((1, P + 1, 8))
    o = oracle.attention(rng.standard_normal((2, 1, 8)), k, v, [P])
    np.testing.assert_allclose(o[0, 0], v[0].mean(axis=0), rtol=1e-13)
    np.testing.assert_allclose(o[1, 0], v[0].mean(axis=0), rtol=1e-13)


def test_attention_one_hot_values_expose_softmax():
    rng = np.random.default_rng(9)
    T = 7
    q = rng.standard_normal((1, T, T))
    k = rng.standard_normal((1, T, T))
    v = np.eye(T)[None]
    o = oracle.attention(q, k, v, np.arange(T))
    s = q[0] @ k[0].T / math.sqrt(T)
    for m in range(T):
        e = np.exp(s[m, :m + 1] - s[m, :m + 1].max())
        np.testing.assert_allclose(o[0, m, :m + 1], e / e.sum(), rtol=1e-13)
        assert np.all(o[0, m, m + 1:] == 0.0)


# ----------------------------------------------------------------- SwiGLU
def test_silu_closed_forms():
    z = np.array([0.0, 1.0, -1.0, 40.0, -40.0])
    s = oracle.silu(z)
    assert s[0] == 0.0
    assert s[1] == pytest.approx(1.0 / (1.0 + math.exp(-1.0)), rel=1e-15)
    assert s[2] == pytest.approx(-1.0 / (1.0 + math.e), rel=1e-15)
    assert s[3] == pytest.approx(40.0, rel=1e-15)
    assert -1e-15 < s[4] < 0.0


def _silu_inverse(y):
    lo, hi = -1.278, 50.0       # silu is increasing above its minimum at z ~ -1.278
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if mid / (1 + math.exp(-mid)) < y:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


def test_swiglu_page_gate_example():
    g = GOLD["swiglu_gate_example"]
    gate_pre = np.array([_silu_inverse(t) for t in g["gate_branch"]])
    np.testing.assert_allclose(oracle.silu(gate_pre), g["gate_branch"], atol=1e-12)
    # a = e_0; W_gate maps it to gate_pre, W_up to the up branch, W_down = identity
    a = np.array([[1.0, 0.0, 0.0]])
    w_gate = np.zeros((3, 3)); w_gate[:, 0] = gate_pre
    w_up = np.zeros((3, 3)); w_up[:, 0] = g["up_branch"]
    out = oracle.swiglu(a, w_gate, w_up, np.eye(3))
    np.testing.assert_allclose(out[0], g["product"], atol=1e-11)
    # roles are not symmetric: swapping gate and up gives something else
    out_sw = oracle.swiglu(a, w_up, w_gate, np.eye(3))
    assert np.abs(out_sw[0] - np.array(g["product"])).max() > 0.1


def test_swiglu_weight_orientation():
    # [out, in] layout: a [1, d] with W_down [d_model, d_ff] must reject a transposed matrix
    rng = np.random.default_rng(10)
    a = rng.standard_normal((2, 5))
    wg, wu, wd = rng.standard_normal((7, 5)), rng.standard_normal((7, 5)), rng.standard_normal((5, 7))
    out = oracle.swiglu(a, wg, wu, wd)
    ref = (oracle.silu(a @ wg.T) * (a @ wu.T)) @ wd.T
    np.testing.assert_allclose(out, ref, rtol=1e-14)
    with pytest.raises(ValueError):
        oracle.swiglu(a, wg, wu, wd.T)


# ----------------------------------------------------------------- the block
def test_block_zero_projections_give_identity():
    cfg = _cfg()
    rng = np.random.default_rng(11)
    w = _rand_weights(cfg, rng)
    for k in ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down"):
        w[k] = np.zeros_like(w[k])
    x = rng.standard_normal((2, 5, cfg.d_model))
    kc = np.zeros((2, cfg.n_kv_heads, 8, cfg.head_dim))
    y, _, _ = oracle.block_forward(cfg, w, x, kc, kc.copy())
    assert np.array_equal(y, x)


def test_block_zero_gate_gives_h_and_zero_wo_gives_x():
    cfg = _cfg()
    rng = np.random.default_rng(12)
    w = _rand_weights(cfg, rng)
    x = rng.standard_normal((1, 6, cfg.d_model))
    kc = np.zeros((1, cfg.n_kv_heads, 8, cfg.head_dim))
    w0 = dict(w, w_gate=np.zeros_like(w["w_gate"]))
    y, _, _, parts = oracle.block_forward(cfg, w0, x, kc, kc.copy(), return_parts=True)
    assert np.array_equal(y, parts["h"])
    w1 = dict(w0, wo=np.zeros_like(w["wo"]))
    y1, _, _ = oracle.block_forward(cfg, w1, x, kc, kc.copy())
    assert np.array_equal(y1, x)


def test_block_causal_invariance_and_row_sampling():
    cfg = _cfg()
    rng = np.random.default_rng(13)
    w = _rand_weights(cfg, rng)
    x = rng.standard_normal((2, 9, cfg.d_model))
    kc = np.zeros((2, cfg.n_kv_heads, 16, cfg.head_dim))
    y, kn, vn = oracle.block_forward(cfg, w, x, kc, kc.copy())
    y5, kn5, _ = oracle.block_forward(cfg, w, x[:, :5], kc, kc.copy())
    np.testing.assert_allclose(y[:, :5], y5, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(kn[:, :, :5], kn5, rtol=1e-13, atol=1e-13)
    ys, _, _ = oracle.block_forward(cfg, w, x, kc, kc.copy(), rows=[0, 4, 8])
    np.testing.assert_allclose(ys, y[:, [0, 4, 8]], rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("scaled", [False, True])
def test_block_prefill_then_decode_equals_longer_prefill(scaled):
    cfg = _cfg(rope_scaling=scaled)
    rng = np.random.default_rng(14)
    w = _rand_weights(cfg, rng)
    T = 7
    x = rng.standard_normal((3, T + 1, cfg.d_model))
    cap = 16
    kc = np.zeros((3, cfg.n_kv_heads, cap, cfg.head_dim))
    vc = np.zeros_like(kc)
    y_full, _, _ = oracle.block_forward(cfg, w, x, kc, vc)
    _, kn, vn = oracle.block_forward(cfg, w, x[:, :T], kc, vc)
    kc2, vc2 = kc.copy(), vc.copy()
    kc2[:, :, :T] = kn
    vc2[:, :, :T] = vn
    y_dec, _, _ = oracle.block_forward(cfg, w, x[:, T:], kc2, vc2, start_pos=T)
    np.testing.assert_allclose(y_dec[:, 0], y_full[:, T], rtol=1e-12, atol=1e-12)


def test_block_against_independent_torch_evaluation():
    """Second fp64 evaluation built from library routines: torch rms_norm, complex
    multiplication for RoPE (the pages' view_as_complex formulation), SDPA with
    repeat_interleave, F.silu."""
    cfg = _cfg(d_model=64, n_heads=8, n_kv_heads=2, head_dim=8, d_ff=80, rope_theta=10000.0)
    rng = np.random.default_rng(15)
    w = _rand_weights(cfg, rng)
    B, T = 2, 12
    x = rng.standard_normal((B, T, cfg.d_model))
    kc = np.zeros((B, cfg.n_kv_heads, 16, cfg.head_dim))
    y, kn, _ = oracle.block_forward(cfg, w, x, kc, kc.copy())

    F = torch.nn.functional
    tw = {k: torch.from_numpy(v) for k, v in w.items()}
    tx = torch.from_numpy(x)
    H, Hkv, hd = cfg.n_heads, cfg.n_kv_heads, cfg.head_dim
    a = F.rms_norm(tx, (cfg.d_model,), weight=tw["attn_norm"], eps=cfg.eps)
    q = (a @ tw["wq"].T).view(B, T, H, hd)
    k = (a @ tw["wk"].T).view(B, T, Hkv, hd)
    v = (a @ tw["wv"].T).view(B, T, Hkv, hd)
    inv = 1.0 / (cfg.rope_theta ** (torch.arange(0, hd, 2, dtype=torch.float32) / hd))
    ang = torch.outer(torch.arange(T, dtype=torch.float32), inv).double()
    rot = torch.polar(torch.ones_like(ang), ang)                     # complex128
    qc = torch.view_as_complex(q.reshape(B, T, H, hd // 2, 2).contiguous())
    kc_ = torch.view_as_complex(k.reshape(B, T, Hkv, hd // 2, 2).contiguous())
    q = torch.view_as_real(qc * rot[None, :, None, :]).reshape(B, T, H, hd)
    k = torch.view_as_real(kc_ * rot[None, :, None, :]).reshape(B, T, Hkv, hd)
    np.testing.assert_allclose(kn, k.permute(0, 2, 1, 3).numpy(), rtol=1e-12, atol=1e-12)
    qh = q.transpose(1, 2)
    kh = k.transpose(1, 2).repeat_interleave(H // Hkv, dim=1)
    vh = v.transpose(1, 2).repeat_interleave(H // Hkv, dim=1)
    o = F.scaled_dot_product_attention(qh, kh, vh, is_causal=True)
    h = tx + o.transpose(1, 2).reshape(B, T, H * hd) @ tw["wo"].T
    a2 = F.rms_norm(h, (cfg.d_model,), weight=tw["ffn_norm"], eps=cfg.eps)
    ref = h + (F.silu(a2 @ tw["w_gate"].T) * (a2 @ tw["w_up"].T)) @ tw["w_down"].T
    np.testing.assert_allclose(y, ref.numpy(), rtol=1e-10, atol=1e-10)


def test_block_brute_force_loops_tiny():
    """Scalar loops over every index on a tiny block (no matrix routines)."""
    cfg = _cfg(d_model=8, n_heads=4, n_kv_heads=2, head_dim=2, d_ff=6, rope_theta=100.0)
    rng = np.random.default_rng(16)
    w = _rand_weights(cfg, rng)
    T = 4
    x = rng.standard_normal((1, T, 8))
    kc = np.zeros((1, 2, 4, 2))
    y, _, _ = oracle.block_forward(cfg, w, x, kc, kc.copy())
    d, H, hd = 8, 4, 2

    def norm(vec, g):
        ms = sum(t * t for t in vec) / len(vec)
        return [vec[i] / math.sqrt(ms + cfg.eps) * g[i] for i in range(len(vec))]

    def lin(vec, W):
        return [sum(W[o][i] * vec[i] for i in range(len(vec))) for o in range(len(W))]

    ws = {k: v.tolist() for k, v in w.items()}
    qs, ks, vs, hs = [], [], [], []
    for t in range(T):
        a = norm(x[0, t].tolist(), ws["attn_norm"])
        q, k, v = lin(a, ws["wq"]), lin(a, ws["wk"]), lin(a, ws["wv"])
        om = float(np.float32(1.0) / np.float32(100.0 ** 0.0))
        phi = float(np.float32(t) * np.float32(om))
        c, s = math.cos(phi), math.sin(phi)
        qs.append([(q[2 * i] * c - q[2 * i + 1] * s, q[2 * i] * s + q[2 * i + 1] * c)[j]
                   for i in range(len(q) // 2) for j in range(2)])
        ks.append([(k[2 * i] * c - k[2 * i + 1] * s, k[2 * i] * s + k[2 * i + 1] * c)[j]
                   for i in range(len(k) // 2) for j in range(2)])
        vs.append(v)
    for t in range(T):
        o = []
        for h in range(H):
            g = h // 2
            sc = [sum(qs[t][h * hd + j] * ks[n][g * hd + j] for j in range(hd)) / math.sqrt(hd)
                  for n in range(t + 1)]
            mx = max(sc)
            e = [math.exp(z - mx) for z in sc]
            o += [sum(e[n] * vs[n][g * hd + j] for n in range(t + 1)) / sum(e) for j in range(hd)]
        h1 = [x[0, t, i] + lin(o, ws["wo"])[i] for i in range(d)]
        a2 = norm(h1, ws["ffn_norm"])
        gt, up = lin(a2, ws["w_gate"]), lin(a2, ws["w_up"])
        u = [gt[i] / (1 + math.exp(-gt[i])) * up[i] for i in range(len(gt))]
        yt = [h1[i] + lin(u, ws["w_down"])[i] for i in range(d)]
        np.testing.assert_allclose(y[0, t], yt, rtol=1e-12, atol=1e-12)
