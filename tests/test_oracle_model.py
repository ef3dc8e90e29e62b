"""CPU pins of the oracle's model forward (embedding, blocks, final RMSNorm, LM
head), against page-printed counts and against properties fixed by the
definition.  No GPU."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import workloads

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_values.json")))


def test_model_param_counts_match_the_pages():
    g = GOLD["model_params_8b"]
    s = g["shape"]
    c = oracle.model_param_counts(s["d_model"], s["n_heads"], s["n_kv_heads"], s["head_dim"], s["d_ff"],
                                  s["n_layers"], s["vocab"])
    assert round(c["total"] / 1e9, 2) == g["value"]["total_billions_2dp"]
    assert round(c["non_embedding"] / 1e9, 2) == g["value"]["non_embedding_billions_2dp"]
    e = GOLD["embedding_params_70b"]
    c70 = oracle.model_param_counts(e["shape"]["d_model"], 64, 8, 128, 28672, 80, e["shape"]["vocab"])
    assert round(c70["embedding"] / 1e9, 2) == e["value"]["billions_2dp"]


def _tiny(n_layers=2, vocab=96, seed=3):
    shp = workloads.BlockShape(d_model=64, n_heads=4, n_kv_heads=2, head_dim=16, d_ff=96, dtype="f32")
    params, gen = workloads.make_model_weights(shp, n_layers, vocab, seed)
    return shp, params, gen


def test_embedding_is_a_row_lookup():
    E = np.arange(12.0).reshape(4, 3)
    x = oracle.embed(E, [[2, 0], [3, 3]])
    assert np.array_equal(x, np.array([[[6, 7, 8], [0, 1, 2]], [[9, 10, 11], [9, 10, 11]]], dtype=np.float64))
    with pytest.raises(ValueError):
        oracle.embed(E, [[4]])
    with pytest.raises(ValueError):
        oracle.embed(E, [[-1]])


def test_zero_layers_is_norm_then_head():
    """No blocks: logits = RMSNorm(E[t]) W_out^T, written out row by row through a
    one-hot product (a different route from the lookup)."""
    shp, params, gen = _tiny(n_layers=0)
    V, d = params["embed"].shape
    tok = torch.randint(0, V, (2, 5), generator=gen)
    logits, _, _ = oracle.model_forward(shp, params, tok, [], [], 0)
    E = params["embed"].double().numpy()
    W = params["lm_head"].double().numpy()
    g = params["final_norm"].double().numpy()
    for b in range(2):
        for t in range(5):
            onehot = np.zeros(V)
            onehot[int(tok[b, t])] = 1.0
            x = onehot @ E
            z = x / np.sqrt(np.mean(x * x) + shp.eps) * g
            assert np.allclose(logits[b, t], W @ z, rtol=1e-12, atol=1e-12)


def test_last_only_is_the_last_row_and_sequences_are_independent():
    shp, params, gen = _tiny()
    V = params["embed"].shape[0]
    B, T = 3, 6
    tok = torch.randint(0, V, (B, T), generator=gen)
    cap = 8
    kc = [torch.zeros(B, shp.n_kv_heads, cap, shp.head_dim) for _ in params["layers"]]
    vc = [torch.zeros_like(k) for k in kc]
    full, _, _ = oracle.model_forward(shp, params, tok, kc, vc, 0)
    last, _, _ = oracle.model_forward(shp, params, tok, kc, vc, 0, last_only=True)
    assert np.array_equal(last, full[:, -1])
    one, _, _ = oracle.model_forward(shp, params, tok[1:2], [k[1:2] for k in kc], [v[1:2] for v in vc], 0)
    assert np.allclose(one[0], full[1], rtol=1e-12, atol=1e-12)


def test_prefill_then_decode_equals_longer_prefill():
    """forward(tokens[:T]) filling the caches, then forward(token T, start_pos=T)
    gives the logits of position T of forward(tokens[:T+1])."""
    shp, params, gen = _tiny(n_layers=3)
    V = params["embed"].shape[0]
    B, T = 2, 7
    tok = torch.randint(0, V, (B, T + 1), generator=gen)
    cap = 16
    kc = [torch.zeros(B, shp.n_kv_heads, cap, shp.head_dim, dtype=torch.float64) for _ in params["layers"]]
    vc = [torch.zeros_like(k) for k in kc]
    long_logits, _, _ = oracle.model_forward(shp, params, tok, kc, vc, 0)
    _, ks, vs = oracle.model_forward(shp, params, tok[:, :T], kc, vc, 0)
    for l in range(len(params["layers"])):
        kc[l][:, :, :T] = torch.from_numpy(ks[l])
        vc[l][:, :, :T] = torch.from_numpy(vs[l])
    step, _, _ = oracle.model_forward(shp, params, tok[:, T:], kc, vc, T)
    assert np.allclose(step[:, 0], long_logits[:, T], rtol=1e-10, atol=1e-10)
