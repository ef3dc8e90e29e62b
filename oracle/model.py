"""Plain fp64 CPU oracle of a Llama-3/3.1 model forward around the blocks.

TEST INFRASTRUCTURE ONLY (same rules as oracle/block.py: imported by tests/,
__graft_entry__.smoke() and bench.py's cpu_baseline leg only; shares nothing
with the HIP library).

What it computes, in the pages' order ([P1] "Llama 3.1 70B": the token
embedding, the stack of transformer layers, the LM head; [P3] "How Llama 3.1
Generates the Next Token": embedding lookup, the blocks, a final RMSNorm and
the unembedding matrix from d_model to the vocabulary; [P4] "Llama 3 8B -
Prepare Q, K, V": forward(tokens, start_pos) with one cache per layer):

  x_0   = E[tokens]                      (one row of the table per token)
  x_l   = block_l(x_{l-1})               (oracle.block.block_forward, with
                                          layer l's cache at start_pos)
  logits = RMSNorm(x_L; g_final) W_out^T (W_out [vocab, d], not tied to E)

Reading: the pages show the LM head on every position; a
caller that samples only needs each sequence's last position, which is the
same rows of the same product (`last_only`).
"""
from __future__ import annotations

from typing import Dict, List, Sequence

import numpy as np
import torch

from .block import block_forward, block_param_counts, rmsnorm, to64

__all__ = ["embed", "model_forward", "model_param_counts"]


def embed(E, tokens) -> np.ndarray:
    """x = E[tokens]: the embedding row of each token id ([P1] token embedding:
    a lookup, no arithmetic).  tokens: integer array [B, T]."""
    t = np.asarray(tokens, dtype=np.int64)
    if t.min() < 0 or t.max() >= E.shape[0]:
        raise ValueError("token id outside the vocabulary")
    if isinstance(E, np.ndarray):
        return to64(E[t])
    return to64(E[torch.from_numpy(t)])         # gather first: only the used rows widen


def model_forward(cfg, params: Dict, tokens, k_caches: Sequence, v_caches: Sequence, start_pos: int = 0,
                  last_only: bool = False):
    """Logits of a model of len(params['layers']) blocks.

    params: 'embed' [V, d], 'layers' (a list of block weight dicts as for
    block_forward), 'final_norm' [d], 'lm_head' [V, d].
    k_caches / v_caches: one [B, n_kv, cap, hd] cache per layer (rows <
    start_pos used).
    Returns (logits [B, T, V] or [B, V] with last_only, new cache rows per layer
    as lists of [B, n_kv, T, hd]).
    """
    x = embed(params["embed"], tokens)                          # [B, T, d]
    ks, vs = [], []
    for l, w in enumerate(params["layers"]):
        x, k_new, v_new = block_forward(cfg, w, x, k_caches[l], v_caches[l], start_pos)
        ks.append(k_new)
        vs.append(v_new)
    if last_only:
        x = x[:, -1]
    z = rmsnorm(x, params["final_norm"], cfg.eps)
    return z @ to64(params["lm_head"]).T, ks, vs


def model_param_counts(d_model, n_heads, n_kv_heads, head_dim, d_ff, n_layers, vocab) -> Dict[str, int]:
    """Parameter counts of the model from its shapes ([P2] section 06: total and
    non-embedding counts of Llama 3.1 8B; the embedding and LM head are separate
    [vocab, d] matrices)."""
    blk = block_param_counts(d_model, n_heads, n_kv_heads, head_dim, d_ff)["block"]
    emb = vocab * d_model
    non_emb = n_layers * blk + d_model                         # blocks + final norm
    return {"embedding": emb, "lm_head": emb, "blocks": n_layers * blk, "final_norm": d_model,
            "non_embedding": non_emb, "total": non_emb + 2 * emb}
