"""Two-level chunk / token selection over a paged, non-contiguous prefix cache.

Prefilling-dLLM (abstract): the prefix is cut into N chunks whose KV is cached once; decoding keeps the
top-K most relevant chunks with token-level sparsity inside each, and attends over the chunk KV where
it lies (non-contiguously); a beginning-of-sequence token leads every chunk and acts as a recurring
attention anchor.

Readings:
  * chunk score = pinned dot product of the predicted-query sum with the chunk's key sum (a tree over
    all of the chunk's tokens in logical order, anchor included);
  * the top-K chunks are chosen per KV head (ties to the lower chunk); the other reading, one chunk
    set per sequence shared by all its KV heads, ranks chunks by their scores summed over the KV
    heads (pinned float32 tree over the heads, zero-padded to a power of two), same tie rule;
  * inside a chosen chunk its anchor (token 0) is always kept and the top ceil(frac * chunk) of the
    remaining tokens by token score (ties to the lower token) are added;
  * unchosen chunks contribute nothing; attention then runs over the kept tokens plus the block's
    own T tokens.
"""
from __future__ import annotations

import numpy as np

from .fp32tree import tree_sum
from .scoring import pool_keys, token_scores, unit_scores
from .selection import topk_indices


def select_chunks(qs, k_logical, chunk_tokens: int, top_k_chunks: int):
    """-> (chunk scores [B][Hkv][n_chunks] f32, chosen [B][Hkv][top_k] ascending int32)."""
    cs = pool_keys(k_logical, chunk_tokens)
    sc = unit_scores(qs, cs)
    B, H, _ = sc.shape
    chosen = np.zeros((B, H, top_k_chunks), dtype=np.int32)
    for b in range(B):
        for g in range(H):
            chosen[b, g] = sorted(topk_indices(sc[b, g], top_k_chunks))
    return sc, chosen


def select_chunks_shared(qs, k_logical, chunk_tokens: int, top_k_chunks: int):
    """Per-sequence reading -> (chunk scores [B][Hkv][n_chunks] f32, summed over the heads [B][n_chunks]
    f32, chosen [B][Hkv][top_k] ascending int32, the same row for every head)."""
    sc = unit_scores(qs, pool_keys(k_logical, chunk_tokens))
    seq = tree_sum(sc, axis=1)
    B, H, _ = sc.shape
    chosen = np.zeros((B, H, top_k_chunks), dtype=np.int32)
    for b in range(B):
        chosen[b, :] = sorted(topk_indices(seq[b], top_k_chunks))
    return sc, seq, chosen


def select_tokens(qs, k_logical, chosen, chunk_tokens: int, keep: int):
    """-> (token scores [B][Hkv][top_k][chunk] f32, kept token ids [B][Hkv][top_k*(1+keep)])."""
    B, H, nc = chosen.shape
    D = k_logical.shape[-1]
    keep = min(keep, chunk_tokens - 1)
    ks = np.stack([np.stack([np.stack([k_logical[b, g, c * chunk_tokens:(c + 1) * chunk_tokens]
                                       for c in chosen[b, g]]) for g in range(H)]) for b in range(B)])
    ts = token_scores(qs, ks.reshape(B, H, nc * chunk_tokens, D)).reshape(B, H, nc, chunk_tokens)
    kept = np.zeros((B, H, nc * (1 + keep)), dtype=np.int32)
    for b in range(B):
        for g in range(H):
            row = []
            for j, c in enumerate(chosen[b, g]):
                base = int(c) * chunk_tokens
                best = topk_indices(ts[b, g, j], keep, exclude=[0])
                row.extend(sorted([base] + [base + t for t in best]))
            kept[b, g] = row
    return ts, kept
