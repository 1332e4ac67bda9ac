"""Pooled-key block scoring against the predicted queries, in pinned float32.

Focus-dLLM (abstract; Elamur "Summary"): the predicted queries pick out the most relevant parts of the
KV cache, so that redundant attention is estimated and skipped.  Prefilling-dLLM (abstract) ranks
whole prefix chunks first, then tokens inside the chosen chunks.

Readings (the pages give no formula):
  * a KV unit (block, page or chunk) is represented by the float32 sum of its keys, summed with the
    pinned tree over its tokens in logical order (a partial last block sums its valid tokens only);
  * the predicted queries of a KV head's q-head group are summed: a tree over the T slots
    (non-predicted slots contribute +0.0), then a tree over the group's q-heads padded to a power of
    two;
  * a unit's score is the pinned float32 dot product of the two sums; the 1/sqrt(D) scale and mean
    pooling are left out because a positive scale does not change the ranking;
  * a token's score (the chunked workload's second level) is the same dot product with that token's
    key.
"""
from __future__ import annotations

import numpy as np

from .fp32tree import tree_dot, tree_sum, values_f32


def pool_keys(k, unit: int) -> np.ndarray:
    """k [B][Hkv][L][D] -> unit sums [B][Hkv][ceil(L/unit)][D] float32 (tree over each unit's tokens)."""
    kf = values_f32(k)
    B, H, L, D = kf.shape
    n = -(-L // unit)
    if n * unit != L:
        kf = np.concatenate([kf, np.zeros((B, H, n * unit - L, D), np.float32)], axis=2)
    blocks = kf.reshape(B, H, n, unit, D)
    return tree_sum(blocks, axis=3)


def gather_logical(pool, page_table, page_tokens: int) -> np.ndarray:
    """Paged pool [n_pages][Hkv][P][D] -> logical [B][Hkv][pages_per_seq * P][D] (copy)."""
    pool = np.asarray(pool)
    pt = np.asarray(page_table)
    B, npp = pt.shape
    _, H, P, D = pool.shape
    assert P == page_tokens
    out = pool[pt.reshape(-1)].reshape(B, npp, H, P, D).transpose(0, 2, 1, 3, 4)
    return out.reshape(B, H, npp * P, D)


def query_sum(q, pred_bits, n_kv_heads: int) -> np.ndarray:
    """q [B][Hq][T][D], pred_bits [B] -> qs [B][Hkv][D] float32."""
    qf = values_f32(q)
    B, Hq, T, D = qf.shape
    G = Hq // n_kv_heads
    sel = np.zeros((B, T), dtype=bool)
    for b in range(B):
        v = int(pred_bits[b])
        sel[b] = [(v >> p) & 1 for p in range(T)]
    masked_q = np.where(sel[:, None, :, None], qf, np.float32(0.0)).astype(np.float32)
    per_head = tree_sum(masked_q, axis=2)                         # [B][Hq][D]
    grouped = per_head.reshape(B, n_kv_heads, G, D)
    return tree_sum(grouped, axis=2)                              # [B][Hkv][D]


def unit_scores(qs, ks) -> np.ndarray:
    """qs [B][Hkv][D], ks [B][Hkv][n][D] -> [B][Hkv][n] float32."""
    return tree_dot(np.asarray(qs, np.float32)[:, :, None, :], ks)


def unit_scores_max(q, pred_bits, ks, n_kv_heads: int) -> np.ndarray:
    """Per-query scoring, a reading the pages leave open next to the summed-query one: a unit's score
    is the largest pinned float32 dot product of one predicted query of the KV head's q-head group
    with the unit's key sum (a unit that matters to any single predicted position ranks high).  +0
    when no position is predicted; a -0 result reads +0.  q [B][Hq][T][D], pred_bits [B], ks
    [B][Hkv][n][D] -> [B][Hkv][n] float32."""
    qf = values_f32(q)
    B, Hq, T, D = qf.shape
    G = Hq // n_kv_heads
    ks = np.asarray(ks, dtype=np.float32)
    out = np.zeros((B, n_kv_heads, ks.shape[2]), dtype=np.float32)
    for b in range(B):
        P = [p for p in range(T) if (int(pred_bits[b]) >> p) & 1]
        for g in range(n_kv_heads):
            best = None
            for j in range(G):
                for p in P:
                    s = tree_dot(qf[b, g * G + j, p][None, :], ks[b, g])
                    best = s if best is None else np.maximum(best, s)
            if best is not None:
                out[b, g] = best + np.float32(0.0)
    return out


def unit_scores_mass(q, pred_bits, ks, n_kv_heads: int, unit: int, ctx_len: int) -> np.ndarray:
    """Softmax-mass scoring, a third reading of how the predicted queries estimate which units
    matter (the pages speak of estimating attention importance): every predicted query of the KV
    head's q-head group attends to the units' mean keys (the key sum divided by the number of tokens
    in the unit; a partial last unit counts its valid tokens) with the attention scale 1/sqrt(D), a
    softmax over all units of the head; a unit's score is the probability mass it receives, summed
    over those queries.  float64 throughout; zeros when nothing is predicted.  q [B][Hq][T][D],
    pred_bits [B], ks [B][Hkv][n][D] -> [B][Hkv][n] float64."""
    qf = values_f32(q).astype(np.float64)
    B, Hq, T, D = qf.shape
    G = Hq // n_kv_heads
    ks64 = np.asarray(ks, dtype=np.float64)
    n = ks64.shape[2]
    counts = np.minimum(unit, ctx_len - unit * np.arange(n)).astype(np.float64)
    assert (counts > 0).all()
    kbar = ks64 / counts[None, None, :, None]
    out = np.zeros((B, n_kv_heads, n), dtype=np.float64)
    for b in range(B):
        P = [p for p in range(T) if (int(pred_bits[b]) >> p) & 1]
        if not P:
            continue
        for g in range(n_kv_heads):
            queries = qf[b, g * G:(g + 1) * G][:, P].reshape(-1, D)
            z = queries @ kbar[b, g].T / np.sqrt(D)
            z -= z.max(axis=1, keepdims=True)
            w = np.exp(z)
            w /= w.sum(axis=1, keepdims=True)
            out[b, g] = w.sum(axis=0)
    return out


def token_scores(qs, k_tokens) -> np.ndarray:
    """qs [B][Hkv][D], k_tokens [B][Hkv][n][D] (bf16 bits or float32) -> [B][Hkv][n] float32."""
    return tree_dot(np.asarray(qs, np.float32)[:, :, None, :], values_f32(k_tokens))
