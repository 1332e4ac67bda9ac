"""Keep the sinks plus the top-K units; exact integer logic.

Focus-dLLM (abstract; Elamur "Summary"): the predicted queries keep only the most relevant KV, sinks
are always preserved, and deeper layers reuse the source layer's sink locations.  Prefilling-dLLM
(abstract): the top-K chunks are kept, with token-level sparsity inside each.

Readings:
  * every block holding a sink token is forced in; K counts the other (non-forced) blocks;
  * ranking is by score, highest first, with -0 equal to +0, NaN below everything, and ties to the
    lower index; K larger than what is left keeps everything;
  * the kept set is reported in ascending order;
  * the other reading of sink retention (token granularity): the sink tokens themselves are kept and
    the top-K blocks are chosen among all blocks.
"""
from __future__ import annotations

import numpy as np

from .fp32tree import order_key


def topk_indices(scores, k: int, exclude=()) -> list[int]:
    """Indices of the k best scores (key desc, index asc), skipping ``exclude``."""
    key = order_key(np.asarray(scores, np.float32)).astype(np.int64)
    ex = set(int(e) for e in exclude)
    cand = [i for i in range(len(key)) if i not in ex]
    cand.sort(key=lambda i: (-key[i], i))
    return cand[: max(0, min(k, len(cand)))]


def select_units(scores, forced, k: int) -> np.ndarray:
    """Forced units plus the top-k of the rest, ascending, as int32."""
    forced = sorted(set(int(f) for f in forced))
    chosen = topk_indices(scores, k, exclude=forced)
    return np.array(sorted(set(forced) | set(chosen)), dtype=np.int32)


def sink_blocks(sink_pos, n_sinks: int, kv_block: int) -> list[int]:
    return sorted(set(int(s) // kv_block for s in list(sink_pos)[: int(n_sinks)]))


def select_token_sinks(scores, sink_pos, n_sinks, kv_block: int, k: int, ctx_len: int):
    """Token-granular sink retention, the other reading of how sinks are kept: the top k blocks of
    all blocks (sink blocks compete like the others), and the sink tokens themselves.  -> list over
    b of list over g of the ascending cached-token ids attended (each id once)."""
    scores = np.asarray(scores)
    B, H, _ = scores.shape
    out = []
    for b in range(B):
        sinks = set()
        if sink_pos is not None:
            sinks = {int(t) for t in list(sink_pos[b])[: int(n_sinks[b])] if 0 <= int(t) < ctx_len}
        row = []
        for g in range(H):
            toks = set(sinks)
            for blk in select_units(scores[b, g], [], k):
                toks.update(range(int(blk) * kv_block, min((int(blk) + 1) * kv_block, ctx_len)))
            row.append(np.array(sorted(toks), dtype=np.int32))
        out.append(row)
    return out


def select_blocks(scores, sink_pos, n_sinks, kv_block: int, k: int):
    """scores [B][Hkv][n_blk] -> list over b of list over g of ascending int32 block ids."""
    scores = np.asarray(scores)
    B, H, _ = scores.shape
    out = []
    for b in range(B):
        forced = sink_blocks(sink_pos[b], n_sinks[b], kv_block) if sink_pos is not None else []
        out.append([select_units(scores[b, g], forced, k) for g in range(H)])
    return out
