"""One layer-step of the method, chaining the oracle's steps in the order the pages give them.

Focus-dLLM (Elamur "Summary"): predict positions from the previous confidence and widen them, let the
predicted queries select KV, keep sinks (found at one layer, reused deeper), keep full attention in
the shallow layers.  Prefilling-dLLM (abstract): top-K chunks, then tokens inside them, over a paged
prefix.

``p`` is any object with the workload attributes (batch, n_q_heads, n_kv_heads, head_dim, ctx_len,
dec_len, kv_block, top_k_pos, window, top_k_blocks, sink_tau, max_sinks and, for the chunked mode,
chunk_tokens, top_k_chunks, tokens_per_chunk_kept, page_tokens).
"""
from __future__ import annotations

import numpy as np

from .attention import attend, blocks_to_tokens
from .chunked import select_chunks, select_chunks_shared, select_tokens
from .predictor import predict_positions
from .scoring import gather_logical, pool_keys, query_sum, unit_scores
from .selection import select_blocks, select_token_sinks
from .sinks import detect_sinks


def focus_layer_step(p, x: dict, mode: str, sinks=None, ks=None, with_output: bool = True,
                     sink_tokens: bool = False) -> dict:
    """mode: "dense" (full attention), "source" (detect sinks here) or "reuse" (take ``sinks``).

    x holds q, k, v, k_dec, v_dec, prev_conf (or None), masked.  ``sinks`` = (sink_pos, n_sinks) from
    the source layer.  ``ks`` = the layer's pooled keys if already computed.
    """
    r: dict = {}
    bits, npred = predict_positions(x.get("prev_conf"), x["masked"], p.top_k_pos, p.window)
    r["pred_mask"], r["n_pred"] = bits, npred
    if mode == "dense":
        if with_output:
            r["out"] = attend(x["q"], x["k"], x["v"], x["k_dec"], x["v_dec"], None)
        return r
    if ks is None:
        ks = pool_keys(x["k"], p.kv_block)
    r["ks"] = ks
    qs = query_sum(x["q"], bits, p.n_kv_heads)
    r["qs"] = qs
    r["scores"] = unit_scores(qs, ks)
    if mode == "source":
        pos, n, over, margin = detect_sinks(x["q"], x["k"], x["k_dec"], bits, p.sink_tau, p.max_sinks)
        r["sink_pos"], r["n_sinks"], r["sink_overflow"], r["sink_margin"] = pos, n, over, margin
    elif mode == "reuse":
        pos, n = sinks
        r["sink_pos"], r["n_sinks"] = pos, n
    else:
        raise ValueError(mode)
    if sink_tokens:   # token-granular sink retention: sinks as tokens, top-K of all blocks
        toks = select_token_sinks(r["scores"], r["sink_pos"], r["n_sinks"], p.kv_block, p.top_k_blocks,
                                  p.ctx_len)
        r["tokens"] = toks
        if with_output:
            r["out"] = attend(x["q"], x["k"], x["v"], x["k_dec"], x["v_dec"], toks)
        return r
    sel = select_blocks(r["scores"], r["sink_pos"], r["n_sinks"], p.kv_block, p.top_k_blocks)
    r["sel"] = sel
    if with_output:
        toks = [[blocks_to_tokens(s, p.kv_block, p.ctx_len) for s in row] for row in sel]
        r["out"] = attend(x["q"], x["k"], x["v"], x["k_dec"], x["v_dec"], toks)
    return r


def chunked_layer_step(p, x: dict, with_output: bool = True, per_sequence: bool = False) -> dict:
    """Chunked, paged workload: x holds q, k_pool, v_pool, page_table, k_dec, v_dec, prev_conf, masked.
    per_sequence: one chunk set per sequence, from the chunk scores summed over the KV heads."""
    r: dict = {}
    bits, npred = predict_positions(x.get("prev_conf"), x["masked"], p.top_k_pos, p.window)
    r["pred_mask"], r["n_pred"] = bits, npred
    kl = gather_logical(x["k_pool"], x["page_table"], p.page_tokens)
    qs = query_sum(x["q"], bits, p.n_kv_heads)
    r["qs"] = qs
    if per_sequence:
        r["chunk_scores"], r["seq_chunk_scores"], r["chunks"] = select_chunks_shared(qs, kl, p.chunk_tokens,
                                                                                     p.top_k_chunks)
    else:
        r["chunk_scores"], r["chunks"] = select_chunks(qs, kl, p.chunk_tokens, p.top_k_chunks)
    r["token_scores"], r["tokens"] = select_tokens(qs, kl, r["chunks"], p.chunk_tokens,
                                                   p.tokens_per_chunk_kept)
    if with_output:
        vl = gather_logical(x["v_pool"], x["page_table"], p.page_tokens)
        B, H = r["tokens"].shape[:2]
        toks = [[r["tokens"][b, g] for g in range(H)] for b in range(B)]
        r["out"] = attend(x["q"], kl, vl, x["k_dec"], x["v_dec"], toks)
    return r


def schedule_modes(p) -> list[str]:
    """Layer modes of a multi-layer step: dense shallow layers, one source layer, reuse below it."""
    modes = []
    for layer in range(p.n_layers):
        if layer < p.dense_layers:
            modes.append("dense")
        elif layer == p.source_layer:
            modes.append("source")
        else:
            modes.append("reuse")
    return modes

