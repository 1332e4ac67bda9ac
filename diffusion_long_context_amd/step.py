"""One layer-step of the method as a chain of libfdllm calls (device buffers come from torch).

Focus-dLLM (Elamur "Summary"): predict positions from the previous confidence and widen them, let the
predicted queries select the KV, keep the sinks (found at one layer, reused in deeper ones) and keep
full attention in the shallow layers.  Prefilling-dLLM (abstract): top-K chunks, then token sparsity
inside each chunk, over a paged prefix.  Nothing here computes: every step is a library call.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from .fdllm import FDL_BF16, Geom, Handle


@dataclass
class FocusParams:
    top_k_pos: int = 4
    window: int = 4
    top_k_blocks: int = 64
    sink_tau: float = 0.03
    max_sinks: int = 64


class FocusStep:
    """Buffers and calls for the Focus-dLLM path on one geometry (contiguous cache)."""

    def __init__(self, h: Handle, g: Geom, fp: FocusParams, device="cuda"):
        self.h, self.g, self.fp = h, g, fp
        B, Hkv = g.batch, g.n_kv_heads
        self.n_blk = -(-g.ctx_len // g.kv_block)
        self.max_sel = max(1, min(self.n_blk, fp.max_sinks + fp.top_k_blocks))
        i32 = dict(dtype=torch.int32, device=device)
        self.pred_mask = torch.zeros(B, dtype=torch.int64, device=device)
        self.n_pred = torch.zeros(B, **i32)
        self.scores = torch.zeros(B, Hkv, max(1, self.n_blk), dtype=torch.float32, device=device)
        self.sink_pos = torch.full((B, fp.max_sinks), -1, **i32)
        self.n_sinks = torch.zeros(B, **i32)
        self.sel_idx = torch.zeros(B, Hkv, self.max_sel, **i32)
        self.n_sel = torch.zeros(B, Hkv, **i32)

    def new_ks(self, device="cuda") -> torch.Tensor:
        g = self.g
        return torch.empty(g.batch, g.n_kv_heads, max(1, self.n_blk), g.head_dim, dtype=torch.float32,
                           device=device)

    def pool(self, k_cache, ks):
        self.h.fdl_pool_keys(self.g, k_cache, None, self.g.kv_block, ks)

    def predict(self, prev_conf, masked):
        self.h.fdl_predict_queries(self.g.batch, self.g.dec_len, prev_conf, masked, self.fp.top_k_pos,
                                   self.fp.window, self.pred_mask, self.n_pred)

    def score(self, q, ks, k_cache=None, k_dec=None, detect_sinks=False, scorer: str = "sum"):
        """scorer "sum": the summed predicted query against each pooled key; "max": the best single
        predicted query (fdl_score_blocks_max); "mass": the softmax mass over the units' mean keys
        (fdl_score_blocks_mass).  Sinks, when asked for, are detected by fdl_score_blocks."""
        if scorer not in ("sum", "max", "mass"):
            raise ValueError(f"unknown scorer {scorer!r}")
        if scorer != "sum":
            if detect_sinks:   # the sink pass also writes summed scores, which the max scores replace
                self.h.fdl_score_blocks(self.g, q, self.pred_mask, ks, self.g.kv_block, self.scores,
                                        k_cache=k_cache, k_dec=k_dec, detect_sinks=True,
                                        sink_tau=self.fp.sink_tau, max_sinks=self.fp.max_sinks,
                                        sink_pos=self.sink_pos, n_sinks=self.n_sinks)
            score = self.h.fdl_score_blocks_max if scorer == "max" else self.h.fdl_score_blocks_mass
            score(self.g, q, self.pred_mask, ks, self.g.kv_block, self.scores)
            return
        self.h.fdl_score_blocks(self.g, q, self.pred_mask, ks, self.g.kv_block, self.scores,
                                k_cache=k_cache, k_dec=k_dec, detect_sinks=detect_sinks,
                                sink_tau=self.fp.sink_tau, max_sinks=self.fp.max_sinks,
                                sink_pos=self.sink_pos if detect_sinks else None,
                                n_sinks=self.n_sinks if detect_sinks else None)

    def select(self):
        self.h.fdl_select_blocks(self.g, self.scores, self.n_blk, self.g.kv_block, self.sink_pos,
                                 self.n_sinks, self.fp.max_sinks, self.fp.top_k_blocks, self.max_sel,
                                 self.sel_idx, self.n_sel)

    def attend(self, q, k, v, k_dec, v_dec, out):
        self.h.fdl_sparse_attn(self.g, q, k, v, k_dec, v_dec, None, self.sel_idx, self.n_sel,
                               self.max_sel, self.g.kv_block, out)

    def dense(self, q, k, v, k_dec, v_dec, out):
        self.h.fdl_dense_attn(self.g, q, k, v, k_dec, v_dec, None, out)

    def select_token_sinks(self):
        """Token-granular sink retention: the top-K of all blocks (no block forced), then the list of
        their tokens merged with the sink tokens outside them (tok_idx / n_tok)."""
        g, fp = self.g, self.fp
        k = min(self.n_blk, fp.top_k_blocks)
        if not hasattr(self, "tok_idx"):
            self.max_tok = max(1, k) * g.kv_block + fp.max_sinks
            self.tok_idx = torch.zeros(g.batch, g.n_kv_heads, self.max_tok, dtype=torch.int32, device=self.scores.device)
            self.n_tok = torch.zeros(g.batch, g.n_kv_heads, dtype=torch.int32, device=self.scores.device)
        self.h.fdl_select_blocks(g, self.scores, self.n_blk, g.kv_block, None, None, 1, k, max(1, k), self.sel_idx,
                                 self.n_sel)
        self.h.fdl_expand_tokens(g, self.sel_idx, self.n_sel, max(1, k), g.kv_block, self.sink_pos, self.n_sinks,
                                 fp.max_sinks, self.tok_idx, self.n_tok, self.max_tok)

    def layer(self, mode: str, q, k, v, k_dec, v_dec, ks, out, scorer: str = "sum", sink_tokens: bool = False):
        """mode: "dense", "source" (detect sinks here) or "reuse" (keep the last source's sinks).
        sink_tokens: keep the sinks as tokens, the top-K from all blocks (select_token_sinks)."""
        if mode == "dense":
            self.dense(q, k, v, k_dec, v_dec, out)
            return
        self.score(q, ks, k_cache=k, k_dec=k_dec, detect_sinks=(mode == "source"), scorer=scorer)
        if sink_tokens:
            self.select_token_sinks()
            self.h.fdl_sparse_attn(self.g, q, k, v, k_dec, v_dec, None, self.tok_idx, self.n_tok, self.max_tok, 1,
                                   out)
            return
        self.select()
        self.attend(q, k, v, k_dec, v_dec, out)


@dataclass
class ChunkParams:
    top_k_pos: int = 4
    window: int = 4
    chunk_tokens: int = 2048
    top_k_chunks: int = 4
    keep_tokens: int = 512


class ChunkedStep:
    """Buffers and calls for the chunked, paged Prefilling-dLLM variant."""

    def __init__(self, h: Handle, g: Geom, cp: ChunkParams, device="cuda"):
        assert g.paged
        self.h, self.g, self.cp = h, g, cp
        B, Hkv = g.batch, g.n_kv_heads
        self.n_chunks = g.ctx_len // cp.chunk_tokens
        self.per_chunk = 1 + cp.keep_tokens
        self.max_tok = cp.top_k_chunks * self.per_chunk
        i32 = dict(dtype=torch.int32, device=device)
        self.pred_mask = torch.zeros(B, dtype=torch.int64, device=device)
        self.n_pred = torch.zeros(B, **i32)
        self.chunk_scores = torch.zeros(B, Hkv, self.n_chunks, dtype=torch.float32, device=device)
        self.chunks = torch.zeros(B, Hkv, cp.top_k_chunks, **i32)
        self.n_chunks_sel = torch.zeros(B, Hkv, **i32)
        self.token_scores = torch.zeros(B, Hkv, cp.top_k_chunks, cp.chunk_tokens, dtype=torch.float32,
                                        device=device)
        self.tokens = torch.zeros(B, Hkv, self.max_tok, **i32)
        self.n_tokens = torch.zeros(B, Hkv, **i32)

    def new_chunk_sums(self, device="cuda"):
        g = self.g
        return torch.empty(g.batch, g.n_kv_heads, self.n_chunks, g.head_dim, dtype=torch.float32,
                           device=device)

    def pool(self, k_pool, page_table, cs):
        self.h.fdl_pool_keys(self.g, k_pool, page_table, self.cp.chunk_tokens, cs)

    def predict(self, prev_conf, masked):
        self.h.fdl_predict_queries(self.g.batch, self.g.dec_len, prev_conf, masked, self.cp.top_k_pos,
                                   self.cp.window, self.pred_mask, self.n_pred)

    def select(self, q, k_pool, page_table, cs, separate: bool = False, per_sequence: bool = False,
               one_launch: bool = True):
        """Level 1 (chunk scores, top chunks per KV head, or with per_sequence=True one chunk set per
        sequence from the scores summed over its KV heads), then level 2 (token scores inside them,
        anchor + top tokens).  Per KV head, both levels run as one launch (fdl_select_chunks_tokens)
        where its shape allows and one_launch is set; otherwise level 1 as two calls and level 2 as
        one call, or with separate=True as the score and select calls."""
        g, cp = self.g, self.cp
        if one_launch and not separate and not per_sequence and self.one_launch_ok():
            self.h.fdl_select_chunks_tokens(g, q, self.pred_mask, cs, k_pool, page_table, cp.chunk_tokens,
                                            cp.top_k_chunks, cp.keep_tokens, self.max_tok, self.chunk_scores,
                                            self.chunks, self.n_chunks_sel, self.token_scores, self.tokens,
                                            self.n_tokens)
            return
        self.h.fdl_score_blocks(g, q, self.pred_mask, cs, cp.chunk_tokens, self.chunk_scores)
        select = self.h.fdl_select_blocks_shared if per_sequence else self.h.fdl_select_blocks
        select(g, self.chunk_scores, self.n_chunks, cp.chunk_tokens, None, None, 1, cp.top_k_chunks, cp.top_k_chunks,
               self.chunks, self.n_chunks_sel)
        if not separate:
            self.h.fdl_score_select_tokens(g, q, self.pred_mask, k_pool, page_table, cp.chunk_tokens, self.chunks,
                                           cp.top_k_chunks, cp.keep_tokens, self.max_tok, self.token_scores,
                                           self.tokens, self.n_tokens)
            return
        self.h.fdl_score_blocks(g, q, self.pred_mask, None, cp.chunk_tokens, self.token_scores,
                                cand_idx=self.chunks, n_cand=cp.top_k_chunks, k_cache=k_pool,
                                page_table=page_table)
        self.h.fdl_select_blocks(g, self.token_scores, self.n_chunks, cp.chunk_tokens, None, None, 1,
                                 cp.keep_tokens, self.max_tok, self.tokens, self.n_tokens,
                                 cand_idx=self.chunks, n_cand=cp.top_k_chunks, force_first=True)

    def one_launch_ok(self) -> bool:
        """The shapes fdl_select_chunks_tokens takes (see its declaration)."""
        g, cp = self.g, self.cp
        page_ok = not g.paged or g.page_tokens >= 16
        return (g.dtype == FDL_BF16 and g.dec_len <= 32 and g.head_dim in (64, 128) and 256 <= cp.chunk_tokens <= 4096
                and page_ok and g.n_q_heads // g.n_kv_heads <= 8 and 1 <= self.n_chunks <= 64
                and 1 <= cp.top_k_chunks <= self.n_chunks)

    def attend(self, q, k_pool, v_pool, page_table, k_dec, v_dec, out):
        self.h.fdl_sparse_attn(self.g, q, k_pool, v_pool, k_dec, v_dec, page_table, self.tokens,
                               self.n_tokens, self.max_tok, 1, out)

    def run(self, q, k_pool, v_pool, page_table, k_dec, v_dec, cs, out, separate: bool = False,
            per_sequence: bool = False, one_launch: bool = True):
        self.select(q, k_pool, page_table, cs, separate, per_sequence, one_launch)
        self.attend(q, k_pool, v_pool, page_table, k_dec, v_dec, out)


def geom_for(cfg, dtype=None, ctx_lens=None) -> Geom:
    """Geom from any object with the workload attributes (batch, n_q_heads, ...); ctx_lens: a device
    int32 tensor [batch] of per-sequence cached lengths (a ragged batch; ctx_len is then the stride
    and the largest length), or None."""
    dt = dtype if dtype is not None else (FDL_BF16 if cfg.dtype == "bf16" else 0)
    paged = bool(getattr(cfg, "paged", False))
    return Geom(batch=cfg.batch, n_q_heads=cfg.n_q_heads, n_kv_heads=cfg.n_kv_heads,
                head_dim=cfg.head_dim, ctx_len=cfg.ctx_len, kv_block=cfg.kv_block,
                dec_len=cfg.dec_len, dtype=dt, paged=int(paged),
                page_tokens=cfg.page_tokens if paged else 0,
                pages_per_seq=(cfg.ctx_len // cfg.page_tokens) if paged else 0,
                n_pages=(cfg.batch * (cfg.ctx_len // cfg.page_tokens)) if paged else 0,
                ctx_lens=ctx_lens)
