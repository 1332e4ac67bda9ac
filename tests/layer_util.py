"""Whole-layer helpers for the GPU tests: run one layer-step through the step drivers and compare
every intermediate the oracle also produces (predicted positions, scores, sinks, selection,
output)."""
from __future__ import annotations

import numpy as np
import torch

from gpu_util import assert_close, dev, host, out_buffer, out_to_f64


def _focus(h, cfg, x, modes=("source", "reuse"), sink_tokens=False):
    from diffusion_long_context_amd.step import FocusParams, FocusStep, geom_for
    g = geom_for(cfg)
    fs = FocusStep(h, g, FocusParams(cfg.top_k_pos, cfg.window, cfg.top_k_blocks, cfg.sink_tau,
                                     cfg.max_sinks))
    t = {k: dev(x[k]) for k in ("q", "k", "v", "k_dec", "v_dec", "masked")}
    pc = dev(x["prev_conf"]) if x.get("prev_conf") is not None else None
    fs.predict(pc, t["masked"])
    ks = fs.new_ks()
    fs.pool(t["k"], ks)
    res = {}
    for mode in modes:
        out = out_buffer(cfg)
        fs.layer(mode, t["q"], t["k"], t["v"], t["k_dec"], t["v_dec"], ks, out, sink_tokens=sink_tokens)
        torch.cuda.synchronize()
        res[mode] = {
            "out": out_to_f64(cfg, out),
            "pred_mask": host(fs.pred_mask).view(np.uint64).copy(),
            "scores": host(fs.scores).copy(),
            "sink_pos": host(fs.sink_pos).copy(),
            "n_sinks": host(fs.n_sinks).copy(),
            "sel": host(fs.sel_idx).copy(),
            "n_sel": host(fs.n_sel).copy(),
        }
        if sink_tokens:
            res[mode]["tokens"] = host(fs.tok_idx).copy()
            res[mode]["n_tok"] = host(fs.n_tok).copy()
    assert h.fdl_get_status() == 0
    return res


def _check_layer(cfg, got, want, margin=None):
    assert np.array_equal(got["pred_mask"], np.asarray(want["pred_mask"], np.uint64))
    if "scores" in want:
        assert np.array_equal(got["scores"].view(np.uint32), want["scores"].view(np.uint32))
    if "sel" in want:
        if margin is None or margin > 1e-4 * cfg.sink_tau:
            ns = int(want["n_sinks"][0])
            for b in range(cfg.batch):
                nsb = int(want["n_sinks"][b])
                assert got["n_sinks"][b] == nsb
                assert got["sink_pos"][b, :nsb].tolist() == want["sink_pos"][b, :nsb].tolist()
            for b in range(cfg.batch):
                for g in range(cfg.n_kv_heads):
                    w = want["sel"][b][g].tolist()
                    assert got["n_sel"][b, g] == len(w)
                    assert got["sel"][b, g, : len(w)].tolist() == w
    assert_close(got["out"], want["out"], cfg.name)


def _chunked(h, cfg, x, per_sequence=False):
    from diffusion_long_context_amd.step import ChunkedStep, ChunkParams, geom_for
    g = geom_for(cfg)
    cs_ = ChunkedStep(h, g, ChunkParams(cfg.top_k_pos, cfg.window, cfg.chunk_tokens, cfg.top_k_chunks,
                                        cfg.tokens_per_chunk_kept))
    t = {k: dev(x[k]) for k in ("q", "k_pool", "v_pool", "page_table", "k_dec", "v_dec", "masked",
                                "prev_conf")}
    cs_.predict(t["prev_conf"], t["masked"])
    cs = cs_.new_chunk_sums()
    cs_.pool(t["k_pool"], t["page_table"], cs)
    out = out_buffer(cfg)
    cs_.run(t["q"], t["k_pool"], t["v_pool"], t["page_table"], t["k_dec"], t["v_dec"], cs, out,
            per_sequence=per_sequence)
    torch.cuda.synchronize()
    assert h.fdl_get_status() == 0
    return {"chunk_scores": host(cs_.chunk_scores), "chunks": host(cs_.chunks),
            "token_scores": host(cs_.token_scores), "tokens": host(cs_.tokens),
            "n_tokens": host(cs_.n_tokens), "out": out_to_f64(cfg, out)}


def _check_chunked(cfg, got, want):
    assert np.array_equal(got["chunk_scores"].view(np.uint32), want["chunk_scores"].view(np.uint32))
    assert np.array_equal(got["chunks"], want["chunks"])
    assert np.array_equal(got["token_scores"].view(np.uint32), want["token_scores"].view(np.uint32))
    assert np.array_equal(got["tokens"], want["tokens"])
    assert np.all(got["n_tokens"] == want["tokens"].shape[-1])
    assert_close(got["out"], want["out"], "chunked")
