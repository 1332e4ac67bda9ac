"""Whole-layer helpers for the GPU tests: run one layer-step through the step drivers and compare
every intermediate the oracle also produces (predicted positions, scores, sinks, selection,
output)."""
from __future__ import annotations

import numpy as np
import torch

from gpu_util import assert_close, dev, host, out_buffer, out_to_f64


def _focus(h, cfg, x, modes=("source", "reuse"), sink_tokens=False, ctx_lens=None):
    from diffusion_long_context_amd.step import FocusParams, FocusStep, geom_for
    g = geom_for(cfg, ctx_lens=dev(np.asarray(ctx_lens, np.int32)) if ctx_lens is not None else None)
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
        if margin is not None:
            # a sink mass within 1e-4 tau of the threshold may land on either side in float32: such
            # inputs are a flagged case, not a pass; none of the seeded workloads is one
            assert margin > 1e-4 * cfg.sink_tau, f"flagged case: sink margin {margin:.3g} within 1e-4 tau"
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


def focus_step_layers(h, cfg, xs, modes, prev_conf, masked, ctx_lens=None):
    """fdl_focus_step over one layer table (xs[l] holds layer l's q, k, v, k_dec, v_dec; modes[l] is
    "dense", "source" or "reuse"), with every sparse layer's scores and selection captured: the step
    is run once with the table cut after each sparse layer (the buffers then hold that layer's
    values), then once in full for the outputs, predicted positions and sinks.  ctx_lens: per-sequence
    cached lengths of a ragged batch, or None.  Returns
    {"layers": {l: (scores, sel, n_sel)}, "outs": [...], "pred_mask", "sink_pos", "n_sinks", "bits"}."""
    from diffusion_long_context_amd.fdllm import (FDL_LAYER_DENSE, FDL_LAYER_REUSE, FDL_LAYER_SOURCE,
                                                  fdl_focus_params)
    from diffusion_long_context_amd.step import geom_for
    g = geom_for(cfg, ctx_lens=dev(np.asarray(ctx_lens, np.int32)) if ctx_lens is not None else None)
    B, Hq, Hkv, D, T, nb, ms = (cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.dec_len,
                                cfg.n_blk, cfg.max_sel_blocks)
    code = {"dense": FDL_LAYER_DENSE, "source": FDL_LAYER_SOURCE, "reuse": FDL_LAYER_REUSE}
    t = [{k: dev(x[k]) for k in ("q", "k", "v", "k_dec", "v_dec")} for x in xs]
    ks = [torch.zeros((B, Hkv, nb, D), dtype=torch.float32, device="cuda") for _ in modes]
    outs = [torch.zeros((B, Hq, T, D), dtype=torch.bfloat16, device="cuda") for _ in modes]
    for l in range(len(modes)):
        h.fdl_pool_keys(g, t[l]["k"], None, cfg.kv_block, ks[l])
    pm = torch.zeros(B, dtype=torch.int64, device="cuda")
    npd = torch.zeros(B, dtype=torch.int32, device="cuda")
    sc = torch.zeros((B, Hkv, nb), dtype=torch.float32, device="cuda")
    sp = torch.full((B, cfg.max_sinks), -1, dtype=torch.int32, device="cuda")
    nsk = torch.zeros(B, dtype=torch.int32, device="cuda")
    sel = torch.zeros((B, Hkv, ms), dtype=torch.int32, device="cuda")
    nsel = torch.zeros((B, Hkv), dtype=torch.int32, device="cuda")
    params = fdl_focus_params(cfg.top_k_pos, cfg.window, cfg.top_k_blocks, cfg.max_sinks, ms, cfg.sink_tau)
    table = h.make_layers(g, [dict(q=t[l]["q"], k_cache=t[l]["k"], v_cache=t[l]["v"], k_dec=t[l]["k_dec"],
                                   v_dec=t[l]["v_dec"], ks=ks[l], out=outs[l], mode=code[m])
                              for l, m in enumerate(modes)])
    pc = dev(prev_conf) if prev_conf is not None else None
    mk = dev(masked)
    res = {"layers": {}}

    def step(n):
        sub = (table._type_ * n)(*table[:n]) if n < len(modes) else table
        h.fdl_focus_step(g, params, pc, mk, sub, pm, npd, sc, sp, nsk, sel, nsel)
        torch.cuda.synchronize()

    for l, m in enumerate(modes):
        if m != "dense":
            step(l + 1)
            res["layers"][l] = (host(sc).copy(), host(sel).copy(), host(nsel).copy())
    step(len(modes))
    st, bits = h.fdl_get_status_bits()
    assert st == 0, st
    res.update(outs=outs, pred_mask=host(pm).view(np.uint64).copy(), n_pred=host(npd).copy(),
               sink_pos=host(sp).copy(), n_sinks=host(nsk).copy(), bits=bits)
    return res


def check_focus_step_layers(cfg, got, xs, modes, prev_conf, masked, what=""):
    """Every layer of a focus_step_layers run against the oracle run one layer at a time: predicted
    positions and sinks bit for bit, every sparse layer's scores and selection bit for bit, outputs
    within tolerance.  Returns the oracle's per-layer results."""
    from gpu_util import bf16_out_to_f64
    from oracle.pipeline import focus_layer_step
    sinks = None
    wants = []
    for l, m in enumerate(modes):
        x = dict(xs[l], prev_conf=prev_conf, masked=masked)
        want = focus_layer_step(cfg, x, m, sinks=sinks)
        wants.append(want)
        assert np.array_equal(got["pred_mask"], np.asarray(want["pred_mask"], np.uint64)), (what, l)
        if "n_pred" in got:
            assert [bin(int(v)).count("1") for v in got["pred_mask"]] == got["n_pred"].tolist(), (what, l)
        if m == "source":
            assert want["sink_margin"] > 1e-4 * cfg.sink_tau, f"flagged case: sink margin {want['sink_margin']:.3g}"
            sinks = (want["sink_pos"], want["n_sinks"])
            for b in range(cfg.batch):
                nsb = int(want["n_sinks"][b])
                assert int(got["n_sinks"][b]) == nsb, (what, b)
                assert got["sink_pos"][b, :nsb].tolist() == want["sink_pos"][b, :nsb].tolist(), (what, b)
        if m != "dense":
            sc, sel, nsel = got["layers"][l]
            assert np.array_equal(sc.view(np.uint32), want["scores"].view(np.uint32)), (what, l)
            for b in range(cfg.batch):
                for gh in range(cfg.n_kv_heads):
                    w = want["sel"][b][gh].tolist()
                    assert int(nsel[b, gh]) == len(w), (what, l, b, gh)
                    assert sel[b, gh, :len(w)].tolist() == w, (what, l, b, gh)
        assert_close(bf16_out_to_f64(got["outs"][l]), want["out"], f"{what} layer {l} ({m})")
    return wants
