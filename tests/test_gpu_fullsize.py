"""Parity at full size.

* The 32K-context, 32-layer step exactly as the benchmark launches it (same workspace, same
  parameters, one fdl_focus_step over all 32 layers, keys pooled by fdl_pool_keys), at three
  generation steps: the first step of the first block (no previous confidence, every position
  predicted), a mid-block step and the last step.  Sampled outputs -- a dense layer, the sink-source
  layer, the first reuse layer and the last one -- are checked element by element against the
  oracle run one layer at a time; the predicted positions and the sinks are checked bit for bit, and
  so are the block scores and the selection of the sink-source layer, the first reuse layer and the
  last layer (the step is run again cut after layers 2 and 3 to read theirs).
* The same step's scores and selection at every one of its 30 sparse layers (generation step 37).
* The chunked, paged 32K workload with batch 4, in full.
"""
import numpy as np
import pytest
import torch

import bench
from gpu_util import assert_close, bf16_out_to_f64, host, require_gpu
from layer_util import _check_chunked, _chunked
from oracle.pipeline import chunked_layer_step, focus_layer_step
from oracle.scoring import pool_keys
from synth import get_config
from synth.gen import make_single, schedule_state

pytestmark = pytest.mark.gpu

STEPS = (0, 37, 255)          # global generation steps (block = step // 32, s = step % 32)
CHECK_LAYERS = (0, 2, 3, 31)  # dense, sink source, first reuse, last reuse


def _bits(t: torch.Tensor) -> np.ndarray:
    return host(t.view(torch.int16)).view(np.uint16)


def test_focus_step_32k_32layer_as_benchmarked():
    require_gpu()
    from diffusion_long_context_amd import Handle
    from diffusion_long_context_amd.fdllm import (FDL_LAYER_DENSE, FDL_LAYER_REUSE, FDL_LAYER_SOURCE,
                                                  fdl_focus_params)
    from diffusion_long_context_amd.step import geom_for
    from synth.device import layer_kv, step_qkv_pool

    cfg = get_config(3)
    g = geom_for(cfg)
    NL, B, Hq, Hkv, D, T = cfg.n_layers, cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.dec_len
    n_blk, max_sel = cfg.n_blk, cfg.max_sel_blocks
    devc = torch.device("cuda")
    h = Handle(workspace_bytes=bench.WORKSPACE_BYTES)
    try:
        K, V = zip(*[layer_kv(cfg, layer, devc) for layer in range(NL)])
        Q, KD, VD = step_qkv_pool(cfg, len(STEPS), devc)
        ks = [torch.zeros((B, Hkv, n_blk, D), dtype=torch.float32, device=devc) for _ in range(NL)]
        outs = [torch.zeros((B, Hq, T, D), dtype=torch.bfloat16, device=devc) for _ in range(NL)]
        pred_mask = torch.zeros(B, dtype=torch.int64, device=devc)
        n_pred = torch.zeros(B, dtype=torch.int32, device=devc)
        scores = torch.zeros((B, Hkv, n_blk), dtype=torch.float32, device=devc)
        sink_pos = torch.full((B, cfg.max_sinks), -1, dtype=torch.int32, device=devc)
        n_sinks = torch.zeros(B, dtype=torch.int32, device=devc)
        sel_idx = torch.zeros((B, Hkv, max_sel), dtype=torch.int32, device=devc)
        n_sel = torch.zeros((B, Hkv), dtype=torch.int32, device=devc)
        params = fdl_focus_params(cfg.top_k_pos, cfg.window, cfg.top_k_blocks, cfg.max_sinks, max_sel,
                                  cfg.sink_tau)
        modes = [FDL_LAYER_DENSE if l < cfg.dense_layers else
                 (FDL_LAYER_SOURCE if l == cfg.source_layer else FDL_LAYER_REUSE) for l in range(NL)]
        for layer in range(NL):
            h.fdl_pool_keys(g, K[layer], None, cfg.kv_block, ks[layer])

        kv_host = {l: (_bits(K[l]), _bits(V[l])) for l in CHECK_LAYERS}
        ks_oracle = {}
        for i, gstep in enumerate(STEPS):
            st = schedule_state(cfg, gstep)
            conf = None if st["prev_conf"] is None else torch.from_numpy(st["prev_conf"]).to(devc)
            masked = torch.from_numpy(st["masked"]).to(devc)
            table = h.make_layers(g, [dict(q=Q[i, l], k_cache=K[l], v_cache=V[l], k_dec=KD[i, l],
                                           v_dec=VD[i, l], ks=ks[l], out=outs[l], mode=m)
                                      for l, m in enumerate(modes)])
            print(f"focus step {gstep} (32 layers)", flush=True)
            h.fdl_focus_step(g, params, conf, masked, table, pred_mask, n_pred, scores, sink_pos, n_sinks,
                             sel_idx, n_sel)
            torch.cuda.synchronize()
            assert h.fdl_get_status() == 0
            got_pred = host(pred_mask).view(np.uint64)
            got_sinks = (host(sink_pos).copy(), host(n_sinks).copy())
            got_sel = (host(sel_idx).copy(), host(n_sel).copy())
            got_out = {l: bf16_out_to_f64(outs[l]) for l in CHECK_LAYERS}
            # scores and selection of every checked sparse layer: the full step leaves the last
            # layer's; the step cut after layer 2 (the sink source) and after layer 3 (the first reuse
            # layer) leaves theirs
            cut = {NL - 1: (host(scores).copy(), got_sel[0], got_sel[1])}
            for lc in (cfg.source_layer, cfg.source_layer + 1):
                sub = (table._type_ * (lc + 1))(*table[:lc + 1])
                h.fdl_focus_step(g, params, conf, masked, sub, pred_mask, n_pred, scores, sink_pos, n_sinks,
                                 sel_idx, n_sel)
                torch.cuda.synchronize()
                assert h.fdl_get_status() == 0
                cut[lc] = (host(scores).copy(), host(sel_idx).copy(), host(n_sel).copy())

            sinks = None
            for l in CHECK_LAYERS:
                k_h, v_h = kv_host[l]
                x = {"q": _bits(Q[i, l]), "k": k_h, "v": v_h, "k_dec": _bits(KD[i, l]),
                     "v_dec": _bits(VD[i, l]), "prev_conf": st["prev_conf"], "masked": st["masked"]}
                mode = ("dense" if l < cfg.dense_layers else "source" if l == cfg.source_layer else "reuse")
                if mode != "dense" and l not in ks_oracle:
                    ks_oracle[l] = pool_keys(k_h, cfg.kv_block)
                want = focus_layer_step(cfg, x, mode, sinks=sinks, ks=ks_oracle.get(l))
                assert np.array_equal(got_pred, np.asarray(want["pred_mask"], np.uint64)), (gstep, l)
                if mode == "source":
                    # the planted sinks sit far above the threshold, so the set is unique
                    assert want["sink_margin"] > 1e-4 * cfg.sink_tau
                    nsb = int(want["n_sinks"][0])
                    assert nsb > 0
                    assert int(got_sinks[1][0]) == nsb
                    assert got_sinks[0][0, :nsb].tolist() == want["sink_pos"][0, :nsb].tolist()
                    sinks = (want["sink_pos"], want["n_sinks"])
                if l in cut:
                    c_scores, c_sel, c_nsel = cut[l]
                    assert np.array_equal(c_scores.view(np.uint32), want["scores"].view(np.uint32)), (gstep, l)
                    for gh in range(Hkv):
                        w = want["sel"][0][gh].tolist()
                        assert int(c_nsel[0, gh]) == len(w), (gstep, l, gh)
                        assert c_sel[0, gh, : len(w)].tolist() == w, (gstep, l, gh)
                assert_close(got_out[l], want["out"], f"step {gstep} layer {l} ({mode})")
    finally:
        h.close()


def test_chunked_paged_32k_batch4_full():
    require_gpu()
    from diffusion_long_context_amd import Handle
    cfg = get_config(4)
    x = make_single(cfg)
    h = Handle(workspace_bytes=512 << 20)
    try:
        print("chunked paged 32K, batch 4", flush=True)
        got = _chunked(h, cfg, x)
        want = chunked_layer_step(cfg, x)
        _check_chunked(cfg, got, want)
    finally:
        h.close()


INDEX_STEPS = (0, 1, 31, 32, 37, 255)   # first and second step, both sides of a block boundary, the last


def test_focus_step_32k_every_sparse_layer_selection():
    """Index parity at every sparse layer of the benchmarked 32K step, at six generation steps (the
    first two, the last of block 0 and the first of block 1, one mid block, the last): each step is
    run cut after each of layers 2 .. 31 and that layer's block scores and selection are compared bit
    for bit with the oracle's, as are the predicted positions and the sinks (scores and selection
    only: the outputs of the sampled layers are checked in the test above)."""
    require_gpu()
    from diffusion_long_context_amd import Handle
    from diffusion_long_context_amd.fdllm import (FDL_LAYER_DENSE, FDL_LAYER_REUSE, FDL_LAYER_SOURCE,
                                                  fdl_focus_params)
    from diffusion_long_context_amd.step import geom_for
    from synth.device import layer_kv, step_qkv_pool

    cfg = get_config(3)
    g = geom_for(cfg)
    NL, B, Hq, Hkv, D, T = cfg.n_layers, cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.dec_len
    n_blk, max_sel = cfg.n_blk, cfg.max_sel_blocks
    devc = torch.device("cuda")
    h = Handle(workspace_bytes=bench.WORKSPACE_BYTES)
    try:
        K, V = zip(*[layer_kv(cfg, layer, devc) for layer in range(NL)])
        Q, KD, VD = step_qkv_pool(cfg, len(INDEX_STEPS), devc)
        ks = [torch.zeros((B, Hkv, n_blk, D), dtype=torch.float32, device=devc) for _ in range(NL)]
        outs = [torch.zeros((B, Hq, T, D), dtype=torch.bfloat16, device=devc) for _ in range(NL)]
        pred_mask = torch.zeros(B, dtype=torch.int64, device=devc)
        n_pred = torch.zeros(B, dtype=torch.int32, device=devc)
        scores = torch.zeros((B, Hkv, n_blk), dtype=torch.float32, device=devc)
        sink_pos = torch.full((B, cfg.max_sinks), -1, dtype=torch.int32, device=devc)
        n_sinks = torch.zeros(B, dtype=torch.int32, device=devc)
        sel_idx = torch.zeros((B, Hkv, max_sel), dtype=torch.int32, device=devc)
        n_sel = torch.zeros((B, Hkv), dtype=torch.int32, device=devc)
        params = fdl_focus_params(cfg.top_k_pos, cfg.window, cfg.top_k_blocks, cfg.max_sinks, max_sel,
                                  cfg.sink_tau)
        modes = [FDL_LAYER_DENSE if l < cfg.dense_layers else
                 (FDL_LAYER_SOURCE if l == cfg.source_layer else FDL_LAYER_REUSE) for l in range(NL)]
        for layer in range(NL):
            h.fdl_pool_keys(g, K[layer], None, cfg.kv_block, ks[layer])
        # the cache side is the same at every step: the oracle's keys and pooled keys once per layer
        k_host = {l: _bits(K[l]) for l in range(cfg.dense_layers, NL)}
        ks_host = {l: pool_keys(k_host[l], cfg.kv_block) for l in k_host}
        for i, gstep in enumerate(INDEX_STEPS):
            st = schedule_state(cfg, gstep)
            conf = None if st["prev_conf"] is None else torch.from_numpy(st["prev_conf"]).to(devc)
            masked = torch.from_numpy(st["masked"]).to(devc)
            table = h.make_layers(g, [dict(q=Q[i, l], k_cache=K[l], v_cache=V[l], k_dec=KD[i, l], v_dec=VD[i, l],
                                           ks=ks[l], out=outs[l], mode=m) for l, m in enumerate(modes)])
            got = {}
            for lc in range(cfg.dense_layers, NL):
                sub = (table._type_ * (lc + 1))(*table[:lc + 1]) if lc + 1 < NL else table
                sink_pos.fill_(-7)   # sentinels: the step must write the list and its length
                n_sinks.fill_(-7)
                h.fdl_focus_step(g, params, conf, masked, sub, pred_mask, n_pred, scores, sink_pos, n_sinks,
                                 sel_idx, n_sel)
                torch.cuda.synchronize()
                assert h.fdl_get_status() == 0
                got[lc] = (host(scores).copy(), host(sel_idx).copy(), host(n_sel).copy(), host(sink_pos).copy(),
                           host(n_sinks).copy())
            got_pred = host(pred_mask).view(np.uint64)
            sinks = None
            print(f"step {gstep}: layers {cfg.dense_layers}..{NL - 1} against the oracle", flush=True)
            for l in range(cfg.dense_layers, NL):
                x = {"q": _bits(Q[i, l]), "k": k_host[l], "v": None, "k_dec": _bits(KD[i, l]), "v_dec": None,
                     "prev_conf": st["prev_conf"], "masked": st["masked"]}
                mode = "source" if l == cfg.source_layer else "reuse"
                want = focus_layer_step(cfg, x, mode, sinks=sinks, ks=ks_host[l], with_output=False)
                assert np.array_equal(got_pred, np.asarray(want["pred_mask"], np.uint64)), (gstep, l)
                if mode == "source":
                    assert want["sink_margin"] > 1e-4 * cfg.sink_tau, (gstep, "flagged case: sink margin")
                    sinks = (want["sink_pos"], want["n_sinks"])
                c_scores, c_sel, c_nsel, c_sp, c_ns = got[l]
                nsk = int(np.asarray(sinks[1])[0])
                want_sp = np.asarray(sinks[0])[0, :nsk].tolist()
                assert int(c_ns[0]) == nsk and c_sp[0, :nsk].tolist() == want_sp, (gstep, l)
                assert np.array_equal(c_scores.view(np.uint32), want["scores"].view(np.uint32)), (gstep, l)
                for gh in range(Hkv):
                    w = want["sel"][0][gh].tolist()
                    assert int(c_nsel[0, gh]) == len(w), (gstep, l, gh)
                    assert c_sel[0, gh, : len(w)].tolist() == w, (gstep, l, gh)
    finally:
        h.close()
