#!/usr/bin/env python3
"""Benchmark of one denoising step of confidence-guided, sink-aware block-sparse attention on the
32K-context, 32-layer workload (LLaDA-8B-shaped attention: 32 heads, head_dim 128, bf16; 32-token
decode blocks; generation of 256 tokens as 8 blocks of 32 steps; layers 0-1 dense, layer 2 finds the
sinks, layers 3-31 reuse them; 64 blocks of 64 tokens kept per head).

A step = one fdl_focus_step call (predict once, then the 32 layers) plus, at the first step of every
generation block, the key pooling of all 32 layers (the cache-side refresh).  Inputs are resident in
HBM before timing: 32 distinct layers of KV cache (16 GiB, far larger than the 256 MB last-level
cache, so every layer reads cold data) and distinct per-(step, layer) queries and block keys/values.

Prints one JSON line (rank 0, N = 1).  The CPU baseline times the oracle on a bounded sample in a
single-threaded child process.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "sparse-attn step us + KV tokens/s at 32K ctx; achieved HBM GB/s vs peak"
PEAK_HBM_GBS = 8000.0
WORKSPACE_BYTES = 256 << 20   # library workspace of the timed handle (sets the attention split count)


# HBM bytes per sparse-attention dispatch, from two rocprofv3 counter runs of this benchmark
# (FETCH_SIZE, WRITE_SIZE; scaled by a 1 GiB copy in the same runs).  Valid only for the kernel
# sources they were taken on: the file records their hash.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "llada8b_32k_32layer_sparse_attn_traffic.json")
KERNEL_SOURCES = ("diffusion_long_context_amd/csrc/attn_mha.hip", "diffusion_long_context_amd/csrc/fdl_device.h")


def measured_traffic():
    try:
        with open(TRAFFIC_FILE) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return d["hbm_bytes_per_dispatch"] if h.hexdigest() == d.get("source_sha256") else None


def log(msg: str):
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


# ------------------------------------------------------------------------------------------------
# CPU baseline: the oracle as it stands, single-threaded, on one layer of the same workload
# ------------------------------------------------------------------------------------------------

def cpu_baseline_child() -> dict:
    import numpy as np

    from oracle.pipeline import focus_layer_step
    from oracle.scoring import pool_keys
    from synth import get_config
    from synth.gen import context_kv, schedule_state, step_qkv

    cfg = get_config(3)
    layer, gstep = 3, 33
    st = schedule_state(cfg, gstep)
    x = dict(step_qkv(cfg, layer, st["block"], st["s"]))
    x.update(context_kv(cfg, layer))
    x["prev_conf"], x["masked"] = st["prev_conf"], st["masked"]
    t = {}
    t0 = time.perf_counter()
    ks = pool_keys(x["k"], cfg.kv_block)
    t["pool"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    r_src = focus_layer_step(cfg, x, "source", ks=ks)
    t["source"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    focus_layer_step(cfg, x, "reuse", sinks=(r_src["sink_pos"], r_src["n_sinks"]), ks=ks)
    t["reuse"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    focus_layer_step(cfg, x, "dense")
    t["dense"] = time.perf_counter() - t0
    step = (cfg.dense_layers * t["dense"] + t["source"]
            + (cfg.n_layers - cfg.dense_layers - 1) * t["reuse"] + cfg.n_layers * t["pool"] / cfg.steps_per_block)
    return {"layer_seconds": t, "step_seconds_extrapolated": step,
            "kv_tokens_per_s": cfg.ctx_len * cfg.n_layers / step}


def cpu_baseline() -> dict | None:
    env = dict(os.environ, OMP_NUM_THREADS="1", OPENBLAS_NUM_THREADS="1", MKL_NUM_THREADS="1")
    env["PYTHONPATH"] = ROOT + os.pathsep + env.get("PYTHONPATH", "")
    try:
        r = subprocess.run([sys.executable, os.path.abspath(__file__), "--cpu-baseline-child"], env=env,
                           capture_output=True, text=True, timeout=600)
    except subprocess.TimeoutExpired:
        log("cpu baseline timed out")
        return None
    if r.returncode != 0:
        log("cpu baseline failed: " + r.stderr[-2000:])
        return None
    d = json.loads(r.stdout.strip().splitlines()[-1])
    lt = d["layer_seconds"]
    return {
        "value": d["kv_tokens_per_s"], "unit": "KV tokens/s", "cores": 1, "kind": "oracle",
        "sample": ("one 32K layer (32 heads) of the same workload, run once as dense, source and reuse "
                   "layer plus its key pooling; step = 2 dense + 1 source + 29 reuse + 32 poolings/32 "
                   f"(measured s: dense {lt['dense']:.2f}, source {lt['source']:.2f}, reuse "
                   f"{lt['reuse']:.2f}, pool {lt['pool']:.2f})"),
        "step_ms_extrapolated": 1e3 * d["step_seconds_extrapolated"],
    }


# ------------------------------------------------------------------------------------------------
# GPU run
# ------------------------------------------------------------------------------------------------

def sparse_launch_bytes(cfg, units: int) -> int:
    """Bytes one select-and-attend launch must move: K and V of the selected 64-token blocks, Q and O,
    the decode block's own K and V, the pooled keys (f32) and the scores and selection it writes."""
    B, Hq, Hkv, D, T, n_blk = cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.dec_len, cfg.n_blk
    unit_bytes = cfg.kv_block * D * 2 * 2
    fixed = (B * Hq * T * D * 2 * 2 + B * Hkv * T * D * 2 * 2 + units * 4 + B * Hkv * 4
             + B * Hkv * n_blk * D * 4 + B * Hkv * n_blk * 4)
    return units * unit_bytes + fixed


def time_decode_loop(h, g, cfg, params, Q, K, V, KD, VD, ks, outs, modes, pred_mask, n_pred, scores, sink_pos,
                     n_sinks, sel_idx, n_sel, reps: int = 3) -> dict:
    """One decode block (steps_per_block steps of all layers, each step followed by the unmask
    update) as one fdl_decode_steps call, eager and replayed from a HIP graph, on a side stream.
    Confidences are seeded U(0, 1); the masked flags start all set and evolve on the device."""
    import torch
    spb, B, T, NL = min(cfg.steps_per_block, Q.shape[0]), cfg.batch, cfg.dec_len, cfg.n_layers
    dev = Q.device
    table = h.make_layers(g, [dict(q=Q[i, l], k_cache=K[l], v_cache=V[l], k_dec=KD[i, l], v_dec=VD[i, l], ks=ks[l],
                                   out=outs[l], mode=m) for i in range(spb) for l, m in enumerate(modes())])
    confs = torch.rand((spb, B, T), generator=torch.Generator(device=dev).manual_seed(7), device=dev)
    masked = torch.ones((B, T), dtype=torch.uint8, device=dev)
    decoded = torch.zeros((spb, B, 1), dtype=torch.int32, device=dev)

    def block():
        h.fdl_decode_steps(g, params, spb, None, confs, masked, 1, decoded, table, pred_mask, n_pred, scores,
                           sink_pos, n_sinks, sel_idx, n_sel)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    res = {}
    with torch.cuda.stream(side):
        masked.fill_(1)
        block()
        side.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            masked.fill_(1)
            block()
        side.synchronize()
        res["eager_ms_per_step"] = 1e3 * (time.perf_counter() - t0) / (reps * spb)
        h.fdl_capture_begin()
        try:
            block()
        finally:
            graph = h.fdl_capture_end()
        try:
            masked.fill_(1)
            h.fdl_graph_launch(graph)
            side.synchronize()
            t0 = time.perf_counter()
            for _ in range(reps):
                masked.fill_(1)
                h.fdl_graph_launch(graph)
            side.synchronize()
            res["graph_ms_per_step"] = 1e3 * (time.perf_counter() - t0) / (reps * spb)
        finally:
            h.fdl_graph_destroy(graph)
    torch.cuda.synchronize()
    assert h.fdl_get_status() == 0
    dec = decoded.cpu().numpy()
    res.update(steps=spb, layers=NL, kv_tokens_per_s_graph=cfg.ctx_len * B * NL / (res["graph_ms_per_step"] * 1e-3),
               decoded_distinct=all(len(set(dec[:, b, 0].tolist())) == spb for b in range(B)),
               masked_left=int(masked.sum().item()))
    return res


def other_workloads(h, dev, steps: int = 10, chunk_runs: int = 20) -> dict:
    """Diagnostics on the other workloads of the benchmark description (not the headline): the 8K MHA
    and 16K grouped-query single-layer configurations (per-layer GPU time of each layer kind through
    fdl_focus_step, 32 layers of one kind per step) and the chunked paged batch-4 32K configuration
    (the whole select-and-attend chain), each with the dense baseline on the same inputs and the
    achieved rate on the bytes the sparse path must move.  Inputs are drawn on the device (seeded)."""
    import torch

    from diffusion_long_context_amd.fdllm import (FDL_LAYER_DENSE, FDL_LAYER_REUSE, FDL_LAYER_SOURCE,
                                                  fdl_focus_params)
    from diffusion_long_context_amd.step import ChunkedStep, ChunkParams, geom_for
    from synth import get_config

    def timed(fn, n):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        fn()   # warm
        torch.cuda.synchronize()
        a.record()
        for _ in range(n):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / n   # us per call

    out = {}
    for ci in (1, 2):
        cfg = get_config(ci)
        g = geom_for(cfg)
        B, Hq, Hkv, D, L, T = cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.ctx_len, cfg.dec_len
        gen = torch.Generator(device=dev).manual_seed(7000 + ci)

        def rn(*shape):
            return torch.randn(*shape, generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)

        q, k, v = rn(B, Hq, T, D), rn(B, Hkv, L, D), rn(B, Hkv, L, D)
        k[:, :, :4] *= 6   # sink keys
        kd, vd = rn(B, Hkv, T, D), rn(B, Hkv, T, D)
        n_blk, max_sel = cfg.n_blk, cfg.max_sel_blocks
        ks = torch.zeros((B, Hkv, n_blk, D), dtype=torch.float32, device=dev)
        h.fdl_pool_keys(g, k, None, cfg.kv_block, ks)
        o = torch.zeros((B, Hq, T, D), dtype=torch.bfloat16, device=dev)
        pred_mask = torch.zeros(B, dtype=torch.int64, device=dev)
        n_pred = torch.zeros(B, dtype=torch.int32, device=dev)
        scores = torch.zeros((B, Hkv, n_blk), dtype=torch.float32, device=dev)
        sink_pos = torch.full((B, cfg.max_sinks), -1, dtype=torch.int32, device=dev)
        n_sinks = torch.zeros(B, dtype=torch.int32, device=dev)
        sel_idx = torch.zeros((B, Hkv, max_sel), dtype=torch.int32, device=dev)
        n_sel = torch.zeros((B, Hkv), dtype=torch.int32, device=dev)
        conf = torch.rand((B, T), generator=gen, device=dev)
        masked = (torch.rand((B, T), generator=gen, device=dev) < 0.5).to(torch.uint8)
        params = fdl_focus_params(cfg.top_k_pos, cfg.window, cfg.top_k_blocks, cfg.max_sinks, max_sel,
                                  cfg.sink_tau)
        per = {}
        for name, mode in (("dense", FDL_LAYER_DENSE), ("source", FDL_LAYER_SOURCE), ("reuse", FDL_LAYER_REUSE)):
            table = h.make_layers(g, [dict(q=q, k_cache=k, v_cache=v, k_dec=kd, v_dec=vd, ks=ks, out=o,
                                           mode=mode)] * 32)
            per[name] = timed(lambda: h.fdl_focus_step(g, params, conf, masked, table, pred_mask, n_pred, scores,
                                                       sink_pos, n_sinks, sel_idx, n_sel), steps) / 32
        assert h.fdl_get_status() == 0
        sel_blocks = int(n_sel.sum())
        reuse_bytes = sparse_launch_bytes(cfg, sel_blocks)
        out[cfg.name] = {
            "layer_us": per, "speedup_reuse_vs_dense": per["dense"] / per["reuse"],
            "reuse_kv_tokens_per_s": B * L / (per["reuse"] * 1e-6),
            "reuse_bytes": reuse_bytes, "reuse_GBps": reuse_bytes / (per["reuse"] * 1e-6) / 1e9,
            "reuse_frac_of_peak": reuse_bytes / (per["reuse"] * 1e-6) / 1e9 / PEAK_HBM_GBS,
            "sel_blocks_per_kv_head": sel_blocks / (B * Hkv)}
        del q, k, v, kd, vd, ks, o
    # chunked, paged: the pool is [n_pages][Hkv][page][D]; each sequence's pages in shuffled order
    cfg = get_config(4)
    g = geom_for(cfg)
    B, Hq, Hkv, D, L, T = cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.ctx_len, cfg.dec_len
    gen = torch.Generator(device=dev).manual_seed(7004)
    n_pages, pps = cfg.n_pages, cfg.pages_per_seq

    def rn(*shape):
        return torch.randn(*shape, generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)

    kp, vp = rn(n_pages, Hkv, cfg.page_tokens, D), rn(n_pages, Hkv, cfg.page_tokens, D)
    pt = torch.randperm(n_pages, generator=gen, device=dev).to(torch.int32).view(B, pps).contiguous()
    q, kd, vd = rn(B, Hq, T, D), rn(B, Hkv, T, D), rn(B, Hkv, T, D)
    conf = torch.rand((B, T), generator=gen, device=dev)
    masked = (torch.rand((B, T), generator=gen, device=dev) < 0.5).to(torch.uint8)
    cs_ = ChunkedStep(h, g, ChunkParams(cfg.top_k_pos, cfg.window, cfg.chunk_tokens, cfg.top_k_chunks,
                                        cfg.tokens_per_chunk_kept))
    cs_.predict(conf, masked)
    cs = cs_.new_chunk_sums()
    cs_.pool(kp, pt, cs)
    o = torch.zeros((B, Hq, T, D), dtype=torch.bfloat16, device=dev)
    t_step = timed(lambda: cs_.run(q, kp, vp, pt, kd, vd, cs, o), chunk_runs)
    t_dense = timed(lambda: h.fdl_dense_attn(g, q, kp, vp, kd, vd, pt, o), chunk_runs)
    assert h.fdl_get_status() == 0
    n_tok = int(cs_.n_tokens.sum())
    kept = cfg.top_k_chunks * cfg.chunk_tokens
    # chunk sums, level-2 token scoring over the chosen chunks' K, the attended tokens' K and V, the
    # own block, Q and O
    step_bytes = (B * Hkv * (cfg.n_chunks * D * 4 + kept * D * 2 + T * D * 4) + n_tok * D * 4
                  + B * Hq * T * D * 4)
    out[cfg.name] = {
        "step_us": t_step, "dense_us": t_dense, "speedup_vs_dense": t_dense / t_step,
        "kv_tokens_per_s": B * L / (t_step * 1e-6), "step_bytes": step_bytes,
        "GBps": step_bytes / (t_step * 1e-6) / 1e9, "frac_of_peak": step_bytes / (t_step * 1e-6) / 1e9 / PEAK_HBM_GBS,
        "tokens_per_kv_head": n_tok / (B * Hkv)}
    del kp, vp, q, kd, vd, o
    # cache side: a full refresh of one 32K layer's cache (new K and V written, keys re-pooled per
    # 64-token block) in one pass, against copying K and V and pooling the cache afterwards
    cfg = get_config(3)
    g = geom_for(cfg)
    B, Hkv, D, L = cfg.batch, cfg.n_kv_heads, cfg.head_dim, cfg.ctx_len
    gen = torch.Generator(device=dev).manual_seed(7003)
    kn, vn = rn(B, Hkv, L, D), rn(B, Hkv, L, D)
    kc, vc = torch.empty_like(kn), torch.empty_like(vn)
    ks = torch.zeros((B, Hkv, cfg.n_blk, D), dtype=torch.float32, device=dev)
    t_fused = timed(lambda: h.fdl_cache_write(g, kn, vn, 0, kc, vc, None, cfg.kv_block, ks), chunk_runs)

    def unfused():
        kc.copy_(kn)
        vc.copy_(vn)
        h.fdl_pool_keys(g, kc, None, cfg.kv_block, ks)

    t_unfused = timed(unfused, chunk_runs)
    assert h.fdl_get_status() == 0
    # scorer readings on the same layer's pooled keys: the summed predicted query (the step's), the
    # best single predicted query and the softmax mass over the units' mean keys
    q = rn(B, cfg.n_q_heads, cfg.dec_len, D)
    conf = torch.rand((B, cfg.dec_len), generator=gen, device=dev)
    masked = (torch.rand((B, cfg.dec_len), generator=gen, device=dev) < 0.5).to(torch.uint8)
    pm = torch.zeros(B, dtype=torch.int64, device=dev)
    npred = torch.zeros(B, dtype=torch.int32, device=dev)
    h.fdl_predict_queries(B, cfg.dec_len, conf, masked, cfg.top_k_pos, cfg.window, pm, npred)
    sc = torch.zeros((B, Hkv, cfg.n_blk), dtype=torch.float32, device=dev)
    t_sum = timed(lambda: h.fdl_score_blocks(g, q, pm, ks, cfg.kv_block, sc), chunk_runs)
    t_max = timed(lambda: h.fdl_score_blocks_max(g, q, pm, ks, cfg.kv_block, sc), chunk_runs)
    t_mass = timed(lambda: h.fdl_score_blocks_mass(g, q, pm, ks, cfg.kv_block, sc), chunk_runs)
    assert h.fdl_get_status() == 0
    out["block_scoring_32k_layer"] = {"summed_query_us": t_sum, "per_query_max_us": t_max,
                                      "softmax_mass_us": t_mass,
                                      "predicted_positions": int(npred.sum())}
    kv_bytes = B * Hkv * L * D * 2
    refresh_bytes = 4 * kv_bytes + B * Hkv * cfg.n_blk * D * 4   # read new K, V; write K, V; write ks
    out["cache_refresh_32k_layer"] = {
        "fused_us": t_fused, "copy_then_pool_us": t_unfused, "speedup": t_unfused / t_fused,
        "bytes": refresh_bytes, "GBps": refresh_bytes / (t_fused * 1e-6) / 1e9,
        "frac_of_peak": refresh_bytes / (t_fused * 1e-6) / 1e9 / PEAK_HBM_GBS}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=32)
    ap.add_argument("--dense-steps", type=int, default=8)
    ap.add_argument("--diag-steps", type=int, default=32)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-workloads", action="store_true", help="skip the other workloads' diagnostics")
    ap.add_argument("--cpu-baseline-child", action="store_true")
    ap.add_argument("--copy-calib-mib", type=int, default=0,
                    help="after the run, one plain elementwise copy of this many MiB (counter calibration)")
    args = ap.parse_args()

    if args.cpu_baseline_child:
        print(json.dumps(cpu_baseline_child()))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the multi-GPU path is not built",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from diffusion_long_context_amd import Handle
    from diffusion_long_context_amd.fdllm import (FDL_LAYER_DENSE, FDL_LAYER_REUSE, FDL_LAYER_SOURCE,
                                                  fdl_focus_params)
    from diffusion_long_context_amd.step import geom_for
    from synth import get_config
    from synth.device import layer_kv, step_qkv_pool
    from synth.gen import schedule_state

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    cfg = get_config(3)
    g = geom_for(cfg)
    NL, B, Hq, Hkv, D, T = cfg.n_layers, cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.dec_len
    n_blk = cfg.n_blk
    spb, gen_steps = cfg.steps_per_block, cfg.n_gen_blocks * cfg.steps_per_block
    h = Handle(workspace_bytes=WORKSPACE_BYTES)
    dev = torch.device("cuda")

    log(f"drawing {NL} layers of KV cache on device")
    K, V = [], []
    for layer in range(NL):
        k, v = layer_kv(cfg, layer, dev)
        K.append(k)
        V.append(v)
    n_total = args.warmup + max(args.steps, args.diag_steps, args.dense_steps)
    log(f"drawing per-step queries for {n_total} steps")
    Q, KD, VD = step_qkv_pool(cfg, n_total, dev)
    conf = torch.zeros((n_total, B, T), dtype=torch.float32)
    masked = torch.zeros((n_total, B, T), dtype=torch.uint8)
    has_prev = []
    for i in range(n_total):
        st = schedule_state(cfg, i % gen_steps)
        has_prev.append(st["prev_conf"] is not None)
        if st["prev_conf"] is not None:
            conf[i] = torch.from_numpy(st["prev_conf"])
        masked[i] = torch.from_numpy(st["masked"])
    conf, masked = conf.to(dev), masked.to(dev)
    ks = [torch.zeros((B, Hkv, n_blk, D), dtype=torch.float32, device=dev) for _ in range(NL)]
    outs = [torch.zeros((B, Hq, T, D), dtype=torch.bfloat16, device=dev) for _ in range(NL)]
    pred_mask = torch.zeros(B, dtype=torch.int64, device=dev)
    n_pred = torch.zeros(B, dtype=torch.int32, device=dev)
    scores = torch.zeros((B, Hkv, n_blk), dtype=torch.float32, device=dev)
    sink_pos = torch.full((B, cfg.max_sinks), -1, dtype=torch.int32, device=dev)
    n_sinks = torch.zeros(B, dtype=torch.int32, device=dev)
    max_sel = cfg.max_sel_blocks
    sel_idx = torch.zeros((B, Hkv, max_sel), dtype=torch.int32, device=dev)
    n_sel = torch.zeros((B, Hkv), dtype=torch.int32, device=dev)
    params = fdl_focus_params(cfg.top_k_pos, cfg.window, cfg.top_k_blocks, cfg.max_sinks, max_sel,
                              cfg.sink_tau)

    def modes(all_dense=False):
        return [FDL_LAYER_DENSE if (all_dense or l < cfg.dense_layers)
                else (FDL_LAYER_SOURCE if l == cfg.source_layer else FDL_LAYER_REUSE) for l in range(NL)]

    def layer_array(i, all_dense=False):
        return h.make_layers(g, [dict(q=Q[i, l], k_cache=K[l], v_cache=V[l], k_dec=KD[i, l], v_dec=VD[i, l],
                                      ks=ks[l], out=outs[l], mode=m) for l, m in enumerate(modes(all_dense))])

    log("building per-step layer tables")
    arrays = [layer_array(i) for i in range(n_total)]
    dense_arrays = [layer_array(i, all_dense=True) for i in range(args.dense_steps)]

    def run(i0, n, tables, pool=True):
        for i in range(i0, i0 + n):
            if pool and (i % gen_steps) % spb == 0:
                for layer in range(NL):
                    h.fdl_pool_keys(g, K[layer], None, cfg.kv_block, ks[layer])
            h.fdl_focus_step(g, params, conf[i] if has_prev[i] else None, masked[i], tables[i], pred_mask,
                             n_pred, scores, sink_pos, n_sinks, sel_idx, n_sel)

    log(f"warmup {args.warmup} steps")
    run(0, args.warmup, arrays)
    torch.cuda.synchronize()
    assert h.fdl_get_status() == 0

    # ---- the timed region: exactly K steps; one pair of HIP events around each step's run of reuse
    # layers (one fused sparse-attention launch per layer, back to back on the library's stream) ----
    log(f"timing {args.steps} steps")
    h.fdl_profile_begin(args.steps + 16, kinds=("reuse_run",), every=1)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run(args.warmup, args.steps, arrays)
    torch.cuda.synchronize()
    t_total = time.perf_counter() - t0
    prof_main = h.fdl_profile_end()
    assert h.fdl_get_status() == 0
    nsel_last = n_sel.cpu().numpy()
    nsinks_last = int(n_sinks.cpu().numpy()[0])

    # ---- diagnostics (not the headline): per-kind breakdown, event overhead, dense baseline -------
    log("diagnostic passes")
    i0 = args.warmup
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run(i0, args.diag_steps, arrays)
    torch.cuda.synchronize()
    t_plain = (time.perf_counter() - t0) / args.diag_steps
    h.fdl_profile_begin(args.diag_steps * (NL * 6 + 8) + 64)
    run(i0, args.diag_steps, arrays)
    prof_all = h.fdl_profile_end()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run(0, args.dense_steps, dense_arrays, pool=False)
    torch.cuda.synchronize()
    t_dense_step = (time.perf_counter() - t0) / args.dense_steps
    assert h.fdl_get_status() == 0
    decode_loop = None if args.no_workloads else time_decode_loop(h, g, cfg, params, Q, K, V, KD, VD, ks, outs, modes,
                                                                  pred_mask, n_pred, scores, sink_pos, n_sinks,
                                                                  sel_idx, n_sel)

    def avg_us(prof, kind):
        tot, cnt = prof[kind]
        return tot / cnt if cnt else None

    sparse_us = avg_us(prof_main, "reuse_run")      # stream time per reuse launch, gaps included
    units = int(nsel_last.sum())                       # selected 64-token blocks over all heads
    unit_bytes = cfg.kv_block * D * 2 * 2              # K + V of one block, bf16
    # the sparse launch scores the blocks itself: pooled keys in, scores and selection out
    launch_bytes = sparse_launch_bytes(cfg, units)
    achieved = launch_bytes / (sparse_us * 1e-6) / 1e9
    ms_per_step = 1e3 * t_total / args.steps
    value = cfg.ctx_len * B * NL * args.steps / t_total
    reuse_layer_us = avg_us(prof_all, "layer_reuse")
    result = {
        "metric": METRIC,
        "value": value,
        "unit": "KV tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "llada8b_32k_32layer", "batch": B, "ctx_len": cfg.ctx_len, "layers": NL,
                   "q_heads": Hq, "kv_heads": Hkv, "head_dim": D, "dec_len": T, "kv_block": cfg.kv_block,
                   "top_k_blocks": cfg.top_k_blocks, "dense_layers": cfg.dense_layers,
                   "sink_source_layer": cfg.source_layer, "gen_len": gen_steps},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": measured_traffic(),
                     "kernel": "attn_mha_kernel<128,false,false,true,false> (block scoring + selection + sparse attention)",
                     "avg_launch_us": sparse_us, "launches": prof_main["reuse_run"][1],
                     "bytes_per_launch": launch_bytes, "units_per_launch": units,
                     "unit_bytes": unit_bytes},
        "sparse_attn_layer_step_us": reuse_layer_us,
        "sparse_attn_layer_kv_tokens_per_s": (cfg.ctx_len * B / (reuse_layer_us * 1e-6)) if reuse_layer_us else None,
        "breakdown_us": {k: avg_us(prof_all, k) for k in prof_all if prof_all[k][1]},
        "event_overhead_ms_per_step": 1e3 * (ms_per_step / 1e3 - t_plain),
        "dense_step_ms": 1e3 * t_dense_step,
        "speedup_vs_dense_hip": t_dense_step / t_plain,
        "sinks_detected": nsinks_last,
        "decode_loop": decode_loop,
        "workloads": None,
        "cpu_baseline": None,
    }
    if not args.no_workloads:
        log("other workloads (diagnostics)")
        del K, V, arrays, dense_arrays
        result["workloads"] = other_workloads(h, dev)
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle, single thread)")
        result["cpu_baseline"] = cpu_baseline()
    if args.copy_calib_mib > 0:
        n = args.copy_calib_mib << 20
        src = torch.ones(n // 2, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.neg(src, out=dst)   # reads n bytes, writes n bytes
        torch.cuda.synchronize()
        log(f"copy calibration: one elementwise kernel read {n} and wrote {n} bytes")
        del src, dst
    print(json.dumps(result), flush=True)
    h.close()


if __name__ == "__main__":
    main()
