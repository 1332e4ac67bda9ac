"""The decode loop on the GPU: fdl_unmask bit for bit against the oracle's unmask update,
fdl_decode_steps (several denoising steps in one call) against the oracle's block schedule and layer
steps, and the same steps captured into a HIP graph and replayed."""
import ctypes

import numpy as np
import pytest
import torch

from gpu_util import assert_close, bf16_out_to_f64, dev, host, require_gpu
from oracle.decode import block_schedule, unmask
from oracle.pipeline import focus_layer_step
from synth import get_config
from synth.gen import make_single

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def h():
    require_gpu()
    from diffusion_long_context_amd import Handle
    hh = Handle(workspace_bytes=512 << 20)
    yield hh
    hh.close()


def _conf(rng, B, T):
    pool = np.array([0.25, 0.5, -0.0, 0.0, np.nan, 1.0, -1.0, np.inf], dtype=np.float32)
    return np.where(rng.random((B, T)) < 0.4, rng.choice(pool, (B, T)),
                    rng.random((B, T)).astype(np.float32)).astype(np.float32)


@pytest.mark.parametrize("B,T,n,p_mask", [
    (4, 32, 1, 0.5), (4, 32, 4, 0.5), (3, 64, 64, 0.7), (5, 1, 1, 1.0), (2, 17, 5, 0.3),
    (8, 32, 0, 0.5), (2, 32, 3, 0.0), (2, 32, 40, 1.0), (300, 32, 2, 0.5),
], ids=["t32-n1", "t32-n4", "t64-all", "t1", "t17-n5", "n0", "none-masked", "all-masked-n40", "b300"])
def test_unmask_bit_exact(h, B, T, n, p_mask):
    rng = np.random.default_rng(B * 1000 + T * 10 + n)
    conf = _conf(rng, B, T)
    masked = (rng.random((B, T)) < p_mask).astype(np.uint8)
    m_d = dev(masked)
    dec_d = torch.full((B, max(n, 1)), 77, dtype=torch.int32, device="cuda")
    h.fdl_unmask(B, T, dev(conf), m_d, n, dec_d if n > 0 else None)
    torch.cuda.synchronize()
    want_m, want_dec = unmask(conf, masked, n)
    assert np.array_equal(host(m_d), want_m)
    if n > 0:
        assert np.array_equal(host(dec_d)[:, :n], want_dec)


def test_unmask_argument_errors(h):
    from diffusion_long_context_amd.fdllm import FdlError
    conf = torch.zeros((2, 32), dtype=torch.float32, device="cuda")
    masked = torch.ones((2, 32), dtype=torch.uint8, device="cuda")
    for B, T, n in ((2, 65, 1), (0, 32, 1), (2, 32, 65), (2, 32, -1)):
        with pytest.raises(FdlError):
            h._check(h.lib.fdl_unmask(h.h, B, T, ctypes.c_void_p(conf.data_ptr()),
                                      ctypes.c_void_p(masked.data_ptr()), n, None))
    with pytest.raises(FdlError):
        h._check(h.lib.fdl_unmask(h.h, 2, 32, None, ctypes.c_void_p(masked.data_ptr()), 1, None))
    torch.cuda.synchronize()
    assert host(masked).all()   # untouched


def _setup(h, S, modes, **kw):
    from diffusion_long_context_amd.fdllm import (FDL_LAYER_DENSE, FDL_LAYER_REUSE, FDL_LAYER_SOURCE,
                                                  fdl_focus_params)
    from diffusion_long_context_amd.step import geom_for
    cfg = get_config(1).with_(**dict(dict(batch=2, n_q_heads=4, n_kv_heads=4, ctx_len=3000, top_k_blocks=12), **kw))
    g = geom_for(cfg)
    B, Hq, Hkv, D, T, nb, ms = (cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.dec_len,
                                cfg.n_blk, cfg.max_sel_blocks)
    code = {"dense": FDL_LAYER_DENSE, "source": FDL_LAYER_SOURCE, "reuse": FDL_LAYER_REUSE}
    xs = [[make_single(cfg, layer=l, step=s) for l in range(len(modes))] for s in range(S)]
    kv = [{k: dev(xs[0][l][k]) for k in ("k", "v")} for l in range(len(modes))]
    ks = [torch.zeros((B, Hkv, nb, D), dtype=torch.float32, device="cuda") for _ in modes]
    for l in range(len(modes)):
        h.fdl_pool_keys(g, kv[l]["k"], None, cfg.kv_block, ks[l])
    own = [[{k: dev(xs[s][l][k]) for k in ("q", "k_dec", "v_dec")} for l in range(len(modes))] for s in range(S)]
    outs = [[torch.zeros((B, Hq, T, D), dtype=torch.bfloat16, device="cuda") for _ in modes] for _ in range(S)]
    table = h.make_layers(g, [dict(q=own[s][l]["q"], k_cache=kv[l]["k"], v_cache=kv[l]["v"], k_dec=own[s][l]["k_dec"],
                                   v_dec=own[s][l]["v_dec"], ks=ks[l], out=outs[s][l], mode=code[m])
                              for s in range(S) for l, m in enumerate(modes)])
    bufs = dict(pm=torch.zeros(B, dtype=torch.int64, device="cuda"), npd=torch.zeros(B, dtype=torch.int32, device="cuda"),
                sc=torch.zeros((B, Hkv, nb), dtype=torch.float32, device="cuda"),
                sp=torch.full((B, cfg.max_sinks), -1, dtype=torch.int32, device="cuda"),
                nsk=torch.zeros(B, dtype=torch.int32, device="cuda"),
                sel=torch.zeros((B, Hkv, ms), dtype=torch.int32, device="cuda"),
                nsel=torch.zeros((B, Hkv), dtype=torch.int32, device="cuda"))
    params = fdl_focus_params(cfg.top_k_pos, cfg.window, cfg.top_k_blocks, cfg.max_sinks, ms, cfg.sink_tau)
    rng = np.random.default_rng(4242)
    confs = rng.random((S, B, T)).astype(np.float32)
    return cfg, g, params, xs, outs, table, bufs, confs


def _decode(h, g, params, S, confs_d, masked_d, n, dec_d, table, b):
    h.fdl_decode_steps(g, params, S, None, confs_d, masked_d, n, dec_d, table, b["pm"], b["npd"], b["sc"], b["sp"],
                       b["nsk"], b["sel"], b["nsel"])


@pytest.mark.parametrize("n", [1, 3])
def test_decode_steps_against_oracle(h, n):
    """Four steps of a block from all-masked, three layers (dense, source, reuse) per step: the
    decoded positions and the final masked flags bit for bit, every layer's output of every step to
    the output tolerance."""
    S, modes = 4, ["dense", "source", "reuse"]
    cfg, g, params, xs, outs, table, b, confs = _setup(h, S, modes)
    B, T = cfg.batch, cfg.dec_len
    masked_d = torch.ones((B, T), dtype=torch.uint8, device="cuda")
    dec_d = torch.full((S, B, n), 99, dtype=torch.int32, device="cuda")
    _decode(h, g, params, S, dev(confs), masked_d, n, dec_d, table, b)
    torch.cuda.synchronize()
    assert h.fdl_get_status() == 0
    states, want_dec = block_schedule(confs, np.ones((B, T), np.uint8), n)
    assert np.array_equal(host(dec_d), want_dec)
    want_last, _ = unmask(confs[-1], states[-1][1], n)
    assert np.array_equal(host(masked_d), want_last)
    for s in range(S):
        prev, m = states[s]
        sinks = None
        for l, mode in enumerate(modes):
            x = dict(xs[s][l], k=xs[0][l]["k"], v=xs[0][l]["v"], prev_conf=prev, masked=m)
            want = focus_layer_step(cfg, x, mode, sinks=sinks)
            if mode == "source":
                assert want["sink_margin"] > 1e-4 * cfg.sink_tau
                sinks = (want["sink_pos"], want["n_sinks"])
            assert_close(bf16_out_to_f64(outs[s][l]), want["out"], f"step {s} layer {l} ({mode})")


def test_graph_replay_equals_eager(h):
    """The same steps captured into one graph on a side stream: every replay (with the masked flags
    reset and the outputs cleared in between, plus unrelated eager work) reproduces the eager run's
    outputs, decoded positions and flags bit for bit."""
    S, modes, n = 3, ["dense", "source", "reuse", "reuse"], 1
    cfg, g, params, xs, outs, table, b, confs = _setup(h, S, modes, n_kv_heads=2, top_k_blocks=10)
    B, T = cfg.batch, cfg.dec_len
    confs_d = dev(confs)
    masked0 = torch.ones((B, T), dtype=torch.uint8, device="cuda")
    masked_d = masked0.clone()
    dec_d = torch.zeros((S, B, n), dtype=torch.int32, device="cuda")
    _decode(h, g, params, S, confs_d, masked_d, n, dec_d, table, b)
    torch.cuda.synchronize()
    assert h.fdl_get_status() == 0
    want_outs = [[o.clone() for o in row] for row in outs]
    want_dec, want_masked, want_sel = dec_d.clone(), masked_d.clone(), b["sel"].clone()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        masked_d.copy_(masked0)
        side.synchronize()
        h.fdl_capture_begin()
        try:
            _decode(h, g, params, S, confs_d, masked_d, n, dec_d, table, b)
        finally:
            graph = h.fdl_capture_end()
    try:
        scratch = torch.ones((B, T), dtype=torch.uint8, device="cuda")
        for rep in range(3):
            with torch.cuda.stream(side):
                masked_d.copy_(masked0)
                dec_d.zero_()
                for row in outs:
                    for o in row:
                        o.zero_()
                h.fdl_graph_launch(graph)
            torch.cuda.synchronize()
            assert h.fdl_get_status() == 0
            assert torch.equal(dec_d, want_dec), rep
            assert torch.equal(masked_d, want_masked), rep
            assert torch.equal(b["sel"], want_sel), rep
            for s in range(S):
                for l in range(len(modes)):
                    assert torch.equal(outs[s][l].view(torch.int16), want_outs[s][l].view(torch.int16)), (rep, s, l)
            # eager work between replays, on the default stream
            h.fdl_unmask(B, T, confs_d[0], scratch, 2, None)
            torch.cuda.synchronize()
            assert int(host(scratch).sum()) == B * (T - 2)
            scratch.fill_(1)
    finally:
        h.fdl_graph_destroy(graph)


def test_capture_rules(h):
    from diffusion_long_context_amd.fdllm import FdlError
    with pytest.raises(FdlError):
        h.fdl_capture_begin()          # the default stream cannot be captured
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        h.fdl_capture_begin()
        try:
            with pytest.raises(FdlError):
                h._check(h.lib.fdl_get_status(h.h))      # no synchronisation while capturing
            with pytest.raises(FdlError):
                h.fdl_capture_begin()                    # one capture at a time
        finally:
            graph = h.fdl_capture_end()                  # an empty graph is a valid graph
        h.fdl_graph_launch(graph)
        h.fdl_graph_destroy(graph)
    torch.cuda.synchronize()
    assert h.fdl_get_status() == 0


def test_decode_steps_validates_every_step_before_launching(h):
    """A bad layer table in the last step is reported before anything runs: the masked flags and
    the outputs of the earlier steps stay untouched."""
    from diffusion_long_context_amd.fdllm import FDL_LAYER_REUSE, FdlError, fdl_layer_io
    S, modes, n = 3, ["dense", "source", "reuse"], 1
    cfg, g, params, xs, outs, table, b, confs = _setup(h, S, modes)
    B, T = cfg.batch, cfg.dec_len
    bad = (fdl_layer_io * len(table))()
    for i in range(len(table)):
        bad[i] = table[i]
    bad[len(table) - 1].ks = None            # a reuse layer without pooled keys
    assert bad[len(table) - 1].mode == FDL_LAYER_REUSE
    masked_d = torch.ones((B, T), dtype=torch.uint8, device="cuda")
    for row in outs:
        for o in row:
            o.fill_(3.0)
    torch.cuda.synchronize()
    with pytest.raises(FdlError):
        h.fdl_decode_steps(g, params, S, None, dev(confs), masked_d, n, None, bad, b["pm"], b["npd"], b["sc"],
                           b["sp"], b["nsk"], b["sel"], b["nsel"])
    torch.cuda.synchronize()
    assert bool((masked_d == 1).all())
    assert all(bool((o == 3.0).all()) for row in outs for o in row)


def test_graph_of_the_chunked_paged_step(h):
    """The chunked, paged select-and-attend chain (chunk scores, chunk selection, level 2 in one
    kernel, paged attention) captured once and replayed: every replay equals the eager run."""
    from diffusion_long_context_amd.step import ChunkedStep, ChunkParams, geom_for
    cfg = get_config(4).with_(batch=2, n_q_heads=4, n_kv_heads=2, ctx_len=4096, chunk_tokens=512)
    g = geom_for(cfg)
    x = make_single(cfg)
    t = {k: dev(x[k]) for k in ("q", "k_pool", "v_pool", "page_table", "k_dec", "v_dec", "masked", "prev_conf")}
    cs_ = ChunkedStep(h, g, ChunkParams(cfg.top_k_pos, cfg.window, cfg.chunk_tokens, cfg.top_k_chunks,
                                        cfg.tokens_per_chunk_kept))
    cs = cs_.new_chunk_sums()
    cs_.pool(t["k_pool"], t["page_table"], cs)
    out = torch.zeros((cfg.batch, cfg.n_q_heads, cfg.dec_len, cfg.head_dim), dtype=torch.bfloat16, device="cuda")

    def step():
        cs_.predict(t["prev_conf"], t["masked"])
        cs_.run(t["q"], t["k_pool"], t["v_pool"], t["page_table"], t["k_dec"], t["v_dec"], cs, out)

    step()
    torch.cuda.synchronize()
    assert h.fdl_get_status() == 0
    want_out, want_tok = out.clone(), cs_.tokens.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        h.fdl_capture_begin()
        try:
            step()
        finally:
            graph = h.fdl_capture_end()
    try:
        for rep in range(3):
            with torch.cuda.stream(side):
                out.zero_()
                cs_.tokens.zero_()
                h.fdl_graph_launch(graph)
            torch.cuda.synchronize()
            assert h.fdl_get_status() == 0
            assert torch.equal(out.view(torch.int16), want_out.view(torch.int16)), rep
            assert torch.equal(cs_.tokens, want_tok), rep
            step()                                # eager work between replays
            torch.cuda.synchronize()
    finally:
        h.fdl_graph_destroy(graph)
