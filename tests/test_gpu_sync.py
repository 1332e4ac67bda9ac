"""Placement of the workgroups that hand data to each other through an XCD's L2.

The fused kernel's splits exchange scores through tagged entries that carry the writer's XCD, and
the last split of a head merges the others' partials after a ticket that counts the takers per XCD;
the sink scan merges its splits' statistics the same way.  With FDL_SAFE_SYNC=1 (read when a handle
is created) nothing is handed over inside a launch.  Both modes must give the same bits -- scores,
sinks, selections and outputs -- and on this hardware the default mode must never find a sibling on
another XCD (no FDL_FLAG_PLACEMENT, no FDL_ESYNC)."""
import numpy as np
import pytest
import torch

from gpu_util import assert_close, host, require_gpu
from synth import get_config
from synth.gen import make_single

pytestmark = pytest.mark.gpu

FLAG_PLACEMENT, FLAG_SPLIT_PLACEMENT = 32, 64


def _run(cfg, xs, modes, safe, monkeypatch):
    from diffusion_long_context_amd import Handle
    from layer_util import focus_step_layers
    if safe:
        monkeypatch.setenv("FDL_SAFE_SYNC", "1")
    else:
        monkeypatch.delenv("FDL_SAFE_SYNC", raising=False)
    h = Handle(workspace_bytes=512 << 20)
    try:
        got = focus_step_layers(h, cfg, xs, modes, xs[0]["prev_conf"], xs[0]["masked"])
    finally:
        h.close()
    got["outs"] = [host(o.view(torch.int16)).copy() for o in got["outs"]]
    return got


@pytest.mark.parametrize("ci,kw", [
    (1, dict(ctx_len=16384, n_q_heads=32, n_kv_heads=32, top_k_blocks=64)),   # the 32K layer's grid
    (1, {}),                                                                   # 8K, 32 heads
    (2, {}),                                                                   # 16K, 28 / 4 heads
    (1, dict(batch=3, n_q_heads=8, n_kv_heads=8, ctx_len=5000, top_k_blocks=20)),
], ids=["16k-32heads", "8k", "16k-gqa7", "b3-ragged"])
def test_safe_mode_is_bit_identical(ci, kw, monkeypatch):
    require_gpu()
    cfg = get_config(ci).with_(**kw)
    modes = ["dense", "source", "reuse", "reuse"]
    xs = [make_single(cfg, layer=l) for l in range(len(modes))]
    print(f"safe-mode comparison {cfg.name} {kw}", flush=True)
    fast = _run(cfg, xs, modes, False, monkeypatch)
    safe = _run(cfg, xs, modes, True, monkeypatch)
    assert fast["bits"] & (FLAG_PLACEMENT | FLAG_SPLIT_PLACEMENT) == 0, fast["bits"]
    assert safe["bits"] == 0, safe["bits"]
    assert np.array_equal(fast["pred_mask"], safe["pred_mask"])
    assert np.array_equal(fast["n_sinks"], safe["n_sinks"]) and np.array_equal(fast["sink_pos"], safe["sink_pos"])
    for l in fast["layers"]:
        for a, b in zip(fast["layers"][l], safe["layers"][l]):
            assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), l
    for l, (a, b) in enumerate(zip(fast["outs"], safe["outs"])):
        assert np.array_equal(a, b), f"layer {l} outputs differ"


def test_safe_mode_standalone_attention(monkeypatch):
    """fdl_sparse_attn and fdl_dense_attn (split partials merged in place, or by the second launch in
    the safe mode): the same bits, and the oracle's values."""
    require_gpu()
    from diffusion_long_context_amd import Handle
    from diffusion_long_context_amd.step import geom_for
    from gpu_util import dev, out_buffer, out_to_f64
    from oracle.attention import attend, blocks_to_tokens
    cfg = get_config(1).with_(n_q_heads=16, n_kv_heads=16)
    x = make_single(cfg)
    g = geom_for(cfg)
    rng = np.random.default_rng(3)
    sel = np.sort(np.stack([[rng.choice(cfg.n_blk, 20, replace=False) for _ in range(16)]]), axis=-1).astype(np.int32)
    res = []
    for safe in (False, True):
        if safe:
            monkeypatch.setenv("FDL_SAFE_SYNC", "1")
        else:
            monkeypatch.delenv("FDL_SAFE_SYNC", raising=False)
        h = Handle()
        try:
            t = {n: dev(x[n]) for n in ("q", "k", "v", "k_dec", "v_dec")}
            o_s, o_d = out_buffer(cfg), out_buffer(cfg)
            h.fdl_sparse_attn(g, t["q"], t["k"], t["v"], t["k_dec"], t["v_dec"], None, dev(sel),
                              dev(np.full((1, 16), 20, np.int32)), 20, cfg.kv_block, o_s)
            h.fdl_dense_attn(g, t["q"], t["k"], t["v"], t["k_dec"], t["v_dec"], None, o_d)
            torch.cuda.synchronize()
            st, bits = h.fdl_get_status_bits()
            assert st == 0 and bits == 0, (st, bits)
            res.append((host(o_s).copy(), host(o_d).copy(), out_to_f64(cfg, o_s), out_to_f64(cfg, o_d)))
        finally:
            h.close()
    assert np.array_equal(res[0][0], res[1][0]) and np.array_equal(res[0][1], res[1][1])
    toks = [[blocks_to_tokens(sel[0, gg], cfg.kv_block, cfg.ctx_len) for gg in range(16)]]
    assert_close(res[0][2], attend(x["q"], x["k"], x["v"], x["k_dec"], x["v_dec"], toks), "sparse")
    assert_close(res[0][3], attend(x["q"], x["k"], x["v"], x["k_dec"], x["v_dec"], None), "dense")
