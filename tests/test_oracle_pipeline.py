"""Layer-to-layer behaviour of the oracle: shallow dense layers, one source layer, sink reuse."""
import numpy as np

from oracle.pipeline import focus_layer_step, schedule_modes
from synth import get_config
from synth.gen import context_kv, schedule_state, step_qkv


def test_schedule_modes_32_layers():
    m = schedule_modes(get_config(3))
    assert m[:2] == ["dense", "dense"] and m[2] == "source" and set(m[3:]) == {"reuse"} and len(m) == 32


def test_reuse_forced_set_equals_source_sinks():
    cfg = get_config(3).with_(n_q_heads=4, n_kv_heads=4, ctx_len=2048, n_layers=5, top_k_blocks=4)
    st = schedule_state(cfg, 1)
    res = {}
    sinks = None
    for layer, mode in enumerate(schedule_modes(cfg)):
        x = dict(step_qkv(cfg, layer, st["block"], st["s"]))
        x.update(context_kv(cfg, layer))
        x["prev_conf"], x["masked"] = st["prev_conf"], st["masked"]
        r = focus_layer_step(cfg, x, mode, sinks=sinks, with_output=False)
        if mode == "source":
            sinks = (r["sink_pos"], r["n_sinks"])
            assert r["n_sinks"][0] >= 1
        res[layer] = r
    F = {int(s) // cfg.kv_block for s in sinks[0][0][: sinks[1][0]]}
    for layer in (3, 4):
        assert np.array_equal(res[layer]["sink_pos"], sinks[0])
        for g in range(cfg.n_kv_heads):
            assert F <= set(res[layer]["sel"][0][g].tolist())
            assert len(res[layer]["sel"][0][g]) == len(F) + cfg.top_k_blocks
