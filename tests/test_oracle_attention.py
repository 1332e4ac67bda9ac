"""Pins of the attention definition: closed form, degenerate cases, a library routine in float64 and a
pure-Python brute force."""
import math

import numpy as np
import pytest
import torch

from oracle.attention import attend, attend_rows


def test_closed_form_three_quarters():
    q = np.array([[math.sqrt(2) * math.log(3.0), 0.0]])
    keys = np.array([[1.0, 0.0], [0.0, 1.0]])
    vals = np.array([[1.0, 0.0], [0.0, 1.0]])
    o = attend_rows(q, keys, vals)
    assert np.allclose(o, [[0.75, 0.25]], atol=1e-15)


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape).astype(np.float32)


def test_constant_v_gives_constant():
    B, H, T, D, L = 1, 2, 4, 8, 16
    v = np.full((B, H, L, D), 0.375, np.float32)
    o = attend(_rand((B, H, T, D), 1), _rand((B, H, L, D), 2), v, _rand((B, H, T, D), 3),
               np.full((B, H, T, D), 0.375, np.float32), None)
    assert np.allclose(o, 0.375, atol=1e-15)


def test_zero_keys_give_mean_of_values():
    B, H, T, D, L = 1, 1, 4, 8, 16
    v, vd = _rand((B, H, L, D), 4), _rand((B, H, T, D), 5)
    o = attend(_rand((B, H, T, D), 6), np.zeros((B, H, L, D), np.float32), v,
               np.zeros((B, H, T, D), np.float32), vd, [[np.array([0, 3, 5])]])
    mean = np.concatenate([v[0, 0, [0, 3, 5]], vd[0, 0]]).astype(np.float64).mean(axis=0)
    assert np.allclose(o[0, 0], mean[None, :], atol=1e-15)


def test_dense_matches_torch_sdpa_float64():
    from synth import get_config
    from synth.gen import make_single
    cfg = get_config(0)
    x = make_single(cfg)
    o = attend(x["q"], x["k"], x["v"], x["k_dec"], x["v_dec"], None)
    q = torch.from_numpy(x["q"].astype(np.float64))
    k = torch.from_numpy(np.concatenate([x["k"], x["k_dec"]], axis=2).astype(np.float64))
    v = torch.from_numpy(np.concatenate([x["v"], x["v_dec"]], axis=2).astype(np.float64))
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v).numpy()
    assert np.allclose(o, ref, atol=1e-12, rtol=0)


def test_gqa_head_mapping_matches_sdpa():
    B, Hq, Hkv, T, D, L = 1, 6, 2, 4, 8, 10
    q, k, v = _rand((B, Hq, T, D), 7), _rand((B, Hkv, L, D), 8), _rand((B, Hkv, L, D), 9)
    kd, vd = _rand((B, Hkv, T, D), 10), _rand((B, Hkv, T, D), 11)
    o = attend(q, k, v, kd, vd, None)
    kk = np.repeat(np.concatenate([k, kd], axis=2), Hq // Hkv, axis=1).astype(np.float64)
    vv = np.repeat(np.concatenate([v, vd], axis=2), Hq // Hkv, axis=1).astype(np.float64)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q.astype(np.float64)), torch.from_numpy(kk), torch.from_numpy(vv)).numpy()
    assert np.allclose(o, ref, atol=1e-12, rtol=0)


def test_all_blocks_selected_equals_dense():
    from synth import get_config
    from synth.gen import make_single
    from oracle.pipeline import focus_layer_step
    cfg = get_config(0).with_(top_k_blocks=16)
    x = make_single(cfg)
    r = focus_layer_step(cfg, x, "source")
    dense = focus_layer_step(cfg, x, "dense")["out"]
    assert all(len(s) == 16 for s in r["sel"][0])
    assert np.allclose(r["out"], dense, atol=1e-13, rtol=0)


def test_brute_force_rows_tiny_workload():
    from synth import get_config
    from synth.gen import make_single
    from oracle.pipeline import focus_layer_step
    cfg = get_config(0)
    x = make_single(cfg)
    r = focus_layer_step(cfg, x, "source")
    D = cfg.head_dim
    for h, i in [(0, 0), (1, 17), (1, 31)]:
        toks = [t for n in r["sel"][0][h] for t in range(n * cfg.kv_block, (n + 1) * cfg.kv_block)]
        keys = [x["k"][0, h, t] for t in toks] + [x["k_dec"][0, h, t] for t in range(cfg.dec_len)]
        vals = [x["v"][0, h, t] for t in toks] + [x["v_dec"][0, h, t] for t in range(cfg.dec_len)]
        qq = [float(v) for v in x["q"][0, h, i]]
        s = [sum(a * float(b) for a, b in zip(qq, kk)) / math.sqrt(D) for kk in keys]
        m = max(s)
        w = [math.exp(v - m) for v in s]
        z = sum(w)
        o = [sum(w[j] * float(vals[j][d]) for j in range(len(w))) / z for d in range(D)]
        assert np.allclose(r["out"][0, h, i], o, atol=1e-12, rtol=0)
