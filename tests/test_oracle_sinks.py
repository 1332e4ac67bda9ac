"""Pins of sink detection: row masses sum to one, planted sinks recovered, pure-Python brute force,
closed form on identical keys."""
import math

import numpy as np
import pytest

from oracle.predictor import predict_positions
from oracle.sinks import detect_sinks, sink_masses


def test_full_row_mass_sums_to_one():
    from synth import get_config
    from synth.gen import make_single
    cfg = get_config(0)
    x = make_single(cfg)
    bits, _ = predict_positions(x["prev_conf"], x["masked"], cfg.top_k_pos, cfg.window)
    a = sink_masses(x["q"], x["k"], x["k_dec"], bits, full_row=True)
    assert np.allclose(a.sum(axis=-1), 1.0, atol=1e-12, rtol=0)


@pytest.mark.parametrize("ci,expected", [(0, [0]), (1, [0, 1, 2, 3]), (2, [0, 1, 2, 3])])
def test_planted_sinks_recovered(ci, expected):
    from synth import get_config
    from synth.gen import make_single
    cfg = get_config(ci)
    x = make_single(cfg)
    bits, _ = predict_positions(x["prev_conf"], x["masked"], cfg.top_k_pos, cfg.window)
    pos, n, over, margin = detect_sinks(x["q"], x["k"], x["k_dec"], bits, cfg.sink_tau, cfg.max_sinks)
    assert pos[0, : n[0]].tolist() == expected and not over[0]
    assert margin > 1e-4 * cfg.sink_tau


def test_brute_force_pure_python():
    rng = np.random.default_rng(21)
    B, Hq, Hkv, T, D, L = 1, 4, 2, 4, 4, 8
    q = rng.standard_normal((B, Hq, T, D)).astype(np.float32)
    k = rng.standard_normal((B, Hkv, L, D)).astype(np.float32)
    kd = rng.standard_normal((B, Hkv, T, D)).astype(np.float32)
    bits = np.array([0b1011], dtype=np.uint64)
    a = sink_masses(q, k, kd, bits)
    P = [0, 1, 3]
    for h in range(Hq):
        g = h // 2
        keys = [list(map(float, k[0, g, t])) for t in range(L)] + [list(map(float, kd[0, g, t])) for t in range(T)]
        acc = [0.0] * L
        for p in P:
            qq = list(map(float, q[0, h, p]))
            s = [sum(x * y for x, y in zip(qq, kk)) / math.sqrt(D) for kk in keys]
            z = sum(math.exp(v) for v in s)
            for t in range(L):
                acc[t] += math.exp(s[t]) / z / len(P)
        assert np.allclose(a[0, h], acc, rtol=0, atol=1e-13)


def test_identical_keys_uniform_mass():
    B, H, T, D, L = 1, 2, 4, 8, 12
    q = np.ones((B, H, T, D), np.float32)
    k = np.full((B, H, L, D), 0.5, np.float32)
    kd = np.full((B, H, T, D), 0.5, np.float32)
    bits = np.array([0b0110], dtype=np.uint64)
    a = sink_masses(q, k, kd, bits)
    assert np.allclose(a, 1.0 / (L + T), atol=1e-15)
    pos, n, _, _ = detect_sinks(q, k, kd, bits, 1.0 / (L + T) - 1e-9, 64)
    assert n[0] == L and pos[0, :L].tolist() == list(range(L))
    pos, n, _, _ = detect_sinks(q, k, kd, bits, 1.0 / (L + T) + 1e-9, 64)
    assert n[0] == 0


def test_overflow_truncates_and_flags():
    B, H, T, D, L = 1, 1, 2, 4, 10
    q = np.zeros((B, H, T, D), np.float32)
    k = np.zeros((B, H, L, D), np.float32)
    kd = np.zeros((B, H, T, D), np.float32)
    pos, n, over, _ = detect_sinks(q, k, kd, np.array([1], np.uint64), 0.01, 4)
    assert over[0] and n[0] == 4 and pos[0].tolist() == [0, 1, 2, 3]


def test_empty_prediction_has_no_sinks():
    q = np.ones((1, 1, 2, 4), np.float32)
    k = np.ones((1, 1, 6, 4), np.float32)
    pos, n, over, _ = detect_sinks(q, k, k[:, :, :2], np.array([0], np.uint64), 0.0, 8)
    assert n[0] == 0
