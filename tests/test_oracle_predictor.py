"""Pins of the past-confidence predictor: hand-worked cases and brute force over k-subsets."""
import itertools
import json
import math
import os

import numpy as np
import pytest

from oracle.predictor import mask_to_positions, predict_positions, top_masked_positions


def test_golden_cases(golden_dir):
    with open(os.path.join(golden_dir, "predictor_cases.json")) as f:
        g = json.load(f)
    conf = np.array([g["conf"]], dtype=np.float32)
    masked = np.array([g["masked"]], dtype=np.uint8)
    for c in g["cases"]:
        bits, n = predict_positions(conf, masked, c["k"], c["w"])
        assert mask_to_positions(bits[0], g["T"]) == c["positions"], c
        assert n[0] == len(c["positions"])


def _better(ca, a, cb, b):
    """a ranks above b: larger confidence (NaN below every number), ties to the lower slot."""
    na, nb = math.isnan(ca), math.isnan(cb)
    if na and nb:
        return a < b
    if na != nb:
        return nb
    if ca != cb:
        return ca > cb
    return a < b


def _brute_topk(conf, masked, k):
    cand = [i for i in range(len(conf)) if masked[i]]
    kk = min(k, len(cand))
    valid = []
    for A in itertools.combinations(cand, kk):
        rest = [b for b in cand if b not in A]
        if all(_better(float(conf[a]), a, float(conf[b]), b) for a in A for b in rest):
            valid.append(set(A))
    assert len(valid) == 1
    return valid[0]


@pytest.mark.parametrize("seed", range(30))
def test_brute_force_small(seed):
    rng = np.random.default_rng(seed)
    T = 12
    conf = rng.choice([0.1, 0.2, 0.5, 0.9, np.nan, -0.0, 0.0], size=T).astype(np.float32)
    masked = (rng.random(T) < 0.6).astype(np.uint8)
    for k in (1, 2, 4):
        top = top_masked_positions(conf, masked, k)
        assert set(top) == _brute_topk(conf, masked, k)
        w = int(rng.integers(0, 3))
        bits, n = predict_positions(conf[None], masked[None], k, w)
        exp = sorted({p for i in top for p in range(i - w, i + w + 1) if 0 <= p < T})
        assert mask_to_positions(bits[0], T) == exp


def test_tiny_workload_brute_force():
    from synth import get_config
    from synth.gen import decode_state
    cfg = get_config(0)
    d = decode_state(cfg)
    top = top_masked_positions(d["prev_conf"][0], d["masked"][0], cfg.top_k_pos)
    assert set(top) == _brute_topk(d["prev_conf"][0], d["masked"][0], cfg.top_k_pos)


def test_no_previous_confidence_predicts_all():
    masked = np.zeros((2, 32), np.uint8)
    bits, n = predict_positions(None, masked, 4, 4)
    assert all(int(b) == (1 << 32) - 1 for b in bits) and list(n) == [32, 32]


def test_nothing_masked_predicts_nothing():
    bits, n = predict_positions(np.ones((1, 32), np.float32), np.zeros((1, 32), np.uint8), 4, 4)
    assert int(bits[0]) == 0 and n[0] == 0


def test_full_width_block_of_64():
    conf = np.linspace(0, 1, 64, dtype=np.float32)[None]
    bits, n = predict_positions(conf, np.ones((1, 64), np.uint8), 1, 2)
    assert mask_to_positions(bits[0], 64) == [61, 62, 63]
