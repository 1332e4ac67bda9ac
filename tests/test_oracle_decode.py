"""Pins of the decode-loop closure (oracle/decode.py): hand-worked cases, an independent brute force,
the argmax special case and the invariants of a whole block."""
import json
import math
import os

import numpy as np
import pytest

from oracle.decode import block_schedule, unmask


def _num(x):
    return float(x) if not isinstance(x, str) else {"nan": math.nan, "-0": -0.0}[x]


@pytest.fixture(scope="module")
def golden(golden_dir):
    with open(os.path.join(golden_dir, "decode_cases.json")) as f:
        return json.load(f)


def test_golden_single_step(golden):
    conf = np.array([golden["conf"]], dtype=np.float32)
    masked = np.array([golden["masked"]], dtype=np.uint8)
    for c in golden["cases"]:
        m2, dec = unmask(conf, masked, c["n"])
        assert dec[0].tolist() == c["decoded"], c["why"]
        assert m2[0].tolist() == c["masked_after"], c["why"]


def test_golden_schedule(golden):
    sc = golden["schedule"]
    confs = np.array([[[_num(x) for x in row]] for row in sc["confs"]], dtype=np.float32)
    m0 = np.array([sc["masked0"]], dtype=np.uint8)
    states, dec = block_schedule(confs, m0, sc["n"])
    assert dec[:, 0].tolist() == sc["decoded"], sc["why"]
    assert states[0][0] is None
    for s in range(1, len(states)):
        assert states[s][0] is confs[s - 1] or np.array_equal(states[s][0], confs[s - 1], equal_nan=True)
    last, _ = unmask(confs[-1], states[-1][1], sc["n"])
    assert last[0].tolist() == sc["masked_after"]


def _brute(conf_row, masked_row, n):
    """Repeatedly take the best remaining masked slot under Python float comparison: a number beats
    NaN, a larger number beats a smaller one (-0 == +0), and among equals the lower slot wins."""
    left = [i for i in range(len(conf_row)) if masked_row[i]]
    out = []
    while left and len(out) < n:
        best = left[0]
        for i in left[1:]:
            a, b = float(conf_row[i]), float(conf_row[best])
            if math.isnan(b) and not math.isnan(a):
                best = i
            elif not math.isnan(a) and not math.isnan(b) and a > b:
                best = i
        out.append(best)
        left.remove(best)
    return out


@pytest.mark.parametrize("seed", range(40))
def test_brute_force_with_ties_nan_and_signed_zero(seed):
    rng = np.random.default_rng(seed)
    B, T = 3, int(rng.integers(1, 65))
    pool = np.array([0.25, 0.5, -0.0, 0.0, np.nan, 1.0, -1.0, np.inf, -np.inf], dtype=np.float32)
    conf = np.where(rng.random((B, T)) < 0.5, rng.choice(pool, (B, T)),
                    rng.random((B, T)).astype(np.float32)).astype(np.float32)
    masked = (rng.random((B, T)) < rng.random()).astype(np.uint8)
    for n in (1, 2, 5, 64):
        m2, dec = unmask(conf, masked, n)
        for b in range(B):
            want = _brute(conf[b], masked[b], n)
            assert dec[b, :len(want)].tolist() == want
            assert (dec[b, len(want):] == -1).all()
            assert m2[b].sum() == masked[b].sum() - len(want)
            assert all(m2[b, i] == 0 for i in want)
            assert all(m2[b, i] == masked[b, i] for i in range(T) if i not in want)


def test_distinct_confidences_reduce_to_argmax():
    rng = np.random.default_rng(7)
    B, T = 16, 32
    conf = rng.permutation(B * T).reshape(B, T).astype(np.float32) / (B * T)
    masked = (rng.random((B, T)) < 0.6).astype(np.uint8)
    masked[:, 0] = 1
    _, dec = unmask(conf, masked, 1)
    want = np.argmax(np.where(masked != 0, conf, -np.inf), axis=1)
    assert dec[:, 0].tolist() == want.tolist()


@pytest.mark.parametrize("T,n", [(32, 1), (32, 3), (17, 4), (64, 1)])
def test_a_block_decodes_every_position_once(T, n):
    """From all masked, ceil(T / n) steps decode every slot exactly once, n per step (the last step
    what is left); a step with nothing masked changes nothing."""
    rng = np.random.default_rng(T * 10 + n)
    B = 2
    S = -(-T // n) + 1
    confs = rng.random((S, B, T)).astype(np.float32)
    states, dec = block_schedule(confs, np.ones((B, T), np.uint8), n)
    for b in range(B):
        got = [int(i) for i in dec[:, b].reshape(-1) if i >= 0]
        assert sorted(got) == list(range(T))
        for s in range(S):
            assert states[s][1][b].sum() == max(T - n * s, 0)
    assert (dec[-1] == -1).all()
