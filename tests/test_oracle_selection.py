"""Pins of block selection: hand-worked case, brute force over subsets, invariants."""
import itertools
import json
import math
import os

import numpy as np
import pytest

from oracle.selection import select_blocks, select_units, topk_indices


def _f(v):
    return {"-0": -0.0, "+0": 0.0}.get(v, v) if isinstance(v, str) else v


def test_golden_cases(golden_dir):
    with open(os.path.join(golden_dir, "selection_cases.json")) as f:
        g = json.load(f)
    s = np.array([_f(v) for v in g["scores"]], dtype=np.float32)
    for c in g["cases"]:
        assert select_units(s, g["forced"], c["k"]).tolist() == c["selected"], c


def _better(sa, a, sb, b):
    na, nb = math.isnan(sa), math.isnan(sb)
    if na and nb:
        return a < b
    if na != nb:
        return nb
    if sa != sb:
        return sa > sb
    return a < b


def _brute(scores, forced, k):
    free = [i for i in range(len(scores)) if i not in forced]
    kk = min(k, len(free))
    valid = []
    for A in itertools.combinations(free, kk):
        rest = [i for i in free if i not in A]
        if all(_better(float(scores[a]), a, float(scores[b]), b) for a in A for b in rest):
            valid.append(sorted(set(A) | set(forced)))
    assert len(valid) == 1
    return valid[0]


def test_brute_force_tiny_workload():
    """Tiny workload shape: 16 blocks, one forced sink block, K = 4 -> C(15,4) = 1365 subsets."""
    from synth import get_config
    from synth.gen import make_single
    from oracle.pipeline import focus_layer_step
    cfg = get_config(0)
    x = make_single(cfg)
    r = focus_layer_step(cfg, x, "source", with_output=False)
    for g in range(cfg.n_kv_heads):
        forced = sorted({int(s) // cfg.kv_block for s in r["sink_pos"][0][: r["n_sinks"][0]]})
        assert r["sel"][0][g].tolist() == _brute(r["scores"][0, g], forced, cfg.top_k_blocks)


@pytest.mark.parametrize("seed", range(20))
def test_brute_force_with_ties_and_specials(seed):
    rng = np.random.default_rng(seed)
    s = rng.choice([1.0, 2.0, -0.0, 0.0, np.nan, -np.inf, 3.5], size=10).astype(np.float32)
    forced = sorted(set(rng.integers(0, 10, size=rng.integers(0, 3)).tolist()))
    for k in (0, 1, 3, 5, 10):
        assert select_units(s, forced, k).tolist() == _brute(s, forced, k)


def test_invariants():
    rng = np.random.default_rng(3)
    B, H, n = 2, 3, 40
    scores = rng.standard_normal((B, H, n)).astype(np.float32)
    sink_pos = np.array([[0, 1, 130, -1], [70, -1, -1, -1]], dtype=np.int32)
    n_sinks = np.array([3, 1], dtype=np.int32)
    for k in (0, 5, 37, 38, 100):
        sel = select_blocks(scores, sink_pos, n_sinks, 64, k)
        for b in range(B):
            F = sorted({int(s) // 64 for s in sink_pos[b][: n_sinks[b]]})
            for g in range(H):
                s = sel[b][g].tolist()
                assert set(F) <= set(s)
                assert s == sorted(set(s))
                assert len(s) == len(F) + min(k, n - len(F))
                if k >= n - len(F):
                    assert s == list(range(n))


def test_topk_excludes():
    s = np.array([5, 4, 3, 2, 1], np.float32)
    assert topk_indices(s, 2, exclude=[0]) == [1, 2]


# ---- token-granular sink retention ------------------------------------------------------------

def test_token_sinks_worked_case():
    """Blocks of 4 tokens, 5 blocks, L = 18 (the last block holds 2 tokens); scores [9, 1, 5, 7, 3],
    sinks at tokens 0, 1 and 9, K = 2.  The top 2 blocks of all five are 0 and 3 (tokens 0-3 and
    12-15); the sinks add token 9 only (0 and 1 are inside block 0): 9 tokens.  With block-granular
    retention block 2 (tokens 8-11) would be forced in and K = 2 would pick blocks 3 and 2."""
    from oracle.selection import select_token_sinks
    sc = np.array([[[9, 1, 5, 7, 3]]], np.float32)
    got = select_token_sinks(sc, np.array([[0, 1, 9, -1]]), np.array([3]), 4, 2, 18)
    assert got[0][0].tolist() == [0, 1, 2, 3, 9, 12, 13, 14, 15]
    got = select_token_sinks(sc, np.array([[17, 16]]), np.array([2]), 4, 1, 18)
    assert got[0][0].tolist() == [0, 1, 2, 3, 16, 17]     # sinks inside the partial last block
    got = select_token_sinks(sc, None, None, 4, 9, 18)
    assert got[0][0].tolist() == list(range(18))           # K above the block count: everything


@pytest.mark.parametrize("seed", range(10))
def test_token_sinks_brute_force(seed):
    """Against an independent formulation: the union of the sink tokens with the tokens of the k
    blocks that beat all others (brute force over k-subsets: best score sum, ties to the
    lexicographically smallest subset, distinct integer scores so the order is total)."""
    from oracle.selection import select_token_sinks
    rng = np.random.default_rng(seed)
    n_blk, bt, k = 7, 8, 3
    L = n_blk * bt - int(rng.integers(0, bt))
    sc = rng.permutation(n_blk).astype(np.float32)[None, None, :]
    sinks = rng.choice(L, 3, replace=False)
    best = max(itertools.combinations(range(n_blk), k), key=lambda c: (sum(sc[0, 0, list(c)]), [-i for i in c]))
    want = sorted(set(sinks.tolist()) | {t for blk in best for t in range(blk * bt, min((blk + 1) * bt, L))})
    got = select_token_sinks(sc, sinks[None, :], np.array([3]), bt, k, L)
    assert got[0][0].tolist() == want
