"""Pins of the per-query (max) scoring reading (oracle/scoring.unit_scores_max)."""
import numpy as np
import pytest

from oracle.scoring import pool_keys, query_sum, unit_scores, unit_scores_max
from synth.gen import round_to_bf16


def _int_bf16(rng, shape, lo=-3, hi=3):
    ints = rng.integers(lo, hi + 1, size=shape)
    return ints, round_to_bf16(ints.astype(np.float32))


@pytest.mark.parametrize("Hq,Hkv", [(2, 2), (8, 2), (28, 4)])
def test_integer_inputs_exact(Hq, Hkv):
    """Integer-valued inputs make every float32 operation exact: the score is the integer maximum."""
    rng = np.random.default_rng(Hq + 10 * Hkv)
    B, T, D, L, bt = 2, 32, 64, 256, 64
    qi, qb = _int_bf16(rng, (B, Hq, T, D))
    ki, kb = _int_bf16(rng, (B, Hkv, L, D))
    bits = np.array([rng.integers(1, 2 ** 32), rng.integers(1, 2 ** 32)], dtype=np.uint64)
    S = unit_scores_max(qb, bits, pool_keys(kb, bt), Hkv)
    G = Hq // Hkv
    kbl = ki.reshape(B, Hkv, L // bt, bt, D).sum(axis=3)
    for b in range(B):
        P = [p for p in range(T) if (int(bits[b]) >> p) & 1]
        for g in range(Hkv):
            want = max(int(qi[b, g * G + j, p] @ kbl[b, g, n]) for j in range(G) for p in P
                       for n in [0])
            cand = np.array([[int(qi[b, g * G + j, p] @ kbl[b, g, n]) for n in range(L // bt)]
                             for j in range(G) for p in P])
            assert np.array_equal(S[b, g], cand.max(axis=0).astype(np.float32)), (b, g)
            assert S[b, g, 0] == want


def test_one_predicted_query_equals_the_summed_reading():
    """With one q-head per KV head and one predicted position, the summed query is that query (the
    tree adds exact zeros), so both readings give the same bits."""
    rng = np.random.default_rng(4)
    B, H, T, D, L = 2, 3, 32, 128, 640
    q = round_to_bf16(rng.standard_normal((B, H, T, D)).astype(np.float32))
    k = round_to_bf16(rng.standard_normal((B, H, L, D)).astype(np.float32))
    bits = np.array([1 << 5, 1 << 31], dtype=np.uint64)
    ks = pool_keys(k, 64)
    a = unit_scores_max(q, bits, ks, H)
    s = unit_scores(query_sum(q, bits, H), ks)
    assert np.array_equal(a.view(np.uint32), (s + np.float32(0)).view(np.uint32))


def test_bounds_and_empty_prediction():
    rng = np.random.default_rng(8)
    B, Hq, Hkv, T, D, L = 1, 4, 2, 16, 32, 320
    q = round_to_bf16(rng.standard_normal((B, Hq, T, D)).astype(np.float32))
    k = round_to_bf16(rng.standard_normal((B, Hkv, L, D)).astype(np.float32))
    ks = pool_keys(k, 32)
    bits = np.array([0b1010000000000101], dtype=np.uint64)
    S = unit_scores_max(q, bits, ks, Hkv)
    # the max is attained by one (head, position) and bounds every other one
    for g in range(Hkv):
        singles = [unit_scores_max(q[:, 2 * g + j:2 * g + j + 1], np.array([1 << p], np.uint64),
                                   ks[:, g:g + 1], 1)[0, 0]
                   for j in range(2) for p in (0, 2, 13, 15)]
        singles = np.stack(singles)
        assert np.all(S[0, g] >= singles.max(axis=0)) and np.all(S[0, g] <= singles.max(axis=0))
    Z = unit_scores_max(q, np.array([0], np.uint64), ks, Hkv)
    assert np.all(Z == 0) and not np.any(np.signbit(Z))
