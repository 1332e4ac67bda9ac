"""Pins of pooled-key scoring: integer-valued inputs make every float32 operation exact, so the result
must equal plain integer arithmetic whatever the order; random inputs stay within the float32 bound."""
import math

import numpy as np
import pytest

from oracle.scoring import gather_logical, pool_keys, query_sum, token_scores, unit_scores
from synth.gen import round_to_bf16


def _int_bf16(rng, shape, lo=-2, hi=2):
    ints = rng.integers(lo, hi + 1, size=shape)
    return ints, round_to_bf16(ints.astype(np.float32))


@pytest.mark.parametrize("Hq,Hkv", [(2, 2), (28, 4), (8, 2)])
def test_integer_inputs_exact(Hq, Hkv):
    rng = np.random.default_rng(Hq * 100 + Hkv)
    B, T, D, L, bt = 2, 32, 128, 256, 64
    qi, qb = _int_bf16(rng, (B, Hq, T, D))
    ki, kb = _int_bf16(rng, (B, Hkv, L, D))
    bits = np.array([rng.integers(0, 2 ** 32), rng.integers(0, 2 ** 32)], dtype=np.uint64)
    ks = pool_keys(kb, bt)
    qs = query_sum(qb, bits, Hkv)
    S = unit_scores(qs, ks)
    G = Hq // Hkv
    for b in range(B):
        P = [p for p in range(T) if (int(bits[b]) >> p) & 1]
        for g in range(Hkv):
            qsum = qi[b, g * G:(g + 1) * G][:, P, :].sum(axis=(0, 1))
            assert np.array_equal(qs[b, g], qsum.astype(np.float32))
            for n in range(L // bt):
                ksum = ki[b, g, n * bt:(n + 1) * bt].sum(axis=0)
                assert np.array_equal(ks[b, g, n], ksum.astype(np.float32))
                assert float(S[b, g, n]) == float(int(np.dot(qsum.astype(np.int64), ksum.astype(np.int64))))


def test_partial_last_block_sums_valid_tokens():
    rng = np.random.default_rng(5)
    ki, kb = _int_bf16(rng, (1, 1, 100, 4))
    ks = pool_keys(kb, 64)
    assert ks.shape == (1, 1, 2, 4)
    assert np.array_equal(ks[0, 0, 1], ki[0, 0, 64:].sum(axis=0).astype(np.float32))


def test_scores_within_float32_bound():
    rng = np.random.default_rng(6)
    B, H, T, D, L, bt = 1, 2, 32, 128, 512, 64
    q = round_to_bf16(rng.standard_normal((B, H, T, D)).astype(np.float32))
    k = round_to_bf16(rng.standard_normal((B, H, L, D)).astype(np.float32))
    bits = np.array([0xF0F0F0F0], dtype=np.uint64)
    ks = pool_keys(k, bt)
    qs = query_sum(q, bits, H)
    S = unit_scores(qs, ks)
    u = 2.0 ** -24
    gam = lambda m: m * u / (1 - m * u)
    for g in range(H):
        for n in range(L // bt):
            exact = math.fsum(float(a) * float(b) for a, b in zip(qs[0, g], ks[0, g, n]))
            bound = gam(8) * math.fsum(abs(float(a) * float(b)) for a, b in zip(qs[0, g], ks[0, g, n]))
            assert abs(float(S[0, g, n]) - exact) <= bound


def test_token_scores_match_unit_scores_at_unit_one():
    rng = np.random.default_rng(7)
    k = round_to_bf16(rng.standard_normal((1, 2, 16, 128)).astype(np.float32))
    qs = rng.standard_normal((1, 2, 128)).astype(np.float32)
    assert np.array_equal(token_scores(qs, k), unit_scores(qs, pool_keys(k, 1)))


def test_chunk_tree_is_tree_of_page_trees():
    rng = np.random.default_rng(8)
    k = round_to_bf16(rng.standard_normal((1, 1, 2048, 8)).astype(np.float32))
    pages = pool_keys(k, 64)                     # [1][1][32][8]
    chunk = pool_keys(k, 2048)[0, 0, 0]
    from oracle.fp32tree import tree_sum
    assert np.array_equal(chunk, tree_sum(pages[0, 0], axis=0))


def test_gather_logical_inverts_page_scatter():
    from synth import get_config
    from synth.gen import to_pages
    cfg = get_config(4).with_(batch=2, n_q_heads=2, n_kv_heads=2, ctx_len=512, chunk_tokens=128)
    rng = np.random.default_rng(9)
    X = rng.integers(0, 60000, size=(2, 2, 512, 128)).astype(np.uint16)
    pt = rng.permutation(cfg.n_pages).astype(np.int32).reshape(2, -1)
    pool = to_pages(cfg, X, pt)
    assert np.array_equal(gather_logical(pool, pt, 64), X)
