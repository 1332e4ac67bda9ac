"""Pins of the softmax-mass scoring reading (oracle/scoring.unit_scores_mass)."""
import math

import numpy as np
import pytest

from oracle.scoring import pool_keys, unit_scores_mass, unit_scores_max
from synth.gen import bf16_bits_to_f32, round_to_bf16


def test_closed_form_three_quarters():
    """Two units of 4 tokens with mean keys e1 and e2, D = 2, one query q = [sqrt(2) ln 3, 0]: the
    scaled logits are ln 3 and 0, so the masses are 3/4 and 1/4."""
    D, unit = 2, 4
    k = np.zeros((1, 1, 8, D), np.float32)
    k[0, 0, :4, 0] = 1.0
    k[0, 0, 4:, 1] = 1.0
    q = np.zeros((1, 1, 1, D), np.float32)
    q[0, 0, 0, 0] = math.sqrt(2.0) * math.log(3.0)
    s = unit_scores_mass(q, np.array([1], np.uint64), pool_keys(k, unit), 1, unit, 8)
    assert abs(s[0, 0, 0] - 0.75) < 1e-6 and abs(s[0, 0, 1] - 0.25) < 1e-6   # q is rounded to float32


def _brute(q, bits, ks, Hkv, unit, L):
    """Pure-Python loops: the same definition, one query and one unit at a time."""
    q = bf16_bits_to_f32(q)
    B, Hq, T, D = q.shape
    G = Hq // Hkv
    n = ks.shape[2]
    out = np.zeros((B, Hkv, n))
    for b in range(B):
        for g in range(Hkv):
            for j in range(G):
                for p in range(T):
                    if not (int(bits[b]) >> p) & 1:
                        continue
                    z = []
                    for u in range(n):
                        c = min(unit, L - unit * u)
                        z.append(sum(float(q[b, g * G + j, p, d]) * float(ks[b, g, u, d]) / c
                                     for d in range(D)) / math.sqrt(D))
                    m = max(z)
                    e = [math.exp(x - m) for x in z]
                    tot = sum(e)
                    for u in range(n):
                        out[b, g, u] += e[u] / tot
    return out


@pytest.mark.parametrize("Hq,Hkv,L,unit", [(2, 2, 200, 32), (4, 1, 130, 16), (6, 2, 96, 32)])
def test_brute_force(Hq, Hkv, L, unit):
    rng = np.random.default_rng(L + Hq)
    B, T, D = 2, 6, 8
    q = round_to_bf16(rng.standard_normal((B, Hq, T, D)).astype(np.float32))
    k = round_to_bf16(rng.standard_normal((B, Hkv, L, D)).astype(np.float32))
    bits = np.array([0b101101, 0b000010], np.uint64)
    ks = pool_keys(k, unit)
    got = unit_scores_mass(q, bits, ks, Hkv, unit, L)
    want = _brute(q, bits, ks, Hkv, unit, L)
    assert np.allclose(got, want, rtol=1e-12, atol=1e-14)


def test_mass_conservation_and_empty_prediction():
    """Every predicted query spreads a mass of one over the units: a head's scores sum to
    G * |P|; nothing predicted gives zeros."""
    rng = np.random.default_rng(3)
    B, Hq, Hkv, T, D, L, unit = 3, 8, 2, 32, 64, 1000, 64
    q = round_to_bf16(rng.standard_normal((B, Hq, T, D)).astype(np.float32))
    k = round_to_bf16(rng.standard_normal((B, Hkv, L, D)).astype(np.float32))
    bits = np.array([0xFFFFFFFF, 0x10001, 0], np.uint64)
    s = unit_scores_mass(q, bits, pool_keys(k, unit), Hkv, unit, L)
    for b, npred in enumerate((32, 2, 0)):
        assert np.allclose(s[b].sum(axis=1), 4 * npred, rtol=1e-12, atol=0)
    assert (s[2] == 0).all()


def test_equal_mean_keys_share_the_mass_equally():
    """Units whose mean keys are equal -- here a partial last unit repeating the others' rows --
    receive equal mass, so the mean divides by the valid token count."""
    rng = np.random.default_rng(5)
    D, unit, n_full = 16, 8, 5
    row = round_to_bf16(rng.standard_normal(D).astype(np.float32))
    L = n_full * unit + 3
    k = np.broadcast_to(row, (1, 1, L, D)).copy()
    q = round_to_bf16(rng.standard_normal((1, 1, 4, D)).astype(np.float32))
    s = unit_scores_mass(q, np.array([0b1011], np.uint64), pool_keys(k, unit), 1, unit, L)
    assert np.allclose(s[0, 0], 3.0 / (n_full + 1), rtol=1e-12)


def test_single_query_ranks_like_the_max_reading():
    """One predicted query per KV head and full units: the softmax is monotone in the logit, and the
    logit is the key-sum dot product over a common positive scale, so the mass ranking is the
    per-query (max) reading's ranking."""
    rng = np.random.default_rng(9)
    B, H, T, D, L, unit = 2, 3, 32, 64, 64 * 40, 64
    q = round_to_bf16(rng.standard_normal((B, H, T, D)).astype(np.float32))
    k = round_to_bf16(rng.standard_normal((B, H, L, D)).astype(np.float32))
    bits = np.array([1 << 7, 1 << 30], np.uint64)
    ks = pool_keys(k, unit)
    mass = unit_scores_mass(q, bits, ks, H, unit, L)
    mx = unit_scores_max(q, bits, ks, H)
    for b in range(B):
        for g in range(H):
            assert np.argsort(-mass[b, g], kind="stable").tolist() == np.argsort(-mx[b, g].astype(np.float64),
                                                                                   kind="stable").tolist()
