"""Pins of the cache write and the pooled keys it leaves (oracle/cache.py)."""
import numpy as np
import pytest

from oracle.cache import touched_units, write_and_pool, write_paged, write_rows
from oracle.scoring import gather_logical, pool_keys
from synth.gen import round_to_bf16


def _bf16(rng, shape):
    return round_to_bf16(rng.standard_normal(shape).astype(np.float32))


@pytest.mark.parametrize("t0,n", [(0, 300), (5, 1), (64, 64), (100, 77), (299, 1)])
def test_write_replaces_exactly_the_range(t0, n):
    rng = np.random.default_rng(t0 + 7 * n)
    B, H, L, D = 2, 3, 300, 8
    old, new = _bf16(rng, (B, H, L, D)), _bf16(rng, (B, H, n, D))
    out = write_rows(old, new, t0)
    assert np.array_equal(out[:, :, t0:t0 + n], new)
    assert np.array_equal(out[:, :, :t0], old[:, :, :t0])
    assert np.array_equal(out[:, :, t0 + n:], old[:, :, t0 + n:])


def test_touched_units_brute_force():
    for unit in (1, 16, 64):
        for t0 in range(0, 200, 7):
            for n in (1, 5, 64, 130):
                want = sorted({(t0 + i) // unit for i in range(n)})
                assert list(touched_units(t0, n, unit)) == want


@pytest.mark.parametrize("unit", [16, 64, 256])
def test_pooled_keys_after_a_write(unit):
    """Touched units equal the pooling of the updated cache; the others keep their old (here
    deliberately stale) values; a full write equals pooling the new rows."""
    rng = np.random.default_rng(unit)
    B, H, L, D = 2, 2, 700, 16
    k, v = _bf16(rng, (B, H, L, D)), _bf16(rng, (B, H, L, D))
    n_units = -(-L // unit)
    stale = rng.standard_normal((B, H, n_units, D)).astype(np.float32)
    t0, n = 130, 200
    kn, vn = _bf16(rng, (B, H, n, D)), _bf16(rng, (B, H, n, D))
    k2, v2, ks = write_and_pool(k, v, kn, vn, t0, unit, stale)
    fresh = pool_keys(k2, unit)
    touched = set(touched_units(t0, n, unit))
    for u in range(n_units):
        want = fresh[:, :, u] if u in touched else stale[:, :, u]
        assert np.array_equal(ks[:, :, u].view(np.uint32), want.view(np.uint32)), u
    assert np.array_equal(v2[:, :, t0:t0 + n], vn)
    # a full write of the whole cache: the pooled keys of the new rows alone
    kf, vf = _bf16(rng, (B, H, L, D)), _bf16(rng, (B, H, L, D))
    _, _, ks_full = write_and_pool(k, v, kf, vf, 0, unit, stale)
    assert np.array_equal(ks_full.view(np.uint32), pool_keys(kf, unit).view(np.uint32))


def test_rewriting_the_same_rows_changes_nothing():
    rng = np.random.default_rng(3)
    B, H, L, D = 1, 2, 256, 8
    k, v = _bf16(rng, (B, H, L, D)), _bf16(rng, (B, H, L, D))
    ks = pool_keys(k, 64)
    k2, v2, ks2 = write_and_pool(k, v, k[:, :, 40:170], v[:, :, 40:170], 40, 64, ks)
    assert np.array_equal(k2, k) and np.array_equal(v2, v)
    assert np.array_equal(ks2.view(np.uint32), ks.view(np.uint32))


def test_paged_write_matches_the_logical_write():
    rng = np.random.default_rng(11)
    B, H, P, npp, D = 2, 2, 16, 6, 8
    n_pages = B * npp
    pool = _bf16(rng, (n_pages, H, P, D))
    pt = rng.permutation(n_pages).astype(np.int32).reshape(B, npp)
    t0, n = 21, 50
    new = _bf16(rng, (B, H, n, D))
    pool2 = write_paged(pool, pt, P, new, t0)
    logical = write_rows(gather_logical(pool, pt, P), new, t0)
    assert np.array_equal(gather_logical(pool2, pt, P), logical)
