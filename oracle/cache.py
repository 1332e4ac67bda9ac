"""Writing new rows into the KV cache, and the pooled keys of the units the write touches.

Focus-dLLM (abstract; Elamur "Summary"): the cache of the context is built once and reused across
denoising steps, and the block scoring ranks its units by their pooled keys.  Prefilling-dLLM
(abstract): the chunk KV sits non-contiguously in a paged cache.  The pages describe no cache-write
procedure; the reading taken here is the plainest one: a write replaces the logical rows [t0, t0 + n)
of every (sequence, KV head) with the new rows, bit for bit, and every unit that holds a written row
gets the pooled key (``scoring.pool_keys``) of the updated cache; units without a written row keep
their pooled keys unchanged.
"""
from __future__ import annotations

import numpy as np

from .scoring import pool_keys


def write_rows(cache, new, t0: int) -> np.ndarray:
    """cache [B][Hkv][L][D], new [B][Hkv][n][D] -> copy of cache with rows [t0, t0 + n) = new."""
    out = np.array(cache, copy=True)
    n = np.asarray(new).shape[2]
    assert 0 <= t0 and t0 + n <= out.shape[2]
    out[:, :, t0:t0 + n] = new
    return out


def write_paged(pool, page_table, page_tokens: int, new, t0: int) -> np.ndarray:
    """Paged pool [n_pages][Hkv][P][D] -> copy with logical rows [t0, t0 + n) of sequence b (pages
    page_table[b]) replaced by new[b]; every row goes to its own page, row by row."""
    out = np.array(pool, copy=True)
    pt = np.asarray(page_table)
    new = np.asarray(new)
    B, H, n, _ = new.shape
    for b in range(B):
        for i in range(n):
            t = t0 + i
            out[pt[b, t // page_tokens], :, t % page_tokens] = new[b, :, i]
    return out


def touched_units(t0: int, n: int, unit: int) -> range:
    """Units holding at least one of the rows [t0, t0 + n)."""
    return range(t0 // unit, (t0 + n - 1) // unit + 1)


def write_and_pool(k_cache, v_cache, k_new, v_new, t0: int, unit: int, ks_old):
    """The write on a contiguous cache plus the pooled keys it leaves: returns (k, v, ks)."""
    k = write_rows(k_cache, k_new, t0)
    v = write_rows(v_cache, v_new, t0)
    ks = np.array(ks_old, dtype=np.float32, copy=True)
    fresh = pool_keys(k, unit)
    for u in touched_units(t0, np.asarray(k_new).shape[2], unit):
        ks[:, :, u] = fresh[:, :, u]
    return k, v, ks
