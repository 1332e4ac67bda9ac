"""fdl_cache_write against the oracle's cache write (oracle/cache.py): the cache rows and the pooled
keys of the touched units bit for bit, the other units untouched."""
import numpy as np
import pytest
import torch

from gpu_util import dev, host, require_gpu
from oracle.cache import touched_units, write_and_pool, write_paged
from oracle.scoring import gather_logical, pool_keys
from synth import get_config
from synth.gen import round_to_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def h():
    require_gpu()
    from diffusion_long_context_amd import Handle
    hh = Handle(workspace_bytes=256 << 20)
    yield hh
    hh.close()


def _vals(rng, shape, f32):
    x = rng.standard_normal(shape).astype(np.float32)
    return x if f32 else round_to_bf16(x)


def _bits(a):
    return a.view(np.uint32) if a.dtype == np.float32 else a


@pytest.mark.parametrize("kw,t0,n,unit", [
    (dict(ctx_len=5000), 0, 5000, 64),                     # a full refresh, ragged last block
    (dict(ctx_len=5000), 100, 77, 64),                     # inside two blocks
    (dict(ctx_len=5000), 4990, 10, 64),                    # the ragged tail
    (dict(ctx_len=4096, head_dim=64), 1000, 900, 32),      # head_dim 64, 32-token units
    (dict(ctx_len=4096), 1500, 300, 2048),                 # chunk units: sub-sums and merge
    (dict(ctx_len=4096), 1500, 300, 16),
], ids=["full", "partial", "tail", "d64-u32", "chunks", "u16"])
def test_cache_write_contiguous(h, kw, t0, n, unit):
    from diffusion_long_context_amd.step import geom_for
    cfg = get_config(1).with_(batch=2, n_q_heads=4, n_kv_heads=4, **kw)
    g = geom_for(cfg)
    rng = np.random.default_rng(t0 + n + unit)
    B, H, L, D = cfg.batch, cfg.n_kv_heads, cfg.ctx_len, cfg.head_dim
    k, v = _vals(rng, (B, H, L, D), False), _vals(rng, (B, H, L, D), False)
    kn, vn = _vals(rng, (B, H, n, D), False), _vals(rng, (B, H, n, D), False)
    n_units = -(-L // unit)
    stale = rng.standard_normal((B, H, n_units, D)).astype(np.float32)
    kc, vc, ks = dev(k), dev(v), dev(stale)
    h.fdl_cache_write(g, dev(kn), dev(vn), t0, kc, vc, None, unit, ks)
    torch.cuda.synchronize()
    assert h.fdl_get_status() == 0
    wk, wv, wks = write_and_pool(k, v, kn, vn, t0, unit, stale)
    assert np.array_equal(host(kc).view(np.uint16), wk)
    assert np.array_equal(host(vc).view(np.uint16), wv)
    assert np.array_equal(host(ks).view(np.uint32), wks.view(np.uint32))


def test_cache_write_without_pooling(h):
    from diffusion_long_context_amd.step import geom_for
    cfg = get_config(1).with_(batch=1, n_q_heads=2, n_kv_heads=2, ctx_len=3000)
    g = geom_for(cfg)
    rng = np.random.default_rng(5)
    k, v = _vals(rng, (1, 2, 3000, 128), False), _vals(rng, (1, 2, 3000, 128), False)
    kn, vn = _vals(rng, (1, 2, 700, 128), False), _vals(rng, (1, 2, 700, 128), False)
    kc, vc = dev(k), dev(v)
    h.fdl_cache_write(g, dev(kn), dev(vn), 1234, kc, vc, None, 64, None)
    torch.cuda.synchronize()
    assert h.fdl_get_status() == 0
    wk, wv, _ = write_and_pool(k, v, kn, vn, 1234, 64, np.zeros((1, 2, 47, 128), np.float32))
    assert np.array_equal(host(kc).view(np.uint16), wk)
    assert np.array_equal(host(vc).view(np.uint16), wv)


@pytest.mark.parametrize("t0,n,unit", [(0, 4096, 512), (700, 300, 512), (640, 64, 64)],
                         ids=["full-chunks", "partial-chunks", "one-page-block"])
def test_cache_write_paged(h, t0, n, unit):
    """Paged pool with shuffled pages: the logical cache after the write and the chunk (or block)
    sums."""
    from diffusion_long_context_amd.step import geom_for
    cfg = get_config(4).with_(batch=2, n_q_heads=4, n_kv_heads=4, ctx_len=4096, chunk_tokens=512)
    g = geom_for(cfg)
    rng = np.random.default_rng(t0 + n)
    P, npp, n_pages = cfg.page_tokens, cfg.pages_per_seq, cfg.n_pages
    B, H, D, L = cfg.batch, cfg.n_kv_heads, cfg.head_dim, cfg.ctx_len
    kp, vp = _vals(rng, (n_pages, H, P, D), False), _vals(rng, (n_pages, H, P, D), False)
    pt = rng.permutation(n_pages).astype(np.int32).reshape(B, npp)
    kn, vn = _vals(rng, (B, H, n, D), False), _vals(rng, (B, H, n, D), False)
    n_units = L // unit
    stale = rng.standard_normal((B, H, n_units, D)).astype(np.float32)
    kc, vc, ks = dev(kp), dev(vp), dev(stale)
    h.fdl_cache_write(g, dev(kn), dev(vn), t0, kc, vc, dev(pt), unit, ks)
    torch.cuda.synchronize()
    assert h.fdl_get_status() == 0
    want_k = write_paged(kp, pt, P, kn, t0)
    want_v = write_paged(vp, pt, P, vn, t0)
    assert np.array_equal(host(kc).view(np.uint16), want_k)
    assert np.array_equal(host(vc).view(np.uint16), want_v)
    fresh = pool_keys(gather_logical(want_k, pt, P), unit)
    touched = set(touched_units(t0, n, unit))
    got = host(ks)
    for u in range(n_units):
        want = fresh[:, :, u] if u in touched else stale[:, :, u]
        assert np.array_equal(got[:, :, u].view(np.uint32), want.view(np.uint32)), u


def test_cache_write_float32(h):
    from diffusion_long_context_amd.step import geom_for
    cfg = get_config(0)
    g = geom_for(cfg)
    rng = np.random.default_rng(9)
    B, H, L, D = cfg.batch, cfg.n_kv_heads, cfg.ctx_len, cfg.head_dim
    k, v = _vals(rng, (B, H, L, D), True), _vals(rng, (B, H, L, D), True)
    kn, vn = _vals(rng, (B, H, 100, D), True), _vals(rng, (B, H, 100, D), True)
    unit = cfg.kv_block
    stale = rng.standard_normal((B, H, -(-L // unit), D)).astype(np.float32)
    kc, vc, ks = dev(k), dev(v), dev(stale)
    h.fdl_cache_write(g, dev(kn), dev(vn), 250, kc, vc, None, unit, ks)
    torch.cuda.synchronize()
    assert h.fdl_get_status() == 0
    wk, wv, wks = write_and_pool(k, v, kn, vn, 250, unit, stale)
    assert np.array_equal(_bits(host(kc)), _bits(wk))
    assert np.array_equal(_bits(host(vc)), _bits(wv))
    assert np.array_equal(host(ks).view(np.uint32), wks.view(np.uint32))


@pytest.mark.parametrize("unit", [64, 512], ids=["block-units", "chunk-units"])
def test_cache_write_bad_page(h, unit):
    """One page-table entry out of range inside the written rows: those rows are written nowhere
    (every page of the pool other than the rows the valid entries own is bit-identical afterwards,
    page 0 included), they count +0 in the pooled keys, and FDL_EINDEX is reported.  fdl_pool_keys
    over the same table pools those rows as +0 too."""
    from diffusion_long_context_amd.fdllm import FDL_EINDEX
    from diffusion_long_context_amd.step import geom_for
    cfg = get_config(4).with_(batch=2, n_q_heads=4, n_kv_heads=4, ctx_len=4096, chunk_tokens=512)
    g = geom_for(cfg)
    rng = np.random.default_rng(77 + unit)
    P, npp, n_pages = cfg.page_tokens, cfg.pages_per_seq, cfg.n_pages
    B, H, D, L = cfg.batch, cfg.n_kv_heads, cfg.head_dim, cfg.ctx_len
    kp, vp = _vals(rng, (n_pages, H, P, D), False), _vals(rng, (n_pages, H, P, D), False)
    pt = rng.permutation(n_pages).astype(np.int32).reshape(B, npp)
    t0, n = 900, 1500                       # logical pages 14 .. 37 of each sequence
    bad_b, bad_j = 1, 20
    orphan = int(pt[bad_b, bad_j])
    pt[bad_b, bad_j] = n_pages + 5
    kn, vn = _vals(rng, (B, H, n, D), False), _vals(rng, (B, H, n, D), False)
    n_units = L // unit
    stale = rng.standard_normal((B, H, n_units, D)).astype(np.float32)
    kc, vc, ks = dev(kp), dev(vp), dev(stale)
    h.fdl_cache_write(g, dev(kn), dev(vn), t0, kc, vc, dev(pt), unit, ks)
    torch.cuda.synchronize()
    assert h.fdl_get_status() == FDL_EINDEX
    # the expected pool: the bad entry redirected to an extra page that is dropped afterwards
    pt_ext = pt.copy()
    pt_ext[bad_b, bad_j] = n_pages
    zero_page = np.zeros((1, H, P, D), np.uint16)
    want_k = write_paged(np.concatenate([kp, zero_page]), pt_ext, P, kn, t0)
    want_v = write_paged(np.concatenate([vp, zero_page]), pt_ext, P, vn, t0)
    got_k, got_v = host(kc).view(np.uint16), host(vc).view(np.uint16)
    assert np.array_equal(got_k, want_k[:n_pages]) and np.array_equal(got_v, want_v[:n_pages])
    assert np.array_equal(got_k[orphan], kp[orphan]) and np.array_equal(got_k[0], want_k[0])
    want_k[n_pages] = 0                     # a row without a page has no key
    fresh = pool_keys(gather_logical(want_k, pt_ext, P), unit)
    touched = set(touched_units(t0, n, unit))
    got = host(ks)
    for u in range(n_units):
        want = fresh[:, :, u] if u in touched else stale[:, :, u]
        assert np.array_equal(got[:, :, u].view(np.uint32), want.view(np.uint32)), u
    # the pooling call on the same table
    ks2 = dev(np.zeros((B, H, n_units, D), np.float32))
    h.fdl_pool_keys(g, kc, dev(pt), unit, ks2)
    torch.cuda.synchronize()
    assert h.fdl_get_status() == FDL_EINDEX
    assert np.array_equal(host(ks2).view(np.uint32), fresh.view(np.uint32))
