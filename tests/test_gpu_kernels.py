"""Per-call GPU parity against the CPU oracle on small and medium inputs.

Indices (predicted positions, pooled keys, scores, selections, sinks) must match bit for bit;
attention outputs must satisfy |o - r| <= 1e-2 + 2e-2 |r| against the float64 oracle computed on
the same bf16 / float32 inputs."""
import numpy as np
import pytest
import torch

from gpu_util import assert_close, dev, host, out_buffer, out_to_f64, require_gpu
from oracle.attention import attend, blocks_to_tokens
from oracle.pipeline import focus_layer_step
from oracle.predictor import predict_positions
from oracle.scoring import pool_keys, query_sum, unit_scores, unit_scores_mass, unit_scores_max
from oracle.selection import select_blocks
from synth import get_config
from synth.gen import make_single

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def h():
    require_gpu()
    from diffusion_long_context_amd import Handle
    hh = Handle(workspace_bytes=256 << 20)
    yield hh
    hh.close()


def _geom(cfg):
    from diffusion_long_context_amd.step import geom_for
    return geom_for(cfg)


def _u64(bits):
    return np.asarray(bits, dtype=np.uint64)


# ---------------------------------------------------------------------------------------------
# predictor
# ---------------------------------------------------------------------------------------------

def _gpu_predict(h, prev_conf, masked, k, w):
    B, T = masked.shape
    pm = torch.zeros(B, dtype=torch.int64, device="cuda")
    npred = torch.zeros(B, dtype=torch.int32, device="cuda")
    h.fdl_predict_queries(B, T, None if prev_conf is None else dev(prev_conf), dev(masked), k, w, pm, npred)
    torch.cuda.synchronize()
    return host(pm).view(np.uint64), host(npred)


@pytest.mark.parametrize("seed", range(6))
def test_predict_random(h, seed):
    rng = np.random.default_rng(seed)
    for T in (1, 7, 32, 33, 64):
        B = 5
        conf = rng.choice([0.1, 0.5, 0.5, 0.9, np.nan, -0.0, 0.0, 0.3], size=(B, T)).astype(np.float32)
        masked = (rng.random((B, T)) < 0.5).astype(np.uint8)
        for k, w in [(0, 0), (1, 0), (4, 2), (4, 4), (100, 70)]:
            got = _gpu_predict(h, conf, masked, k, w)
            want = predict_positions(conf, masked, k, w)
            assert np.array_equal(got[0], _u64(want[0])), (T, k, w)
            assert np.array_equal(got[1], want[1])


def test_predict_edge_cases(h):
    T = 32
    masked = np.ones((2, T), np.uint8)
    got = _gpu_predict(h, None, masked, 4, 4)
    assert all(int(v) == (1 << 32) - 1 for v in got[0])
    got = _gpu_predict(h, np.ones((2, T), np.float32), np.zeros((2, T), np.uint8), 4, 4)
    assert list(got[0]) == [0, 0] and list(got[1]) == [0, 0]


@pytest.mark.parametrize("ci", [0, 1, 2, 4])
def test_predict_workloads(h, ci):
    from synth.gen import decode_state
    cfg = get_config(ci)
    d = decode_state(cfg)
    got = _gpu_predict(h, d["prev_conf"], d["masked"], cfg.top_k_pos, cfg.window)
    want = predict_positions(d["prev_conf"], d["masked"], cfg.top_k_pos, cfg.window)
    assert np.array_equal(got[0], _u64(want[0])) and np.array_equal(got[1], want[1])


# ---------------------------------------------------------------------------------------------
# pooled keys and scores
# ---------------------------------------------------------------------------------------------

def _small_bf16(**kw):
    return get_config(1).with_(**kw)


@pytest.mark.parametrize("cfg", [
    get_config(0),
    _small_bf16(n_q_heads=4, n_kv_heads=4, ctx_len=1000, kv_block=64),       # ragged last block
    _small_bf16(n_q_heads=4, n_kv_heads=2, ctx_len=777, kv_block=16, head_dim=64),
    _small_bf16(n_q_heads=2, n_kv_heads=2, ctx_len=4096, kv_block=2048),     # chunk-sized units
    _small_bf16(n_q_heads=2, n_kv_heads=2, ctx_len=5000, kv_block=1024),     # ragged last chunk
], ids=["tiny", "ragged", "d64", "chunk", "chunk-ragged"])
def test_pool_and_scores_bit_exact(h, cfg):
    x = make_single(cfg)
    g = _geom(cfg)
    n_units = -(-cfg.ctx_len // cfg.kv_block)
    ks = torch.zeros(cfg.batch, cfg.n_kv_heads, n_units, cfg.head_dim, dtype=torch.float32, device="cuda")
    h.fdl_pool_keys(g, dev(x["k"]), None, cfg.kv_block, ks)
    want_ks = pool_keys(x["k"], cfg.kv_block)
    bits, _ = predict_positions(x["prev_conf"], x["masked"], cfg.top_k_pos, cfg.window)
    pm = dev(_u64(bits))
    sc = torch.zeros(cfg.batch, cfg.n_kv_heads, n_units, dtype=torch.float32, device="cuda")
    h.fdl_score_blocks(g, dev(x["q"]), pm, ks, cfg.kv_block, sc)
    torch.cuda.synchronize()
    assert np.array_equal(host(ks).view(np.uint32), want_ks.view(np.uint32))
    want_sc = unit_scores(query_sum(x["q"], bits, cfg.n_kv_heads), want_ks)
    assert np.array_equal(host(sc).view(np.uint32), want_sc.view(np.uint32))


def test_pool_chunks_one_pass_fallback():
    """With too little workspace for the sub-unit sums, chunk pooling runs in one pass: same bits."""
    require_gpu()
    from diffusion_long_context_amd import Handle
    # sub-unit sums: 8 heads x 313 runs x 512 B = 1.28 MB > the 1 MiB of scratch of the smallest workspace
    cfg = _small_bf16(n_q_heads=8, n_kv_heads=8, ctx_len=20000, kv_block=2048)
    x = make_single(cfg)
    hs = Handle(workspace_bytes=2 << 20)
    try:
        ks = torch.zeros(cfg.batch, cfg.n_kv_heads, 10, cfg.head_dim, dtype=torch.float32, device="cuda")
        hs.fdl_pool_keys(_geom(cfg), dev(x["k"]), None, cfg.kv_block, ks)
        torch.cuda.synchronize()
        assert hs.fdl_get_status() == 0
        assert np.array_equal(host(ks).view(np.uint32), pool_keys(x["k"], cfg.kv_block).view(np.uint32))
    finally:
        hs.close()


@pytest.mark.parametrize("kw,bits", [
    (dict(n_q_heads=4, n_kv_heads=4, ctx_len=3000), None),
    (dict(n_q_heads=28, n_kv_heads=4, ctx_len=4096), None),
    (dict(n_q_heads=8, n_kv_heads=2, ctx_len=2000, head_dim=64, dec_len=20), None),
    (dict(n_q_heads=4, n_kv_heads=2, ctx_len=1000), [0]),
    (dict(n_q_heads=4, n_kv_heads=1, ctx_len=1000), [(1 << 32) - 1]),
], ids=["mha", "gqa7", "gqa4-d64-T20", "nothing-predicted", "all-predicted"])
def test_scores_max_bit_exact(h, kw, bits):
    """Per-query (max) scores against the oracle, bit for bit, and the selection they lead to."""
    cfg = _small_bf16(**kw)
    x = make_single(cfg)
    g = _geom(cfg)
    if bits is None:
        bits, _ = predict_positions(x["prev_conf"], x["masked"], cfg.top_k_pos, cfg.window)
    bits = _u64(bits)
    n_units = -(-cfg.ctx_len // 64)
    ks = torch.zeros(cfg.batch, cfg.n_kv_heads, n_units, cfg.head_dim, dtype=torch.float32, device="cuda")
    h.fdl_pool_keys(g, dev(x["k"]), None, 64, ks)
    sc = torch.zeros(cfg.batch, cfg.n_kv_heads, n_units, dtype=torch.float32, device="cuda")
    h.fdl_score_blocks_max(g, dev(x["q"]), dev(bits), ks, 64, sc)
    torch.cuda.synchronize()
    assert h.fdl_get_status() == 0
    want = unit_scores_max(x["q"], bits, pool_keys(x["k"], 64), cfg.n_kv_heads)
    assert np.array_equal(host(sc).view(np.uint32), want.view(np.uint32))
    k = min(8, n_units)
    sel = torch.zeros(cfg.batch, cfg.n_kv_heads, k, dtype=torch.int32, device="cuda")
    nsel = torch.zeros(cfg.batch, cfg.n_kv_heads, dtype=torch.int32, device="cuda")
    h.fdl_select_blocks(g, sc, n_units, 64, None, None, 1, k, k, sel, nsel)
    torch.cuda.synchronize()
    ws = select_blocks(want, np.full((cfg.batch, 1), -1, np.int32), np.zeros(cfg.batch, np.int32), 64, k)
    for b in range(cfg.batch):
        for gg in range(cfg.n_kv_heads):
            assert host(sel)[b, gg, :host(nsel)[b, gg]].tolist() == ws[b][gg].tolist()


@pytest.mark.parametrize("kw,bits", [
    (dict(n_q_heads=4, n_kv_heads=4, ctx_len=3000), None),
    (dict(n_q_heads=28, n_kv_heads=4, ctx_len=4096), None),
    (dict(n_q_heads=8, n_kv_heads=2, ctx_len=2000, head_dim=64, dec_len=20), None),
    (dict(n_q_heads=4, n_kv_heads=2, ctx_len=1000), [0]),
    (dict(n_q_heads=4, n_kv_heads=1, ctx_len=1000), [(1 << 32) - 1]),
    (dict(n_q_heads=2, n_kv_heads=2, ctx_len=32768), None),
], ids=["mha", "gqa7", "gqa4-d64-T20", "nothing-predicted", "all-predicted", "32k"])
def test_scores_mass(h, kw, bits):
    """Softmax-mass scores against the float64 oracle.  float32 logits of 64- and 128-term dot
    products carry a relative error of a few 1e-6 of the logit's terms, which moves each
    probability by about as much relatively: |gpu - oracle| <= 1e-4 |oracle| + 1e-6.  The selection
    made from the GPU scores is a valid top-k of the oracle's (no unselected unit beats a selected
    one by more than that tolerance) and equals the oracle's own where its k-th and (k+1)-th scores
    are further apart."""
    cfg = _small_bf16(**kw)
    x = make_single(cfg)
    g = _geom(cfg)
    if bits is None:
        bits, _ = predict_positions(x["prev_conf"], x["masked"], cfg.top_k_pos, cfg.window)
    bits = _u64(bits)
    n_units = -(-cfg.ctx_len // 64)
    ks = torch.zeros(cfg.batch, cfg.n_kv_heads, n_units, cfg.head_dim, dtype=torch.float32, device="cuda")
    h.fdl_pool_keys(g, dev(x["k"]), None, 64, ks)
    sc = torch.full((cfg.batch, cfg.n_kv_heads, n_units), 7.0, dtype=torch.float32, device="cuda")
    h.fdl_score_blocks_mass(g, dev(x["q"]), dev(bits), ks, 64, sc)
    torch.cuda.synchronize()
    assert h.fdl_get_status() == 0
    want = unit_scores_mass(x["q"], bits, pool_keys(x["k"], 64), cfg.n_kv_heads, 64, cfg.ctx_len)
    got = host(sc).astype(np.float64)
    err = np.abs(got - want) - (1e-4 * np.abs(want) + 1e-6)
    assert err.max() <= 0, float(err.max())
    G = cfg.n_q_heads // cfg.n_kv_heads
    for b in range(cfg.batch):
        npred = bin(int(bits[b])).count("1")
        assert np.allclose(got[b].sum(axis=1), G * npred, rtol=1e-4, atol=1e-6)
    k = min(8, n_units)
    sel = torch.zeros(cfg.batch, cfg.n_kv_heads, k, dtype=torch.int32, device="cuda")
    nsel = torch.zeros(cfg.batch, cfg.n_kv_heads, dtype=torch.int32, device="cuda")
    h.fdl_select_blocks(g, sc, n_units, 64, None, None, 1, k, k, sel, nsel)
    torch.cuda.synchronize()
    ws = select_blocks(want.astype(np.float32), np.full((cfg.batch, 1), -1, np.int32),
                       np.zeros(cfg.batch, np.int32), 64, k)
    for b in range(cfg.batch):
        for gg in range(cfg.n_kv_heads):
            chosen = host(sel)[b, gg, :host(nsel)[b, gg]].tolist()
            assert len(chosen) == k and chosen == sorted(set(chosen))
            w = want[b, gg]
            tol = 2e-4 * np.abs(w).max() + 2e-6
            rest = np.delete(w, chosen)
            assert rest.size == 0 or w[chosen].min() >= rest.max() - tol, (b, gg)
            srt = np.sort(w)[::-1]
            if k < n_units and srt[k - 1] - srt[k] > tol:
                assert chosen == ws[b][gg].tolist(), (b, gg)


@pytest.mark.parametrize("Hkv,n,k,sinks", [(1, 16, 4, False), (3, 100, 10, True), (8, 700, 40, True),
                                           (32, 16, 4, False), (5, 3000, 64, True)],
                         ids=["h1", "h3-sinks", "h8-sinks-700", "h32", "h5-radix"])
def test_select_shared_bit_exact(h, Hkv, n, k, sinks):
    """One selection per sequence from the scores summed over the KV heads: every head's row equals
    the oracle's selection on the pinned head sum (ties, signed zeros and NaN included)."""
    from oracle.fp32tree import tree_sum
    from diffusion_long_context_amd.step import geom_for
    rng = np.random.default_rng(Hkv * 1000 + n)
    B = 3
    cfg = _small_bf16(batch=B, n_q_heads=Hkv, n_kv_heads=Hkv, ctx_len=n * 64)
    g = geom_for(cfg)
    pool = np.array([0.5, -0.0, 0.0, np.nan, 1.0, -1.0], np.float32)
    sc = np.where(rng.random((B, Hkv, n)) < 0.3, rng.choice(pool, (B, Hkv, n)),
                  rng.standard_normal((B, Hkv, n)).astype(np.float32)).astype(np.float32)
    sc[0, :, : n // 2] = 0.25        # exact ties across a whole half
    max_sinks = 4
    sp = np.full((B, max_sinks), -1, np.int32)
    ns = np.zeros(B, np.int32)
    if sinks:
        for b in range(B):
            pos = sorted(rng.choice(n * 64, 3, replace=False).tolist())
            sp[b, :3], ns[b] = pos, 3
    max_sel = max_sinks + k
    sel = torch.full((B, Hkv, max_sel), -7, dtype=torch.int32, device="cuda")
    nsel = torch.zeros((B, Hkv), dtype=torch.int32, device="cuda")
    h.fdl_select_blocks_shared(g, dev(sc), n, 64, dev(sp) if sinks else None, dev(ns) if sinks else None,
                               max_sinks, k, max_sel, sel, nsel)
    torch.cuda.synchronize()
    assert h.fdl_get_status() == 0
    seq = tree_sum(sc, axis=1)[:, None, :]
    want = select_blocks(seq, sp if sinks else None, ns, 64, k)
    for b in range(B):
        w = want[b][0].tolist()
        for gg in range(Hkv):
            assert int(host(nsel)[b, gg]) == len(w)
            assert host(sel)[b, gg, :len(w)].tolist() == w, (b, gg)


def test_scores_all_positions_predicted(h):
    cfg = _small_bf16(n_q_heads=8, n_kv_heads=1, ctx_len=640, dec_len=20)
    x = make_single(cfg)
    g = _geom(cfg)
    ks = torch.zeros(1, 1, 10, 128, dtype=torch.float32, device="cuda")
    h.fdl_pool_keys(g, dev(x["k"]), None, 64, ks)
    bits = _u64([(1 << 20) - 1])
    sc = torch.zeros(1, 1, 10, dtype=torch.float32, device="cuda")
    h.fdl_score_blocks(g, dev(x["q"]), dev(bits), ks, 64, sc)
    torch.cuda.synchronize()
    want = unit_scores(query_sum(x["q"], bits, 1), pool_keys(x["k"], 64))
    assert np.array_equal(host(sc).view(np.uint32), want.view(np.uint32))


# ---------------------------------------------------------------------------------------------
# selection on crafted scores (ties, -0/+0, NaN, forced sinks)
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("seed,n", [(0, 300), (1, 300), (2, 300), (3, 300), (4, 200), (5, 200), (6, 2000)])
def test_select_crafted(h, seed, n):
    """n <= 256 with K <= 64 takes the sort-and-threshold form, the rest the radix select."""
    rng = np.random.default_rng(seed)
    B, Hkv = 2, 3
    cfg = _small_bf16(batch=B, n_q_heads=Hkv, n_kv_heads=Hkv, ctx_len=n * 64)
    g = _geom(cfg)
    scores = rng.choice([1.0, 2.0, -0.0, 0.0, np.nan, -np.inf, 3.5, 1e-40, -1e-40], size=(B, Hkv, n))
    scores = scores.astype(np.float32)
    scores[0, 0] = rng.standard_normal(n).astype(np.float32)
    max_sinks = 8
    sink_pos = np.full((B, max_sinks), -1, np.int32)
    sink_pos[0, :3] = [0, 70, 71]
    sink_pos[1, :1] = [64 * (n - 1) + 5]
    n_sinks = np.array([3, 1], np.int32)
    for k in (0, 1, 17, 64, n - 3, n - 1, 500):
        max_sel = min(n, max_sinks + k)
        sel = torch.zeros(B, Hkv, max_sel, dtype=torch.int32, device="cuda")
        nsel = torch.zeros(B, Hkv, dtype=torch.int32, device="cuda")
        h.fdl_select_blocks(g, dev(scores), n, 64, dev(sink_pos), dev(n_sinks), max_sinks, k, max_sel,
                            sel, nsel)
        torch.cuda.synchronize()
        want = select_blocks(scores, sink_pos, n_sinks, 64, k)
        s, c = host(sel), host(nsel)
        for b in range(B):
            for gg in range(Hkv):
                assert c[b, gg] == len(want[b][gg]), (k, b, gg)
                assert s[b, gg, : c[b, gg]].tolist() == want[b][gg].tolist(), (k, b, gg)


# ---------------------------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("cfg", [
    get_config(0),
    _small_bf16(n_q_heads=4, n_kv_heads=4, ctx_len=1000),
    _small_bf16(n_q_heads=8, n_kv_heads=4, ctx_len=1500, head_dim=64),
    _small_bf16(n_q_heads=7, n_kv_heads=1, ctx_len=2000, dec_len=20),
    _small_bf16(batch=2, n_q_heads=8, n_kv_heads=1, ctx_len=300, dec_len=32),
    _small_bf16(n_q_heads=2, n_kv_heads=2, ctx_len=0),
], ids=["tiny", "mha-ragged", "gqa2-d64", "gqa7-T20", "gqa8-b2", "empty-ctx"])
def test_dense_attention(h, cfg):
    x = make_single(cfg)
    g = _geom(cfg)
    out = out_buffer(cfg)
    h.fdl_dense_attn(g, dev(x["q"]), dev(x["k"]) if cfg.ctx_len else None,
                     dev(x["v"]) if cfg.ctx_len else None, dev(x["k_dec"]), dev(x["v_dec"]), None, out)
    torch.cuda.synchronize()
    ref = attend(x["q"], x["k"], x["v"], x["k_dec"], x["v_dec"], None)
    assert_close(out_to_f64(cfg, out), ref, "dense")


@pytest.mark.parametrize("cfg", [
    get_config(0),
    _small_bf16(n_q_heads=4, n_kv_heads=4, ctx_len=1000, top_k_blocks=5),
    _small_bf16(n_q_heads=8, n_kv_heads=2, ctx_len=1500, head_dim=64, kv_block=32, top_k_blocks=9),
    _small_bf16(n_q_heads=7, n_kv_heads=1, ctx_len=4096, dec_len=32, top_k_blocks=12),
    _small_bf16(n_q_heads=2, n_kv_heads=2, ctx_len=2048, top_k_blocks=32),   # everything selected
    # many tiles per wave: one workgroup per head (256 heads), and 4 splits per head
    _small_bf16(batch=4, n_q_heads=64, n_kv_heads=64, ctx_len=4096, top_k_blocks=40),
    _small_bf16(batch=2, n_q_heads=32, n_kv_heads=32, ctx_len=8192, top_k_blocks=48),
], ids=["tiny", "mha-ragged", "gqa4-d64-bt32", "gqa7", "all-blocks", "mha-1split-10tiles",
        "mha-4splits-3tiles"])
def test_sparse_attention_with_oracle_selection(h, cfg):
    x = make_single(cfg)
    g = _geom(cfg)
    r = focus_layer_step(cfg, x, "source")
    n_blk = -(-cfg.ctx_len // cfg.kv_block)
    max_sel = max(len(s) for row in r["sel"] for s in row) + 3
    sel = np.full((cfg.batch, cfg.n_kv_heads, max_sel), -7, np.int32)
    nsel = np.zeros((cfg.batch, cfg.n_kv_heads), np.int32)
    for b in range(cfg.batch):
        for gg in range(cfg.n_kv_heads):
            s = r["sel"][b][gg]
            sel[b, gg, : len(s)] = s
            nsel[b, gg] = len(s)
    out = out_buffer(cfg)
    h.fdl_sparse_attn(g, dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["k_dec"]), dev(x["v_dec"]), None,
                      dev(sel), dev(nsel), max_sel, cfg.kv_block, out)
    torch.cuda.synchronize()
    assert_close(out_to_f64(cfg, out), r["out"], "sparse")
    if max_sel >= n_blk:
        dense = attend(x["q"], x["k"], x["v"], x["k_dec"], x["v_dec"], None)
        assert_close(out_to_f64(cfg, out), dense, "sparse==dense")
