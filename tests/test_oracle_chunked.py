"""Pins of the chunked, paged variant: all chunks + all tokens reduces to dense attention; the physical
page order cannot change any result; anchors are always kept."""
import numpy as np

from oracle.attention import attend
from oracle.pipeline import chunked_layer_step
from synth import get_config
from synth.gen import make_single, to_pages


def _small():
    return get_config(4).with_(batch=2, n_q_heads=4, n_kv_heads=2, ctx_len=1024, chunk_tokens=256)


def test_counts_and_anchor():
    cfg = _small()
    x = make_single(cfg)
    r = chunked_layer_step(cfg, x, with_output=False)
    keep = cfg.tokens_per_chunk_kept
    assert r["tokens"].shape == (2, 2, cfg.top_k_chunks * (1 + keep))
    for b in range(2):
        for g in range(2):
            toks = r["tokens"][b, g].tolist()
            assert toks == sorted(set(toks))
            for c in r["chunks"][b, g]:
                inside = [t for t in toks if c * cfg.chunk_tokens <= t < (c + 1) * cfg.chunk_tokens]
                assert len(inside) == 1 + keep and inside[0] == c * cfg.chunk_tokens


def test_all_chunks_all_tokens_is_dense():
    cfg = _small().with_(top_k_chunks=4, token_keep_frac=1.0)
    x = make_single(cfg)
    r = chunked_layer_step(cfg, x)
    assert cfg.tokens_per_chunk_kept == cfg.chunk_tokens - 1   # every non-anchor token
    dense = attend(x["q"], x["k"], x["v"], x["k_dec"], x["v_dec"], None)
    for b in range(2):
        for g in range(2):
            assert sorted(set(r["tokens"][b, g].tolist())) == list(range(cfg.ctx_len))
    assert np.allclose(r["out"], dense, atol=1e-13, rtol=0)


def test_page_order_invariance():
    cfg = _small()
    x = make_single(cfg)
    ident = np.arange(cfg.n_pages, dtype=np.int32).reshape(cfg.batch, -1)
    y = dict(x)
    y["page_table"] = ident
    y["k_pool"] = to_pages(cfg, x["k"], ident)
    y["v_pool"] = to_pages(cfg, x["v"], ident)
    r1 = chunked_layer_step(cfg, x)
    r2 = chunked_layer_step(cfg, y)
    assert not np.array_equal(x["page_table"], ident)
    for key in ("chunk_scores", "chunks", "token_scores", "tokens", "out"):
        assert np.array_equal(r1[key], r2[key]), key


def test_anchor_keys_are_strong():
    cfg = _small()
    x = make_single(cfg)
    # the generator repeats one anchor per (sequence, head) at every chunk head
    for c in range(cfg.n_chunks):
        assert np.array_equal(x["k"][:, :, c * cfg.chunk_tokens], x["k"][:, :, 0])
