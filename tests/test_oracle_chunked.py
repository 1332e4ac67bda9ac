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


# ---- the per-sequence reading of the chunk selection ------------------------------------------

def _int_case(rng, B, H, n_chunks, chunk, D):
    from synth.gen import round_to_bf16
    qs = rng.integers(-3, 4, size=(B, H, D)).astype(np.float32)
    ki = rng.integers(-2, 3, size=(B, H, n_chunks * chunk, D))
    return qs, ki, round_to_bf16(ki.astype(np.float32))


def test_shared_chunks_integer_brute_force():
    """Integer-valued inputs: every float32 sum is exact, so the sequence score is the Python-integer
    sum over heads of q.(key sum); the chosen set is its top-k (ties to the lower chunk), the same
    for every head."""
    from oracle.chunked import select_chunks_shared
    rng = np.random.default_rng(21)
    B, H, n_chunks, chunk, D, K = 3, 5, 9, 8, 16, 4
    qs, ki, kb = _int_case(rng, B, H, n_chunks, chunk, D)
    _, seq, chosen = select_chunks_shared(qs, kb, chunk, K)
    for b in range(B):
        exact = [sum(int(qs[b, g].astype(np.int64) @ ki[b, g, c * chunk:(c + 1) * chunk].sum(axis=0))
                     for g in range(H)) for c in range(n_chunks)]
        assert seq[b].tolist() == [float(e) for e in exact]
        want = sorted(sorted(range(n_chunks), key=lambda c: (-exact[c], c))[:K])
        for g in range(H):
            assert chosen[b, g].tolist() == want


def test_shared_chunks_one_head_equals_per_head():
    from oracle.chunked import select_chunks, select_chunks_shared
    rng = np.random.default_rng(22)
    qs = rng.standard_normal((2, 1, 32)).astype(np.float32)
    from synth.gen import round_to_bf16
    k = round_to_bf16(rng.standard_normal((2, 1, 12 * 16, 32)).astype(np.float32))
    sc1, ch1 = select_chunks(qs, k, 16, 5)
    sc2, seq, ch2 = select_chunks_shared(qs, k, 16, 5)
    assert np.array_equal(ch1, ch2) and np.array_equal(seq, sc1[:, 0]) and np.array_equal(sc1, sc2)


def test_shared_chunks_in_the_layer_step():
    """The per-sequence layer step keeps the anchor plus the top tokens inside chunks common to all
    heads, and with every chunk chosen both readings keep the same tokens."""
    cfg = get_config(4).with_(batch=2, n_q_heads=4, n_kv_heads=2, ctx_len=4096, chunk_tokens=512)
    x = make_single(cfg)
    r = chunked_layer_step(cfg, x, with_output=False, per_sequence=True)
    for b in range(cfg.batch):
        rows = r["chunks"][b]
        assert all(rows[g].tolist() == rows[0].tolist() for g in range(cfg.n_kv_heads))
    allc = cfg.with_(top_k_chunks=cfg.ctx_len // cfg.chunk_tokens)
    a = chunked_layer_step(allc, x, with_output=False, per_sequence=True)
    p = chunked_layer_step(allc, x, with_output=False, per_sequence=False)
    assert np.array_equal(a["tokens"], p["tokens"])


# ---- level 2 (tokens inside the chosen chunks), pinned independently of the oracle's code ------

def test_select_tokens_hand_worked():
    """One head, head_dim 2, four chunks of four tokens, query sum (1, 0): a token's score is the
    first component of its key, a chunk's score the sum of those.  Chunk sums 4, 6, 3, 8 choose
    chunks 1 and 3 (a strict, non-adjacent subset).  Chunk 1 = (-5, 2, 7, 2): the anchor (token 4)
    is kept although it scores lowest, then token 6 (7) and, of the tie 2 = 2 between tokens 5 and
    7, the lower token 5.  Chunk 3 = (8, 1, -1, 0): the anchor (token 12) scores highest but is kept
    once; the best two others are tokens 13 (1) and 15 (0)."""
    from oracle.chunked import select_chunks, select_tokens
    s = [1, 1, 1, 1, -5, 2, 7, 2, 0, 0, 0, 3, 8, 1, -1, 0]
    k = np.zeros((1, 1, 16, 2), dtype=np.float32)
    k[0, 0, :, 0] = s
    k[0, 0, :, 1] = [3] * 16          # ignored by the query sum below
    qs = np.array([[[1.0, 0.0]]], dtype=np.float32)
    sc, chosen = select_chunks(qs, k, 4, 2)
    assert sc[0, 0].tolist() == [4.0, 6.0, 3.0, 8.0]
    assert chosen[0, 0].tolist() == [1, 3]
    ts, kept = select_tokens(qs, k, chosen, 4, 2)
    assert ts[0, 0].tolist() == [[-5.0, 2.0, 7.0, 2.0], [8.0, 1.0, -1.0, 0.0]]
    assert kept[0, 0].tolist() == [4, 5, 6, 12, 13, 15]


def _brute_layer(cfg, q_int, k_int, pt, chunk, K, keep):
    """Python-integer brute force of the chunked selection: predicted query sum over all positions
    and all heads of a group, chunk scores, top-K chunks, then anchor + top-keep other tokens of
    every chosen chunk (ties to the lower chunk / token).  k_int is the logical [B][Hkv][L][D]."""
    B, Hq, T, D = q_int.shape
    Hkv = k_int.shape[1]
    G = Hq // Hkv
    L = k_int.shape[2]
    n_chunks = L // chunk
    out_chunks, out_tokens = [], []
    for b in range(B):
        rc, rt = [], []
        for g in range(Hkv):
            qs = [sum(int(q_int[b, g * G + m, p, d]) for m in range(G) for p in range(T)) for d in range(D)]
            tok = [sum(qs[d] * int(k_int[b, g, t, d]) for d in range(D)) for t in range(L)]
            csum = [sum(tok[c * chunk:(c + 1) * chunk]) for c in range(n_chunks)]
            chosen = sorted(sorted(range(n_chunks), key=lambda c: (-csum[c], c))[:K])
            row = []
            for c in chosen:
                others = sorted(range(c * chunk + 1, (c + 1) * chunk), key=lambda t: (-tok[t], t))[:keep]
                row.extend(sorted([c * chunk] + others))
            rc.append(chosen)
            rt.append(row)
        out_chunks.append(rc)
        out_tokens.append(rt)
    return out_chunks, out_tokens


def test_select_tokens_integer_brute_force():
    """Integer-valued queries and keys small enough that every float32 product and sum is exact, so
    the oracle's chunk and token choices must equal a Python-integer brute force under any order.
    Chunks are a strict subset (2 of 8), pages shuffled, several KV heads with two query heads each;
    a ranking turned around, or a chosen chunk's tokens scored under another slot, fails."""
    from types import SimpleNamespace

    from oracle.pipeline import chunked_layer_step
    from synth.gen import round_to_bf16, to_pages
    for seed in range(6):
        rng = np.random.default_rng(1000 + seed)
        B, Hq, Hkv, T, D, chunk, n_chunks, K, keep, page = 2, 6, 3, 4, 8, 16, 8, 2, 3, 4
        L = chunk * n_chunks
        q_int = rng.integers(-2, 3, size=(B, Hq, T, D))
        k_int = rng.integers(-3, 4, size=(B, Hkv, L, D))
        p = SimpleNamespace(top_k_pos=4, window=0, n_kv_heads=Hkv, chunk_tokens=chunk, top_k_chunks=K,
                            tokens_per_chunk_kept=keep, page_tokens=page)
        npp = L // page
        pt = rng.permutation(B * npp).astype(np.int32).reshape(B, npp)
        cfg = SimpleNamespace(batch=B, n_kv_heads=Hkv, ctx_len=L, head_dim=D, n_pages=B * npp, page_tokens=page)
        kb = round_to_bf16(k_int.astype(np.float32))
        x = {"q": round_to_bf16(q_int.astype(np.float32)), "k_pool": to_pages(cfg, kb, pt),
             "v_pool": to_pages(cfg, kb, pt), "page_table": pt, "k_dec": kb[:, :, :T], "v_dec": kb[:, :, :T],
             "prev_conf": None, "masked": np.ones((B, T), dtype=np.uint8)}
        r = chunked_layer_step(p, x, with_output=False)
        want_c, want_t = _brute_layer(cfg, q_int, k_int, pt, chunk, K, keep)
        assert r["chunks"].tolist() == want_c, seed
        assert r["tokens"].tolist() == want_t, seed
        # the chosen chunks are a strict subset, and the kept tokens are not simply the first ones
        assert all(len(c) == K for row in want_c for c in row)
