"""Seeded numpy generators for every input of the five workloads.

Recipe (the same for every tensor): a numpy ``Generator`` seeded with
``SeedSequence([cfg.seed, layer, block, step, tag])`` draws float64 values, which are cast to float32
and, for the bf16 workloads, rounded to bf16 with round-to-nearest-even.  bf16 tensors are returned
as their ``uint16`` bit patterns; the tiny workload stays float32.  Both the CPU oracle and the HIP
path consume exactly these bit patterns.

Nothing here predicts, scores, selects or attends: the module only draws and lays out data.
"""
from __future__ import annotations

import numpy as np

from .configs import Config

TAG_Q, TAG_K, TAG_V, TAG_KDEC, TAG_VDEC = 0, 1, 2, 3, 4
TAG_CONF, TAG_MASK, TAG_SINKDIR, TAG_PLANT, TAG_PAGEPERM, TAG_ANCHOR = 5, 6, 7, 8, 9, 10


def rng_for(cfg: Config, layer: int, block: int, step: int, tag: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([cfg.seed, layer, block, step, tag]))


def round_to_bf16(x) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even.  Inputs are finite."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(u16) -> np.ndarray:
    """bf16 bit patterns -> float32 (exact)."""
    u = np.asarray(u16, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32)


def _finish(cfg: Config, x64: np.ndarray) -> np.ndarray:
    f32 = x64.astype(np.float32)
    return f32 if cfg.dtype == "f32" else round_to_bf16(f32)


def as_f32(cfg: Config, t: np.ndarray) -> np.ndarray:
    """Stored tensor (float32 or bf16 bits) -> float32 values, for the generator's own use."""
    return t if cfg.dtype == "f32" else bf16_bits_to_f32(t)


# ----------------------------------------------------------------------------------------------
# Per-step inputs: queries of the current block and the block's own keys / values
# ----------------------------------------------------------------------------------------------

def step_qkv(cfg: Config, layer: int = 0, block: int = 0, step: int = 0) -> dict:
    """Q [B][Hq][T][D], Kdec / Vdec [B][Hkv][T][D], all ~ N(0, 1)."""
    B, Hq, Hkv, T, D = cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.dec_len, cfg.head_dim
    q = rng_for(cfg, layer, block, step, TAG_Q).standard_normal((B, Hq, T, D))
    kd = rng_for(cfg, layer, block, step, TAG_KDEC).standard_normal((B, Hkv, T, D))
    vd = rng_for(cfg, layer, block, step, TAG_VDEC).standard_normal((B, Hkv, T, D))
    return {"q": _finish(cfg, q), "k_dec": _finish(cfg, kd), "v_dec": _finish(cfg, vd)}


def decode_state(cfg: Config, layer: int = 0, block: int = 0, step: int = 0) -> dict:
    """Previous-step confidence [B][T] float32 and the masked flags [B][T] uint8.

    ``n_masked`` positions per sequence are masked, chosen by a seeded permutation.  Confidence is
    U(0,1) or Beta(2,5) over all T slots; only masked slots are ever read.
    """
    B, T = cfg.batch, cfg.dec_len
    r = rng_for(cfg, layer, block, step, TAG_MASK)
    masked = np.zeros((B, T), dtype=np.uint8)
    for b in range(B):
        perm = r.permutation(T)
        masked[b, perm[: cfg.n_masked]] = 1
    rc = rng_for(cfg, layer, block, step, TAG_CONF)
    conf = rc.random((B, T)) if cfg.conf_dist == "uniform" else rc.beta(2.0, 5.0, (B, T))
    return {"prev_conf": conf.astype(np.float32), "masked": masked}


# ----------------------------------------------------------------------------------------------
# Cached context: keys / values with planted sinks (and, for the GQA workload, planted blocks)
# ----------------------------------------------------------------------------------------------

def _context_kv64(cfg: Config, layer: int, b: int, rk, rv):
    """float64 keys / values of one sequence [Hkv][L][D] with the workload's sink structure."""
    Hkv, L, D = cfg.n_kv_heads, cfg.ctx_len, cfg.head_dim
    k = rk.standard_normal((Hkv, L, D))
    v = rv.standard_normal((Hkv, L, D))
    if cfg.sink_kind == "shared_dir_x8":
        # key 0 of every head is turned onto one seeded unit direction, with 8x its own norm
        u = rng_for(cfg, layer, 0, 0, TAG_SINKDIR).standard_normal(D)
        u /= np.linalg.norm(u)
        for g in range(Hkv):
            k[g, 0, :] = 8.0 * np.linalg.norm(k[g, 0, :]) * u
    elif cfg.sink_kind == "first4_x6":
        k[:, :4, :] *= 6.0
    elif cfg.sink_kind == "anchors":
        # one BOS anchor per (sequence, head), repeated at the head of every chunk
        ra = rng_for(cfg, layer, b, 0, TAG_ANCHOR)
        ak = 6.0 * ra.standard_normal((Hkv, D))
        av = ra.standard_normal((Hkv, D))
        for c in range(cfg.n_chunks):
            k[:, c * cfg.chunk_tokens, :] = ak
            v[:, c * cfg.chunk_tokens, :] = av
    return k, v


def context_kv(cfg: Config, layer: int = 0) -> dict:
    """Logical cache K, V [B][Hkv][L][D] (float32 or bf16 bits)."""
    B, Hkv, L, D = cfg.batch, cfg.n_kv_heads, cfg.ctx_len, cfg.head_dim
    dt = np.float32 if cfg.dtype == "f32" else np.uint16
    K = np.empty((B, Hkv, L, D), dtype=dt)
    V = np.empty((B, Hkv, L, D), dtype=dt)
    rk = rng_for(cfg, layer, 0, 0, TAG_K)
    rv = rng_for(cfg, layer, 0, 0, TAG_V)
    for b in range(B):
        k, v = _context_kv64(cfg, layer, b, rk, rv)
        K[b] = _finish(cfg, k)
        del k
        V[b] = _finish(cfg, v)
        del v
    return {"k": K, "v": V}


def plant_blocks(cfg: Config, K: np.ndarray, q: np.ndarray, layer: int = 0) -> np.ndarray:
    """Plant ``planted_blocks`` relevant blocks per KV head (in place on a copy; returns block ids).

    Planted keys are ``c*u_g + sqrt(1-c^2)*eps`` with eps ~ N(0,1)^D and u_g = sqrt(D) times the unit
    direction of the mean query of group g (over its q-heads and all T positions), so their
    correlation with the group's queries is about c.  Blocks are drawn among 1..n_blk-1 (block 0
    holds the sinks).  Returns the planted block ids [B][Hkv][n].
    """
    B, Hkv, D, G, bt = cfg.batch, cfg.n_kv_heads, cfg.head_dim, cfg.group, cfg.kv_block
    c = cfg.planted_corr
    r = rng_for(cfg, layer, 0, 0, TAG_PLANT)
    qf = as_f32(cfg, q).astype(np.float64)
    out = np.zeros((B, Hkv, cfg.planted_blocks), dtype=np.int64)
    for b in range(B):
        for g in range(Hkv):
            m = qf[b, g * G:(g + 1) * G].reshape(-1, D).mean(axis=0)
            u = np.sqrt(D) * m / np.linalg.norm(m)
            blocks = np.sort(r.choice(np.arange(1, cfg.n_blk), size=cfg.planted_blocks, replace=False))
            out[b, g] = blocks
            for n in blocks:
                eps = r.standard_normal((bt, D))
                kk = c * u[None, :] + np.sqrt(1.0 - c * c) * eps
                K[b, g, n * bt:(n + 1) * bt] = _finish(cfg, kk)
    return out


# ----------------------------------------------------------------------------------------------
# Paged pool for the chunked workload
# ----------------------------------------------------------------------------------------------

def page_table(cfg: Config, layer: int = 0) -> np.ndarray:
    """[B][pages_per_seq] int32: logical page i of sequence b lives in physical page pt[b, i]."""
    perm = rng_for(cfg, layer, 0, 0, TAG_PAGEPERM).permutation(cfg.n_pages).astype(np.int32)
    return perm.reshape(cfg.batch, cfg.pages_per_seq)


def to_pages(cfg: Config, X: np.ndarray, pt: np.ndarray) -> np.ndarray:
    """Logical [B][Hkv][L][D] -> pool [n_pages][Hkv][page_tokens][D] through the page table."""
    B, Hkv, L, D, P = cfg.batch, cfg.n_kv_heads, cfg.ctx_len, cfg.head_dim, cfg.page_tokens
    pool = np.zeros((cfg.n_pages, Hkv, P, D), dtype=X.dtype)
    for b in range(B):
        xb = X[b].reshape(Hkv, L // P, P, D)
        pool[pt[b]] = xb.transpose(1, 0, 2, 3)
    return pool


# ----------------------------------------------------------------------------------------------
# The multi-layer, multi-step schedule of the 32K workload
# ----------------------------------------------------------------------------------------------

def schedule_state(cfg: Config, step: int) -> dict:
    """Decode state of global step ``step`` (block j = step // steps_per_block, s = step % it).

    Each generation block draws an unmask order (a seeded permutation of the T slots); at step s the
    first s slots of that order are already decoded, the rest are masked.  Every step draws a fresh
    U(0,1) confidence vector; the predictor of step s reads the one drawn at step s-1 of the same
    block, and step 0 of a block has none (``prev_conf`` is None).
    """
    T, spb = cfg.dec_len, cfg.steps_per_block
    j, s = divmod(step, spb)
    order = rng_for(cfg, 0, j, 0, TAG_MASK).permutation(T)
    masked = np.ones((cfg.batch, T), dtype=np.uint8)
    masked[:, order[:s]] = 0
    prev = None
    if s > 0:
        prev = rng_for(cfg, 0, j, s - 1, TAG_CONF).random((cfg.batch, T)).astype(np.float32)
    return {"block": j, "s": s, "prev_conf": prev, "masked": masked}


# ----------------------------------------------------------------------------------------------
# One whole single-layer workload
# ----------------------------------------------------------------------------------------------

def make_single(cfg: Config, layer: int = 0, block: int = 0, step: int = 0) -> dict:
    """Every input of one layer-step of a single-layer workload (tiny, 8K, 16K GQA, chunked)."""
    d = {}
    d.update(step_qkv(cfg, layer, block, step))
    d.update(decode_state(cfg, layer, block, step))
    d.update(context_kv(cfg, layer))
    if cfg.planted_blocks:
        d["planted"] = plant_blocks(cfg, d["k"], d["q"], layer)
    if cfg.paged:
        pt = page_table(cfg, layer)
        d["page_table"] = pt
        d["k_pool"] = to_pages(cfg, d["k"], pt)
        d["v_pool"] = to_pages(cfg, d["v"], pt)
    return d
