"""Attention-sink detection at the source layer, in float64.

Focus-dLLM (abstract; Elamur "Summary" and "Key points"): highly influential attention sinks are
always kept when pruning, and because sink locations stay consistent from layer to layer they are
found once and reused in deeper layers.

Readings (the pages give no detection rule):
  * for q-head h and predicted position p, the attention row is the softmax of q_p . k_t / sqrt(D)
    over every cached token t in [0, L) and the block's own T tokens;
  * a cached token's mass for head h is the mean of its row weights over the predicted positions;
  * a cached token is a sink if, for at least one q-head, that mass reaches tau;
  * the sink list of a sequence is the union over all q-heads, ascending, truncated to max_sinks
    (truncation is an overflow the GPU reports);
  * no predicted positions -> no sinks.
"""
from __future__ import annotations

import numpy as np

from .fp32tree import values_f32
from .predictor import mask_to_positions


def sink_masses(q, k, k_dec, pred_bits, full_row: bool = False) -> np.ndarray:
    """Per-(q-head, token) mean softmax mass, float64: [B][Hq][L] over the cached tokens, or
    [B][Hq][L+T] with the block's own tokens appended when ``full_row`` (zeros if P is empty)."""
    qf = values_f32(q).astype(np.float64)
    kf = values_f32(k).astype(np.float64)
    kd = values_f32(k_dec).astype(np.float64)
    B, Hq, T, D = qf.shape
    Hkv, L = kf.shape[1], kf.shape[2]
    G = Hq // Hkv
    out = np.zeros((B, Hq, L + T if full_row else L), dtype=np.float64)
    for b in range(B):
        P = mask_to_positions(pred_bits[b], T)
        if not P:
            continue
        for h in range(Hq):
            g = h // G
            keys = np.concatenate([kf[b, g], kd[b, g]], axis=0)       # [L+T][D]
            s = (qf[b, h, P, :] @ keys.T) / np.sqrt(D)                # [|P|][L+T]
            m = s.max(axis=1, keepdims=True)
            w = np.exp(s - m)
            w /= w.sum(axis=1, keepdims=True)
            out[b, h] = w.mean(axis=0) if full_row else w[:, :L].mean(axis=0)
    return out


def detect_sinks(q, k, k_dec, pred_bits, tau: float, max_sinks: int):
    """Returns (sink_pos [B][max_sinks] int32 padded with -1, n_sinks [B] int32,
    overflow [B] bool, margin float: min |mass - tau| over every (head, token))."""
    a = sink_masses(q, k, k_dec, pred_bits)
    B = a.shape[0]
    pos = np.full((B, max_sinks), -1, dtype=np.int32)
    n = np.zeros(B, dtype=np.int32)
    over = np.zeros(B, dtype=bool)
    T = np.asarray(q).shape[2]
    for b in range(B):
        if not mask_to_positions(pred_bits[b], T):
            continue
        hit = np.nonzero((a[b] >= tau).any(axis=0))[0]
        over[b] = len(hit) > max_sinks
        hit = hit[:max_sinks]
        pos[b, : len(hit)] = hit
        n[b] = len(hit)
    margin = float(np.abs(a - tau).min()) if a.size else float("inf")
    return pos, n, over, margin
