"""Bidirectional softmax attention of the decode block's queries over a set of KV tokens, float64.

Focus-dLLM (abstract; Elamur "Summary"): diffusion LLMs attend bidirectionally; the sparse step runs
the same attention over only the selected KV, and shallow layers keep full attention.  This module is
the plain definition, O_i = sum_j softmax_j(q_i . k_j / sqrt(D)) v_j, with no blocking and no online
softmax.

Readings: every one of the T block queries attends (not only the predicted ones); the block's own T
keys / values are always attended; later, still-masked blocks are not part of the KV (the KV is the
cached context plus the current block).
"""
from __future__ import annotations

import numpy as np

from .fp32tree import values_f32


def attend_rows(q, keys, vals) -> np.ndarray:
    """q [T][D], keys / vals [N][D] (float64) -> [T][D] float64."""
    D = q.shape[-1]
    s = (q @ keys.T) / np.sqrt(D)
    m = s.max(axis=1, keepdims=True)
    w = np.exp(s - m)
    w /= w.sum(axis=1, keepdims=True)
    return w @ vals


def blocks_to_tokens(block_ids, kv_block: int, ctx_len: int) -> np.ndarray:
    toks = [np.arange(n * kv_block, min((n + 1) * kv_block, ctx_len)) for n in block_ids]
    return np.concatenate(toks) if toks else np.zeros(0, dtype=np.int64)


def attend(q, k, v, k_dec, v_dec, token_sets) -> np.ndarray:
    """Sparse (or dense) attention.

    q [B][Hq][T][D]; k, v logical [B][Hkv][L][D]; k_dec, v_dec [B][Hkv][T][D];
    token_sets[b][g] = ascending cached-token ids attended by KV head g (None = all L).
    Returns O [B][Hq][T][D] float64.
    """
    qf = values_f32(q).astype(np.float64)
    kf, vf = values_f32(k), values_f32(v)
    kd = values_f32(k_dec).astype(np.float64)
    vd = values_f32(v_dec).astype(np.float64)
    B, Hq, T, D = qf.shape
    Hkv = kf.shape[1]
    G = Hq // Hkv
    out = np.zeros((B, Hq, T, D), dtype=np.float64)
    for b in range(B):
        for g in range(Hkv):
            ts = token_sets[b][g] if token_sets is not None else None
            if ts is None:
                kc, vc = kf[b, g], vf[b, g]
            else:
                ts = np.asarray(ts, dtype=np.int64)
                kc, vc = kf[b, g, ts], vf[b, g, ts]
            keys = np.concatenate([kc.astype(np.float64), kd[b, g]], axis=0)
            vals = np.concatenate([vc.astype(np.float64), vd[b, g]], axis=0)
            for h in range(g * G, (g + 1) * G):
                out[b, h] = attend_rows(qf[b, h], keys, vals)
    return out
