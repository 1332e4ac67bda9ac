"""Closing the denoising loop: the positions a step decodes and the masked set it leaves behind.

Test infrastructure: only tests/, the smoke check and the benchmark's CPU baseline use this module.

Focus-dLLM (Elamur "Summary"): a diffusion LLM decodes a block by denoising its masked positions
step after step; ("Key points") the tokens decoded at a step are the highest-confidence ones among
those still masked (the predictor's recall is measured against them), and generation length equals
the number of steps (256), i.e. one position is decoded per step.

Readings taken where the pages are silent:
  * after a step, the n (default 1) masked positions of highest confidence in that step's confidence
    vector are decoded (their masked flag drops to 0); fewer masked positions than n: all of them;
    none masked: nothing changes;
  * the ranking is the predictor's: higher confidence first, ties to the lower position, NaN below
    every number, -0 equal to +0 (``predictor.top_masked_positions``);
  * the next step's predictor reads this step's confidence, and step 0 of a block has none.
"""
from __future__ import annotations

import numpy as np

from .predictor import top_masked_positions


def unmask(conf, masked, n_unmask: int = 1):
    """conf [B][T] float32, masked [B][T] -> (new masked [B][T] uint8, decoded [B][n_unmask] int32
    in rank order, -1 past the number decoded)."""
    masked = np.asarray(masked)
    B, T = masked.shape
    out = (masked != 0).astype(np.uint8)
    dec = np.full((B, max(n_unmask, 0)), -1, dtype=np.int32)
    for b in range(B):
        chosen = top_masked_positions(conf[b], masked[b], n_unmask) if n_unmask > 0 else []
        for r, i in enumerate(chosen):
            out[b, i] = 0
            dec[b, r] = i
    return out, dec


def block_schedule(confs, masked0, n_unmask: int = 1, prev_conf0=None):
    """The decode state of every step of one block.

    confs [S][B][T]: the confidence each step produces.  Step s runs with (prev_conf_s, masked_s),
    where prev_conf_0 = prev_conf0 (None: the first step of a block), prev_conf_s = confs[s-1], and
    masked_{s+1} = unmask(confs[s], masked_s).  Returns the list of (prev_conf_s, masked_s) and the
    decoded positions [S][B][n_unmask]."""
    confs = np.asarray(confs, dtype=np.float32)
    S = confs.shape[0]
    m = (np.asarray(masked0) != 0).astype(np.uint8)
    states, decoded = [], []
    for s in range(S):
        states.append((prev_conf0 if s == 0 else confs[s - 1], m.copy()))
        m, d = unmask(confs[s], m, n_unmask)
        decoded.append(d)
    return states, np.stack(decoded) if decoded else np.zeros((0,) + m.shape[:1] + (n_unmask,), np.int32)
