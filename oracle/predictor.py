"""Past-confidence-guided prediction of the positions about to be unmasked.

Focus-dLLM (abstract; Elamur "Summary" and "Key points"): a token's confidence at one denoising step
predicts its confidence at the next, so the previous step's confidence is used to guess which masked
positions will be decoded next; the guesses are then widened into local windows, and the queries at
those positions are the "predicted queries".  The Key points use the four highest-confidence tokens
that are still masked.

Readings taken where the pages are silent:
  * candidates are the positions still masked at the current step; they are ranked by the previous
    step's confidence, highest first, ties to the lower position; NaN ranks below every number;
  * the first min(k, #masked) candidates are kept and each is widened to [i-w, i+w] clipped to the
    decode block [0, T); the predicted set is the union; already-decoded positions inside a window
    are predicted queries too;
  * with no previous confidence (first step of a block) every position of the block is predicted;
  * with nothing masked the predicted set is empty.
"""
from __future__ import annotations

import numpy as np

from .fp32tree import order_key


def top_masked_positions(conf_row, masked_row, k: int) -> list[int]:
    """The k highest-confidence masked positions of one sequence, in rank order."""
    conf = np.asarray(conf_row, dtype=np.float32)
    key = order_key(conf).astype(np.int64)
    cand = [i for i in range(len(conf)) if masked_row[i]]
    cand.sort(key=lambda i: (-key[i], i))
    return cand[: min(k, len(cand))]


def predict_positions(prev_conf, masked, top_k: int, window: int):
    """Returns (pred_mask [B] uint64 bitmask over the T slots, n_pred [B] int32)."""
    masked = np.asarray(masked)
    B, T = masked.shape
    assert T <= 64
    bits = np.zeros(B, dtype=np.uint64)
    npred = np.zeros(B, dtype=np.int32)
    for b in range(B):
        if prev_conf is None:
            chosen_set = set(range(T))
        else:
            chosen_set = set()
            for i in top_masked_positions(prev_conf[b], masked[b], top_k):
                for p in range(i - window, i + window + 1):
                    if 0 <= p < T:
                        chosen_set.add(p)
        v = 0
        for p in chosen_set:
            v |= 1 << p
        bits[b] = np.uint64(v)
        npred[b] = len(chosen_set)
    return bits, npred


def mask_to_positions(bits, T: int) -> list[int]:
    v = int(bits)
    return [p for p in range(T) if (v >> p) & 1]
