"""Exact float32 building blocks of the oracle: bf16 decoding, the pinned summation tree and the
order key used for every top-k.

Reading (the pages fix no summation order): every float32 sum in the scoring path is an
"adjacent-pair tree" -- the operand list is padded with +0.0 to a power of two, then level by level
element 2j is added to element 2j+1.  Products are rounded to float32 before they are added.
numpy's elementwise float32 ``+`` and ``*`` are single IEEE-754 round-to-nearest-even operations,
so this code pins every bit of the result; numpy reductions (``sum``, ``dot``, ``matmul``) are never
used on float32 here because their order is unspecified.
"""
from __future__ import annotations

import numpy as np


def bf16_to_f32(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float32; exact (the 16 bits become the high half)."""
    b = np.asarray(bits)
    assert b.dtype == np.uint16, b.dtype
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def values_f32(x) -> np.ndarray:
    """Input tensor as float32 values: bf16 bits are decoded, float32 passes through."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return bf16_to_f32(x)
    assert x.dtype == np.float32, x.dtype
    return x


def tree_sum(x, axis: int = -1) -> np.ndarray:
    """Pinned float32 adjacent-pair tree over ``axis`` (zero-padded to a power of two)."""
    a = np.moveaxis(np.asarray(x, dtype=np.float32), axis, -1)
    n = a.shape[-1]
    if n == 0:
        return np.zeros(a.shape[:-1], dtype=np.float32)
    m = 1 << (n - 1).bit_length()
    if m != n:
        pad = np.zeros(a.shape[:-1] + (m - n,), dtype=np.float32)
        a = np.concatenate([a, pad], axis=-1)
    while a.shape[-1] > 1:
        a = a[..., 0::2] + a[..., 1::2]
    return a[..., 0]


def tree_dot(x, y) -> np.ndarray:
    """Pinned float32 dot product over the last axis: tree over fl32(x_d * y_d).  Broadcasts."""
    prod = np.multiply(np.asarray(x, dtype=np.float32), np.asarray(y, dtype=np.float32),
                       dtype=np.float32)
    return tree_sum(prod, axis=-1)


def order_key(x) -> np.ndarray:
    """float32 -> uint32 key whose unsigned order is the numeric order.

    -0.0 and +0.0 map to the same key; every NaN maps to 0, below -inf, and all NaNs are equal.
    """
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32).copy()
    u[u == np.uint32(0x80000000)] = 0  # -0 -> +0
    neg = (u >> np.uint32(31)) == 1
    key = np.where(neg, ~u, u | np.uint32(0x80000000)).astype(np.uint32)
    key[np.isnan(f)] = 0
    return key
