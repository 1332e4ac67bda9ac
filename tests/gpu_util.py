"""Helpers shared by the GPU tests: device transfer, tolerance check, handle fixture."""
from __future__ import annotations

import numpy as np
import pytest
import torch

ATOL, RTOL = 1e-2, 2e-2   # |o - r| <= ATOL + RTOL * |r|, elementwise, against the float64 oracle


def require_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a visible GPU")


def dev(x, dtype=None):
    """numpy -> device tensor.  bf16 bit patterns (uint16) travel as int16."""
    a = np.ascontiguousarray(x)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    if a.dtype == np.uint64:
        a = a.view(np.int64)
    t = torch.from_numpy(a)
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def bf16_out_to_f64(t: torch.Tensor) -> np.ndarray:
    u = host(t.view(torch.int16)).view(np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def assert_close(out, ref, what=""):
    o = np.asarray(out, np.float64)
    r = np.asarray(ref, np.float64)
    err = np.abs(o - r)
    bad = err > ATOL + RTOL * np.abs(r)
    if bad.any():
        i = np.unravel_index(np.argmax(err - (ATOL + RTOL * np.abs(r))), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} elements out of tolerance; "
                             f"worst at {i}: got {o[i]}, want {r[i]}; max abs err {err.max():.3g}")
    return float(err.max())


def out_buffer(cfg, device="cuda"):
    shape = (cfg.batch, cfg.n_q_heads, cfg.dec_len, cfg.head_dim)
    if cfg.dtype == "f32":
        return torch.zeros(shape, dtype=torch.float32, device=device)
    return torch.zeros(shape, dtype=torch.int16, device=device)


def out_to_f64(cfg, t):
    return host(t).astype(np.float64) if cfg.dtype == "f32" else bf16_out_to_f64(t)
