"""Seeded on-device generation of the 32K multi-layer workload for timing runs.

Same recipe as ``synth.gen`` (N(0,1) values, the first 4 cached keys of every head scaled by 6,
bf16 rounding to nearest even), but drawn by torch's device generator so that 16 GiB of KV cache
appear in seconds.  Values differ from the numpy draws; parity tests use ``synth.gen``.
Only draws and scales random numbers: none of the method's arithmetic is here.
"""
from __future__ import annotations

import torch

from .configs import Config

TAG_K, TAG_V, TAG_STEP = 1, 2, 11


def _gen(cfg: Config, layer: int, tag: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed((cfg.seed * 1_000_003 + layer) * 101 + tag)
    return g


def layer_kv(cfg: Config, layer: int, device="cuda"):
    """K, V [B][Hkv][L][D] bf16 for one layer."""
    shape = (cfg.batch, cfg.n_kv_heads, cfg.ctx_len, cfg.head_dim)
    k = torch.randn(shape, generator=_gen(cfg, layer, TAG_K, device), device=device, dtype=torch.float32)
    if cfg.sink_kind == "first4_x6":
        k[:, :, :4] *= 6.0
    kb = k.to(torch.bfloat16)
    del k
    v = torch.randn(shape, generator=_gen(cfg, layer, TAG_V, device), device=device, dtype=torch.float32)
    vb = v.to(torch.bfloat16)
    return kb, vb


def step_qkv_pool(cfg: Config, n_steps: int, device="cuda"):
    """Q [n_steps][L][B][Hq][T][D], Kdec / Vdec [n_steps][L][B][Hkv][T][D] bf16, drawn per layer."""
    B, Hq, Hkv, T, D, NL = cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.dec_len, cfg.head_dim, cfg.n_layers
    q = torch.empty((n_steps, NL, B, Hq, T, D), dtype=torch.bfloat16, device=device)
    kd = torch.empty((n_steps, NL, B, Hkv, T, D), dtype=torch.bfloat16, device=device)
    vd = torch.empty((n_steps, NL, B, Hkv, T, D), dtype=torch.bfloat16, device=device)
    for layer in range(NL):
        g = _gen(cfg, layer, TAG_STEP, device)
        q[:, layer] = torch.randn((n_steps, B, Hq, T, D), generator=g, device=device).to(torch.bfloat16)
        kd[:, layer] = torch.randn((n_steps, B, Hkv, T, D), generator=g, device=device).to(torch.bfloat16)
        vd[:, layer] = torch.randn((n_steps, B, Hkv, T, D), generator=g, device=device).to(torch.bfloat16)
    return q, kd, vd
