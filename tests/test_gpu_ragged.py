"""Ragged batches: sequences of different cached lengths in one launch.

The geometry carries a device array ctx_lens[B]; sequence b has L_b = ctx_lens[b] cached tokens,
its rows still ctx_len apart in the cache, its unit count ceil(L_b / kv_block) (a partial last
block when L_b is not a multiple), and the sink scan covers its own L_b tokens.  Every sequence must
give what the oracle gives for that sequence alone (its own slice of the inputs, ctx_len = L_b):
predicted positions, sinks and selections bit for bit, scores bit for bit on its own units and +0
past them, outputs within the bf16 tolerance.  The cache rows past each L_b hold NaN, so that any
read of them shows in the outputs."""
import numpy as np
import pytest
import torch

from gpu_util import assert_close, require_gpu
from layer_util import _focus, check_focus_step_layers, focus_step_layers
from synth import get_config
from synth.gen import make_single

pytestmark = pytest.mark.gpu

BF16_NAN = np.uint16(0x7FC0)


def _ragged(cfg, lens, layer=0):
    """make_single's inputs with the cache rows past each sequence's length set to NaN."""
    x = make_single(cfg, layer=layer)
    nan = BF16_NAN if cfg.dtype == "bf16" else np.float32(np.nan)
    for name in ("k", "v"):
        a = x[name].copy()
        for b, lb in enumerate(lens):
            a[b, :, lb:] = nan
        x[name] = a
    return x


def _slice(cfg, x, b, lb):
    """Sequence b alone: batch 1, ctx_len = lb."""
    xb = {}
    for k, v in x.items():
        if v is None or k == "planted":
            continue
        xb[k] = v[b:b + 1, :, :lb] if k in ("k", "v") else v[b:b + 1]
    return cfg.with_(batch=1, ctx_len=lb), xb


def _check_seq(cfg, got, want, b, lb, what):
    """One sequence of a ragged run against the oracle's batch-1 result."""
    nb = -(-lb // cfg.kv_block)
    assert int(got["pred_mask"][b]) == int(np.asarray(want["pred_mask"], np.uint64)[0]), what
    sc = got["scores"][b]
    assert np.array_equal(sc[:, :nb].view(np.uint32), want["scores"][0].view(np.uint32)), what
    assert np.all(sc[:, nb:].view(np.uint32) == 0), f"{what}: scores past the sequence's units"
    nsb = int(want["n_sinks"][0])
    assert int(got["n_sinks"][b]) == nsb, what
    assert got["sink_pos"][b, :nsb].tolist() == want["sink_pos"][0, :nsb].tolist(), what
    for g in range(cfg.n_kv_heads):
        w = want["sel"][0][g].tolist()
        assert int(got["n_sel"][b, g]) == len(w), (what, g)
        assert got["sel"][b, g, :len(w)].tolist() == w, (what, g)
    assert_close(got["out"][b:b + 1], want["out"], what)


CASES = {
    # 8K, 8 heads: one full sequence, one with a partial last block, one shorter than the top-K
    "8k-mha": (1, dict(batch=3, n_q_heads=8, n_kv_heads=8), [8192, 5000, 1000]),
    # 16K GQA (7 query heads per KV head): the grouped kernels
    "16k-gqa7": (2, dict(batch=3, n_q_heads=14, n_kv_heads=2), [16384, 9001, 2100]),
    # float32 path
    "tiny-f32": (0, dict(batch=3), [512, 300, 45]),
    # a sequence with no cached token at all (its own block only) between two others
    "8k-empty": (1, dict(batch=3, n_q_heads=8, n_kv_heads=8), [8192, 0, 1000]),
    # the 32K layer's shapes (64 blocks kept per KV head) at 8 heads
    "32k": (3, dict(batch=2, n_q_heads=8, n_kv_heads=8), [32768, 20000]),
}


@pytest.mark.parametrize("case", list(CASES))
def test_ragged_standalone_calls(case):
    """Pooling, scoring with sink detection, selection and sparse attention as separate calls."""
    require_gpu()
    from diffusion_long_context_amd import Handle
    from oracle.pipeline import focus_layer_step
    ci, kw, lens = CASES[case]
    cfg = get_config(ci).with_(**kw)
    x = _ragged(cfg, lens)
    print(f"ragged standalone {case} lens={lens}", flush=True)
    h = Handle()
    try:
        got = _focus(h, cfg, x, modes=("source", "reuse"), ctx_lens=lens)
    finally:
        h.close()
    for b, lb in enumerate(lens):
        cb, xb = _slice(cfg, x, b, lb)
        src = focus_layer_step(cb, xb, "source")
        assert src["sink_margin"] > 1e-4 * cfg.sink_tau, f"flagged case: sink margin {src['sink_margin']:.3g}"
        _check_seq(cfg, got["source"], src, b, lb, f"{case} b={b} source")
        reu = focus_layer_step(cb, xb, "reuse", sinks=(src["sink_pos"], src["n_sinks"]))
        _check_seq(cfg, got["reuse"], reu, b, lb, f"{case} b={b} reuse")


@pytest.mark.parametrize("case", ["8k-mha", "16k-gqa7", "8k-empty", "32k"])
def test_ragged_focus_step(case):
    """fdl_focus_step over dense, source and reuse layers: each sequence against the oracle's
    layer-by-layer run of that sequence alone."""
    require_gpu()
    from diffusion_long_context_amd import Handle
    ci, kw, lens = CASES[case]
    cfg = get_config(ci).with_(**kw)
    modes = ["dense", "source", "reuse", "reuse"]
    # the source layer takes the inputs seeded for layer 0, whose sink margins are clear of the
    # threshold in every sequence (seeded layer 1 of the 8K case has one within 1e-4 tau)
    xs = [_ragged(cfg, lens, layer=l) for l in (3, 0, 1, 2)]
    print(f"ragged focus step {case} lens={lens}", flush=True)
    h = Handle(workspace_bytes=512 << 20)
    try:
        got = focus_step_layers(h, cfg, xs, modes, xs[0]["prev_conf"], xs[0]["masked"], ctx_lens=lens)
    finally:
        h.close()
    for b, lb in enumerate(lens):
        slices = [_slice(cfg, x, b, lb) for x in xs]
        cb = slices[0][0]
        one = {"layers": {l: tuple(a[b:b + 1, :, :-(-lb // cfg.kv_block)] if i == 0 else a[b:b + 1]
                                   for i, a in enumerate(v)) for l, v in got["layers"].items()},
               "outs": [o[b:b + 1] for o in got["outs"]],
               "pred_mask": got["pred_mask"][b:b + 1], "n_pred": got["n_pred"][b:b + 1], "sink_pos": got["sink_pos"][b:b + 1],
               "n_sinks": got["n_sinks"][b:b + 1]}
        for l, v in got["layers"].items():
            assert np.all(v[0][b, :, -(-lb // cfg.kv_block):].view(np.uint32) == 0), (case, b, l)
        check_focus_step_layers(cb, one, [s[1] for s in slices], modes, slices[0][1]["prev_conf"],
                                slices[0][1]["masked"], what=f"{case} b={b}")


def test_ragged_lengths_checked():
    """A length outside [0, ctx_len] is clamped into it on the device (no fault, no read past the
    stride); ctx_lens with a paged cache, or with a call that takes no ragged batch, is
    FDL_EUNSUPPORTED."""
    require_gpu()
    from diffusion_long_context_amd import Handle
    from diffusion_long_context_amd.fdllm import FDL_EUNSUPPORTED, FdlError
    from diffusion_long_context_amd.step import geom_for
    from gpu_util import dev
    cfg = get_config(1).with_(batch=3, n_q_heads=4, n_kv_heads=4)
    lens_dev = dev(np.array([9000, -5, 4096], np.int32))
    x = _ragged(cfg, [8192, 0, 4096])
    h = Handle()
    try:
        g = geom_for(cfg, ctx_lens=lens_dev)
        ks = torch.zeros((3, 4, cfg.n_blk, cfg.head_dim), dtype=torch.float32, device="cuda")
        h.fdl_pool_keys(g, dev(x["k"]), None, cfg.kv_block, ks)
        torch.cuda.synchronize()
        assert h.fdl_get_status() == 0
        kh = ks.cpu().numpy()
        assert np.all(np.isfinite(kh[0])) and np.all(kh[1] == 0) and np.all(kh[2, :, 64:] == 0)
        pm = torch.full((3,), 0xF, dtype=torch.int64, device="cuda")
        with pytest.raises(FdlError) as e:
            h.fdl_score_blocks_max(g, dev(x["q"]), pm, ks, cfg.kv_block,
                                   torch.zeros((3, 4, cfg.n_blk), dtype=torch.float32, device="cuda"))
        assert e.value.status == FDL_EUNSUPPORTED
    finally:
        h.close()
