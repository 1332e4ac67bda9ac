"""The seeded generators: bf16 rounding, reproducibility and the workloads' planted structure."""
import numpy as np

from synth import get_config
from synth.gen import bf16_bits_to_f32, make_single, round_to_bf16, schedule_state, step_qkv


def test_round_to_bf16_nearest_even():
    one = np.float32(1.0)
    cases = [
        (1.0, 0x3F80),
        (1 + 2 ** -8, 0x3F80),               # tie -> even (down)
        (1 + 3 * 2 ** -8, 0x3F82),           # tie -> even (up)
        (1 + 2 ** -8 + 2 ** -20, 0x3F81),
        (-2.5, 0xC020),
        (0.0, 0x0000),
        (-0.0, 0x8000),
    ]
    got = round_to_bf16(np.array([v for v, _ in cases], dtype=np.float32))
    assert [int(g) for g in got] == [b for _, b in cases]
    assert one == bf16_bits_to_f32(np.uint16(0x3F80))


def test_reproducible():
    cfg = get_config(1)
    a = step_qkv(cfg, 0, 0, 0)
    b = step_qkv(cfg, 0, 0, 0)
    c = step_qkv(cfg, 1, 0, 0)
    assert np.array_equal(a["q"], b["q"]) and not np.array_equal(a["q"], c["q"])


def test_tiny_sink_direction():
    cfg = get_config(0)
    x = make_single(cfg)
    k0 = x["k"][0, :, 0].astype(np.float64)
    u0 = k0[0] / np.linalg.norm(k0[0])
    u1 = k0[1] / np.linalg.norm(k0[1])
    assert np.allclose(u0, u1, atol=1e-6)          # shared direction
    assert np.linalg.norm(k0[0]) > 5 * np.linalg.norm(x["k"][0, 0, 1])


def test_masked_count_and_schedule():
    cfg = get_config(1)
    x = make_single(cfg)
    assert int(x["masked"].sum()) == cfg.n_masked
    c3 = get_config(3)
    for step in (0, 1, 31, 32, 255):
        st = schedule_state(c3, step)
        assert int(st["masked"].sum()) == c3.dec_len - st["s"]
        assert (st["prev_conf"] is None) == (st["s"] == 0)
