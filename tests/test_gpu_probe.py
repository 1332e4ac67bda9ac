"""fdl_bandwidth_probe, the streaming reference of the benchmark: every mode reads exactly the bytes it
claims to (the xor of its per-wave checksums equals the xor of those words, taken on the host), the
copy is exact, and malformed calls are FDL_EINVAL."""
import numpy as np
import pytest
import torch

from gpu_util import require_gpu

pytestmark = pytest.mark.gpu


def _xor_all(words: np.ndarray) -> int:
    return int(np.bitwise_xor.reduce(words.astype(np.uint32).ravel(), initial=np.uint32(0)))


def _checksum(chk: torch.Tensor, n_words: int) -> int:
    return _xor_all(chk[:n_words].cpu().numpy().view(np.uint32))


@pytest.fixture(scope="module")
def setup():
    require_gpu()
    from diffusion_long_context_amd import Handle
    h = Handle()
    n = 48 << 20   # bytes: not a multiple of any grid's stride, so the tails run too
    g = torch.Generator(device="cpu").manual_seed(11)
    src = torch.randint(-(1 << 31), (1 << 31) - 1, (n // 4,), dtype=torch.int32, generator=g).cuda()
    yield h, src, src.cpu().numpy().view(np.uint32)
    h.close()


@pytest.mark.parametrize("n_blocks", [0, 768, 1000])
def test_read_modes_read_every_word(setup, n_blocks):
    from diffusion_long_context_amd.fdllm import FDL_PROBE_READ, FDL_PROBE_READ_LDS
    h, src, words = setup
    nb = n_blocks or 4 * torch.cuda.get_device_properties(0).multi_processor_count
    chk = torch.zeros(nb * 8, dtype=torch.int32, device="cuda")
    h.fdl_bandwidth_probe(FDL_PROBE_READ, src, chk, n_blocks)
    torch.cuda.synchronize()
    assert _checksum(chk, nb * 8) == _xor_all(words)
    # LDS DMA: each wave folds the first 64 words of every 1 KiB fetch it made
    chk.zero_()
    h.fdl_bandwidth_probe(FDL_PROBE_READ_LDS, src, chk, n_blocks)
    torch.cuda.synchronize()
    assert _checksum(chk, nb * 8) == _xor_all(words.reshape(-1, 256)[:, :64])
    assert h.fdl_get_status() == 0


def test_tiles_mode_reads_its_regions(setup):
    """Workgroup w streams bytes [w r, (w + 1) r) of each half (r = half / n_blocks rounded down to
    8 KiB) as 8 KiB K + 8 KiB V tiles; each wave folds, per tile, the first 64 words of every other
    KiB of K and of V."""
    from diffusion_long_context_amd.fdllm import FDL_PROBE_TILES
    h, src, words = setup
    for nb in (0, 100):
        n_wg = nb or torch.cuda.get_device_properties(0).multi_processor_count
        half = words.size * 4 // 2
        region = (half // n_wg) & ~8191
        chk = torch.zeros(n_wg * 8, dtype=torch.int32, device="cuda")
        h.fdl_bandwidth_probe(FDL_PROBE_TILES, src, chk, nb)
        torch.cuda.synchronize()
        want = 0
        for part in (words[: half // 4], words[half // 4:]):
            tiles = part[: n_wg * region // 4].reshape(-1, 2048)   # 8 KiB per tile
            want ^= _xor_all(np.concatenate([tiles[:, 512 * j: 512 * j + 64] for j in range(4)], axis=1))
        assert _checksum(chk, n_wg * 8) == want
    assert h.fdl_get_status() == 0


def test_copy_is_exact(setup):
    from diffusion_long_context_amd.fdllm import FDL_PROBE_COPY
    h, src, _ = setup
    dst = torch.zeros_like(src)
    h.fdl_bandwidth_probe(FDL_PROBE_COPY, src, dst, 333)
    torch.cuda.synchronize()
    assert torch.equal(dst, src)


def test_malformed_calls_are_einval(setup):
    from diffusion_long_context_amd.fdllm import FDL_EINVAL, FDL_PROBE_READ, FDL_PROBE_TILES, FdlError
    h, src, _ = setup
    chk = torch.zeros(1 << 16, dtype=torch.int32, device="cuda")
    for mode, s, d, nb in ((4, src, chk, 0),                        # unknown mode
                           (FDL_PROBE_READ, src[:100], chk, 0),     # not a multiple of 1 KiB
                           (FDL_PROBE_READ, src, chk[:8], 0),       # checksum words do not fit
                           (FDL_PROBE_TILES, src[:4096], chk, 0),   # 16 KiB: no tile per workgroup
                           (FDL_PROBE_READ, src, chk, -1)):
        with pytest.raises(FdlError) as e:
            h.fdl_bandwidth_probe(mode, s, d, nb)
        assert e.value.status == FDL_EINVAL
