"""The C ABI library loads and exports every symbol include/libfdllm.h declares; host-side argument
checks that need no GPU (NULL handle / NULL arguments) return FDL_EINVAL."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    with open(os.path.join(ROOT, "include", "libfdllm.h")) as f:
        src = f.read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(fdl_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    from diffusion_long_context_amd.fdllm import LIB_PATH, load
    if not os.path.exists(LIB_PATH):
        pytest.fail("libfdllm.so is not built: run `python -m diffusion_long_context_amd.build`")
    return load()


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert len(names) >= 12, names
    for n in names:
        assert hasattr(lib, n), n


def test_binding_covers_every_declaration():
    from diffusion_long_context_amd.fdllm import EXPORTED
    assert sorted(EXPORTED) == _declared()


def test_null_handle_is_einval(lib):
    from diffusion_long_context_amd.fdllm import FDL_EINVAL
    assert lib.fdl_destroy(None) == FDL_EINVAL
    assert lib.fdl_get_status(None) == FDL_EINVAL
    assert lib.fdl_set_stream(None, None) == FDL_EINVAL
    assert lib.fdl_predict_queries(None, 1, 32, None, None, 4, 4, None, None) == FDL_EINVAL
    assert lib.fdl_pool_keys(None, None, None, None, 64, None) == FDL_EINVAL
    assert lib.fdl_cache_write(None, None, None, None, 0, 1, None, None, None, 64, None) == FDL_EINVAL
    assert lib.fdl_score_blocks(None, None, None, None, None, 64, None, 0, None, None, None, None, 0,
                                0.03, 64, None, None) == FDL_EINVAL
    assert lib.fdl_select_blocks(None, None, None, 0, 64, None, None, 0, None, 0, 4, 0, 4, None,
                                 None) == FDL_EINVAL
    assert lib.fdl_score_select_tokens(None, None, None, None, None, None, 2048, None, 4, 512, 2052, None, None,
                                       None) == FDL_EINVAL
    assert lib.fdl_select_chunks_tokens(None, None, None, None, None, None, None, 2048, 4, 512, 2052, None, None,
                                        None, None, None, None) == FDL_EINVAL
    assert lib.fdl_score_blocks_max(None, None, None, None, None, 64, None) == FDL_EINVAL
    assert lib.fdl_sparse_attn(None, None, None, None, None, None, None, None, None, None, 1, 64,
                               None) == FDL_EINVAL
    assert lib.fdl_dense_attn(None, None, None, None, None, None, None, None, None) == FDL_EINVAL
    assert lib.fdl_create(None, None, 0) == FDL_EINVAL
    # the measurement and diagnostic calls check their handle first as well
    assert lib.fdl_bandwidth_probe(None, 0, None, 1024, None, 1024, 0) == FDL_EINVAL
    assert lib.fdl_set_phase_buffer(None, None, 0) == FDL_EINVAL
    assert lib.fdl_profile_begin(None, 1, 0, 1) == FDL_EINVAL
    assert lib.fdl_profile_end(None, None, None) == FDL_EINVAL
    assert lib.fdl_unmask(None, 1, 32, None, None, 1, None) == FDL_EINVAL
    assert lib.fdl_capture_begin(None) == FDL_EINVAL


def test_status_strings(lib):
    for s in range(-7, 1):
        assert lib.fdl_status_string(s)
    assert lib.fdl_last_error(None) == b"no handle"


def test_product_path_does_not_import_oracle():
    pkg = os.path.join(ROOT, "diffusion_long_context_amd")
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".hip", ".h", ".cpp")):
                with open(os.path.join(dirpath, fn)) as f:
                    src = f.read()
                assert "import oracle" not in src and "from oracle" not in src, fn
                assert "oracle/" not in src, fn
