"""libfdllm: confidence-guided, sink-aware block-sparse attention for diffusion-LLM decoding over a
long cached bidirectional KV context, on AMD MI355X (gfx950).

The compute lives in ``libfdllm.so`` (HIP kernels behind a C ABI, ``include/libfdllm.h``);
``fdllm`` is its ctypes binding and ``step`` chains the calls of one layer-step.
"""
from .fdllm import (FDL_BF16, FDL_F32, FdlError, Geom, Handle, load)  # noqa: F401

__all__ = ["FDL_BF16", "FDL_F32", "FdlError", "Geom", "Handle", "load"]
