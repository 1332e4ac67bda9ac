"""Thin Python binding of libfdllm (ctypes).

Argument marshalling only: every function below checks that the tensors it is handed are CUDA
(HIP) tensors, contiguous and large enough for the geometry, then passes raw device pointers and the
current torch stream to the C call of the same name.  All arithmetic runs in the library's HIP
kernels.  PyTorch only provides device memory and the stream.

The library must have been built (``python -m diffusion_long_context_amd.build``); loading fails
loudly otherwise -- there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# FDLLM_LIB selects another build of the same library (the phase-stamp, debug or sanitized variant)
LIB_PATH = os.environ.get("FDLLM_LIB") or os.path.join(_HERE, "libfdllm.so")

FDL_OK, FDL_EINVAL, FDL_ENOMEM, FDL_EHIP, FDL_EOVERFLOW, FDL_EUNSUPPORTED, FDL_EINDEX = 0, -1, -2, -3, -4, -5, -6
FDL_ESYNC = -7
FDL_F32, FDL_BF16 = 0, 1

EXPORTED = (
    "fdl_create", "fdl_destroy", "fdl_set_stream", "fdl_get_status", "fdl_get_status_bits",
    "fdl_status_string",
    "fdl_last_error", "fdl_pool_keys", "fdl_cache_write", "fdl_predict_queries", "fdl_score_blocks",
    "fdl_score_blocks_max", "fdl_score_blocks_mass", "fdl_select_blocks", "fdl_select_blocks_shared", "fdl_expand_tokens", "fdl_score_select_tokens", "fdl_select_chunks_tokens", "fdl_sparse_attn", "fdl_dense_attn", "fdl_focus_step",
    "fdl_unmask", "fdl_decode_steps", "fdl_capture_begin", "fdl_capture_end", "fdl_graph_launch",
    "fdl_graph_destroy", "fdl_profile_begin", "fdl_profile_end", "fdl_bandwidth_probe",
    "fdl_sparse_attn_noalloc", "fdl_set_phase_buffer", "fdl_phase_stamps_built",
)

FDL_LAYER_DENSE, FDL_LAYER_SOURCE, FDL_LAYER_REUSE = 0, 1, 2
FDL_PROBE_READ, FDL_PROBE_READ_LDS, FDL_PROBE_COPY, FDL_PROBE_TILES = 0, 1, 2, 3
PROF_KINDS = ("predict", "pool", "score", "sinks", "select", "sparse_attn", "dense_attn",
              "layer_dense", "layer_source", "layer_reuse", "reuse_run")


class FdlError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"libfdllm status {status}: {msg}")
        self.status = status


class fdl_geom(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "n_q_heads", "n_kv_heads", "head_dim", "ctx_len", "kv_block", "dec_len", "dtype",
        "paged", "page_tokens", "pages_per_seq", "n_pages")] + [("ctx_lens", ctypes.c_void_p)]


class fdl_layer_io(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p),
                ("k_dec", ctypes.c_void_p), ("v_dec", ctypes.c_void_p), ("ks", ctypes.c_void_p),
                ("out", ctypes.c_void_p), ("mode", ctypes.c_int32)]


class fdl_focus_params(ctypes.Structure):
    _fields_ = [("top_k_pos", ctypes.c_int32), ("window", ctypes.c_int32),
                ("top_k_blocks", ctypes.c_int32), ("max_sinks", ctypes.c_int32),
                ("max_sel", ctypes.c_int32), ("sink_tau", ctypes.c_float)]


_P = ctypes.c_void_p
_I = ctypes.c_int32
_SIGS = {
    "fdl_create": (_I, [ctypes.POINTER(_P), _P, ctypes.c_size_t]),
    "fdl_destroy": (_I, [_P]),
    "fdl_set_stream": (_I, [_P, _P]),
    "fdl_get_status": (_I, [_P]),
    "fdl_get_status_bits": (_I, [_P, ctypes.POINTER(ctypes.c_uint32)]),
    "fdl_status_string": (ctypes.c_char_p, [_I]),
    "fdl_last_error": (ctypes.c_char_p, [_P]),
    "fdl_pool_keys": (_I, [_P, ctypes.POINTER(fdl_geom), _P, _P, _I, _P]),
    "fdl_cache_write": (_I, [_P, ctypes.POINTER(fdl_geom), _P, _P, _I, _I, _P, _P, _P, _I, _P]),
    "fdl_predict_queries": (_I, [_P, _I, _I, _P, _P, _I, _I, _P, _P]),
    "fdl_score_blocks": (_I, [_P, ctypes.POINTER(fdl_geom), _P, _P, _P, _I, _P, _I, _P, _P, _P, _P, _I,
                              ctypes.c_float, _I, _P, _P]),
    "fdl_score_blocks_max": (_I, [_P, ctypes.POINTER(fdl_geom), _P, _P, _P, _I, _P]),
    "fdl_score_blocks_mass": (_I, [_P, ctypes.POINTER(fdl_geom), _P, _P, _P, _I, _P]),
    "fdl_select_blocks": (_I, [_P, ctypes.POINTER(fdl_geom), _P, _I, _I, _P, _P, _I, _P, _I, _I, _I, _I,
                               _P, _P]),
    "fdl_expand_tokens": (_I, [_P, ctypes.POINTER(fdl_geom), _P, _P, _I, _I, _P, _P, _I, _P, _P, _I]),
    "fdl_select_blocks_shared": (_I, [_P, ctypes.POINTER(fdl_geom), _P, _I, _I, _P, _P, _I, _I, _I, _P, _P]),
    "fdl_score_select_tokens": (_I, [_P, ctypes.POINTER(fdl_geom), _P, _P, _P, _P, _I, _P, _I, _I, _I, _P, _P,
                                     _P]),
    "fdl_select_chunks_tokens": (_I, [_P, ctypes.POINTER(fdl_geom), _P, _P, _P, _P, _P, _I, _I, _I, _I, _P, _P,
                                      _P, _P, _P, _P]),
    "fdl_sparse_attn": (_I, [_P, ctypes.POINTER(fdl_geom), _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _P]),
    "fdl_dense_attn": (_I, [_P, ctypes.POINTER(fdl_geom), _P, _P, _P, _P, _P, _P, _P]),
    "fdl_focus_step": (_I, [_P, ctypes.POINTER(fdl_geom), ctypes.POINTER(fdl_focus_params), _P, _P, _I,
                            ctypes.POINTER(fdl_layer_io), _P, _P, _P, _P, _P, _P, _P]),
    "fdl_unmask": (_I, [_P, _I, _I, _P, _P, _I, _P]),
    "fdl_decode_steps": (_I, [_P, ctypes.POINTER(fdl_geom), ctypes.POINTER(fdl_focus_params), _I, _P, _P, _P, _I,
                              _P, _I, ctypes.POINTER(fdl_layer_io), _P, _P, _P, _P, _P, _P, _P]),
    "fdl_capture_begin": (_I, [_P]),
    "fdl_capture_end": (_I, [_P, ctypes.POINTER(_P)]),
    "fdl_graph_launch": (_I, [_P, _P]),
    "fdl_graph_destroy": (_I, [_P]),
    "fdl_profile_begin": (_I, [_P, _I, ctypes.c_uint32, _I]),
    "fdl_profile_end": (_I, [_P, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]),
    "fdl_bandwidth_probe": (_I, [_P, _I, _P, ctypes.c_size_t, _P, ctypes.c_size_t, _I]),
    "fdl_set_phase_buffer": (_I, [_P, _P, ctypes.c_int64]),
    "fdl_phase_stamps_built": (_I, []),
    "fdl_sparse_attn_noalloc": (_I, [_P, ctypes.POINTER(fdl_geom), _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _P, _P]),
}

_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libfdllm.so once; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise FdlError(FDL_EINVAL, f"{path} not found: build it with "
                                   "`python -m diffusion_long_context_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


@dataclass(frozen=True)
class Geom:
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ctx_len: int
    kv_block: int
    dec_len: int
    dtype: int = FDL_BF16
    paged: int = 0
    page_tokens: int = 0
    pages_per_seq: int = 0
    n_pages: int = 0
    ctx_lens: object = None   # device int32 tensor [batch] of per-sequence lengths, or None

    def c(self) -> fdl_geom:
        ints = [int(getattr(self, f)) for f, _ in fdl_geom._fields_[:-1]]
        return fdl_geom(*ints, _ptr(self.ctx_lens, 4 * self.batch, "ctx_lens"))

    @property
    def elem(self) -> int:
        return 4 if self.dtype == FDL_F32 else 2

    @property
    def kv_elems(self) -> int:
        if self.paged:
            return self.n_pages * self.n_kv_heads * self.page_tokens * self.head_dim
        return self.batch * self.n_kv_heads * self.ctx_len * self.head_dim


def _ptr(t, nbytes: int | None = None, name: str = "tensor"):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if nbytes is not None and t.numel() * t.element_size() < nbytes:
        raise ValueError(f"{name} holds {t.numel() * t.element_size()} bytes, needs {nbytes}")
    return ctypes.c_void_p(t.data_ptr())


def _stream_ptr():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def fdl_sparse_attn_noalloc(g: "Geom", q, k_cache, v_cache, k_dec, v_dec, page_table, sel_idx, n_sel,
                            max_sel: int, sel_unit_tokens: int, out, status=None):
    """The allocation-free sparse attention on the current torch stream (no handle); raises FdlError
    with the status code on an argument error."""
    lib = load()
    B, D, Hkv = g.batch, g.head_dim, g.n_kv_heads
    qbytes = B * g.n_q_heads * g.dec_len * D * g.elem
    dbytes = B * Hkv * g.dec_len * D * g.elem
    kv = g.kv_elems * g.elem if g.ctx_len > 0 else None
    st = lib.fdl_sparse_attn_noalloc(
        _stream_ptr(), ctypes.byref(g.c()), _ptr(q, qbytes, "q"), _ptr(k_cache, kv, "k_cache"),
        _ptr(v_cache, kv, "v_cache"), _ptr(k_dec, dbytes, "k_dec"), _ptr(v_dec, dbytes, "v_dec"),
        _ptr(page_table, 4 * B * g.pages_per_seq if g.paged else None, "page_table"),
        _ptr(sel_idx, 4 * B * Hkv * max_sel, "sel_idx"), _ptr(n_sel, 4 * B * Hkv, "n_sel"), max_sel,
        sel_unit_tokens, _ptr(out, qbytes, "out"), _ptr(status, 4, "status"))
    if st != FDL_OK:
        raise FdlError(st, lib.fdl_status_string(st).decode())


class Handle:
    """An fdl_handle bound to the current device and torch stream."""

    def __init__(self, workspace_bytes: int = 0):
        lib = load()
        h = ctypes.c_void_p()
        st = lib.fdl_create(ctypes.byref(h), _stream_ptr(), workspace_bytes)
        if st != FDL_OK:
            raise FdlError(st, lib.fdl_status_string(st).decode())
        self.h = h
        self.lib = lib

    def close(self):
        if self.h:
            self.lib.fdl_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _check(self, st: int):
        if st != FDL_OK:
            msg = self.lib.fdl_last_error(self.h).decode() or self.lib.fdl_status_string(st).decode()
            raise FdlError(st, msg)

    def sync_stream(self):
        self.lib.fdl_set_stream(self.h, _stream_ptr())

    # ---- the C calls ------------------------------------------------------------------------

    def fdl_get_status(self) -> int:
        self.sync_stream()
        return self.lib.fdl_get_status(self.h)

    def fdl_get_status_bits(self) -> tuple[int, int]:
        """(status, raw FDL_FLAG_* bits); clears them like fdl_get_status."""
        self.sync_stream()
        bits = ctypes.c_uint32(0)
        st = self.lib.fdl_get_status_bits(self.h, ctypes.byref(bits))
        return st, bits.value

    def fdl_pool_keys(self, g: Geom, k_cache, page_table, unit_tokens: int, ks):
        self.sync_stream()
        n_units = -(-g.ctx_len // unit_tokens)
        self._check(self.lib.fdl_pool_keys(
            self.h, ctypes.byref(g.c()), _ptr(k_cache, g.kv_elems * g.elem, "k_cache"),
            _ptr(page_table, 4 * g.batch * g.pages_per_seq if g.paged else None, "page_table"),
            unit_tokens, _ptr(ks, 4 * g.batch * g.n_kv_heads * n_units * g.head_dim, "ks")))

    def fdl_cache_write(self, g: Geom, k_new, v_new, t0: int, k_cache, v_cache, page_table, unit_tokens: int,
                        ks=None):
        """Write rows [t0, t0 + n_tok) of k_new / v_new [B][Hkv][n_tok][D] into the cache and, with ks,
        re-pool the units they touch."""
        self.sync_stream()
        B, Hkv, D = g.batch, g.n_kv_heads, g.head_dim
        n_tok = k_new.shape[2]
        nbytes = B * Hkv * n_tok * D * g.elem
        n_units = -(-g.ctx_len // unit_tokens)
        self._check(self.lib.fdl_cache_write(
            self.h, ctypes.byref(g.c()), _ptr(k_new, nbytes, "k_new"), _ptr(v_new, nbytes, "v_new"), t0, n_tok,
            _ptr(k_cache, g.kv_elems * g.elem, "k_cache"), _ptr(v_cache, g.kv_elems * g.elem, "v_cache"),
            _ptr(page_table, 4 * B * g.pages_per_seq if g.paged else None, "page_table"), unit_tokens,
            _ptr(ks, 4 * B * Hkv * n_units * D, "ks") if ks is not None else None))

    def fdl_predict_queries(self, batch: int, dec_len: int, prev_conf, masked, top_k: int, window: int,
                            pred_mask, n_pred):
        self.sync_stream()
        self._check(self.lib.fdl_predict_queries(
            self.h, batch, dec_len, _ptr(prev_conf, 4 * batch * dec_len, "prev_conf"),
            _ptr(masked, batch * dec_len, "masked"), top_k, window,
            _ptr(pred_mask, 8 * batch, "pred_mask"), _ptr(n_pred, 4 * batch, "n_pred")))

    def fdl_score_blocks(self, g: Geom, q, pred_mask, ks, unit_tokens: int, scores, cand_idx=None,
                         n_cand: int = 0, k_cache=None, k_dec=None, page_table=None,
                         detect_sinks: bool = False, sink_tau: float = 0.03, max_sinks: int = 64,
                         sink_pos=None, n_sinks=None):
        self.sync_stream()
        B, Hkv, D = g.batch, g.n_kv_heads, g.head_dim
        n_units = -(-g.ctx_len // unit_tokens)
        qbytes = B * g.n_q_heads * g.dec_len * D * g.elem
        sbytes = 4 * B * Hkv * (n_cand * unit_tokens if cand_idx is not None else n_units)
        self._check(self.lib.fdl_score_blocks(
            self.h, ctypes.byref(g.c()), _ptr(q, qbytes, "q"), _ptr(pred_mask, 8 * B, "pred_mask"),
            _ptr(ks, 4 * B * Hkv * n_units * D if cand_idx is None else None, "ks"), unit_tokens,
            _ptr(cand_idx, 4 * B * Hkv * n_cand, "cand_idx"), n_cand,
            _ptr(k_cache, g.kv_elems * g.elem, "k_cache"),
            _ptr(k_dec, B * Hkv * g.dec_len * D * g.elem, "k_dec"),
            _ptr(page_table, 4 * B * g.pages_per_seq if g.paged else None, "page_table"),
            _ptr(scores, sbytes, "scores"), 1 if detect_sinks else 0, float(sink_tau), max_sinks,
            _ptr(sink_pos, 4 * B * max_sinks, "sink_pos"), _ptr(n_sinks, 4 * B, "n_sinks")))

    def fdl_score_blocks_max(self, g: Geom, q, pred_mask, ks, unit_tokens: int, scores):
        self.sync_stream()
        B, Hkv = g.batch, g.n_kv_heads
        n_units = -(-g.ctx_len // unit_tokens)
        self._check(self.lib.fdl_score_blocks_max(
            self.h, ctypes.byref(g.c()), _ptr(q, B * g.n_q_heads * g.dec_len * g.head_dim * g.elem, "q"),
            _ptr(pred_mask, 8 * B, "pred_mask"), _ptr(ks, 4 * B * Hkv * n_units * g.head_dim, "ks"), unit_tokens,
            _ptr(scores, 4 * B * Hkv * n_units, "scores")))

    def fdl_score_blocks_mass(self, g: Geom, q, pred_mask, ks, unit_tokens: int, scores):
        self.sync_stream()
        B, Hkv = g.batch, g.n_kv_heads
        n_units = -(-g.ctx_len // unit_tokens)
        self._check(self.lib.fdl_score_blocks_mass(
            self.h, ctypes.byref(g.c()), _ptr(q, B * g.n_q_heads * g.dec_len * g.head_dim * g.elem, "q"),
            _ptr(pred_mask, 8 * B, "pred_mask"), _ptr(ks, 4 * B * Hkv * n_units * g.head_dim, "ks"), unit_tokens,
            _ptr(scores, 4 * B * Hkv * n_units, "scores")))

    def fdl_select_blocks(self, g: Geom, scores, n_units: int, unit_tokens: int, sink_pos, n_sinks,
                          max_sinks: int, top_k: int, max_sel: int, sel_idx, n_sel, cand_idx=None,
                          n_cand: int = 0, force_first: bool = False):
        self.sync_stream()
        B, Hkv = g.batch, g.n_kv_heads
        sbytes = 4 * B * Hkv * (n_cand * unit_tokens if cand_idx is not None else n_units)
        self._check(self.lib.fdl_select_blocks(
            self.h, ctypes.byref(g.c()), _ptr(scores, sbytes, "scores"), n_units, unit_tokens,
            _ptr(sink_pos, 4 * B * max_sinks, "sink_pos"), _ptr(n_sinks, 4 * B, "n_sinks"), max_sinks,
            _ptr(cand_idx, 4 * B * Hkv * n_cand, "cand_idx"), n_cand, top_k, 1 if force_first else 0,
            max_sel, _ptr(sel_idx, 4 * B * Hkv * max_sel, "sel_idx"), _ptr(n_sel, 4 * B * Hkv, "n_sel")))

    def fdl_select_blocks_shared(self, g: Geom, scores, n_units: int, unit_tokens: int, sink_pos, n_sinks,
                                 max_sinks: int, top_k: int, max_sel: int, sel_idx, n_sel):
        self.sync_stream()
        B, Hkv = g.batch, g.n_kv_heads
        self._check(self.lib.fdl_select_blocks_shared(
            self.h, ctypes.byref(g.c()), _ptr(scores, 4 * B * Hkv * n_units, "scores"), n_units, unit_tokens,
            _ptr(sink_pos, 4 * B * max_sinks, "sink_pos"), _ptr(n_sinks, 4 * B, "n_sinks"), max_sinks, top_k,
            max_sel, _ptr(sel_idx, 4 * B * Hkv * max_sel, "sel_idx"), _ptr(n_sel, 4 * B * Hkv, "n_sel")))

    def fdl_expand_tokens(self, g: Geom, sel_idx, n_sel, max_sel: int, unit_tokens: int, sink_pos, n_sinks,
                          max_sinks: int, tok_idx, n_tok, max_tok: int):
        self.sync_stream()
        B, Hkv = g.batch, g.n_kv_heads
        self._check(self.lib.fdl_expand_tokens(
            self.h, ctypes.byref(g.c()), _ptr(sel_idx, 4 * B * Hkv * max_sel, "sel_idx"), _ptr(n_sel, 4 * B * Hkv, "n_sel"),
            max_sel, unit_tokens, _ptr(sink_pos, 4 * B * max_sinks, "sink_pos"), _ptr(n_sinks, 4 * B, "n_sinks"),
            max_sinks, _ptr(tok_idx, 4 * B * Hkv * max_tok, "tok_idx"), _ptr(n_tok, 4 * B * Hkv, "n_tok"), max_tok))

    def fdl_score_select_tokens(self, g: Geom, q, pred_mask, k_cache, page_table, unit_tokens: int, cand_idx,
                                n_cand: int, top_k: int, max_sel: int, scores, sel_idx, n_sel):
        self.sync_stream()
        B, Hkv = g.batch, g.n_kv_heads
        self._check(self.lib.fdl_score_select_tokens(
            self.h, ctypes.byref(g.c()), _ptr(q, B * g.n_q_heads * g.dec_len * g.head_dim * g.elem, "q"),
            _ptr(pred_mask, 8 * B, "pred_mask"), _ptr(k_cache, g.kv_elems * g.elem, "k_cache"),
            _ptr(page_table, 4 * B * g.pages_per_seq if g.paged else None, "page_table"), unit_tokens,
            _ptr(cand_idx, 4 * B * Hkv * n_cand, "cand_idx"), n_cand, top_k, max_sel,
            _ptr(scores, 4 * B * Hkv * n_cand * unit_tokens, "scores"), _ptr(sel_idx, 4 * B * Hkv * max_sel, "sel_idx"),
            _ptr(n_sel, 4 * B * Hkv, "n_sel")))

    def fdl_select_chunks_tokens(self, g: Geom, q, pred_mask, chunk_sums, k_cache, page_table, chunk_tokens: int,
                                 top_k_chunks: int, top_k: int, max_sel: int, chunk_scores, chunks, n_chunks_sel,
                                 token_scores, sel_idx, n_sel):
        self.sync_stream()
        B, Hkv = g.batch, g.n_kv_heads
        nc = g.ctx_len // chunk_tokens
        self._check(self.lib.fdl_select_chunks_tokens(
            self.h, ctypes.byref(g.c()), _ptr(q, B * g.n_q_heads * g.dec_len * g.head_dim * g.elem, "q"),
            _ptr(pred_mask, 8 * B, "pred_mask"), _ptr(chunk_sums, 4 * B * Hkv * nc * g.head_dim, "chunk_sums"),
            _ptr(k_cache, g.kv_elems * g.elem, "k_cache"),
            _ptr(page_table, 4 * B * g.pages_per_seq if g.paged else None, "page_table"), chunk_tokens,
            top_k_chunks, top_k, max_sel, _ptr(chunk_scores, 4 * B * Hkv * nc, "chunk_scores"),
            _ptr(chunks, 4 * B * Hkv * top_k_chunks, "chunks"), _ptr(n_chunks_sel, 4 * B * Hkv, "n_chunks_sel"),
            _ptr(token_scores, 4 * B * Hkv * top_k_chunks * chunk_tokens, "token_scores"),
            _ptr(sel_idx, 4 * B * Hkv * max_sel, "sel_idx"), _ptr(n_sel, 4 * B * Hkv, "n_sel")))

    def _attn_ptrs(self, g: Geom, q, k_cache, v_cache, k_dec, v_dec, page_table, out):
        B, D = g.batch, g.head_dim
        qbytes = B * g.n_q_heads * g.dec_len * D * g.elem
        dbytes = B * g.n_kv_heads * g.dec_len * D * g.elem
        kv = g.kv_elems * g.elem if g.ctx_len > 0 else None
        return (_ptr(q, qbytes, "q"), _ptr(k_cache, kv, "k_cache"), _ptr(v_cache, kv, "v_cache"),
                _ptr(k_dec, dbytes, "k_dec"), _ptr(v_dec, dbytes, "v_dec"),
                _ptr(page_table, 4 * B * g.pages_per_seq if g.paged else None, "page_table"),
                _ptr(out, qbytes, "out"))

    def fdl_sparse_attn(self, g: Geom, q, k_cache, v_cache, k_dec, v_dec, page_table, sel_idx, n_sel,
                        max_sel: int, sel_unit_tokens: int, out):
        self.sync_stream()
        qp, kp, vp, kdp, vdp, ptp, op = self._attn_ptrs(g, q, k_cache, v_cache, k_dec, v_dec, page_table, out)
        B, Hkv = g.batch, g.n_kv_heads
        self._check(self.lib.fdl_sparse_attn(
            self.h, ctypes.byref(g.c()), qp, kp, vp, kdp, vdp, ptp,
            _ptr(sel_idx, 4 * B * Hkv * max_sel, "sel_idx"), _ptr(n_sel, 4 * B * Hkv, "n_sel"),
            max_sel, sel_unit_tokens, op))

    def fdl_dense_attn(self, g: Geom, q, k_cache, v_cache, k_dec, v_dec, page_table, out):
        self.sync_stream()
        qp, kp, vp, kdp, vdp, ptp, op = self._attn_ptrs(g, q, k_cache, v_cache, k_dec, v_dec, page_table, out)
        self._check(self.lib.fdl_dense_attn(self.h, ctypes.byref(g.c()), qp, kp, vp, kdp, vdp, ptp, op))

    # ---- whole step and timing ------------------------------------------------------------------

    def make_layers(self, g: Geom, layers) -> "ctypes.Array":
        """layers: list of dicts with q, k_cache, v_cache, k_dec, v_dec, ks (or None), out, mode.
        Returns a ctypes array that fdl_focus_step can be called with repeatedly."""
        B, D = g.batch, g.head_dim
        qbytes = B * g.n_q_heads * g.dec_len * D * g.elem
        dbytes = B * g.n_kv_heads * g.dec_len * D * g.elem
        kv = g.kv_elems * g.elem if g.ctx_len > 0 else None
        n_blk = -(-g.ctx_len // g.kv_block)
        arr = (fdl_layer_io * len(layers))()
        for i, L in enumerate(layers):
            arr[i] = fdl_layer_io(
                _ptr(L["q"], qbytes, "q"), _ptr(L["k_cache"], kv, "k_cache"), _ptr(L["v_cache"], kv, "v_cache"),
                _ptr(L["k_dec"], dbytes, "k_dec"), _ptr(L["v_dec"], dbytes, "v_dec"),
                _ptr(L.get("ks"), 4 * B * g.n_kv_heads * n_blk * D, "ks"), _ptr(L["out"], qbytes, "out"),
                int(L["mode"]))
        return arr

    def fdl_focus_step(self, g: Geom, params: fdl_focus_params, prev_conf, masked, layers_arr, pred_mask,
                       n_pred, scores, sink_pos, n_sinks, sel_idx, n_sel):
        """One denoising step over len(layers_arr) layers (see make_layers).  Pointers are trusted to
        have been checked by make_layers / the caller's allocation."""
        self.sync_stream()
        B, Hkv = g.batch, g.n_kv_heads
        n_blk = -(-g.ctx_len // g.kv_block)
        self._check(self.lib.fdl_focus_step(
            self.h, ctypes.byref(g.c()), ctypes.byref(params), _ptr(prev_conf, 4 * B * g.dec_len, "prev_conf"),
            _ptr(masked, B * g.dec_len, "masked"), len(layers_arr), layers_arr,
            _ptr(pred_mask, 8 * B, "pred_mask"), _ptr(n_pred, 4 * B, "n_pred"),
            _ptr(scores, 4 * B * Hkv * n_blk, "scores"), _ptr(sink_pos, 4 * B * params.max_sinks, "sink_pos"),
            _ptr(n_sinks, 4 * B, "n_sinks"), _ptr(sel_idx, 4 * B * Hkv * params.max_sel, "sel_idx"),
            _ptr(n_sel, 4 * B * Hkv, "n_sel")))

    # ---- the decode loop ---------------------------------------------------------------------

    def fdl_unmask(self, batch: int, dec_len: int, conf, masked, n_unmask: int = 1, decoded=None):
        self.sync_stream()
        self._check(self.lib.fdl_unmask(self.h, batch, dec_len, _ptr(conf, 4 * batch * dec_len, "conf"),
                                        _ptr(masked, batch * dec_len, "masked"), n_unmask,
                                        _ptr(decoded, 4 * batch * n_unmask, "decoded")))

    def fdl_decode_steps(self, g: Geom, params: fdl_focus_params, n_steps: int, prev_conf0, conf, masked,
                         n_unmask: int, decoded, layers_arr, pred_mask, n_pred, scores, sink_pos, n_sinks,
                         sel_idx, n_sel):
        """n_steps steps of one block: layers_arr holds n_steps tables of equal length, step-major
        (make_layers over the concatenated lists)."""
        self.sync_stream()
        if n_steps > 0 and len(layers_arr) % n_steps:
            raise ValueError("layers_arr must hold n_steps tables of equal length")
        n_layers = len(layers_arr) // n_steps if n_steps > 0 else 0
        B, T, Hkv = g.batch, g.dec_len, g.n_kv_heads
        n_blk = -(-g.ctx_len // g.kv_block)
        self._check(self.lib.fdl_decode_steps(
            self.h, ctypes.byref(g.c()), ctypes.byref(params), n_steps, _ptr(prev_conf0, 4 * B * T, "prev_conf0"),
            _ptr(conf, 4 * n_steps * B * T, "conf"), _ptr(masked, B * T, "masked"), n_unmask,
            _ptr(decoded, 4 * n_steps * B * n_unmask, "decoded"), n_layers, layers_arr,
            _ptr(pred_mask, 8 * B, "pred_mask"), _ptr(n_pred, 4 * B, "n_pred"),
            _ptr(scores, 4 * B * Hkv * n_blk, "scores"), _ptr(sink_pos, 4 * B * params.max_sinks, "sink_pos"),
            _ptr(n_sinks, 4 * B, "n_sinks"), _ptr(sel_idx, 4 * B * Hkv * params.max_sel, "sel_idx"),
            _ptr(n_sel, 4 * B * Hkv, "n_sel")))

    def fdl_capture_begin(self):
        """Start capturing the current torch stream (not the default stream)."""
        self.sync_stream()
        self._check(self.lib.fdl_capture_begin(self.h))

    def fdl_capture_end(self) -> ctypes.c_void_p:
        out = _P()
        self._check(self.lib.fdl_capture_end(self.h, ctypes.byref(out)))
        return out

    def fdl_graph_launch(self, graph):
        self.sync_stream()
        self._check(self.lib.fdl_graph_launch(self.h, graph))

    def fdl_graph_destroy(self, graph):
        self._check(self.lib.fdl_graph_destroy(graph))

    def fdl_profile_begin(self, max_records: int, kinds=PROF_KINDS, every: int = 1):
        self.sync_stream()
        mask = 0
        for k in kinds:
            mask |= 1 << PROF_KINDS.index(k)
        self._check(self.lib.fdl_profile_begin(self.h, max_records, mask, every))

    def fdl_profile_end(self) -> dict:
        self.sync_stream()
        tot = (ctypes.c_double * len(PROF_KINDS))()
        cnt = (ctypes.c_int64 * len(PROF_KINDS))()
        self._check(self.lib.fdl_profile_end(self.h, tot, cnt))
        return {k: (tot[i], cnt[i]) for i, k in enumerate(PROF_KINDS)}

    def fdl_bandwidth_probe(self, mode: int, src, dst, n_blocks: int = 0):
        """Stream all of src once (mode FDL_PROBE_READ / _READ_LDS / _COPY); see the header."""
        self.sync_stream()
        nbytes = src.numel() * src.element_size()
        self._check(self.lib.fdl_bandwidth_probe(self.h, mode, _ptr(src, None, "src"), nbytes,
                                                 _ptr(dst, None, "dst"), dst.numel() * dst.element_size(),
                                                 n_blocks))

    def fdl_set_phase_buffer(self, stamps=None):
        """Phase timestamps of the fused kernel into stamps (device int64 tensor) or off (None)."""
        n = stamps.numel() if stamps is not None else 0
        self._check(self.lib.fdl_set_phase_buffer(self.h, _ptr(stamps, None, "stamps"), n))
