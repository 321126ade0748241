"""ctypes binding of libmiattn (argument marshalling only).

Every entry point has the name and argument order of its C declaration in
``include/miattn.h``. Tensor arguments may be torch tensors (their
``data_ptr()`` is passed) or raw integer device addresses; ``stream`` may be a
``torch.cuda.Stream``, a raw ``hipStream_t`` integer, or None for torch's
current stream. A non-OK status raises :class:`MiattnError` carrying the
library's message. All compute happens in the HIP library; when it is not
built or cannot be loaded, every call fails loudly.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("MIATTN_LIB", os.path.join(_PKG, "libmiattn.so"))

MIATTN_OK = 0
MIATTN_ERR_INVALID_ARG = 1
MIATTN_ERR_UNSUPPORTED = 2
MIATTN_ERR_HIP = 3

EXPORTS = ("attn_fwd", "attn_fwd_window", "attn_fwd_ext", "attn_fwd_varlen",
           "attn_fwd_varlen_ext", "attn_bwd",
           "attn_bwd_workspace_size",
           "attn_fwd_decode_workspace_size",
           "attn_fwd_decode", "attn_fwd_decode_noalloc",
           "attn_fwd_decode_paged", "miattn_last_error", "miattn_version")


class MiattnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"libmiattn status {status}: {message}")
        self.status = status
        self.message = message


_lib = None


def bind_to_torch_runtime():
    """Import torch (when installed) before a HIP library is loaded.

    torch ships its own HIP runtime (libamdhip64, soname .so.7, loaded by its
    file name). A library that needs libamdhip64.so.7 and is loaded after
    torch binds to that same runtime; loaded before torch, it brings in the
    system runtime, torch then loads its own, and a process with two HIP
    (and two HSA) runtimes sees the GPU in only one of them: streams and
    device memory from torch would not belong to the runtime the kernels
    are launched on."""
    try:
        import torch  # noqa: F401
    except ImportError:
        pass


def load(path: str = LIB_PATH):
    """Load the library (building it first if no build exists), after torch
    so that both use one HIP runtime."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        from . import build as _build
        _build.build(out=path)
    bind_to_torch_runtime()
    L = ctypes.CDLL(path)
    vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    L.attn_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, vp]
    L.attn_fwd.restype = i
    L.attn_fwd_window.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, f, vp]
    L.attn_fwd_window.restype = i
    L.attn_fwd_ext.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, f, vp, f, vp]
    L.attn_fwd_ext.restype = i
    L.attn_fwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, i, f, vp]
    L.attn_fwd_varlen.restype = i
    L.attn_fwd_varlen_ext.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, i,
                                      i, f, vp, f, vp]
    L.attn_fwd_varlen_ext.restype = i
    L.attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, vp,
                           ctypes.c_size_t, vp]
    L.attn_bwd.restype = i
    L.attn_bwd_workspace_size.argtypes = [i, i, i]
    L.attn_bwd_workspace_size.restype = ctypes.c_size_t
    L.attn_fwd_decode_workspace_size.argtypes = [i, i, i, i]
    L.attn_fwd_decode_workspace_size.restype = ctypes.c_size_t
    L.attn_fwd_decode.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp,
                                  ctypes.c_size_t, vp]
    L.attn_fwd_decode.restype = i
    L.attn_fwd_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp]
    L.attn_fwd_decode_noalloc.restype = i
    L.attn_fwd_decode_paged.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, f,
                                        vp, ctypes.c_size_t, vp]
    L.attn_fwd_decode_paged.restype = i
    L.miattn_last_error.argtypes = []
    L.miattn_last_error.restype = ctypes.c_char_p
    L.miattn_version.argtypes = []
    L.miattn_version.restype = i
    _lib = L
    return L


def _addr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(s):
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _check(rc: int):
    if rc != MIATTN_OK:
        raise MiattnError(rc, miattn_last_error())


def attn_fwd(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, d, causal, scale, stream=None):
    _check(load().attn_fwd(_addr(q), _addr(k), _addr(v), _addr(o), _addr(lse), int(B),
                           int(Hq), int(Hkv), int(Sq), int(Sk), int(d), int(bool(causal)),
                           float(scale), _stream(stream)))


def attn_fwd_window(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, d, causal, window_left, scale,
                    stream=None):
    _check(load().attn_fwd_window(_addr(q), _addr(k), _addr(v), _addr(o), _addr(lse), int(B),
                                  int(Hq), int(Hkv), int(Sq), int(Sk), int(d),
                                  int(bool(causal)), int(window_left), float(scale),
                                  _stream(stream)))


def attn_fwd_ext(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, d, causal, window_left, softcap,
                 alibi_slopes, scale, stream=None):
    _check(load().attn_fwd_ext(_addr(q), _addr(k), _addr(v), _addr(o), _addr(lse), int(B),
                               int(Hq), int(Hkv), int(Sq), int(Sk), int(d), int(bool(causal)),
                               int(window_left), float(softcap), _addr(alibi_slopes),
                               float(scale), _stream(stream)))


def attn_fwd_varlen(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, B, total_q, total_k,
                    max_seqlen_q, max_seqlen_k, Hq, Hkv, d, causal, scale, stream=None):
    _check(load().attn_fwd_varlen(_addr(q), _addr(k), _addr(v), _addr(o), _addr(lse),
                                  _addr(cu_seqlens_q), _addr(cu_seqlens_k), int(B), int(total_q),
                                  int(total_k), int(max_seqlen_q), int(max_seqlen_k), int(Hq),
                                  int(Hkv), int(d), int(bool(causal)), float(scale),
                                  _stream(stream)))


def attn_fwd_varlen_ext(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, B, total_q, total_k,
                        max_seqlen_q, max_seqlen_k, Hq, Hkv, d, causal, window_left, softcap,
                        alibi_slopes, scale, stream=None):
    _check(load().attn_fwd_varlen_ext(_addr(q), _addr(k), _addr(v), _addr(o), _addr(lse),
                                      _addr(cu_seqlens_q), _addr(cu_seqlens_k), int(B),
                                      int(total_q), int(total_k), int(max_seqlen_q),
                                      int(max_seqlen_k), int(Hq), int(Hkv), int(d),
                                      int(bool(causal)), int(window_left), float(softcap),
                                      _addr(alibi_slopes), float(scale), _stream(stream)))


def attn_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, Sq, Sk, d, causal, scale,
             workspace, workspace_bytes, stream=None):
    _check(load().attn_bwd(_addr(q), _addr(k), _addr(v), _addr(o), _addr(lse), _addr(dout),
                           _addr(dq), _addr(dk), _addr(dv), int(B), int(Hq), int(Hkv), int(Sq),
                           int(Sk), int(d), int(bool(causal)), float(scale), _addr(workspace),
                           int(workspace_bytes), _stream(stream)))


def attn_bwd_workspace_size(B, Hq, Sq) -> int:
    return int(load().attn_bwd_workspace_size(int(B), int(Hq), int(Sq)))


def attn_fwd_decode_workspace_size(B, Hq, d, num_splits) -> int:
    return int(load().attn_fwd_decode_workspace_size(int(B), int(Hq), int(d), int(num_splits)))


def attn_fwd_decode(q, k_cache, v_cache, kv_lens, o, lse, B, Hq, Hkv, S_cap, d, num_splits,
                    scale, workspace, workspace_bytes, stream=None):
    _check(load().attn_fwd_decode(_addr(q), _addr(k_cache), _addr(v_cache), _addr(kv_lens),
                                  _addr(o), _addr(lse), int(B), int(Hq), int(Hkv), int(S_cap),
                                  int(d), int(num_splits), float(scale), _addr(workspace),
                                  int(workspace_bytes), _stream(stream)))


def attn_fwd_decode_noalloc(q, k_cache, v_cache, kv_lens, o, lse, B, Hq, Hkv, S_cap, d,
                            num_splits, scale, stream=None):
    _check(load().attn_fwd_decode_noalloc(_addr(q), _addr(k_cache), _addr(v_cache),
                                          _addr(kv_lens), _addr(o), _addr(lse), int(B), int(Hq),
                                          int(Hkv), int(S_cap), int(d), int(num_splits),
                                          float(scale), _stream(stream)))


def attn_fwd_decode_paged(q, k_pages, v_pages, block_table, kv_lens, o, lse, B, Hq, Hkv,
                          num_pages, page_size, max_pages_per_seq, d, num_splits, scale,
                          workspace, workspace_bytes, stream=None):
    _check(load().attn_fwd_decode_paged(_addr(q), _addr(k_pages), _addr(v_pages),
                                        _addr(block_table), _addr(kv_lens), _addr(o), _addr(lse),
                                        int(B), int(Hq), int(Hkv), int(num_pages), int(page_size),
                                        int(max_pages_per_seq), int(d), int(num_splits),
                                        float(scale), _addr(workspace), int(workspace_bytes),
                                        _stream(stream)))


def miattn_last_error() -> str:
    msg = load().miattn_last_error()
    return msg.decode() if msg else ""


def miattn_version() -> int:
    return int(load().miattn_version())
