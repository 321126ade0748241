"""The f64 CPU oracle for softmax attention -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The product library never loads it and
it imports nothing from the product package.

Two implementations live here:

* ``attn_oracle.c`` (through ctypes): the plain two-pass definition of
  softmax attention in double precision, for prefill and decode.
* ``monoid.py``: the online-softmax monoid of the tang paper (§2.2
  "Comprehensions and monoids", §2.5 "Schedules": split on any associative
  monoid), written separately, used to pin that folding the reduction in any
  split/merge order reproduces the two-pass result.

Both read the same bf16 bit patterns the GPU reads.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (OpenMP, -O2, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-shared", "-fPIC",
                        "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        L = ctypes.CDLL(_LIB)
        u16p = ctypes.POINTER(ctypes.c_uint16)
        f64p = ctypes.POINTER(ctypes.c_double)
        i64p = ctypes.POINTER(ctypes.c_int64)
        i32p = ctypes.POINTER(ctypes.c_int32)
        c_int = ctypes.c_int
        L.oracle_attn_fwd.argtypes = [u16p, u16p, u16p, c_int, c_int, c_int, c_int,
                                      c_int, c_int, c_int, ctypes.c_float, i64p,
                                      ctypes.c_int64, f64p, f64p, c_int]
        L.oracle_attn_fwd.restype = c_int
        L.oracle_attn_fwd_window.argtypes = [u16p, u16p, u16p, c_int, c_int, c_int, c_int,
                                             c_int, c_int, c_int, c_int, ctypes.c_float, i64p,
                                             ctypes.c_int64, f64p, f64p, c_int]
        L.oracle_attn_fwd_window.restype = c_int
        f32p = ctypes.POINTER(ctypes.c_float)
        L.oracle_attn_fwd_ext.argtypes = [u16p, u16p, u16p, c_int, c_int, c_int, c_int,
                                          c_int, c_int, c_int, c_int, ctypes.c_float, f32p,
                                          ctypes.c_float, i64p, ctypes.c_int64, f64p, f64p,
                                          c_int]
        L.oracle_attn_fwd_ext.restype = c_int
        L.oracle_attn_decode.argtypes = [u16p, u16p, u16p, i32p, c_int, c_int, c_int,
                                         c_int, c_int, ctypes.c_float, f64p, f64p,
                                         c_int]
        L.oracle_attn_decode.restype = c_int
        L.oracle_attn_probs.argtypes = [u16p, u16p, c_int, c_int, c_int, c_int, c_int,
                                        c_int, c_int, ctypes.c_float, ctypes.c_int64,
                                        f64p]
        L.oracle_attn_probs.restype = c_int
        L.oracle_max_threads.argtypes = []
        L.oracle_max_threads.restype = c_int
        _lib = L
    return _lib


def _ptr(a, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _u16(a):
    a = np.ascontiguousarray(a, dtype=np.uint16)
    return a


def max_threads() -> int:
    return int(lib().oracle_max_threads())


def attn_fwd(q_bits, k_bits, v_bits, causal: bool, scale: float, rows=None,
             nthreads: int = 0, window: int = -1, softcap: float = 0.0, alibi=None):
    """Two-pass f64 attention on bf16 bit arrays.

    q_bits: [B,Hq,Sq,d], k_bits / v_bits: [B,Hkv,Sk,d] (uint16).
    rows: optional flat row ids ((b*Hq + h)*Sq + i). window >= 0 hides keys
    j < i + Sk - Sq - window from row i (sliding window); < 0: none.
    softcap > 0 caps each scaled score s to softcap * tanh(s / softcap);
    alibi (float32 [Hq]) subtracts alibi[h] * |i + Sk - Sq - j| from it.
    Returns (o, lse) as f64: o has shape [B,Hq,Sq,d] and lse [B,Hq,Sq] when
    rows is None, else [len(rows), d] and [len(rows)].
    """
    q = _u16(q_bits)
    k = _u16(k_bits)
    v = _u16(v_bits)
    B, Hq, Sq, d = q.shape
    Bk, Hkv, Sk, dk = k.shape
    assert Bk == B and dk == d and v.shape == k.shape
    if rows is None:
        n = B * Hq * Sq
        rows_p = None
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        n = rows.shape[0]
        rows_p = _ptr(rows, ctypes.c_int64)
    o = np.empty((max(n, 1), d), dtype=np.float64)
    lse = np.empty(max(n, 1), dtype=np.float64)
    if alibi is not None:
        alibi = np.ascontiguousarray(alibi, dtype=np.float32)
        assert alibi.shape == (Hq,)
    al_p = _ptr(alibi, ctypes.c_float) if alibi is not None else None
    rc = lib().oracle_attn_fwd_ext(_ptr(q, ctypes.c_uint16), _ptr(k, ctypes.c_uint16),
                                   _ptr(v, ctypes.c_uint16), B, Hq, Hkv, Sq, Sk, d,
                                   int(bool(causal)), int(window), float(softcap), al_p,
                                   float(scale), rows_p, n, _ptr(o, ctypes.c_double),
                                   _ptr(lse, ctypes.c_double), int(nthreads))
    if rc != 0:
        raise ValueError("oracle_attn_fwd rejected its arguments")
    o, lse = o[:n], lse[:n]
    if rows is None:
        return o.reshape(B, Hq, Sq, d), lse.reshape(B, Hq, Sq)
    return o, lse


def attn_decode(q_bits, kc_bits, vc_bits, lens, scale: float, nthreads: int = 0):
    """Two-pass f64 decode attention. q: [B,Hq,d]; caches [B,Hkv,S_cap,d]."""
    q = _u16(q_bits)
    kc = _u16(kc_bits)
    vc = _u16(vc_bits)
    lens = np.ascontiguousarray(lens, dtype=np.int32)
    B, Hq, d = q.shape
    Bk, Hkv, S_cap, dk = kc.shape
    assert Bk == B and dk == d and vc.shape == kc.shape and lens.shape == (B,)
    o = np.empty((max(B * Hq, 1), d), dtype=np.float64)
    lse = np.empty(max(B * Hq, 1), dtype=np.float64)
    rc = lib().oracle_attn_decode(_ptr(q, ctypes.c_uint16), _ptr(kc, ctypes.c_uint16),
                                  _ptr(vc, ctypes.c_uint16), _ptr(lens, ctypes.c_int32),
                                  B, Hq, Hkv, S_cap, d, float(scale),
                                  _ptr(o, ctypes.c_double), _ptr(lse, ctypes.c_double),
                                  int(nthreads))
    if rc != 0:
        raise ValueError("oracle_attn_decode rejected its arguments")
    return o[:B * Hq].reshape(B, Hq, d), lse[:B * Hq].reshape(B, Hq)


def attn_fwd_varlen(q_bits, k_bits, v_bits, cu_q, cu_k, causal: bool, scale: float,
                    nthreads: int = 0, window: int = -1, softcap: float = 0.0, alibi=None):
    """A packed batch of sequences: q [Hq, total_q, d], k / v [Hkv, total_k, d];
    sequence b is rows cu_q[b] .. cu_q[b+1]-1 against keys cu_k[b] .. cu_k[b+1]-1,
    each the attention of attn_fwd on its own (with the same window, soft cap
    and ALiBi slopes, taken against the sequence's own lengths). Returns
    o [Hq, total_q, d] and lse [Hq, total_q] (f64)."""
    q = _u16(q_bits)
    k = _u16(k_bits)
    v = _u16(v_bits)
    Hq, total_q, d = q.shape
    Hkv, total_k, _ = k.shape
    o = np.zeros((Hq, total_q, d), dtype=np.float64)
    lse = np.full((Hq, total_q), -np.inf, dtype=np.float64)
    for b in range(len(cu_q) - 1):
        q0, q1, k0, k1 = int(cu_q[b]), int(cu_q[b + 1]), int(cu_k[b]), int(cu_k[b + 1])
        if q1 == q0:
            continue
        ob, lb = attn_fwd(q[None, :, q0:q1], k[None, :, k0:k1], v[None, :, k0:k1], causal,
                          scale, nthreads=nthreads, window=window, softcap=softcap, alibi=alibi)
        o[:, q0:q1] = ob[0]
        lse[:, q0:q1] = lb[0]
    return o, lse


def gather_pages(pool_bits, block_table, lens, page_size: int):
    """The gather view of a paged cache (tang paper, §2.1 "Views": a read whose
    source coordinate comes from an index tensor; paged KV caches are its
    example). pool [num_pages, Hkv, P, d], block_table [B, max_pages] ->
    the contiguous cache [B, Hkv, max_pages * P, d] with

        K[b, g, r, :] = pool[block_table[b, r // P], g, r % P, :]

    for r < lens[b] and zero bits elsewhere. Entries outside [0, num_pages)
    are clamped into it, as the C interface defines for bad entries."""
    pool = _u16(pool_bits)
    table = np.asarray(block_table, dtype=np.int64)
    num_pages, Hkv, P, d = pool.shape
    assert P == page_size
    B, max_pages = table.shape
    out = np.zeros((B, Hkv, max_pages * P, d), dtype=np.uint16)
    for b in range(B):
        for r in range(int(lens[b])):
            page = min(max(int(table[b, r // P]), 0), num_pages - 1)
            out[b, :, r, :] = pool[page, :, r % P, :]
    return out


def attn_decode_paged(q_bits, k_pool_bits, v_pool_bits, block_table, lens, page_size: int,
                      scale: float, nthreads: int = 0):
    """Decode attention over a paged cache: the two-pass f64 decode of the
    gathered cache."""
    kc = gather_pages(k_pool_bits, block_table, lens, page_size)
    vc = gather_pages(v_pool_bits, block_table, lens, page_size)
    return attn_decode(q_bits, kc, vc, lens, scale, nthreads)


def attn_probs(q_bits, k_bits, causal: bool, scale: float, row: int):
    """Probability row p[Sk] of flat query row ``row`` (masked keys are 0)."""
    q = _u16(q_bits)
    k = _u16(k_bits)
    B, Hq, Sq, d = q.shape
    _, Hkv, Sk, _ = k.shape
    p = np.empty(max(Sk, 1), dtype=np.float64)
    rc = lib().oracle_attn_probs(_ptr(q, ctypes.c_uint16), _ptr(k, ctypes.c_uint16),
                                 B, Hq, Hkv, Sq, Sk, d, int(bool(causal)), float(scale),
                                 int(row), _ptr(p, ctypes.c_double))
    if rc != 0:
        raise ValueError("oracle_attn_probs rejected its arguments")
    return p[:Sk]
