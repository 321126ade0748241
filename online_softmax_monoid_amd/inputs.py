"""Seeded synthetic inputs shared by the HIP path's callers and the oracle.

This module holds no attention arithmetic. It draws Gaussian values with
numpy's PCG64 generator, rounds them to bfloat16 bit patterns
(round-to-nearest-even, the rounding the tang paper's emulating interpreter
uses, §4 "Precision is a schedule"), and describes the five workloads the
library is measured and checked on. Both the GPU path (through torch device
tensors) and the f64 oracle (through host arrays) read the very same bit
patterns produced here.

Recipe (one generator per workload, ``seed = 20261200 + workload id``):
  * prefill: draw Q, K, V in that order as float32 ``standard_normal``,
    multiply by the workload's ``std`` (exact for 0.5 and 1.0), round to
    bf16;
  * decode: first draw the per-stream lengths with ``integers(lo, hi,
    endpoint=True)``, then Q, then every stream's valid K rows (stream by
    stream, all kv-heads of a stream in one draw), then the same for V;
    padding rows beyond a stream's length hold a caller-chosen bf16 pattern
    (0 for timing, NaN for the exactness checks).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

BF16_NAN = np.uint16(0x7FC0)
SEED_BASE = 20261200


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 bit patterns (round to nearest even).

    NaN maps to the canonical quiet NaN 0x7FC0; infinities stay infinities.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    rounded = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
               >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        rounded[nan] = BF16_NAN
    return rounded


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 exactly."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


def f32_to_bf16_bits_scalar(x: float) -> int:
    return int(bf16_bits(np.array([x], dtype=np.float32))[0])


def default_scale(d: int) -> float:
    """1/sqrt(d) rounded to float32: the value handed to both sides."""
    return float(np.float32(1.0 / math.sqrt(d)))


@dataclasses.dataclass(frozen=True)
class Prefill:
    """A prefill workload: Q/O are [B, Hq, Sq, d], K/V are [B, Hkv, Sk, d]."""
    wid: int
    name: str
    B: int
    Hq: int
    Hkv: int
    Sq: int
    Sk: int
    d: int
    causal: tuple  # the causal settings the workload runs with
    std: float = 1.0
    sampled_rows_per_head: Optional[int] = None  # None: check every row

    @property
    def seed(self) -> int:
        return SEED_BASE + self.wid

    @property
    def scale(self) -> float:
        return default_scale(self.d)

    def flops(self, causal: bool) -> float:
        """Algorithmic flops: 4*B*Hq*Sq*Sk*d, halved when causal."""
        f = 4.0 * self.B * self.Hq * self.Sq * self.Sk * self.d
        return f / 2 if causal else f


@dataclasses.dataclass(frozen=True)
class Decode:
    """A decode workload: Q/O are [B, Hq, d]; the caches are [B, Hkv, S_cap, d]."""
    wid: int
    name: str
    B: int
    Hq: int
    Hkv: int
    d: int
    len_lo: int
    len_hi: int
    S_cap: int
    num_splits: int
    std: float = 1.0

    @property
    def seed(self) -> int:
        return SEED_BASE + self.wid

    @property
    def scale(self) -> float:
        return default_scale(self.d)


WORKLOADS = {
    1: Prefill(1, "tiny non-causal B1 H2 S128 d64", 1, 2, 2, 128, 128, 64, (False,)),
    2: Prefill(2, "MHA B4 H16 S1024 d64", 4, 16, 16, 1024, 1024, 64, (True, False)),
    3: Prefill(3, "Llama-class causal prefill B2 H32 S4096 d128", 2, 32, 32, 4096,
               4096, 128, (True,), std=0.5),
    4: Prefill(4, "long-context GQA B1 Hq16 Hkv2 S44032 d256 causal", 1, 16, 2,
               44032, 44032, 256, (True,), sampled_rows_per_head=512),
    5: Decode(5, "batched split-KV decode B32 Hq32 Hkv8 d128 len U[1024,8192]",
              32, 32, 8, 128, 1024, 8192, 8192, 16),
}


def draw_prefill_bits(seed: int, B: int, Hq: int, Hkv: int, Sq: int, Sk: int,
                      d: int, std: float = 1.0):
    """Q, K, V as bf16 bit arrays (uint16) of shapes [B,Hq,Sq,d], [B,Hkv,Sk,d]."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = []
    for shape in ((B, Hq, Sq, d), (B, Hkv, Sk, d), (B, Hkv, Sk, d)):
        x = rng.standard_normal(size=shape, dtype=np.float32)
        if std != 1.0:
            x *= np.float32(std)
        out.append(bf16_bits(x))
    return tuple(out)


def prefill_inputs(w: Prefill):
    return draw_prefill_bits(w.seed, w.B, w.Hq, w.Hkv, w.Sq, w.Sk, w.d, w.std)


def prefill_inputs_f32(w: Prefill):
    """The unrounded float32 draws of a workload (same generator, same order)."""
    rng = np.random.Generator(np.random.PCG64(w.seed))
    out = []
    for shape in ((w.B, w.Hq, w.Sq, w.d), (w.B, w.Hkv, w.Sk, w.d),
                  (w.B, w.Hkv, w.Sk, w.d)):
        x = rng.standard_normal(size=shape, dtype=np.float32)
        if w.std != 1.0:
            x *= np.float32(w.std)
        out.append(x)
    return tuple(out)


def sampled_rows(w: Prefill, rows_per_head: int, extra_edges: bool = True):
    """Flat row indices ((b*Hq + h)*Sq + i) checked for a large workload.

    Per head, ``rows_per_head`` distinct query positions drawn with a second
    generator seeded ``seed + 1``; the first and last positions are added as
    edge rows.
    """
    rng = np.random.Generator(np.random.PCG64(w.seed + 1))
    rows = []
    for b in range(w.B):
        for h in range(w.Hq):
            pick = rng.choice(w.Sq, size=min(rows_per_head, w.Sq), replace=False)
            pick = set(int(i) for i in pick)
            if extra_edges:
                pick.update((0, w.Sq - 1))
            base = (b * w.Hq + h) * w.Sq
            rows.extend(base + i for i in sorted(pick))
    return np.asarray(rows, dtype=np.int64)


def draw_decode_bits(seed: int, B: int, Hq: int, Hkv: int, d: int, len_lo: int,
                     len_hi: int, S_cap: int, std: float = 1.0,
                     pad_bits: int = 0, lens: Optional[np.ndarray] = None):
    """lens[int32 B], Q bits [B,Hq,d], K/V cache bits [B,Hkv,S_cap,d].

    Rows at or beyond a stream's length hold ``pad_bits``.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    if lens is None:
        lens = rng.integers(len_lo, len_hi, size=B, endpoint=True)
    lens = np.asarray(lens, dtype=np.int32)
    assert lens.shape == (B,) and (lens >= 0).all() and (lens <= S_cap).all()

    def draw(shape):
        x = rng.standard_normal(size=shape, dtype=np.float32)
        if std != 1.0:
            x *= np.float32(std)
        return bf16_bits(x)

    q = draw((B, Hq, d))
    kc = np.full((B, Hkv, S_cap, d), pad_bits, dtype=np.uint16)
    vc = np.full((B, Hkv, S_cap, d), pad_bits, dtype=np.uint16)
    for cache in (kc, vc):
        for b in range(B):
            n = int(lens[b])
            if n:
                cache[b, :, :n, :] = draw((Hkv, n, d))
    return lens, q, kc, vc


def decode_inputs(w: Decode, pad_bits: int = 0):
    return draw_decode_bits(w.seed, w.B, w.Hq, w.Hkv, w.d, w.len_lo, w.len_hi,
                            w.S_cap, w.std, pad_bits=pad_bits)


def paged_layout(seed: int, lens: np.ndarray, page_size: int, max_pages: int,
                 spare_pages: int = 0):
    """A random page assignment for a paged cache: block table [B, max_pages]
    int32 and the pool size.

    Stream b's logical pages 0 .. ceil(lens[b] / page_size) - 1 get distinct
    pool pages in a seeded random order; ``spare_pages`` more pool pages
    belong to no stream. Table entries past a stream's last page hold -1
    (never used). No attention arithmetic happens here: this only decides
    where rows are stored.
    """
    lens = np.asarray(lens, dtype=np.int64)
    used = (lens + page_size - 1) // page_size
    assert (used <= max_pages).all()
    num_pages = int(used.sum()) + int(spare_pages)
    rng = np.random.Generator(np.random.PCG64(seed))
    perm = rng.permutation(num_pages).astype(np.int32)
    table = np.full((len(lens), max_pages), -1, dtype=np.int32)
    pos = 0
    for b, n in enumerate(used):
        table[b, :n] = perm[pos:pos + n]
        pos += int(n)
    return table, num_pages


def scatter_to_pages(cache_bits: np.ndarray, table: np.ndarray, num_pages: int,
                     page_size: int, fill_bits: int = 0) -> np.ndarray:
    """Store a contiguous cache [B, Hkv, S_cap, d] in a page pool
    [num_pages, Hkv, page_size, d] by the block table (entries < 0 skipped);
    pool rows no table entry reaches hold ``fill_bits``."""
    B, Hkv, S_cap, d = cache_bits.shape
    pool = np.full((num_pages, Hkv, page_size, d), fill_bits, dtype=np.uint16)
    for b in range(B):
        for p, page in enumerate(table[b]):
            if page < 0:
                continue
            lo = p * page_size
            n = max(0, min(page_size, S_cap - lo))
            pool[page, :, :n, :] = cache_bits[b, :, lo:lo + n, :]
    return pool
