"""GPU: a seeded sweep of small random shapes, forward (plain, with a
sliding window, soft cap and ALiBi drawn at random, and packed variable-length
batches), backward and decode (contiguous and paged), against the f64
oracles.

The shape lists are drawn once from a fixed PCG64 stream, so the cases (and
their test ids) are the same on every run. The lengths are drawn so that most
are not multiples of the 32-key tile or of the 8 rows of a copy block, and
include 1: every ragged end of the tile and copy layouts at head dimensions
64, 128 and 256, with and without the causal mask, with MHA and grouped
heads. Bounds as in the parity tests: forward O max-abs 1e-2, O rel-RMS 4e-3,
LSE max-abs 1e-3, rows that see no key exactly (+0, -inf); backward per
gradient tensor rel-RMS <= 8e-3 and max-abs <= 1.2e-2 of its largest
magnitude. The paged decode must also equal the contiguous decode bit for bit
(pool pages no stream owns hold NaN bits).
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
from oracle import backward as bw
from online_softmax_monoid_amd import inputs
from tests import harness as H

pytestmark = pytest.mark.gpu
REL_RMS, MAX_REL = 8e-3, 1.2e-2


def _note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _bits(seed, shape, std=1.0):
    rng = np.random.Generator(np.random.PCG64(seed))
    return inputs.bf16_bits(rng.standard_normal(size=shape, dtype=np.float32) * np.float32(std))


def _draw_shapes(seed, n, max_len):
    rng = np.random.Generator(np.random.PCG64(seed))
    out = []
    for _ in range(n):
        d = int(rng.choice([64, 128, 256]))
        hkv = int(rng.integers(1, 3))
        g = int(rng.choice([1, 2, 4]))
        b = int(rng.integers(1, 3))
        sq = int(rng.integers(1, max_len + 1))
        sk = sq if rng.random() < 0.5 else int(rng.integers(1, max_len + 1))
        causal = bool(rng.random() < 0.6)
        out.append((b, hkv * g, hkv, sq, sk, d, causal))
    return out


FWD = _draw_shapes(20261211, 30, 300)
BWD = _draw_shapes(20261212, 12, 160)


def _draw_decode(seed, n):
    """(seed, lens, Hq, Hkv, d, page size, splits): lengths from 0 to 700,
    with an empty stream or a one-row stream forced into two of every three
    cases, and 1 to 16 query heads per kv-head."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = []
    for i in range(n):
        B = int(rng.integers(1, 7))
        lens = rng.integers(0, 701, size=B)
        if i % 3 == 0:
            lens[0] = 0
        if i % 3 == 1:
            lens[-1] = 1
        hkv = int(rng.integers(1, 5))
        g = int(rng.choice([1, 2, 4, 8, 16]))
        d = int(rng.choice([64, 128, 256]))
        P = int(rng.choice([16, 32, 64]))
        splits = int(rng.integers(1, 25))
        out.append((seed + 7 * i, [int(x) for x in lens], hkv * g, hkv, d, P, splits))
    return out


DEC = _draw_decode(20261213, 16)


def _draw_ext(seed, n):
    """Forward shapes with a sliding window, a soft cap and ALiBi slopes,
    each present or not at random (at least one of them in every case)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = []
    for b, hq, hkv, sq, sk, d, causal in _draw_shapes(seed + 1, n, 300):
        while True:
            window = int(rng.integers(0, 200)) if rng.random() < 0.5 else -1
            softcap = float(rng.uniform(5.0, 50.0)) if rng.random() < 0.5 else 0.0
            alibi = bool(rng.random() < 0.5)
            if window >= 0 or softcap > 0.0 or alibi:
                break
        out.append((b, hq, hkv, sq, sk, d, causal, window, round(softcap, 3), alibi))
    return out


EXT = _draw_ext(20261214, 16)


def _draw_varlen(seed, n):
    """Packed batches: 1-8 sequences of 0-400 query rows, each with 0-200
    more keys than rows (a chunk against its cache), and the variants drawn
    as in _draw_ext (any of them may be absent here)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = []
    for i in range(n):
        nseq = int(rng.integers(1, 9))
        lq = [int(x) for x in rng.integers(0, 401, size=nseq)]
        extra = [int(x) for x in rng.integers(0, 201, size=nseq)]
        hkv = int(rng.integers(1, 3))
        g = int(rng.choice([1, 2, 4]))
        d = int(rng.choice([64, 128, 256]))
        causal = bool(rng.random() < 0.6)
        window = int(rng.integers(0, 200)) if rng.random() < 0.3 else -1
        softcap = round(float(rng.uniform(5.0, 50.0)), 3) if rng.random() < 0.3 else 0.0
        alibi = bool(rng.random() < 0.3)
        out.append((seed + 11 * i, lq, extra, hkv * g, hkv, d, causal, window, softcap, alibi))
    return out


VARLEN = _draw_varlen(20261215, 10)


@pytest.mark.parametrize("i", range(len(FWD)))
def test_forward_sweep(i):
    B, Hq, Hkv, Sq, Sk, d, causal = FWD[i]
    label = f"fwd sweep {i} {FWD[i]}"
    seed = 9000 + 10 * i
    q = _bits(seed, (B, Hq, Sq, d))
    k = _bits(seed + 1, (B, Hkv, Sk, d))
    v = _bits(seed + 2, (B, Hkv, Sk, d))
    scale = inputs.default_scale(d)
    _note(f"[gpu] {label}")
    o, lse, guards = H.run_fwd(q, k, v, causal, scale)
    assert guards, f"{label}: write outside the logical outputs"
    o_ref, lse_ref = oracle.attn_fwd(q, k, v, causal, scale)
    m = H.metrics(o, lse, o_ref, lse_ref)
    _note(f"[gpu] {label}: {m}")
    H.assert_parity(m, label)


@pytest.mark.parametrize("i", range(len(BWD)))
def test_backward_sweep(i):
    B, Hq, Hkv, Sq, Sk, d, causal = BWD[i]
    label = f"bwd sweep {i} {BWD[i]}"
    seed = 9500 + 10 * i
    q = _bits(seed, (B, Hq, Sq, d), 0.5)
    k = _bits(seed + 1, (B, Hkv, Sk, d), 0.5)
    v = _bits(seed + 2, (B, Hkv, Sk, d))
    do = _bits(seed + 3, (B, Hq, Sq, d))
    scale = inputs.default_scale(d)
    o_ref, lse_ref = oracle.attn_fwd(q, k, v, causal, scale)
    o_bits = inputs.bf16_bits(o_ref.astype(np.float32))
    lse = lse_ref.astype(np.float32)
    _note(f"[gpu] {label}")
    dq, dk, dv, guards = H.run_bwd(q, k, v, o_bits, lse, do, causal, scale)
    assert guards, f"{label}: write outside the gradients"
    rq, rk, rv = bw.attn_bwd(q, k, v, do, causal, scale)
    for name, got, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        m = H.grad_metrics(got, ref)
        _note(f"[gpu] {label} {name}: {m}")
        assert m["finite"], f"{label} {name}: non-finite"
        if not np.any(ref):
            # nothing reaches this gradient (every row sees no key, or no
            # row sees any key of it): it must be exactly zero
            assert not np.any(got), f"{label} {name}: expected exact zeros"
            continue
        assert m["rel_rms"] <= REL_RMS, f"{label} {name}: {m}"
        assert m["max_abs_rel"] <= MAX_REL, f"{label} {name}: {m}"


@pytest.mark.parametrize("i", range(len(DEC)))
def test_decode_sweep(i):
    seed, lens, Hq, Hkv, d, P, splits = DEC[i]
    lens = np.asarray(lens, dtype=np.int32)
    label = f"decode sweep {i} B={len(lens)} Hq={Hq} Hkv={Hkv} d={d} P={P} splits={splits}"
    nan = int(inputs.BF16_NAN)
    max_pages = max(1, int((lens.max() + P - 1) // P))
    S_cap = max_pages * P
    _, q, kc, vc = inputs.draw_decode_bits(seed, len(lens), Hq, Hkv, d, 0, 0, S_cap, lens=lens,
                                           pad_bits=nan)
    scale = inputs.default_scale(d)
    _note(f"[gpu] {label} lens={lens.tolist()}")
    o, lse, guards = H.run_decode(q, kc, vc, lens, scale, splits)
    assert guards, f"{label}: write outside the logical outputs"
    o_ref, lse_ref = oracle.attn_decode(q, kc, vc, lens, scale)
    m = H.metrics(o, lse, o_ref, lse_ref)
    _note(f"[gpu] {label}: {m}")
    H.assert_parity(m, label)
    assert m["empty_rows"] == Hq * int((lens == 0).sum())
    # the same rows in a page pool, in a seeded random page order
    table, npg = inputs.paged_layout(seed + 1, lens, P, max_pages, spare_pages=3)
    kp = inputs.scatter_to_pages(kc, table, npg, P, fill_bits=nan)
    vp = inputs.scatter_to_pages(vc, table, npg, P, fill_bits=nan)
    op, lp, guards = H.run_decode_paged(q, kp, vp, table, lens, P, scale, splits)
    assert guards, f"{label} paged: write outside the logical outputs"
    assert np.array_equal(op, o), f"{label}: paged O differs from the contiguous decode"
    assert np.array_equal(lp.view(np.uint32), lse.view(np.uint32)), f"{label}: paged LSE differs"


@pytest.mark.parametrize("i", range(len(EXT)))
def test_forward_variants_sweep(i):
    B, Hq, Hkv, Sq, Sk, d, causal, window, softcap, alibi = EXT[i]
    label = f"fwd variant sweep {i} {EXT[i]}"
    seed = 9800 + 10 * i
    std = 0.5 if alibi else 1.0
    q = _bits(seed, (B, Hq, Sq, d), std)
    k = _bits(seed + 1, (B, Hkv, Sk, d), std)
    v = _bits(seed + 2, (B, Hkv, Sk, d))
    slopes = (2.0 ** (-8.0 * (np.arange(Hq) + 1) / Hq)).astype(np.float32) if alibi else None
    scale = inputs.default_scale(d)
    _note(f"[gpu] {label}")
    o, lse, guards = H.run_fwd_ext(q, k, v, causal, scale, window, softcap, slopes)
    assert guards, f"{label}: write outside the logical outputs"
    o_ref, lse_ref = oracle.attn_fwd(q, k, v, causal, scale, window=window, softcap=softcap,
                                     alibi=slopes)
    m = H.metrics(o, lse, o_ref, lse_ref)
    _note(f"[gpu] {label}: {m}")
    H.assert_parity(m, label)


@pytest.mark.parametrize("i", range(len(VARLEN)))
def test_varlen_sweep(i):
    from tests.test_gpu_varlen import _run_ext

    seed, lq, extra, Hq, Hkv, d, causal, window, softcap, alibi = VARLEN[i]
    lk = [a + b for a, b in zip(lq, extra)]
    cu_q = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
    std = 0.5 if alibi else 1.0
    q = _bits(seed, (Hq, int(cu_q[-1]), d), std)
    k = _bits(seed + 1, (Hkv, int(cu_k[-1]), d), std)
    v = _bits(seed + 2, (Hkv, int(cu_k[-1]), d))
    slopes = (2.0 ** (-8.0 * (np.arange(Hq) + 1) / Hq)).astype(np.float32) if alibi else None
    scale = inputs.default_scale(d)
    label = f"varlen sweep {i} {VARLEN[i]}"
    _note(f"[gpu] {label}")
    o, lse, guards = _run_ext(q, k, v, cu_q, cu_k, max(lq), max(lk), causal, scale, window,
                              softcap, slopes)
    assert guards, f"{label}: write outside the logical outputs"
    o_ref, lse_ref = oracle.attn_fwd_varlen(q, k, v, cu_q, cu_k, causal, scale, window=window,
                                            softcap=softcap, alibi=slopes)
    m = H.metrics(o, lse, o_ref, lse_ref)
    _note(f"[gpu] {label}: {m}")
    H.assert_parity(m, label)
