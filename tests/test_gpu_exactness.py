"""GPU: what masking guarantees bit for bit, one-hot scores, and key order.

* Masked and hidden positions. Scores of masked keys are selected to -inf, so
  any bits in K at a masked key never reach an output, and K/V rows that no
  row of a work item can see (past the last key, above a causal item's last
  row, below a sliding window's first tile) are never read at all. Each case
  runs twice, once with finite values and once with NaN / inf planted at such
  positions, and the rows they are hidden from must agree bitwise. (A
  non-finite V value at a key masked for only some rows of a partially
  visible tile is the one exception the C interface states: its exact zero
  weight times NaN is NaN.)
* One-hot scores (the tang paper, §2.2 "Comprehensions and monoids": softmax
  of a row with one distinguished score): with orthogonal keys every score is
  exactly 0 except the distinguished key's L, so p* = e^L / (e^L + n - 1),
  LSE = ln(e^L + n - 1) and O = p* v* + (1 - p*) mean of the other values,
  in closed form.
* Key order (§2.5 "Schedules": a reduction over an associative and
  commutative monoid may be taken in any order): permuting the keys and
  values together leaves non-causal prefill and split decode within the
  tolerances of the unpermuted oracle result.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
from online_softmax_monoid_amd import inputs, miattn
from tests import harness as H

pytestmark = pytest.mark.gpu

NAN = int(inputs.BF16_NAN)
PINF = 0x7F80


def _note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _bits(seed, shape, std=1.0):
    rng = np.random.Generator(np.random.PCG64(seed))
    return inputs.bf16_bits(rng.standard_normal(size=shape, dtype=np.float32) * np.float32(std))


def _same(a, b):
    return np.array_equal(a, b)


def _same_lse(a, b):
    return np.array_equal(np.asarray(a, np.float32).view(np.uint32),
                          np.asarray(b, np.float32).view(np.uint32))


@pytest.mark.parametrize("d", [64, 128, 256])
def test_nan_keys_at_masked_positions(d):
    """Causal: K rows from key J on hold NaN. Every row i < J masks them
    (partly inside its diagonal tile, partly in tiles above it), so rows
    i < J are bit-identical to the run with finite keys."""
    S, J = 300, 100
    q = _bits(9001, (1, 2, S, d))
    k = _bits(9002, (1, 2, S, d))
    v = _bits(9003, (1, 2, S, d))
    s = inputs.default_scale(d)
    o0, l0, g0 = H.run_fwd(q, k, v, True, s)
    k2 = k.copy()
    k2[:, :, J:] = NAN
    o1, l1, g1 = H.run_fwd(q, k2, v, True, s)
    assert g0 and g1
    assert _same(o1[:, :, :J], o0[:, :, :J]) and _same_lse(l1[:, :, :J], l0[:, :, :J])
    # rows that see a NaN key propagate it (they do not pass for empty rows)
    assert np.all(np.isnan(l1[:, :, J:]))


@pytest.mark.parametrize("d", [64, 128, 256])
def test_nonfinite_kv_in_tiles_above_the_diagonal(d):
    """Causal: K = NaN and V = +inf from key J on, with J a multiple of every
    kernel's query-tile height (128 or 256 rows). No row i < J sees those keys
    and no work item holding such rows reads their tiles, so rows i < J are
    bit-identical to the finite run."""
    S, J = 600, 512
    q = _bits(9011, (1, 2, S, d))
    k = _bits(9012, (1, 1, S, d))
    v = _bits(9013, (1, 1, S, d))
    s = inputs.default_scale(d)
    o0, l0, _ = H.run_fwd(q, k, v, True, s)
    k2, v2 = k.copy(), v.copy()
    k2[:, :, J:] = NAN
    v2[:, :, J:] = PINF
    o1, l1, g1 = H.run_fwd(q, k2, v2, True, s)
    assert g1
    assert _same(o1[:, :, :J], o0[:, :, :J]) and _same_lse(l1[:, :, :J], l0[:, :, :J])


@pytest.mark.parametrize("d", [64, 128, 256])
def test_nonfinite_kv_below_the_window(d):
    """Causal sliding window of W = 100 keys: rows from R = 512 on (a
    query-tile boundary of every kernel) see keys from 412 on, so their work
    items start at the 32- or 64-key tile holding key 412 (key 384) and never
    read below it. K and V of keys below 320 are NaN / -inf: rows i >= R are
    bit-identical to the finite run."""
    S, W, R, lo = 700, 100, 512, 320
    q = _bits(9021, (1, 2, S, d))
    k = _bits(9022, (1, 2, S, d))
    v = _bits(9023, (1, 2, S, d))
    s = inputs.default_scale(d)
    o0, l0, _ = H.run_fwd(q, k, v, True, s, window=W)
    k2, v2 = k.copy(), v.copy()
    k2[:, :, :lo] = NAN
    v2[:, :, :lo] = 0xFF80  # -inf
    o1, l1, g1 = H.run_fwd(q, k2, v2, True, s, window=W)
    assert g1
    assert _same(o1[:, :, R:], o0[:, :, R:]) and _same_lse(l1[:, :, R:], l0[:, :, R:])


def _run_with_tail(q, k, v, causal, scale, tail_bits):
    """attn_fwd with K and V each followed in memory by 4096 elements of
    tail_bits (B = Hkv = 1, so the tail lies right after the last key)."""
    import torch
    B, Hq, Sq, d = q.shape
    _, Hkv, Sk, _ = k.shape
    assert B == 1 and Hkv == 1
    tail = np.full(4096, tail_bits, dtype=np.uint16)
    kd = H.dev_bits(np.concatenate([k.reshape(-1), tail]))
    vd = H.dev_bits(np.concatenate([v.reshape(-1), tail]))
    n = B * Hq * Sq
    o, lse = H.nan_out(n * d, n)
    miattn.attn_fwd(H.dev_bits(q), kd, vd, o, lse, B, Hq, Hkv, Sq, Sk, d, causal, scale)
    torch.cuda.synchronize()
    return H.host_bits(o)[:n * d], lse.cpu().numpy()[:n]


@pytest.mark.parametrize("d,causal", [(64, False), (128, False), (256, False), (128, True),
                                      (256, True)])
def test_nan_past_the_last_key_is_never_read(d, causal):
    """Sk = 300 (a ragged last tile): NaN right after the last key row of K
    and V in memory changes no output bit."""
    Sq, Sk = 200, 300
    q = _bits(9031, (1, 4, Sq, d))
    k = _bits(9032, (1, 1, Sk, d))
    v = _bits(9033, (1, 1, Sk, d))
    s = inputs.default_scale(d)
    o0, l0 = _run_with_tail(q, k, v, causal, s, 0)
    o1, l1 = _run_with_tail(q, k, v, causal, s, NAN)
    assert _same(o0, o1) and _same_lse(l0, l1)
    assert not np.any(np.isnan(l1))


def _one_hot_case(rng, n_rows, Sk, d, jstar, b_val):
    """Queries a_i e_0 (a_i in [0.25, 1.5]), keys orthogonal to e_0 except key
    jstar = b e_0: row i's scores are exactly 0 except a_i b at jstar."""
    a = inputs.bf16_bits(rng.uniform(0.25, 1.5, size=n_rows).astype(np.float32))
    q = np.zeros((n_rows, d), dtype=np.uint16)
    q[:, 0] = a
    k = inputs.bf16_bits(rng.standard_normal(size=(Sk, d), dtype=np.float32))
    k[:, 0] = 0
    k[jstar] = 0
    k[jstar, 0] = inputs.f32_to_bf16_bits_scalar(b_val)
    return q, k, inputs.bf16_to_f32(a).astype(np.float64)


def _one_hot_expected(a, b, scale, v, jstar):
    """Closed form for rows whose n = Sk keys are all visible."""
    vf = inputs.bf16_to_f32(v).astype(np.float64)
    n = vf.shape[0]
    L = np.float64(np.float32(scale)) * a * np.float64(b)
    pstar = 1.0 / (1.0 + (n - 1) * np.exp(-L))
    rest = (vf.sum(axis=0) - vf[jstar]) / (n - 1)
    o = pstar[:, None] * vf[jstar][None, :] + (1.0 - pstar)[:, None] * rest[None, :]
    lse = L + np.log1p((n - 1) * np.exp(-L))
    return o, lse


@pytest.mark.parametrize("d", [64, 128, 256])
def test_one_hot_scores_prefill(d):
    Sq, Sk, jstar, b = 150, 200, 77, 24.0
    rng = np.random.Generator(np.random.PCG64(9100 + d))
    q, k, a = _one_hot_case(rng, Sq, Sk, d, jstar, b)
    v = _bits(9101 + d, (Sk, d))
    s = inputs.default_scale(d)
    o, lse, guards = H.run_fwd(q[None, None], k[None, None], v[None, None], False, s)
    assert guards
    o_ref, l_ref = _one_hot_expected(a, b, s, v, jstar)
    m = H.metrics(o[0, 0], lse[0, 0], o_ref, l_ref)
    _note(f"[gpu] one-hot prefill d={d}: {m}")
    H.assert_parity(m, f"one-hot prefill d={d}")


def test_one_hot_scores_decode():
    d, Hq, Hkv, B, jstar, b = 128, 8, 2, 3, 401, 24.0
    lens = np.array([1000, 600, 402], dtype=np.int32)
    S_cap = 1024
    rng = np.random.Generator(np.random.PCG64(9200))
    q = np.zeros((B, Hq, d), dtype=np.uint16)
    kc = np.zeros((B, Hkv, S_cap, d), dtype=np.uint16)
    vc = _bits(9201, (B, Hkv, S_cap, d))
    a_all = np.zeros((B, Hq))
    for bb in range(B):
        qq, kk, a = _one_hot_case(rng, Hq, S_cap, d, jstar, b)
        q[bb] = qq
        a_all[bb] = a
        for g in range(Hkv):
            kc[bb, g] = kk
    s = inputs.default_scale(d)
    o, lse, guards = H.run_decode(q, kc, vc, lens, s, 16)
    assert guards
    G = Hq // Hkv
    o_ref = np.zeros((B, Hq, d))
    l_ref = np.zeros((B, Hq))
    for bb in range(B):
        n = int(lens[bb])
        for h in range(Hq):
            oo, ll = _one_hot_expected(a_all[bb, h:h + 1], b, s, vc[bb, h // G, :n], jstar)
            o_ref[bb, h], l_ref[bb, h] = oo[0], ll[0]
    m = H.metrics(o, lse, o_ref, l_ref)
    _note(f"[gpu] one-hot decode: {m}")
    H.assert_parity(m, "one-hot decode")


@pytest.mark.parametrize("d", [64, 128, 256])
def test_key_permutation_prefill(d):
    """Non-causal, GQA, ragged: the keys and values permuted together give
    the unpermuted oracle result."""
    B, Hq, Hkv, Sq, Sk = 2, 4, 2, 100, 333
    q = _bits(9300 + d, (B, Hq, Sq, d))
    k = _bits(9301 + d, (B, Hkv, Sk, d))
    v = _bits(9302 + d, (B, Hkv, Sk, d))
    perm = np.random.Generator(np.random.PCG64(9303 + d)).permutation(Sk)
    s = inputs.default_scale(d)
    o, lse, guards = H.run_fwd(q, k[:, :, perm], v[:, :, perm], False, s)
    assert guards
    o_ref, l_ref = oracle.attn_fwd(q, k, v, False, s)
    m = H.metrics(o, lse, o_ref, l_ref)
    _note(f"[gpu] permuted keys d={d}: {m}")
    H.assert_parity(m, f"permuted keys d={d}")


def test_key_permutation_decode():
    """Each stream's valid cache rows permuted (K and V together): the split
    ranges then hold other keys, and the combined result is still the
    unpermuted oracle's."""
    d, Hq, Hkv, S_cap = 128, 16, 4, 2048
    lens = np.array([2048, 1500, 333, 64, 1], dtype=np.int32)
    _, q, kc, vc = inputs.draw_decode_bits(9400, len(lens), Hq, Hkv, d, 0, 0, S_cap, lens=lens)
    rng = np.random.Generator(np.random.PCG64(9401))
    kp, vp = kc.copy(), vc.copy()
    for b, n in enumerate(lens):
        perm = rng.permutation(int(n))
        kp[b, :, :n] = kc[b, :, perm].transpose(1, 0, 2)
        vp[b, :, :n] = vc[b, :, perm].transpose(1, 0, 2)
    s = inputs.default_scale(d)
    o, lse, guards = H.run_decode(q, kp, vp, lens, s, 16)
    assert guards
    o_ref, l_ref = oracle.attn_decode(q, kc, vc, lens, s)
    m = H.metrics(o, lse, o_ref, l_ref)
    _note(f"[gpu] permuted decode keys: {m}")
    H.assert_parity(m, "permuted decode keys")
