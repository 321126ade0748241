"""GPU: prefill with a score modifier (attn_fwd_ext): soft cap and ALiBi,
alone and with a sliding window, against the f64 oracle.

The soft cap replaces each scaled score s by cap * tanh(s / cap); ALiBi
subtracts slope_h * |i + Sk - Sq - j|, with the geometric slopes
2^(-8 (h + 1) / Hq). Cases cover head dimensions 64, 128 and 256, causal and
not, Sq != Sk, GQA and ragged sizes; the two variant rows of the pages'
table (n = 2k, d = 64) run at full size. Tolerances as for attn_fwd.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
from online_softmax_monoid_amd import inputs
from tests import harness as H

pytestmark = pytest.mark.gpu


def _note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _rand_bits(seed, shape, std=1.0):
    rng = np.random.Generator(np.random.PCG64(seed))
    return inputs.bf16_bits(rng.standard_normal(size=shape, dtype=np.float32) * np.float32(std))


def alibi_slopes(Hq):
    return (2.0 ** (-8.0 * (np.arange(Hq) + 1) / Hq)).astype(np.float32)


def _check(seed, B, Hq, Hkv, Sq, Sk, d, causal, window, softcap, alibi, std, label):
    q = _rand_bits(seed, (B, Hq, Sq, d), std)
    k = _rand_bits(seed + 1, (B, Hkv, Sk, d), std)
    v = _rand_bits(seed + 2, (B, Hkv, Sk, d), std)
    scale = inputs.default_scale(d)
    _note(f"[gpu] {label}: running the HIP path")
    o, lse, guards = H.run_fwd_ext(q, k, v, causal, scale, window, softcap, alibi)
    assert guards, f"{label}: write outside the logical outputs"
    o_ref, lse_ref = oracle.attn_fwd(q, k, v, causal, scale, window=window, softcap=softcap,
                                     alibi=alibi)
    m = H.metrics(o, lse, o_ref, lse_ref)
    _note(f"[gpu] {label}: {m}")
    H.assert_parity(m, label)


SOFTCAP = [
    # B, Hq, Hkv, Sq, Sk, d, causal, window, cap
    (1, 4, 2, 300, 300, 128, True, -1, 5.0),
    (1, 4, 4, 257, 400, 128, False, -1, 2.0),
    (1, 4, 1, 300, 300, 256, True, -1, 30.0),
    (2, 4, 4, 190, 260, 256, False, -1, 4.0),
    (1, 4, 2, 333, 333, 64, False, -1, 5.0),
    (2, 8, 2, 500, 500, 128, True, 100, 5.0),
    (1, 4, 4, 200, 200, 64, True, 50, 3.0),
]


@pytest.mark.parametrize("case", SOFTCAP)
def test_softcap_parity(case):
    B, Hq, Hkv, Sq, Sk, d, causal, window, cap = case
    _check(6000 + SOFTCAP.index(case), B, Hq, Hkv, Sq, Sk, d, causal, window, cap, None, 1.0,
           f"softcap {case}")


ALIBI = [
    # B, Hq, Hkv, Sq, Sk, d, causal, window
    (1, 8, 2, 300, 300, 128, True, -1),
    (1, 8, 8, 257, 400, 128, False, -1),
    (1, 4, 1, 300, 300, 256, True, -1),
    (1, 8, 4, 333, 333, 64, False, -1),
    (2, 8, 2, 500, 500, 128, True, 100),
    (1, 4, 4, 200, 200, 64, True, 64),
    (1, 4, 2, 150, 80, 128, True, -1),     # Sq > Sk: leading rows see no key
]


@pytest.mark.parametrize("case", ALIBI)
def test_alibi_parity(case):
    B, Hq, Hkv, Sq, Sk, d, causal, window = case
    _check(6100 + ALIBI.index(case), B, Hq, Hkv, Sq, Sk, d, causal, window, 0.0,
           alibi_slopes(Hq), 0.5, f"alibi {case}")


BOTH = [
    # B, Hq, Hkv, Sq, Sk, d, causal, window, softcap
    (1, 4, 2, 300, 300, 64, True, -1, 20.0),
    (2, 4, 4, 190, 333, 128, False, -1, 30.0),
    (1, 8, 2, 257, 257, 256, True, -1, 10.0),
    (1, 4, 4, 500, 500, 128, True, 64, 15.0),
]


@pytest.mark.parametrize("case", BOTH)
def test_softcap_and_alibi_together(case):
    """Soft cap, then ALiBi, then the mask (and a window in the last case)."""
    B, Hq, Hkv, Sq, Sk, d, causal, window, softcap = case
    _check(7700 + BOTH.index(case), B, Hq, Hkv, Sq, Sk, d, causal, window, softcap,
           alibi_slopes(Hq), 1.0, f"softcap+alibi {case}")


# the two score-variant rows of the pages' table (§7.3: forward, n = 2k,
# d = 64; batch and heads not stated there, 4 x 16 here), every row
def test_softcap_workload_d64_n2k_full():
    _check(6200, 4, 16, 16, 2048, 2048, 64, False, -1, 30.0, None, 1.0, "softcap d64 n2k")


def test_alibi_workload_d64_n2k_full():
    _check(6300, 4, 16, 16, 2048, 2048, 64, False, -1, 0.0, alibi_slopes(16), 1.0,
           "alibi d64 n2k")
