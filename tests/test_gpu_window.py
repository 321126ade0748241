"""GPU: prefill with a sliding window (attn_fwd_window) against the f64 oracle.

Row i sees keys [i + Sk - Sq - W, i + Sk - Sq] (causal) or from
i + Sk - Sq - W on (not causal). Cases cover head dimensions 64 (the simple
kernel), 128 and 256 (the persistent kernel), windows narrower than, equal to
and wider than a 32-key tile, Sq < Sk and Sq > Sk, rows whose window holds no
key, GQA, and more work items than resident workgroups. Tolerances as for
attn_fwd: O max-abs 1e-2, O rel-RMS 4e-3, LSE max-abs 1e-3; rows with no key
exactly (+0, -inf).
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


def _inputs(seed, B, Hq, Hkv, Sq, Sk, d, std=1.0):
    return (_rand_bits(seed, (B, Hq, Sq, d), std), _rand_bits(seed + 1, (B, Hkv, Sk, d), std),
            _rand_bits(seed + 2, (B, Hkv, Sk, d), std))


WINDOW = [
    # B, Hq, Hkv, Sq, Sk, d, causal, window
    (1, 4, 2, 300, 300, 128, True, 0),
    (1, 4, 2, 300, 300, 128, True, 31),
    (1, 8, 8, 1000, 1000, 128, True, 100),
    (2, 16, 4, 700, 1100, 128, True, 257),   # Sq < Sk
    (1, 4, 4, 500, 200, 128, True, 64),      # Sq > Sk: leading rows see no key
    (1, 2, 2, 400, 400, 128, False, 50),     # window without the causal bound
    (1, 2, 2, 300, 100, 128, False, 10),     # windows past the last key: empty rows
    (8, 64, 8, 256, 512, 128, True, 40),     # many items per persistent workgroup
    (1, 4, 1, 600, 600, 256, True, 200),
    (1, 4, 4, 333, 333, 256, False, 1),
    (4, 32, 4, 200, 200, 256, True, 32),
    (1, 4, 2, 300, 300, 64, True, 0),
    (2, 4, 2, 700, 700, 64, True, 128),
    (1, 4, 4, 250, 250, 64, False, 33),
    (1, 2, 1, 300, 120, 64, True, 5),
]


@pytest.mark.parametrize("case", WINDOW)
def test_window_parity(case):
    B, Hq, Hkv, Sq, Sk, d, causal, W = case
    seed = 5000 + WINDOW.index(case)
    q, k, v = _inputs(seed, B, Hq, Hkv, Sq, Sk, d, 0.5)
    scale = inputs.default_scale(d)
    label = f"window {case}"
    _note(f"[gpu] {label}: running the HIP path")
    o, lse, guards = H.run_fwd(q, k, v, causal, scale, window=W)
    assert guards, f"{label}: write outside the logical outputs"
    o_ref, lse_ref = oracle.attn_fwd(q, k, v, causal, scale, window=W)
    m = H.metrics(o, lse, o_ref, lse_ref)
    _note(f"[gpu] {label}: {m}")
    H.assert_parity(m, label)


@pytest.mark.parametrize("d", [64, 128, 256])
def test_wide_window_equals_attn_fwd(d):
    """A window wider than every row's keys changes nothing, bit for bit."""
    B, Hq, Hkv, Sq, Sk = 1, 4, 2, 300, 350
    q, k, v = _inputs(60 + d, B, Hq, Hkv, Sq, Sk, d)
    scale = inputs.default_scale(d)
    for causal in (False, True):
        o0, l0, _ = H.run_fwd(q, k, v, causal, scale)
        o1, l1, _ = H.run_fwd(q, k, v, causal, scale, window=Sq + Sk)
        assert np.array_equal(o0, o1)
        assert np.array_equal(l0.view(np.uint32), l1.view(np.uint32))


# The sliding-window row of the pages' variant table (§7.3: window 128, forward,
# n = 8k, d = 64; batch and heads are not stated: 4 x 16 here), every row, and a
# Mistral-class long window at d = 128 on sampled rows.
def test_window_workload_d64_w128_full():
    B, H_, S, d, W = 4, 16, 8192, 64, 128
    q, k, v = _inputs(7100, B, H_, H_, S, S, d)
    scale = inputs.default_scale(d)
    _note("[gpu] window d64 W128 S8192: running the HIP path")
    o, lse, guards = H.run_fwd(q, k, v, True, scale, window=W)
    assert guards
    o_ref, lse_ref = oracle.attn_fwd(q, k, v, True, scale, window=W)
    m = H.metrics(o, lse, o_ref, lse_ref)
    _note(f"[gpu] window d64 W128 S8192: {m}")
    H.assert_parity(m, "window d64 W128")


def test_window_workload_d128_w4096_sampled():
    B, H_, S, d, W = 1, 32, 16384, 128, 4096
    q = _rand_bits(7200, (B, H_, S, d), 0.5)
    k = _rand_bits(7201, (B, 8, S, d), 0.5)
    v = _rand_bits(7202, (B, 8, S, d), 0.5)
    scale = inputs.default_scale(d)
    _note("[gpu] window d128 W4096 S16384 GQA 4: running the HIP path")
    o, lse, guards = H.run_fwd(q, k, v, True, scale, window=W)
    assert guards
    rng = np.random.Generator(np.random.PCG64(7203))
    rows = np.unique(np.concatenate([h * S + np.concatenate(
        [rng.choice(S, 256, replace=False), [0, W - 1, W, W + 1, S - 1]])
        for h in range(B * H_)])).astype(np.int64)
    o_ref, lse_ref = oracle.attn_fwd(q, k, v, True, scale, rows=rows, window=W)
    m = H.metrics(o.reshape(-1, d)[rows], lse.reshape(-1)[rows], o_ref, lse_ref)
    _note(f"[gpu] window d128 W4096: {m}")
    H.assert_parity(m, "window d128 W4096")
