"""GPU: the attention backward (attn_bwd) against the f64 backward oracle.

O and LSE, the backward's inputs from the forward, come from the oracle
(O rounded to bf16, LSE to f32) so that the backward is checked on its own;
one case feeds it the GPU forward's outputs instead. The expected gradients
are the oracle's f64 dQ, dK, dV from Q, K, V and dO alone.

Tolerance, per gradient tensor: relative RMS error <= 8e-3 and max-abs error
<= 1.2e-2 of the tensor's largest magnitude. The error budget: the kernels
round four quantities to bf16 (RNE, relative error up to 2^-8 and about
2^-9 / sqrt(3) = 1.1e-3 RMS each): P and dS before their MFMAs, O (read for
D_i = dO_i . O_i) and the gradients themselves. Summed over many rows with
independent signs these give about 1.6e-3 RMS for dV (P and the result) and
about 2.2e-3 for dK and dQ (dS, O through D, the result), plus the f32
accumulation (1e-6). dS = P (dP - D) cancels where dP is close to D, which
scales one term's relative error up, so single elements reach a few times the
RMS. Measured on every case: rel-RMS 2.1-2.9e-3, max 2.5-4.3e-3 of the tensor
maximum; the bounds sit at about three times that, so an error one rounding
larger than the budget fails.
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


def _check(q, k, v, do, causal, scale, label, o_bits=None, lse=None):
    if o_bits is None:
        o_ref, lse_ref = oracle.attn_fwd(q, k, v, causal, scale)
        o_bits = inputs.bf16_bits(o_ref.astype(np.float32))
        lse = lse_ref.astype(np.float32)
    _note(f"[gpu] {label}: running the HIP backward")
    dq, dk, dv, guards = H.run_bwd(q, k, v, o_bits, lse, do, causal, scale)
    assert guards, f"{label}: write outside the gradients"
    rq, rk, rv = bw.attn_bwd(q, k, v, do, causal, scale)
    for name, got, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        m = H.grad_metrics(got, ref)
        _note(f"[gpu] {label} {name}: {m}")
        assert m["finite"], f"{label} {name}: non-finite"
        assert m["rel_rms"] <= REL_RMS, f"{label} {name}: {m}"
        assert m["max_abs_rel"] <= MAX_REL, f"{label} {name}: {m}"


BWD = [
    # B, Hq, Hkv, Sq, Sk, d, causal
    (1, 2, 2, 64, 64, 64, True),
    (1, 2, 2, 77, 129, 64, False),
    (2, 4, 2, 300, 300, 128, True),
    (1, 4, 1, 129, 300, 128, True),    # Sq < Sk
    (1, 2, 2, 200, 77, 128, True),     # Sq > Sk: leading rows see no key
    (1, 4, 4, 190, 190, 128, False),
    (2, 6, 3, 257, 257, 64, True),
    (1, 2, 2, 64, 64, 256, True),
    (1, 4, 2, 130, 300, 256, False),   # GQA, Sq < Sk, ragged
    (2, 4, 1, 257, 257, 256, True),    # GQA 4
    (1, 2, 2, 200, 77, 256, True),     # Sq > Sk: leading rows see no key
]


@pytest.mark.parametrize("case", BWD)
def test_backward_parity(case):
    B, Hq, Hkv, Sq, Sk, d, causal = case
    seed = 8000 + 10 * BWD.index(case)
    q = _bits(seed, (B, Hq, Sq, d), 0.5)
    k = _bits(seed + 1, (B, Hkv, Sk, d), 0.5)
    v = _bits(seed + 2, (B, Hkv, Sk, d))
    do = _bits(seed + 3, (B, Hq, Sq, d))
    _check(q, k, v, do, causal, inputs.default_scale(d), f"bwd {case}")


@pytest.mark.parametrize("d", [128, 256])
def test_backward_after_the_gpu_forward(d):
    """The whole step on the GPU: attn_fwd's O and LSE feed attn_bwd."""
    B, Hq, Hkv, S = 1, 8, 2, 512
    q = _bits(8100 + d, (B, Hq, S, d), 0.5)
    k = _bits(8101 + d, (B, Hkv, S, d), 0.5)
    v = _bits(8102 + d, (B, Hkv, S, d))
    do = _bits(8103 + d, (B, Hq, S, d))
    scale = inputs.default_scale(d)
    o_bits, lse, _ = H.run_fwd(q, k, v, True, scale)
    _check(q, k, v, do, True, scale, f"bwd after gpu fwd d={d}", o_bits=o_bits, lse=lse)


def test_backward_workload_full_size_sampled_heads():
    """The bench's backward: the prefill workload (B2 H32 S4096 d128 causal),
    the GPU forward's O and LSE feeding the backward, in the bench's launch
    configuration; four (batch, head) slices checked against the oracle,
    which computes them from Q, K, V and dO alone (one query head per
    kv-head)."""
    w = inputs.WORKLOADS[3]
    q, k, v = inputs.prefill_inputs(w)
    do = _bits(w.seed + 11, (w.B, w.Hq, w.Sq, w.d))
    _note("[gpu] backward workload: forward then backward on the GPU")
    o_bits, lse, _ = H.run_fwd(q, k, v, True, w.scale)
    dq, dk, dv, guards = H.run_bwd(q, k, v, o_bits, lse, do, True, w.scale)
    assert guards
    for b, h in ((0, 0), (0, 17), (1, 6), (1, 31)):
        sl = (slice(b, b + 1), slice(h, h + 1))
        rq, rk, rv = bw.attn_bwd(q[sl], k[sl], v[sl], do[sl], True, w.scale)
        for name, got, ref in (("dq", dq[sl], rq), ("dk", dk[sl], rk), ("dv", dv[sl], rv)):
            m = H.grad_metrics(got, ref)
            _note(f"[gpu] backward workload b={b} h={h} {name}: {m}")
            assert m["finite"] and m["rel_rms"] <= REL_RMS and m["max_abs_rel"] <= MAX_REL, m


@pytest.mark.parametrize("d", [128, 256])
def test_backward_gqa_full(d):
    """Grouped-query heads at a size with many query tiles per key tile:
    B1 Hq8 Hkv2 S2048 causal, forward and backward on the GPU, every element
    of dQ, dK and dV against the oracle (dK and dV of a kv-head sum over its
    four query heads)."""
    B, Hq, Hkv, S = 1, 8, 2, 2048
    q = _bits(8300 + d, (B, Hq, S, d), 0.5)
    k = _bits(8301 + d, (B, Hkv, S, d), 0.5)
    v = _bits(8302 + d, (B, Hkv, S, d))
    do = _bits(8303 + d, (B, Hq, S, d))
    scale = inputs.default_scale(d)
    o_bits, lse, _ = H.run_fwd(q, k, v, True, scale)
    _check(q, k, v, do, True, scale, f"bwd gqa full d={d}", o_bits=o_bits, lse=lse)


@pytest.mark.parametrize("Sq,Sk,d", [(40, 0, 128), (0, 40, 128), (40, 0, 256), (0, 40, 256)])
def test_backward_degenerate_lengths(Sq, Sk, d):
    """No keys: dQ is exactly zero (no row sees a key). No queries: dK and dV
    are exactly zero (no query sees a key)."""
    B, Hq, Hkv = 1, 4, 2
    q = _bits(8200, (B, Hq, Sq, d))
    k = _bits(8201, (B, Hkv, Sk, d))
    v = _bits(8202, (B, Hkv, Sk, d))
    do = _bits(8203, (B, Hq, Sq, d))
    o_bits = np.zeros((B, Hq, Sq, d), dtype=np.uint16)
    lse = np.full((B, Hq, Sq), -np.inf, dtype=np.float32)
    dq, dk, dv, guards = H.run_bwd(q, k, v, o_bits, lse, do, True, inputs.default_scale(d))
    assert guards
    assert not dq.any() and not dk.any() and not dv.any()


def test_backward_d256_bench_shape_sampled_heads():
    """The bench's head-dimension-256 backward (B2 H16 S4096 d256 causal, the
    same seeded draws), the GPU forward's O and LSE feeding it, in that launch
    configuration; two (batch, head) slices against the oracle."""
    B, NH, S, d = 2, 16, 4096, 256
    q, k, v = inputs.draw_prefill_bits(7400, B, NH, NH, S, S, d, 0.5)
    (do,) = inputs.draw_prefill_bits(7401, B, NH, NH, S, S, d)[:1]
    scale = inputs.default_scale(d)
    _note("[gpu] backward d256 bench shape: forward then backward on the GPU")
    o_bits, lse, _ = H.run_fwd(q, k, v, True, scale)
    dq, dk, dv, guards = H.run_bwd(q, k, v, o_bits, lse, do, True, scale)
    assert guards
    for b, h in ((0, 3), (1, 12)):
        sl = (slice(b, b + 1), slice(h, h + 1))
        rq, rk, rv = bw.attn_bwd(q[sl], k[sl], v[sl], do[sl], True, scale)
        for name, got, ref in (("dq", dq[sl], rq), ("dk", dk[sl], rk), ("dv", dv[sl], rv)):
            m = H.grad_metrics(got, ref)
            _note(f"[gpu] backward d256 bench shape b={b} h={h} {name}: {m}")
            assert m["finite"] and m["rel_rms"] <= REL_RMS and m["max_abs_rel"] <= MAX_REL, m

