"""GPU parity: the HIP path through the C ABI against the f64 oracle.

Every case draws seeded bf16 inputs, runs libmiattn on the GPU with
NaN-prefilled outputs and guard regions, and compares with the oracle on the
same bits at O max-abs 1e-2, O rel-RMS 4e-3 and LSE max-abs 1e-3; rows with
no visible key must be exactly (+0, -inf). The five workloads run at full
size in the launch configuration the bench times; the long-context workload
(B1 Hq16 Hkv2 S44032 d256) is checked on 512 sampled rows per head plus the
first and last row, every row of the others is checked.
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


def _check_full(q, k, v, causal, scale, label):
    _note(f"[gpu] {label}: shape q{q.shape} k{k.shape} causal={causal}")
    o, lse, guards = H.run_fwd(q, k, v, causal, scale)
    assert guards, f"{label}: write outside the logical outputs"
    o_ref, lse_ref = oracle.attn_fwd(q, k, v, causal, scale)
    m = H.metrics(o, lse, o_ref, lse_ref)
    _note(f"[gpu] {label}: {m}")
    H.assert_parity(m, label)
    return o, lse


@pytest.mark.parametrize("wid,causal", [(1, False), (2, True), (2, False), (3, True)])
def test_workload_full_rows(wid, causal):
    w = inputs.WORKLOADS[wid]
    q, k, v = inputs.prefill_inputs(w)
    _check_full(q, k, v, causal, w.scale, f"workload {wid} causal={causal}")


def test_workload1_against_unrounded_fp32_draws():
    """The tiny workload is drawn in fp32; the GPU reads its bf16 rounding.
    For information the error against the oracle on the unrounded draws
    (exact f32 bits widened) is also within the tolerances."""
    w = inputs.WORKLOADS[1]
    q, k, v = inputs.prefill_inputs(w)
    o, lse, _ = H.run_fwd(q, k, v, False, w.scale)
    qf, kf, vf = inputs.prefill_inputs_f32(w)
    # an f64 reference on the unrounded fp32 values, via torch CPU f64
    import torch
    t = [torch.from_numpy(x.astype(np.float64)) for x in (qf, kf, vf)]
    ref = torch.nn.functional.scaled_dot_product_attention(*t, scale=w.scale).numpy()
    s = w.scale * (t[0] @ t[1].transpose(-1, -2).contiguous())
    lref = torch.logsumexp(s, dim=-1).numpy()
    m = H.metrics(o, lse, ref, lref)
    _note(f"[gpu] workload 1 vs fp32 draws: {m}")
    assert m["o_rel_rms"] <= H.O_REL_RMS and m["o_max_abs"] <= H.O_MAX_ABS


@pytest.mark.parametrize("wid,rows_per_head", [(4, 512)])
def test_workload_sampled_rows(wid, rows_per_head):
    w = inputs.WORKLOADS[wid]
    _note(f"[gpu] workload {wid}: drawing inputs")
    q, k, v = inputs.prefill_inputs(w)
    causal = w.causal[0]
    _note(f"[gpu] workload {wid}: running the HIP path")
    o, lse, guards = H.run_fwd(q, k, v, causal, w.scale)
    assert guards
    rows = inputs.sampled_rows(w, rows_per_head)
    _note(f"[gpu] workload {wid}: oracle on {rows.size} sampled rows")
    o_ref, lse_ref = oracle.attn_fwd(q, k, v, causal, w.scale, rows=rows)
    m = H.metrics(o.reshape(-1, w.d)[rows], lse.reshape(-1)[rows], o_ref, lse_ref)
    _note(f"[gpu] workload {wid}: {m}")
    H.assert_parity(m, f"workload {wid}")
    # every row was written (NaN prefill)
    assert not np.any(o == H.NAN_BF16) and not np.any(np.isnan(lse))


RAGGED = [
    # B, Hq, Hkv, Sq, Sk, d, causal
    (1, 2, 2, 300, 300, 64, True),
    (1, 2, 2, 300, 300, 128, False),
    (2, 4, 2, 257, 257, 256, True),
    (1, 8, 1, 100, 333, 128, True),   # Sq < Sk: bottom-right causal alignment
    (1, 2, 1, 200, 77, 64, True),     # Sq > Sk: leading rows see no key
    (1, 2, 2, 1, 1, 128, False),
    (1, 2, 2, 5, 0, 64, False),       # Sk = 0: every row empty
    (1, 2, 2, 5, 0, 256, True),
    (3, 3, 1, 33, 65, 256, False),
    (1, 1, 1, 129, 129, 128, True),
    (2, 6, 3, 190, 190, 64, False),
    (1, 4, 4, 64, 1000, 256, True),
]


@pytest.mark.parametrize("case", RAGGED)
def test_ragged_and_edge_shapes(case):
    B, Hq, Hkv, Sq, Sk, d, causal = case
    seed = 1000 + RAGGED.index(case)
    q = _rand_bits(seed, (B, Hq, Sq, d))
    k = _rand_bits(seed + 1, (B, Hkv, Sk, d))
    v = _rand_bits(seed + 2, (B, Hkv, Sk, d))
    _check_full(q, k, v, causal, inputs.default_scale(d), f"ragged {case}")


# Several work items per persistent workgroup (more items than the device
# holds workgroups), where the copy stream runs from one item into the next:
# items shorter than the four-tile ring (some first tiles copied in the
# previous item, the rest in the item's own prologue), items that see no key
# at all (Sq > Sk causal: the first query tile), GQA groups, and a number of
# (batch, kv-head) units that is not a multiple of the 8 XCDs (the other tile
# order). The last two are checked on sampled rows. Values are drawn with
# standard deviation 0.5, as in the Llama-class workload: a row that sees only
# one or two keys has |O| up to the largest |v|, and where that passes 4 the
# bf16 rounding of O alone (half an ulp, 2^-6) exceeds the 1e-2 bound.
PERSIST = [
    # B, Hq, Hkv, Sq, Sk, d, causal, rows sampled per head (0: all)
    (8, 64, 8, 256, 64, 128, False, 0),     # 512 items of 2 tiles
    (8, 64, 8, 256, 100, 128, True, 0),     # 4 tiles, leading rows empty
    (4, 64, 4, 512, 40, 128, True, 0),      # items of 0 and 2 tiles, alternating
    (8, 32, 4, 256, 64, 256, False, 0),     # head dimension 256: 512 items of 2 tiles
    (8, 32, 8, 256, 40, 256, True, 0),      # 256: items of 0 and 2 tiles
    (2, 48, 16, 1536, 1536, 128, True, 96),  # GQA 3, items of 8 .. 48 tiles
    (3, 30, 3, 2048, 2048, 128, True, 64),  # 9 units: not a multiple of 8
]


@pytest.mark.parametrize("case", PERSIST)
def test_persistent_item_walk(case):
    B, Hq, Hkv, Sq, Sk, d, causal, per_head = case
    seed = 3000 + PERSIST.index(case)
    q = _rand_bits(seed, (B, Hq, Sq, d), 0.5)
    k = _rand_bits(seed + 1, (B, Hkv, Sk, d), 0.5)
    v = _rand_bits(seed + 2, (B, Hkv, Sk, d), 0.5)
    scale = inputs.default_scale(d)
    if per_head == 0:
        _check_full(q, k, v, causal, scale, f"persistent {case}")
        return
    _note(f"[gpu] persistent {case}: running the HIP path")
    o, lse, guards = H.run_fwd(q, k, v, causal, scale)
    assert guards
    rng = np.random.Generator(np.random.PCG64(seed + 3))
    rows = np.sort(np.concatenate([h * Sq + rng.choice(Sq, per_head, replace=False)
                                   for h in range(B * Hq)]))
    o_ref, lse_ref = oracle.attn_fwd(q, k, v, causal, scale, rows=rows)
    m = H.metrics(o.reshape(-1, d)[rows], lse.reshape(-1)[rows], o_ref, lse_ref)
    _note(f"[gpu] persistent {case}: {m}")
    H.assert_parity(m, f"persistent {case}")
    assert not np.any(o == H.NAN_BF16) and not np.any(np.isnan(lse))


def test_gqa_is_bitwise_repeated_mha():
    q = _rand_bits(21, (1, 8, 150, 128))
    k = _rand_bits(22, (1, 2, 150, 128))
    v = _rand_bits(23, (1, 2, 150, 128))
    s = inputs.default_scale(128)
    o1, l1, _ = H.run_fwd(q, k, v, True, s)
    o2, l2, _ = H.run_fwd(q, np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1), True, s)
    assert np.array_equal(o1, o2) and np.array_equal(l1.view(np.uint32), l2.view(np.uint32))


@pytest.mark.parametrize("d", [64, 128, 256])
def test_causal_first_row_and_masked_key_exactness(d):
    S, jstar = 200, 70
    q = _rand_bits(31, (1, 2, S, d))
    k = _rand_bits(32, (1, 2, S, d))
    v = _rand_bits(33, (1, 2, S, d))
    s = inputs.default_scale(d)
    o, lse, _ = H.run_fwd(q, k, v, True, s)
    # row 0 sees only key 0: p = 1 exactly, so O equals V row 0 bit for bit
    assert np.array_equal(o[:, :, 0], v[:, :, 0])
    # changing key j* (finite values) must leave every row i < j* bit-identical
    k2, v2 = k.copy(), v.copy()
    k2[:, :, jstar] = _rand_bits(34, (1, 2, d), std=3.0)
    v2[:, :, jstar] = _rand_bits(35, (1, 2, d), std=3.0)
    o2, lse2, _ = H.run_fwd(q, k2, v2, True, s)
    assert np.array_equal(o2[:, :, :jstar], o[:, :, :jstar])
    assert np.array_equal(lse2[:, :, :jstar].view(np.uint32), lse[:, :, :jstar].view(np.uint32))
    assert not np.array_equal(o2[:, :, jstar:], o[:, :, jstar:])


@pytest.mark.parametrize("d,causal", [(64, False), (128, True), (256, True)])
def test_constant_values_give_that_constant(d, causal):
    """Constant V: O equals the constant up to the bf16 rounding of P (the
    value contraction sums bf16 probabilities, the normaliser their f32 sum):
    within one bf16 ulp everywhere, exactly where a row sees a single key."""
    q = _rand_bits(41, (2, 2, 150, d), std=2.0)
    k = _rand_bits(42, (2, 2, 150, d), std=2.0)
    cval = -1.71875
    c = inputs.f32_to_bf16_bits_scalar(cval)
    v = np.full((2, 2, 150, d), c, dtype=np.uint16)
    o, _, _ = H.run_fwd(q, k, v, causal, inputs.default_scale(d))
    of = inputs.bf16_to_f32(o).astype(np.float64)
    assert np.max(np.abs(of - cval)) <= 2.0 ** -7 * 2  # one bf16 ulp at |c| in [1, 2)
    assert np.mean(o == c) > 0.9
    if causal:
        assert np.all(o[:, :, 0] == c)


def test_zero_keys_give_uniform_average():
    S, d = 190, 128
    q = _rand_bits(51, (1, 2, S, d))
    k = np.zeros((1, 2, S, d), dtype=np.uint16)
    v = _rand_bits(52, (1, 2, S, d))
    o, lse, _ = H.run_fwd(q, k, v, True, inputs.default_scale(d))
    n = np.arange(1, S + 1, dtype=np.float64)
    assert np.max(np.abs(lse - np.log(n))) <= H.LSE_MAX_ABS
    vf = inputs.bf16_to_f32(v).astype(np.float64)
    ref = np.cumsum(vf, axis=2) / n[None, None, :, None]
    m = H.metrics(o, lse, ref, np.log(n)[None, None, :].repeat(2, axis=1))
    H.assert_parity(m, "zero keys")


def test_deterministic_across_runs():
    w = inputs.WORKLOADS[2]
    q, k, v = inputs.prefill_inputs(w)
    o1, l1, _ = H.run_fwd(q, k, v, True, w.scale)
    o2, l2, _ = H.run_fwd(q, k, v, True, w.scale)
    assert np.array_equal(o1, o2) and np.array_equal(l1.view(np.uint32), l2.view(np.uint32))


# ------------------------------------------------------------------ decode --
def test_decode_workload_full():
    w = inputs.WORKLOADS[5]
    _note("[gpu] decode workload: drawing inputs")
    lens, q, kc, vc = inputs.decode_inputs(w)
    _note(f"[gpu] decode workload: lens sum {int(lens.sum())}")
    o, lse, guards = H.run_decode(q, kc, vc, lens, w.scale, w.num_splits)
    assert guards
    o_ref, lse_ref = oracle.attn_decode(q, kc, vc, lens, w.scale)
    m = H.metrics(o, lse, o_ref, lse_ref)
    _note(f"[gpu] decode workload: {m}")
    H.assert_parity(m, "decode workload")


@pytest.mark.parametrize("d,Hq,Hkv,splits", [(128, 32, 8, 16), (64, 4, 4, 3), (256, 8, 1, 7),
                                              (128, 6, 2, 1), (64, 3, 1, 40),
                                              # query-head groups wider than the 16 MFMA
                                              # columns: 20 = 16 + 4 and 34 = 16 + 16 + 2
                                              (128, 40, 2, 5), (64, 34, 1, 4),
                                              # more splits than a wave has lanes
                                              (64, 4, 2, 100)])
def test_decode_edge_lengths(d, Hq, Hkv, splits):
    lens = np.array([0, 1, 3, 15, 16, 17, 200, 511], dtype=np.int32)
    S_cap = 511
    lens_, q, kc, vc = inputs.draw_decode_bits(77 + d + splits, len(lens), Hq, Hkv, d, 0, 0,
                                               S_cap, lens=lens)
    s = inputs.default_scale(d)
    o, lse, guards = H.run_decode(q, kc, vc, lens, s, splits)
    assert guards
    o_ref, lse_ref = oracle.attn_decode(q, kc, vc, lens, s)
    m = H.metrics(o, lse, o_ref, lse_ref)
    _note(f"[gpu] decode d={d} Hq={Hq} Hkv={Hkv} splits={splits}: {m}")
    H.assert_parity(m, "decode edges")
    assert m["empty_rows"] == Hq  # the stream of length 0


def test_decode_many_streams():
    """More streams than one wave can rank by length (they then go in index
    order), with lengths spread over [0, S_cap]."""
    rng = np.random.Generator(np.random.PCG64(4242))
    lens = rng.integers(0, 300, size=70, endpoint=True).astype(np.int32)
    lens[[3, 40]] = 0
    _, q, kc, vc = inputs.draw_decode_bits(4243, 70, 8, 2, 128, 0, 0, 300, lens=lens)
    s = inputs.default_scale(128)
    o, lse, guards = H.run_decode(q, kc, vc, lens, s, 6)
    assert guards
    o_ref, lse_ref = oracle.attn_decode(q, kc, vc, lens, s)
    m = H.metrics(o, lse, o_ref, lse_ref)
    _note(f"[gpu] decode 70 streams: {m}")
    H.assert_parity(m, "decode many streams")
    assert m["empty_rows"] == 2 * 8


def test_decode_padding_is_never_read():
    lens = np.array([5, 300, 1024, 17], dtype=np.int32)
    args = (99, 4, 16, 4, 128, 0, 0, 1024)
    _, q, kc0, vc0 = inputs.draw_decode_bits(*args, lens=lens, pad_bits=0)
    _, _, kcn, vcn = inputs.draw_decode_bits(*args, lens=lens, pad_bits=int(inputs.BF16_NAN))
    s = inputs.default_scale(128)
    o0, l0, _ = H.run_decode(q, kc0, vc0, lens, s, 16)
    on, ln, _ = H.run_decode(q, kcn, vcn, lens, s, 16, ws_fill=0.0)
    assert np.array_equal(o0, on) and np.array_equal(l0.view(np.uint32), ln.view(np.uint32))
    # decode equals the prefill kernel's Sq = 1 forward within tolerance
    o_ref, lse_ref = oracle.attn_decode(q, kc0, vc0, lens, s)
    H.assert_parity(H.metrics(o0, l0, o_ref, lse_ref), "decode padding")


def test_decode_lengths_clamped_on_device():
    lens = np.array([-5, 2000], dtype=np.int32)  # clamp to [0, S_cap = 64]
    _, q, kc, vc = inputs.draw_decode_bits(5, 2, 4, 2, 64, 0, 0, 64,
                                           lens=np.array([0, 64], dtype=np.int32))
    s = inputs.default_scale(64)
    o, lse, _ = H.run_decode(q, kc, vc, lens, s, 4)
    o_ref, lse_ref = oracle.attn_decode(q, kc, vc, np.array([0, 64], dtype=np.int32), s)
    H.assert_parity(H.metrics(o, lse, o_ref, lse_ref), "decode clamp")


# Scores that make the running reference move late or far. Every query row is
# the same +-1 vector u and key jstar is gamma * u, so row i's score for jstar
# is gamma * sqrt(d) above the O(1) scores of the random keys: 33 (gamma = 2)
# or 200 (gamma = 12) log2 units at d = 128. The first makes a tile's row sums
# exceed the reference's bound when jstar arrives in the middle of the keys;
# the second overflows them to inf. Sq > Sk with causal leaves the first rows
# of the first waves without any visible key. All values are exact in bf16.
REF_CASES = [
    # (d, causal, Sq, Sk, jstar, gamma)
    (128, True, 1000, 1000, 700, 2.0),
    (128, False, 600, 1000, 700, 2.0),
    (128, True, 1000, 1000, 5, 2.0),
    (128, True, 1000, 1000, 700, 12.0),
    (256, True, 700, 700, 450, 2.0),
    (256, False, 300, 700, 450, 12.0),
    (128, True, 300, 200, 150, 2.0),
    (256, True, 300, 200, 150, 2.0),
]


@pytest.mark.parametrize("case", REF_CASES)
def test_reference_moves_late_or_far(case):
    d, causal, Sq, Sk, jstar, gamma = case
    seed = 2000 + REF_CASES.index(case)
    rng = np.random.Generator(np.random.PCG64(seed))
    u = np.where(rng.random(d) < 0.5, -1.0, 1.0).astype(np.float32)
    q = inputs.bf16_bits(np.broadcast_to(u, (1, 2, Sq, d)).copy())
    kf = rng.standard_normal(size=(1, 1, Sk, d), dtype=np.float32) * np.float32(0.5)
    kf[0, 0, jstar, :] = np.float32(gamma) * u
    k = inputs.bf16_bits(kf)
    v = _rand_bits(seed + 1, (1, 1, Sk, d))
    _check_full(q, k, v, causal, inputs.default_scale(d), f"reference {case}")
