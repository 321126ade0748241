"""Pins of the f64 backward oracle (CPU only), against facts other than itself:
central finite differences of the forward, torch's float64 autograd of its
own attention (a library special case), grouped-query heads as repeated
multi-head keys, and the closed forms of a single visible key."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from oracle import backward as bw
from online_softmax_monoid_amd import inputs


def _rand(rng, shape, std=1.0):
    return rng.standard_normal(size=shape) * std


@pytest.mark.parametrize("causal", [False, True])
def test_backward_matches_finite_differences(causal):
    """d/dx of L = sum(O * G) by central differences, every element of Q, K, V."""
    rng = np.random.Generator(np.random.PCG64(40 + causal))
    B, Hq, Hkv, Sq, Sk, d = 1, 2, 1, 4, 6, 3
    q, k, v = _rand(rng, (B, Hq, Sq, d)), _rand(rng, (B, Hkv, Sk, d)), _rand(rng, (B, Hkv, Sk, d))
    G = _rand(rng, (B, Hq, Sq, d))
    scale = 0.7
    dq, dk, dv = bw.backward_f64(q, k, v, G, causal, scale)
    eps = 1e-6
    for x, dx in ((q, dq), (k, dk), (v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            old = x[idx]
            x[idx] = old + eps
            lp = np.sum(bw.forward_f64(q, k, v, causal, scale)[0] * G)
            x[idx] = old - eps
            lm = np.sum(bw.forward_f64(q, k, v, causal, scale)[0] * G)
            x[idx] = old
            num[idx] = (lp - lm) / (2 * eps)
        np.testing.assert_allclose(dx, num, rtol=1e-6, atol=1e-8)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_matches_torch_f64_autograd(causal):
    torch = pytest.importorskip("torch")
    rng = np.random.Generator(np.random.PCG64(50 + causal))
    B, H, Sq, Sk, d = 2, 3, 7, 7, 5
    q, k, v = _rand(rng, (B, H, Sq, d)), _rand(rng, (B, H, Sk, d)), _rand(rng, (B, H, Sk, d))
    do = _rand(rng, (B, H, Sq, d))
    scale = 0.3
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    to = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal,
                                                          scale=scale)
    to.backward(torch.tensor(do, dtype=torch.float64))
    dq, dk, dv = bw.backward_f64(q, k, v, do, causal, scale)
    for mine, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        np.testing.assert_allclose(mine, ref.numpy(), rtol=1e-10, atol=1e-12)


def test_backward_gqa_sums_over_the_group():
    """GQA gradients equal those of multi-head attention with each kv-head
    repeated, with dK and dV summed over the repeats."""
    rng = np.random.Generator(np.random.PCG64(60))
    B, Hq, Hkv, S, d = 1, 4, 2, 6, 3
    q, k, v = _rand(rng, (B, Hq, S, d)), _rand(rng, (B, Hkv, S, d)), _rand(rng, (B, Hkv, S, d))
    do = _rand(rng, (B, Hq, S, d))
    dq, dk, dv = bw.backward_f64(q, k, v, do, True, 0.5)
    kr, vr = np.repeat(k, 2, axis=1), np.repeat(v, 2, axis=1)
    dq2, dkr, dvr = bw.backward_f64(q, kr, vr, do, True, 0.5)
    np.testing.assert_allclose(dq, dq2, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(dk, dkr.reshape(B, Hkv, 2, S, d).sum(axis=2), rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(dv, dvr.reshape(B, Hkv, 2, S, d).sum(axis=2), rtol=1e-13, atol=1e-15)


def test_backward_single_key_closed_form():
    """Causal row 0 sees key 0 alone: O_0 = v_0, so dV_0 gets dO_0 in full
    from row 0, and the softmax of one key has zero gradient: row 0 adds
    nothing to dQ or dK."""
    rng = np.random.Generator(np.random.PCG64(61))
    q, k, v = _rand(rng, (1, 1, 1, 4)), _rand(rng, (1, 1, 1, 4)), _rand(rng, (1, 1, 1, 4))
    do = _rand(rng, (1, 1, 1, 4))
    dq, dk, dv = bw.backward_f64(q, k, v, do, True, 0.9)
    assert np.allclose(dv, do, rtol=0, atol=1e-15)
    assert np.allclose(dq, 0.0, atol=1e-15) and np.allclose(dk, 0.0, atol=1e-15)


def test_backward_forward_agrees_with_the_c_oracle():
    """The backward's own f64 forward equals the C oracle's two-pass forward
    on the same bf16 bits (empty rows included)."""
    rng = np.random.Generator(np.random.PCG64(62))
    qb = inputs.bf16_bits(rng.standard_normal((1, 2, 9, 8), dtype=np.float32))
    kb = inputs.bf16_bits(rng.standard_normal((1, 1, 6, 8), dtype=np.float32))
    vb = inputs.bf16_bits(rng.standard_normal((1, 1, 6, 8), dtype=np.float32))
    o_c, l_c = oracle.attn_fwd(qb, kb, vb, True, 0.25)
    o_p, l_p = bw.forward_f64(bw._f64(qb), bw._f64(kb), bw._f64(vb), True, 0.25)
    np.testing.assert_allclose(o_p, o_c, rtol=1e-13, atol=1e-15)
    assert np.array_equal(np.isneginf(l_p), np.isneginf(l_c))
    fin = np.isfinite(l_c)
    np.testing.assert_allclose(l_p[fin], l_c[fin], rtol=1e-13)
