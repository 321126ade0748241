"""f64 oracle of the attention backward -- TEST INFRASTRUCTURE ONLY.

Gradients of O = softmax(scale Q K^T + mask) V with respect to Q, K and V,
given the upstream gradient dO, written out as the plain definition in double
precision (NumPy matrix products as the only library steps). The tang paper
(§3, "Gradients are comprehensions") derives the flash backward from the
forward comprehension and states the identity it rests on: the softmax
gradient needs only the row statistic D_i = sum_j P_ij dP_ij, which equals
dO_i . O_i, so P is recomputed from the saved log-sum-exp instead of stored:

    P_ij  = exp(scale q_i . k_j - LSE_i)     (0 for masked keys)
    dV_j  = sum_i P_ij dO_i
    dP_ij = dO_i . v_j
    D_i   = dO_i . O_i
    dS_ij = P_ij (dP_ij - D_i)
    dQ_i  = scale sum_j dS_ij k_j
    dK_j  = scale sum_i dS_ij q_i

With grouped-query heads the key/value gradients of a kv-head sum over the
query heads that read it. Masks follow the forward (bottom-right causal). A
row with no visible key has P = 0 and contributes nothing.

Only the test suite may import this module; it shares nothing with the HIP
library.
"""
from __future__ import annotations

import numpy as np


def _f64(bits):
    """bf16 bit patterns widened exactly: bits << 16 is the float32 pattern."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def visible_mask(Sq: int, Sk: int, causal: bool) -> np.ndarray:
    """[Sq, Sk] boolean: key j visible to query i (bottom-right causal)."""
    i = np.arange(Sq)[:, None]
    j = np.arange(Sk)[None, :]
    if not causal:
        return np.ones((Sq, Sk), dtype=bool)
    return j <= i + (Sk - Sq)


def forward_f64(q, k, v, causal: bool, scale: float):
    """Two-pass softmax attention on f64 arrays q [B,Hq,Sq,d], k/v [B,Hkv,Sk,d];
    returns (O, LSE) with O = 0, LSE = -inf on rows with no visible key."""
    B, Hq, Sq, d = q.shape
    Hkv, Sk = k.shape[1], k.shape[2]
    G = Hq // Hkv
    vis = visible_mask(Sq, Sk, causal)
    o = np.zeros((B, Hq, Sq, d))
    lse = np.full((B, Hq, Sq), -np.inf)
    for b in range(B):
        for h in range(Hq):
            s = scale * (q[b, h] @ k[b, h // G].T)
            s = np.where(vis, s, -np.inf)
            m = s.max(axis=1, initial=-np.inf)
            live = np.isfinite(m)
            w = np.where(vis & live[:, None], np.exp(s - np.where(live, m, 0.0)[:, None]), 0.0)
            l = w.sum(axis=1)
            o[b, h, live] = (w[live] @ v[b, h // G]) / l[live, None]
            lse[b, h, live] = m[live] + np.log(l[live])
    return o, lse


def backward_f64(q, k, v, do, causal: bool, scale: float, o=None, lse=None):
    """Gradients (dQ, dK, dV) of the attention forward on f64 arrays, given
    dO [B,Hq,Sq,d]. O and LSE are recomputed unless given."""
    B, Hq, Sq, d = q.shape
    Hkv, Sk = k.shape[1], k.shape[2]
    G = Hq // Hkv
    if o is None or lse is None:
        o, lse = forward_f64(q, k, v, causal, scale)
    vis = visible_mask(Sq, Sk, causal)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            live = np.isfinite(lse[b, h])
            s = scale * (q[b, h] @ k[b, g].T)
            p = np.where(vis & live[:, None],
                         np.exp(s - np.where(live, lse[b, h], 0.0)[:, None]), 0.0)
            dv[b, g] += p.T @ do[b, h]
            dp = do[b, h] @ v[b, g].T
            D = np.sum(do[b, h] * o[b, h], axis=1)
            ds = p * (dp - D[:, None])
            dq[b, h] = scale * (ds @ k[b, g])
            dk[b, g] += scale * (ds.T @ q[b, h])
    return dq, dk, dv


def attn_bwd(q_bits, k_bits, v_bits, do_bits, causal: bool, scale: float):
    """The backward on the bf16 bit patterns the GPU reads (widened exactly);
    returns f64 (dQ, dK, dV)."""
    return backward_f64(_f64(q_bits), _f64(k_bits), _f64(v_bits), _f64(do_bits), causal,
                        float(np.float32(scale)))
