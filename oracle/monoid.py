"""The online-softmax monoid in f64 -- TEST INFRASTRUCTURE ONLY.

The tang paper (§2.2 "Comprehensions and monoids") makes online softmax a
reduction whose state is the running maximum together with the sum rescaled
to it, and attention carries the weighted value vector along in the same
state. Written out, the state of a set of keys is

    (m, l, a) = (max_j s_j,  sum_j exp(s_j - m),  sum_j exp(s_j - m) v_j)

and two states over disjoint key sets combine as

    M = max(m1, m2)
    (m1, l1, a1) (+) (m2, l2, a2) = (M, l1 e^(m1-M) + l2 e^(m2-M),
                                        a1 e^(m1-M) + a2 e^(m2-M))

with the convention that a side whose m is -inf contributes nothing. The
identity is (-inf, 0, 0): the paper's Lean proof (§6 "Verification") covers a
commutative semigroup and says the compiler supplies the identity, which this
convention realises. A key j enters as the leaf (s_j, 1, v_j). The finished
value is O = a / l and LSE = m + ln l; the empty set finishes to (0, -inf).

§2.5 "Schedules" states that splitting the reduce space across threads and
tree-combining is valid for any associative monoid, including this one; the
tests fold the leaves in random trees and random orders and compare against
the two-pass definition in ``attn_oracle.c``.

Scores are formed with numpy's f64 matrix-vector product (a library primitive
used as one step); everything else is the combine above.
"""
from __future__ import annotations

import math
from typing import Sequence, Tuple

import numpy as np

State = Tuple[float, float, np.ndarray]


def identity(d: int) -> State:
    return (-math.inf, 0.0, np.zeros(d, dtype=np.float64))


def leaf(s: float, v: np.ndarray) -> State:
    return (float(s), 1.0, np.asarray(v, dtype=np.float64).copy())


def combine(x: State, y: State) -> State:
    m1, l1, a1 = x
    m2, l2, a2 = y
    M = max(m1, m2)
    if M == -math.inf:
        return (-math.inf, 0.0, np.zeros_like(a1))
    w1 = 0.0 if m1 == -math.inf else math.exp(m1 - M)
    w2 = 0.0 if m2 == -math.inf else math.exp(m2 - M)
    return (M, l1 * w1 + l2 * w2, a1 * w1 + a2 * w2)


def finish(x: State):
    m, l, a = x
    if l == 0.0:
        return np.zeros_like(a), -math.inf
    return a / l, m + math.log(l)


def fold(states: Sequence[State], d: int) -> State:
    acc = identity(d)
    for st in states:
        acc = combine(acc, st)
    return acc


def fold_tree(states: Sequence[State], d: int, rng: np.random.Generator) -> State:
    """Combine the states as a random binary tree (random split points)."""
    states = list(states)
    if not states:
        return identity(d)
    if len(states) == 1:
        return states[0]
    cut = int(rng.integers(1, len(states)))
    return combine(fold_tree(states[:cut], d, rng), fold_tree(states[cut:], d, rng))


def widen(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> f64, exactly."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def row_leaves(q_row_bits, k_bits, v_bits, nkeys: int, scale: float):
    """Leaves (s_j, 1, v_j) of one query row over keys 0..nkeys-1.

    k_bits / v_bits: [Sk, d] bit arrays of the row's kv-head.
    """
    q = widen(q_row_bits)
    K = widen(k_bits[:nkeys])
    V = widen(v_bits[:nkeys])
    s = float(scale) * (K @ q)
    return [leaf(s[j], V[j]) for j in range(nkeys)]


def split_bounds(n: int, num_splits: int):
    """Balanced split s covers keys [floor(s*n/ns), floor((s+1)*n/ns))."""
    return [((s * n) // num_splits, ((s + 1) * n) // num_splits)
            for s in range(num_splits)]


def decode_split(q_bits, kc_bits, vc_bits, lens, scale: float, num_splits: int):
    """Split-KV decode: fold each split, then combine the partial states.

    q: [B,Hq,d]; caches [B,Hkv,S_cap,d]; returns (o [B,Hq,d], lse [B,Hq]).
    """
    B, Hq, d = q_bits.shape
    Hkv = kc_bits.shape[1]
    G = Hq // Hkv
    o = np.zeros((B, Hq, d))
    lse = np.zeros((B, Hq))
    for b in range(B):
        n = int(lens[b])
        for h in range(Hq):
            g = h // G
            leaves = row_leaves(q_bits[b, h], kc_bits[b, g], vc_bits[b, g], n, scale)
            partials = [fold(leaves[lo:hi], d) for lo, hi in split_bounds(n, num_splits)]
            o[b, h], lse[b, h] = finish(fold(partials, d))
    return o, lse
