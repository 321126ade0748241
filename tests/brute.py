"""Brute-force softmax attention for tiny inputs (pure Python, no numpy).

Independent of the oracle: it uses the textbook form of softmax, with no
maximum subtracted,

    p_j = exp(s_j) / sum_k exp(s_k),   O = sum_j p_j v_j,   LSE = ln sum_k exp(s_k),

sums with ``math.fsum`` (exactly rounded), and its own bf16 widening, mask and
head map. ``mp_attention`` repeats the computation in mpmath at 50 digits as a
second referee. Only small scores are fed to it, so exp cannot overflow.
"""
from __future__ import annotations

import math
import struct


def bf16_value(bits: int) -> float:
    return struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]


def _visible(i, j, Sq, Sk, causal, window=-1):
    # bottom-right aligned causal mask: key j is visible to query i iff
    # j - i <= Sk - Sq; a sliding window further needs j - i >= Sk - Sq - window
    if causal and j - i > Sk - Sq:
        return False
    return window < 0 or j - i >= Sk - Sq - window


def attention(q, k, v, causal, scale, window=-1, softcap=0.0, alibi=None):
    """q: nested lists [B][Hq][Sq][d] of bf16 bits; k, v: [B][Hkv][Sk][d].

    Returns (o, lse) as nested lists of Python floats.
    """
    B, Hq, Sq, d = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    Hkv, Sk = len(k[0]), len(k[0][0])
    group = Hq // Hkv
    o = [[[None] * Sq for _ in range(Hq)] for _ in range(B)]
    lse = [[[None] * Sq for _ in range(Hq)] for _ in range(B)]
    for b in range(B):
        for h in range(Hq):
            kvh = h // group
            for i in range(Sq):
                keys = [j for j in range(Sk) if _visible(i, j, Sq, Sk, causal, window)]
                if not keys:
                    o[b][h][i] = [0.0] * d
                    lse[b][h][i] = -math.inf
                    continue
                e = {}
                for j in keys:
                    dot = math.fsum(bf16_value(q[b][h][i][t]) * bf16_value(k[b][kvh][j][t])
                                    for t in range(d))
                    sj = scale * dot
                    if softcap > 0:
                        sj = softcap * math.tanh(sj / softcap)
                    if alibi is not None:
                        sj -= alibi[h] * abs(i + Sk - Sq - j)
                    e[j] = math.exp(sj)
                z = math.fsum(e.values())
                o[b][h][i] = [math.fsum(e[j] * bf16_value(v[b][kvh][j][t]) for j in keys) / z
                              for t in range(d)]
                lse[b][h][i] = math.log(z)
    return o, lse


def mp_attention(q, k, v, causal, scale, dps=50):
    import mpmath
    mpmath.mp.dps = dps
    B, Hq, Sq, d = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    Hkv, Sk = len(k[0]), len(k[0][0])
    group = Hq // Hkv
    sc = mpmath.mpf(scale)
    o = [[[None] * Sq for _ in range(Hq)] for _ in range(B)]
    lse = [[[None] * Sq for _ in range(Hq)] for _ in range(B)]
    for b in range(B):
        for h in range(Hq):
            kvh = h // group
            for i in range(Sq):
                keys = [j for j in range(Sk) if _visible(i, j, Sq, Sk, causal)]
                if not keys:
                    o[b][h][i] = [mpmath.mpf(0)] * d
                    lse[b][h][i] = -mpmath.inf
                    continue
                e = {}
                for j in keys:
                    dot = mpmath.fsum(mpmath.mpf(bf16_value(q[b][h][i][t]))
                                      * mpmath.mpf(bf16_value(k[b][kvh][j][t]))
                                      for t in range(d))
                    e[j] = mpmath.exp(sc * dot)
                z = mpmath.fsum(e.values())
                o[b][h][i] = [mpmath.fsum(e[j] * mpmath.mpf(bf16_value(v[b][kvh][j][t]))
                                          for j in keys) / z for t in range(d)]
                lse[b][h][i] = mpmath.log(z)
    return o, lse
