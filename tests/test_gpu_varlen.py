"""GPU: packed variable-length batches (attn_fwd_varlen, and attn_fwd_varlen_ext
with windows, soft caps and ALiBi) against the f64 oracle.

Sequences of 0 to 1000 query rows and as many or more keys (a chunk of new
queries against its cached prefix), causal and not, head dimensions 64, 128
and 256, GQA; max_seqlen_q above the longest sequence (the launch's items past a
sequence's end are skipped); more work items than resident workgroups. A
batch of equal lengths must match attn_fwd on the same data bit for bit.
Tolerances as for attn_fwd.
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


def _bits(seed, shape, std=0.5):
    rng = np.random.Generator(np.random.PCG64(seed))
    return inputs.bf16_bits(rng.standard_normal(size=shape, dtype=np.float32) * np.float32(std))


def _run(q, k, v, cu_q, cu_k, max_q, max_k, causal, scale):
    torch = H.torch_mod()
    Hq, total_q, d = q.shape
    Hkv, total_k, _ = k.shape
    n = Hq * total_q
    o, lse = H.nan_out(n * d, n)
    cq = torch.tensor(cu_q, dtype=torch.int32, device="cuda")
    ck = torch.tensor(cu_k, dtype=torch.int32, device="cuda")
    H.miattn.attn_fwd_varlen(H.dev_bits(q), H.dev_bits(k), H.dev_bits(v), o, lse, cq, ck,
                             len(cu_q) - 1, total_q, total_k, max_q, max_k, Hq, Hkv, d, causal,
                             scale)
    torch.cuda.synchronize()
    ob = H.host_bits(o)
    lh = lse.cpu().numpy()
    guards = bool(np.all(ob[n * d:] == H.NAN_BF16) and np.all(np.isnan(lh[n:])))
    return ob[:n * d].reshape(Hq, total_q, d), lh[:n].reshape(Hq, total_q), guards


VARLEN = [
    # seed, query lengths, extra cached keys per sequence, Hq, Hkv, d, causal
    (1, [0, 1, 31, 32, 33, 257, 700], [0, 0, 0, 5, 100, 0, 64], 4, 2, 128, True),
    (2, [0, 1, 31, 32, 33, 257, 700], [0, 3, 0, 0, 0, 9, 0], 4, 2, 128, False),
    (3, [5, 300, 129, 1000], [0, 200, 0, 17], 4, 1, 256, True),
    (4, [64, 65, 190], [1, 0, 300], 2, 2, 256, False),
    (5, [0, 1, 31, 33, 127, 129, 700], [0, 2, 0, 40, 0, 9, 64], 4, 2, 64, True),
    (6, [5, 300, 129], [0, 200, 17], 6, 3, 64, False),
    # Hq a multiple of 8: the walk gives a kv-head's query heads one XCD
    # (Hkv a multiple of 8) or an equal share of the XCDs (Hkv dividing 8)
    (7, [33, 300, 129, 5], [0, 64, 17, 0], 8, 1, 128, True),
    (8, [190, 64, 257], [3, 0, 40], 16, 2, 128, True),
    (9, [77, 300], [0, 100], 16, 16, 64, False),
    (10, [129, 31, 400], [9, 0, 0], 8, 4, 256, True),
]


@pytest.mark.parametrize("case", VARLEN)
def test_varlen_parity(case):
    seed, lq, extra, Hq, Hkv, d, causal = case
    lk = [a + b for a, b in zip(lq, extra)]
    cu_q = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
    q = _bits(seed * 10, (Hq, int(cu_q[-1]), d))
    k = _bits(seed * 10 + 1, (Hkv, int(cu_k[-1]), d))
    v = _bits(seed * 10 + 2, (Hkv, int(cu_k[-1]), d))
    scale = inputs.default_scale(d)
    label = f"varlen {case}"
    _note(f"[gpu] {label}: running the HIP path")
    o, lse, guards = _run(q, k, v, cu_q, cu_k, max(lq) + 100, max(lk) + 100, causal, scale)
    assert guards, f"{label}: write outside the logical outputs"
    o_ref, lse_ref = oracle.attn_fwd_varlen(q, k, v, cu_q, cu_k, causal, scale)
    m = H.metrics(o, lse, o_ref, lse_ref)
    _note(f"[gpu] {label}: {m}")
    H.assert_parity(m, label)


@pytest.mark.parametrize("d", [64, 128, 256])
def test_varlen_equal_lengths_match_attn_fwd(d):
    B, Hq, Hkv, S = 3, 4, 2, 300
    q = _bits(40 + d, (B, Hq, S, d))
    k = _bits(41 + d, (B, Hkv, S, d))
    v = _bits(42 + d, (B, Hkv, S, d))
    pack = lambda x: np.ascontiguousarray(x.transpose(1, 0, 2, 3).reshape(x.shape[1], -1, d))
    cu = (np.arange(B + 1) * S).astype(np.int32)
    scale = inputs.default_scale(d)
    for causal in (False, True):
        o0, l0, _ = H.run_fwd(q, k, v, causal, scale)
        o1, l1, guards = _run(pack(q), pack(k), pack(v), cu, cu, S, S, causal, scale)
        assert guards
        assert np.array_equal(o1, o0.transpose(1, 0, 2, 3).reshape(Hq, B * S, d))
        assert np.array_equal(l1.view(np.uint32),
                              l0.transpose(1, 0, 2).reshape(Hq, B * S).view(np.uint32))


def test_varlen_many_sequences_sampled():
    """40 sequences, lengths U[0, 1200], GQA 4: more items than resident
    workgroups; every sequence's rows checked on a sample."""
    rng = np.random.Generator(np.random.PCG64(77))
    lq = rng.integers(0, 1200, size=40, endpoint=True)
    lk = lq + rng.integers(0, 300, size=40, endpoint=True)
    cu_q = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
    Hq, Hkv, d = 16, 4, 128
    q = _bits(78, (Hq, int(cu_q[-1]), d))
    k = _bits(79, (Hkv, int(cu_k[-1]), d))
    v = _bits(80, (Hkv, int(cu_k[-1]), d))
    scale = inputs.default_scale(d)
    _note("[gpu] varlen 40 sequences: running the HIP path")
    o, lse, guards = _run(q, k, v, cu_q, cu_k, int(lq.max()), int(lk.max()), True, scale)
    assert guards
    # two sampled rows per (head, sequence) plus its first and last
    picks = []
    for b in range(40):
        if lq[b] == 0:
            continue
        rows = {0, int(lq[b]) - 1, *rng.integers(0, lq[b], size=2).tolist()}
        picks += [(b, r) for r in sorted(rows)]
    o_ref = np.zeros((Hq, len(picks), d))
    l_ref = np.zeros((Hq, len(picks)))
    o_got = np.zeros((Hq, len(picks), d), dtype=np.uint16)
    l_got = np.zeros((Hq, len(picks)), dtype=np.float32)
    for n, (b, r) in enumerate(picks):
        q0, k0, k1 = int(cu_q[b]), int(cu_k[b]), int(cu_k[b + 1])
        # the row's own attention: Sq = lq[b], Sk = lk[b], row r of the sequence
        rows = np.arange(Hq) * int(lq[b]) + r
        ob, lb = oracle.attn_fwd(q[None, :, q0:q0 + int(lq[b])], k[None, :, k0:k1],
                                 v[None, :, k0:k1], True, scale, rows=rows)
        o_ref[:, n], l_ref[:, n] = ob, lb
        o_got[:, n], l_got[:, n] = o[:, q0 + r], lse[:, q0 + r]
    m = H.metrics(o_got, l_got, o_ref, l_ref)
    _note(f"[gpu] varlen 40 sequences: {m}")
    H.assert_parity(m, "varlen 40 sequences")


def test_varlen_more_than_64_sequences():
    """70 sequences (past what a wave ranks in its lanes): the walk over the
    plain item space that skips items past each sequence's end."""
    rng = np.random.Generator(np.random.PCG64(90))
    lq = rng.integers(0, 300, size=70, endpoint=True)
    lk = lq + rng.integers(0, 100, size=70, endpoint=True)
    lq[[5, 33]] = 0
    cu_q = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
    Hq, Hkv, d = 4, 2, 128
    q = _bits(91, (Hq, int(cu_q[-1]), d))
    k = _bits(92, (Hkv, int(cu_k[-1]), d))
    v = _bits(93, (Hkv, int(cu_k[-1]), d))
    scale = inputs.default_scale(d)
    _note("[gpu] varlen 70 sequences: running the HIP path")
    o, lse, guards = _run(q, k, v, cu_q, cu_k, int(lq.max()), int(lk.max()), True, scale)
    assert guards
    o_ref, lse_ref = oracle.attn_fwd_varlen(q, k, v, cu_q, cu_k, True, scale)
    m = H.metrics(o, lse, o_ref, lse_ref)
    _note(f"[gpu] varlen 70 sequences: {m}")
    H.assert_parity(m, "varlen 70 sequences")


def test_varlen_bench_configuration_sampled():
    """The bench's packed chunked prefill (16 sequences of U[512, 4096]
    queries against prefixes of U[0, 2048] keys, Hq 32, Hkv 8, d 128,
    causal), in the bench's launch configuration; rows sampled per sequence
    and head against the oracle."""
    rng = np.random.Generator(np.random.PCG64(7300))
    lq = rng.integers(512, 4096, size=16, endpoint=True)
    lk = lq + rng.integers(0, 2048, size=16, endpoint=True)
    cu_q = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
    Hq, Hkv, d = 32, 8, 128
    q, k, v = inputs.draw_prefill_bits(7301, 1, Hq, Hkv, int(lq.sum()), int(lk.sum()), d)
    q, k, v = q[0], k[0], v[0]
    scale = inputs.default_scale(d)
    _note("[gpu] varlen bench configuration: running the HIP path")
    o, lse, guards = _run(q, k, v, cu_q, cu_k, int(lq.max()), int(lk.max()), True, scale)
    assert guards
    pick = np.random.Generator(np.random.PCG64(7302))
    o_ref, l_ref, o_got, l_got = [], [], [], []
    for b in range(16):
        q0, k0, k1, n = int(cu_q[b]), int(cu_k[b]), int(cu_k[b + 1]), int(lq[b])
        rows_b = np.unique(np.concatenate([[0, n - 1], pick.integers(0, n, size=6)]))
        rows = (np.arange(Hq)[:, None] * n + rows_b[None, :]).reshape(-1)
        ob, lb = oracle.attn_fwd(q[None, :, q0:q0 + n], k[None, :, k0:k1], v[None, :, k0:k1],
                                 True, scale, rows=rows)
        o_ref.append(ob)
        l_ref.append(lb)
        o_got.append(o[:, q0 + rows_b].reshape(-1, d))
        l_got.append(lse[:, q0 + rows_b].reshape(-1))
    m = H.metrics(np.concatenate(o_got), np.concatenate(l_got), np.concatenate(o_ref),
                  np.concatenate(l_ref))
    _note(f"[gpu] varlen bench configuration: {m}")
    H.assert_parity(m, "varlen bench configuration")


# ---- packed batches with the score and mask variants (attn_fwd_varlen_ext) ----------

def _run_ext(q, k, v, cu_q, cu_k, max_q, max_k, causal, scale, window, softcap, alibi):
    torch = H.torch_mod()
    Hq, total_q, d = q.shape
    Hkv, total_k, _ = k.shape
    n = Hq * total_q
    o, lse = H.nan_out(n * d, n)
    cq = torch.tensor(cu_q, dtype=torch.int32, device="cuda")
    ck = torch.tensor(cu_k, dtype=torch.int32, device="cuda")
    ad = None if alibi is None else torch.from_numpy(np.ascontiguousarray(alibi, np.float32)).cuda()
    H.miattn.attn_fwd_varlen_ext(H.dev_bits(q), H.dev_bits(k), H.dev_bits(v), o, lse, cq, ck,
                                 len(cu_q) - 1, total_q, total_k, max_q, max_k, Hq, Hkv, d,
                                 causal, window, softcap, ad, scale)
    torch.cuda.synchronize()
    ob = H.host_bits(o)
    lh = lse.cpu().numpy()
    guards = bool(np.all(ob[n * d:] == H.NAN_BF16) and np.all(np.isnan(lh[n:])))
    return ob[:n * d].reshape(Hq, total_q, d), lh[:n].reshape(Hq, total_q), guards


def _slopes(Hq):
    return (2.0 ** (-8.0 * (np.arange(Hq) + 1) / Hq)).astype(np.float32)


VARLEN_EXT = [
    # seed, query lengths, extra cached keys, Hq, Hkv, d, causal, window, softcap, ALiBi
    (11, [0, 1, 31, 33, 257, 700], [0, 0, 5, 100, 0, 64], 4, 2, 128, True, 64, 0.0, False),
    (12, [5, 300, 129], [0, 200, 17], 4, 2, 128, False, 100, 0.0, False),
    (13, [1, 33, 300, 0], [0, 9, 40, 3], 4, 2, 128, True, -1, 30.0, False),
    (14, [1, 33, 300], [3, 0, 100], 4, 1, 64, True, -1, 0.0, True),
    (15, [64, 190, 513], [1, 0, 300], 2, 2, 256, False, -1, 20.0, True),
    (16, [31, 257, 700], [0, 64, 5], 6, 3, 64, True, 128, 50.0, True),
    (17, [129, 0, 400], [20, 7, 0], 4, 2, 256, True, 32, 0.0, True),
]


@pytest.mark.parametrize("case", VARLEN_EXT)
def test_varlen_ext_parity(case):
    """Windows, soft caps and ALiBi on packed batches: each sequence takes the
    variant against its own lengths; against the f64 oracle per sequence."""
    seed, lq, extra, Hq, Hkv, d, causal, window, softcap, use_alibi = case
    lk = [a + b for a, b in zip(lq, extra)]
    cu_q = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
    q = _bits(seed * 10, (Hq, int(cu_q[-1]), d))
    k = _bits(seed * 10 + 1, (Hkv, int(cu_k[-1]), d))
    v = _bits(seed * 10 + 2, (Hkv, int(cu_k[-1]), d))
    al = _slopes(Hq) if use_alibi else None
    scale = inputs.default_scale(d)
    label = f"varlen ext {case}"
    _note(f"[gpu] {label}: running the HIP path")
    o, lse, guards = _run_ext(q, k, v, cu_q, cu_k, max(lq) + 40, max(lk) + 40, causal, scale,
                              window, softcap, al)
    assert guards, f"{label}: write outside the logical outputs"
    o_ref, lse_ref = oracle.attn_fwd_varlen(q, k, v, cu_q, cu_k, causal, scale, window=window,
                                            softcap=softcap, alibi=al)
    m = H.metrics(o, lse, o_ref, lse_ref)
    _note(f"[gpu] {label}: {m}")
    H.assert_parity(m, label)


@pytest.mark.parametrize("d", [64, 128, 256])
def test_varlen_ext_equal_lengths_match_attn_fwd_ext(d):
    """A packed batch of equal lengths under every variant at once gives
    attn_fwd_ext's outputs bit for bit."""
    B, Hq, Hkv, S = 3, 4, 2, 300
    q = _bits(50 + d, (B, Hq, S, d))
    k = _bits(51 + d, (B, Hkv, S, d))
    v = _bits(52 + d, (B, Hkv, S, d))
    pack = lambda x: np.ascontiguousarray(x.transpose(1, 0, 2, 3).reshape(x.shape[1], -1, d))
    cu = (np.arange(B + 1) * S).astype(np.int32)
    scale = inputs.default_scale(d)
    al = _slopes(Hq)
    for causal, window, softcap in ((True, 77, 30.0), (False, 40, 0.0)):
        _note(f"[gpu] varlen ext equal lengths d={d} causal={causal}: running the HIP path")
        o0, l0, _ = H.run_fwd_ext(q, k, v, causal, scale, window=window, softcap=softcap,
                                  alibi=al)
        o1, l1, guards = _run_ext(pack(q), pack(k), pack(v), cu, cu, S, S, causal, scale, window,
                                  softcap, al)
        assert guards
        assert np.array_equal(o1, o0.transpose(1, 0, 2, 3).reshape(Hq, B * S, d))
        assert np.array_equal(l1.view(np.uint32),
                              l0.transpose(1, 0, 2).reshape(Hq, B * S).view(np.uint32))
