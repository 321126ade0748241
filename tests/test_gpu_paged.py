"""GPU: split-KV decode over a paged KV cache (attn_fwd_decode_paged).

A paged cache is the gather view of the contiguous one, so two checks apply to
every case: bit-for-bit equality with attn_fwd_decode on the contiguous cache
that holds the same rows (same splits, same kernels apart from the addresses
of the copies), and parity with the f64 oracle's decode of the gathered
cache at O max-abs 1e-2, O rel-RMS 4e-3, LSE max-abs 1e-3. Pool pages no
stream owns hold NaN bits, so a copy from a wrong page shows up.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
from online_softmax_monoid_amd import inputs
from tests import harness as H

pytestmark = pytest.mark.gpu
NAN = int(inputs.BF16_NAN)


def _note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _same_bits(o1, l1, o2, l2, label):
    assert np.array_equal(o1, o2), f"{label}: O differs from the contiguous decode"
    assert np.array_equal(l1.view(np.uint32), l2.view(np.uint32)), f"{label}: LSE differs"


def _paged_case(seed, lens, Hq, Hkv, d, P, splits, spare=5, table_junk=False):
    lens = np.asarray(lens, dtype=np.int32)
    max_pages = max(1, int((lens.max() + P - 1) // P) + 1)
    S_cap = max_pages * P
    _, q, kc, vc = inputs.draw_decode_bits(seed, len(lens), Hq, Hkv, d, 0, 0, S_cap, lens=lens,
                                           pad_bits=NAN)
    table, npg = inputs.paged_layout(seed + 1, lens, P, max_pages, spare_pages=spare)
    kp = inputs.scatter_to_pages(kc, table, npg, P, fill_bits=NAN)
    vp = inputs.scatter_to_pages(vc, table, npg, P, fill_bits=NAN)
    if table_junk:  # entries past each stream's last page: never used
        table = np.where(table < 0, np.int32(1 << 30), table).astype(np.int32)
        table[:, -1] = -7
    scale = inputs.default_scale(d)
    label = f"paged B={len(lens)} Hq={Hq} Hkv={Hkv} d={d} P={P} splits={splits}"
    _note(f"[gpu] {label}: running the HIP path")
    o, lse, guards = H.run_decode_paged(q, kp, vp, table, lens, P, scale, splits)
    assert guards, f"{label}: write outside the logical outputs"
    oc, lc, _ = H.run_decode(q, kc, vc, lens, scale, splits)
    _same_bits(o, lse, oc, lc, label)
    o_ref, lse_ref = oracle.attn_decode_paged(q, kp, vp, table, lens, P, scale)
    m = H.metrics(o, lse, o_ref, lse_ref)
    _note(f"[gpu] {label}: {m}")
    H.assert_parity(m, label)
    assert m["empty_rows"] == Hq * int((lens == 0).sum())


PAGED = [
    # seed, lens, Hq, Hkv, d, page size, splits
    (11, [0, 1, 15, 16, 17, 100, 257, 600], 8, 2, 128, 16, 4),
    (12, [0, 1, 15, 16, 17, 100, 257, 600], 8, 2, 128, 16, 16),
    (13, [3, 64, 65, 500], 4, 4, 64, 64, 3),
    (14, [1, 31, 33, 290], 8, 1, 256, 32, 5),
    (15, [255, 256, 257, 1000], 40, 2, 128, 256, 7),   # 20 heads per kv-head
    (16, [7, 2000, 48, 1500], 16, 4, 128, 128, 1),     # one split per stream
]


@pytest.mark.parametrize("case", PAGED)
def test_paged_decode_matches_contiguous_and_oracle(case):
    seed, lens, Hq, Hkv, d, P, splits = case
    _paged_case(seed, lens, Hq, Hkv, d, P, splits)


def test_paged_decode_ignores_unused_table_entries():
    """Entries past a stream's last page (here 2^30 and -7) are never used;
    the three entries a block reads are clamped, so reading them is safe."""
    _paged_case(21, [0, 5, 40, 33, 130], 8, 2, 128, 16, 6, table_junk=True)


def test_paged_decode_clamps_bad_entries():
    """An entry outside [0, num_pages) reads the nearest pool page instead of
    memory outside the pool (the values are then those of that page)."""
    lens = np.array([40, 70], dtype=np.int32)
    P, d, Hq, Hkv = 16, 128, 4, 2
    _, q, kc, vc = inputs.draw_decode_bits(31, 2, Hq, Hkv, d, 0, 0, 80, lens=lens)
    table, npg = inputs.paged_layout(32, lens, P, 5, spare_pages=2)
    kp = inputs.scatter_to_pages(kc, table, npg, P)
    vp = inputs.scatter_to_pages(vc, table, npg, P)
    table[0, 1] = -3
    table[1, 2] = npg + 40
    scale = inputs.default_scale(d)
    o, lse, guards = H.run_decode_paged(q, kp, vp, table, lens, P, scale, 4)
    assert guards
    kg = oracle.gather_pages(kp, table, lens, P)
    vg = oracle.gather_pages(vp, table, lens, P)
    oc, lc, _ = H.run_decode(q, kg, vg, lens, scale, 4)
    _same_bits(o, lse, oc, lc, "paged clamp")
    o_ref, lse_ref = oracle.attn_decode(q, kg, vg, lens, scale)
    H.assert_parity(H.metrics(o, lse, o_ref, lse_ref), "paged clamp")


def test_paged_decode_without_pages():
    """max_pages_per_seq = 0: every stream is empty, pools and table unused."""
    torch = H.torch_mod()
    B, Hq, Hkv, d = 3, 4, 2, 64
    q = inputs.bf16_bits(np.ones((B, Hq, d), np.float32))
    o, lse = H.nan_out(B * Hq * d, B * Hq)
    lens = torch.full((B,), 9, dtype=torch.int32, device="cuda")
    nbytes = H.miattn.attn_fwd_decode_workspace_size(B, Hq, d, 2)
    ws = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda")
    H.miattn.attn_fwd_decode_paged(H.dev_bits(q), 0, 0, 0, lens, o, lse, B, Hq, Hkv, 0, 16, 0,
                                   d, 2, 0.125, ws, nbytes)
    torch.cuda.synchronize()
    ob = H.host_bits(o)[:B * Hq * d]
    lh = lse.cpu().numpy()[:B * Hq]
    assert np.all(ob == 0) and np.all(np.isneginf(lh))


def test_paged_decode_workload_full():
    """The batched decode workload (32 streams, lengths U[1024, 8192], 16
    splits) stored in 16-key pages in random pool order."""
    w = inputs.WORKLOADS[5]
    P = 16
    _note("[gpu] paged decode workload: drawing inputs")
    lens, q, kc, vc = inputs.decode_inputs(w, pad_bits=NAN)
    table, npg = inputs.paged_layout(w.seed + 7, lens, P, w.S_cap // P, spare_pages=64)
    kp = inputs.scatter_to_pages(kc, table, npg, P, fill_bits=NAN)
    vp = inputs.scatter_to_pages(vc, table, npg, P, fill_bits=NAN)
    _note(f"[gpu] paged decode workload: {npg} pages of {P} keys")
    o, lse, guards = H.run_decode_paged(q, kp, vp, table, lens, P, w.scale, w.num_splits)
    assert guards
    oc, lc, _ = H.run_decode(q, kc, vc, lens, w.scale, w.num_splits)
    _same_bits(o, lse, oc, lc, "paged decode workload")
    o_ref, lse_ref = oracle.attn_decode(q, kc, vc, lens, w.scale)
    m = H.metrics(o, lse, o_ref, lse_ref)
    _note(f"[gpu] paged decode workload: {m}")
    H.assert_parity(m, "paged decode workload")
