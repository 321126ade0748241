"""GPU: attn_fwd_decode_noalloc, the decode entry point that allocates
nothing (its split partials live in the library's fixed device scratch),
against attn_fwd_decode with a caller workspace, through the C ABI.

Both run the same kernels, so their outputs must agree bit for bit; the first
call is also checked against the f64 oracle at the decode tolerances. Two
calls in a row, the second with a smaller input (other shape, head dimension
and split count), show that what the first left in the scratch does not leak
into the second. A request whose partials exceed the scratch is rejected
before anything is launched.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
from online_softmax_monoid_amd import inputs, miattn
from tests import harness as H

pytestmark = pytest.mark.gpu

SCRATCH_BYTES = 16 << 20


def _note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _run_noalloc(q, kc, vc, lens, scale, splits):
    import torch
    B, Hq, d = q.shape
    _, Hkv, S_cap, _ = kc.shape
    ld = torch.from_numpy(np.ascontiguousarray(lens, dtype=np.int32)).to("cuda")
    n = B * Hq
    o, lse = H.nan_out(n * d, n)
    miattn.attn_fwd_decode_noalloc(H.dev_bits(q), H.dev_bits(kc), H.dev_bits(vc), ld, o, lse, B,
                                   Hq, Hkv, S_cap, d, splits, scale)
    torch.cuda.synchronize()
    ob = H.host_bits(o)
    lh = lse.cpu().numpy()
    guards = bool(np.all(ob[n * d:] == H.NAN_BF16) and np.all(np.isnan(lh[n:])))
    return ob[:n * d].reshape(B, Hq, d), lh[:n].reshape(B, Hq), guards


def _same(o1, l1, o2, l2):
    return np.array_equal(o1, o2) and np.array_equal(l1.view(np.uint32), l2.view(np.uint32))


def test_noalloc_matches_the_workspace_entry_on_two_calls():
    # first call: the batched decode workload (32 streams, Hq 32, Hkv 8, d 128,
    # lengths U[1024, 8192], 16 splits): 8.5 MB of partials
    w = inputs.WORKLOADS[5]
    lens, q, kc, vc = inputs.decode_inputs(w, pad_bits=int(inputs.BF16_NAN))
    need = miattn.attn_fwd_decode_workspace_size(w.B, w.Hq, w.d, w.num_splits)
    assert need <= SCRATCH_BYTES
    _note(f"[gpu] noalloc call 1: B={w.B} Hq={w.Hq} d={w.d} splits={w.num_splits} "
          f"({need} bytes of partials)")
    o1, l1, g1 = _run_noalloc(q, kc, vc, lens, w.scale, w.num_splits)
    o1w, l1w, g1w = H.run_decode(q, kc, vc, lens, w.scale, w.num_splits)
    assert g1 and g1w
    assert _same(o1, l1, o1w, l1w)
    o_ref, l_ref = oracle.attn_decode(q, kc, vc, lens, w.scale)
    m = H.metrics(o1, l1, o_ref, l_ref)
    _note(f"[gpu] noalloc call 1 vs oracle: {m}")
    H.assert_parity(m, "noalloc call 1")

    # second call, smaller: 5 streams (one empty), Hq 8, Hkv 2, d 256, 7 splits
    lens2 = np.array([700, 0, 1, 333, 1024], dtype=np.int32)
    _, q2, kc2, vc2 = inputs.draw_decode_bits(9500, 5, 8, 2, 256, 0, 0, 1024, lens=lens2,
                                              pad_bits=int(inputs.BF16_NAN))
    s2 = inputs.default_scale(256)
    _note("[gpu] noalloc call 2: B=5 Hq=8 Hkv=2 d=256 splits=7")
    o2, l2, g2 = _run_noalloc(q2, kc2, vc2, lens2, s2, 7)
    o2w, l2w, g2w = H.run_decode(q2, kc2, vc2, lens2, s2, 7)
    assert g2 and g2w
    assert _same(o2, l2, o2w, l2w)
    m2 = H.metrics(o2, l2, *oracle.attn_decode(q2, kc2, vc2, lens2, s2))
    _note(f"[gpu] noalloc call 2 vs oracle: {m2}")
    H.assert_parity(m2, "noalloc call 2")
    assert m2["empty_rows"] == 8


def test_noalloc_rejects_partials_beyond_the_scratch():
    import torch
    B, Hq, Hkv, d, splits = 64, 64, 8, 256, 16
    assert miattn.attn_fwd_decode_workspace_size(B, Hq, d, splits) > SCRATCH_BYTES
    q = torch.zeros(B * Hq * d, dtype=torch.int16, device="cuda")
    kc = torch.zeros(B * Hkv * 16 * d, dtype=torch.int16, device="cuda")
    lens = torch.full((B,), 16, dtype=torch.int32, device="cuda")
    o, lse = H.nan_out(B * Hq * d, B * Hq)
    with pytest.raises(miattn.MiattnError) as exc:
        miattn.attn_fwd_decode_noalloc(q, kc, kc, lens, o, lse, B, Hq, Hkv, 16, d, splits,
                                       inputs.default_scale(d))
    assert exc.value.status == miattn.MIATTN_ERR_UNSUPPORTED
    assert "scratch" in exc.value.message
    torch.cuda.synchronize()
    assert np.all(H.host_bits(o) == H.NAN_BF16)  # nothing was launched
