"""GPU: the library's launches captured in a HIP graph (torch.cuda.CUDAGraph)
and replayed.

A serving loop captures one prefill and one decode step and replays them on
new inputs; a training-style step captures a forward and its backward beside
a paged and an allocation-free decode. The entry points launch kernels only on the caller's stream and
record no memset or allocation, so they capture. Each replay runs after
eager work of its own (new inputs copied in, an eager call on other buffers,
a host synchronisation), and every replay's outputs must equal, bit for bit,
an eager call on the same inputs.
"""
from __future__ import annotations

import numpy as np
import pytest

from online_softmax_monoid_amd import inputs
from tests import harness as H

pytestmark = pytest.mark.gpu


def _bits(seed, shape, std=1.0):
    rng = np.random.Generator(np.random.PCG64(seed))
    return inputs.bf16_bits(rng.standard_normal(size=shape, dtype=np.float32) * np.float32(std))


def test_prefill_and_decode_replay_in_a_graph():
    torch = H.torch_mod()
    M = H.miattn
    # prefill: B1 Hq8 Hkv2 S700 d128 causal; decode: B6 Hq8 Hkv2 d128, 4 splits
    B, Hq, Hkv, S, d = 1, 8, 2, 700, 128
    DB, S_cap, ns = 6, 600, 4
    scale = inputs.default_scale(d)
    dev = lambda a: H.dev_bits(a)
    q, k, v = dev(_bits(1, (B, Hq, S, d))), dev(_bits(2, (B, Hkv, S, d))), dev(_bits(3, (B, Hkv, S, d)))
    o = torch.empty(B * Hq * S * d, dtype=torch.int16, device="cuda")
    lse = torch.empty(B * Hq * S, dtype=torch.float32, device="cuda")
    lens = torch.tensor([0, 1, 33, 300, 599, 600], dtype=torch.int32, device="cuda")
    dq = dev(_bits(4, (DB, Hq, d)))
    kc, vc = dev(_bits(5, (DB, Hkv, S_cap, d))), dev(_bits(6, (DB, Hkv, S_cap, d)))
    do = torch.empty(DB * Hq * d, dtype=torch.int16, device="cuda")
    dlse = torch.empty(DB * Hq, dtype=torch.float32, device="cuda")
    wsb = M.attn_fwd_decode_workspace_size(DB, Hq, d, ns)
    ws = torch.empty(wsb // 4, dtype=torch.float32, device="cuda")

    def step(stream):
        M.attn_fwd(q, k, v, o, lse, B, Hq, Hkv, S, S, d, True, scale, stream)
        M.attn_fwd_decode(dq, kc, vc, lens, do, dlse, DB, Hq, Hkv, S_cap, d, ns, scale, ws, wsb,
                          stream)

    side = torch.cuda.Stream()
    step(side)  # warm-up outside the capture (per-device launch shapes are cached)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        step(side)
    torch.cuda.synchronize()

    # eager copies of the outputs on separate buffers
    o2, lse2 = torch.empty_like(o), torch.empty_like(lse)
    do2, dlse2 = torch.empty_like(do), torch.empty_like(dlse)
    ws2 = torch.empty_like(ws)
    cur = torch.cuda.current_stream()
    for rep in range(4):
        # new inputs, copied in eagerly, then a host synchronisation
        q.copy_(dev(_bits(100 + rep, (B, Hq, S, d))))
        dq.copy_(dev(_bits(200 + rep, (DB, Hq, d))))
        o.fill_(0x7FC0)
        do.fill_(0x7FC0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        M.attn_fwd(q, k, v, o2, lse2, B, Hq, Hkv, S, S, d, True, scale, cur)
        M.attn_fwd_decode(dq, kc, vc, lens, do2, dlse2, DB, Hq, Hkv, S_cap, d, ns, scale, ws2,
                          wsb, cur)
        torch.cuda.synchronize()
        assert torch.equal(o, o2), f"replay {rep}: prefill O differs from eager"
        assert torch.equal(lse.view(torch.int32), lse2.view(torch.int32)), f"replay {rep}: LSE"
        assert torch.equal(do, do2), f"replay {rep}: decode O differs from eager"
        assert torch.equal(dlse.view(torch.int32), dlse2.view(torch.int32)), f"replay {rep}"


def test_backward_and_paged_decode_replay_in_a_graph():
    """A training-style step (forward, then the backward from its O and LSE)
    and a paged decode and an allocation-free decode, captured together and
    replayed four times on new inputs, each replay bit for bit equal to the
    same calls made eagerly."""
    torch = H.torch_mod()
    M = H.miattn
    B, Hq, Hkv, S, d = 1, 4, 2, 300, 128
    DB, S_cap, ns, P = 5, 256, 4, 16
    scale = inputs.default_scale(d)
    dev = lambda a: H.dev_bits(a)
    q, k, v = dev(_bits(11, (B, Hq, S, d))), dev(_bits(12, (B, Hkv, S, d))), dev(_bits(13, (B, Hkv, S, d)))
    dout = dev(_bits(14, (B, Hq, S, d)))
    nq, nk = B * Hq * S * d, B * Hkv * S * d
    bufs = lambda: (torch.empty(nq, dtype=torch.int16, device="cuda"),
                    torch.empty(B * Hq * S, dtype=torch.float32, device="cuda"),
                    torch.empty(nq, dtype=torch.int16, device="cuda"),
                    torch.empty(nk, dtype=torch.int16, device="cuda"),
                    torch.empty(nk, dtype=torch.int16, device="cuda"))
    wbb = M.attn_bwd_workspace_size(B, Hq, S)
    lens_h = np.array([0, 1, 17, 200, 256], dtype=np.int64)
    table, num_pages = inputs.paged_layout(21, lens_h, P, S_cap // P, spare_pages=3)
    kc, vc = _bits(15, (DB, Hkv, S_cap, d)), _bits(16, (DB, Hkv, S_cap, d))
    kp = dev(inputs.scatter_to_pages(kc, table, num_pages, P))
    vp = dev(inputs.scatter_to_pages(vc, table, num_pages, P))
    kcd, vcd = dev(kc), dev(vc)
    tab = torch.from_numpy(np.ascontiguousarray(table, dtype=np.int32)).cuda()
    lens = torch.from_numpy(lens_h.astype(np.int32)).cuda()
    dq_in = dev(_bits(17, (DB, Hq, d)))
    wdb = M.attn_fwd_decode_workspace_size(DB, Hq, d, ns)
    dec_bufs = lambda: (torch.empty(DB * Hq * d, dtype=torch.int16, device="cuda"),
                        torch.empty(DB * Hq, dtype=torch.float32, device="cuda"),
                        torch.empty(DB * Hq * d, dtype=torch.int16, device="cuda"),
                        torch.empty(DB * Hq, dtype=torch.float32, device="cuda"),
                        torch.empty(wdb // 4, dtype=torch.float32, device="cuda"))

    def step(stream, fb, wsb, db_):
        o, lse, dq, dk, dv = fb
        M.attn_fwd(q, k, v, o, lse, B, Hq, Hkv, S, S, d, True, scale, stream)
        M.attn_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, S, S, d, True, scale, wsb, wbb,
                   stream)
        po, plse, no, nlse, wsd = db_
        M.attn_fwd_decode_paged(dq_in, kp, vp, tab, lens, po, plse, DB, Hq, Hkv, num_pages, P,
                                S_cap // P, d, ns, scale, wsd, wdb, stream)
        M.attn_fwd_decode_noalloc(dq_in, kcd, vcd, lens, no, nlse, DB, Hq, Hkv, S_cap, d, ns, scale,
                                  stream)

    gb, gw, gd = bufs(), torch.empty(wbb // 4, dtype=torch.float32, device="cuda"), dec_bufs()
    eb, ew, ed = bufs(), torch.empty(wbb // 4, dtype=torch.float32, device="cuda"), dec_bufs()
    side = torch.cuda.Stream()
    step(side, gb, gw, gd)  # warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        step(side, gb, gw, gd)
    torch.cuda.synchronize()
    cur = torch.cuda.current_stream()
    for rep in range(4):
        q.copy_(dev(_bits(300 + rep, (B, Hq, S, d))))
        dout.copy_(dev(_bits(400 + rep, (B, Hq, S, d))))
        dq_in.copy_(dev(_bits(500 + rep, (DB, Hq, d))))
        for t in gb + gd[:4]:
            t.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        step(cur, eb, ew, ed)
        torch.cuda.synchronize()
        for name, a_, b_ in zip(("o", "lse", "dq", "dk", "dv"), gb, eb):
            assert torch.equal(a_.view(torch.int32) if a_.dtype == torch.float32 else a_,
                               b_.view(torch.int32) if b_.dtype == torch.float32 else b_), \
                f"replay {rep}: {name} differs from eager"
        for name, a_, b_ in zip(("paged o", "paged lse", "noalloc o", "noalloc lse"), gd[:4], ed[:4]):
            assert torch.equal(a_.view(torch.int32) if a_.dtype == torch.float32 else a_,
                               b_.view(torch.int32) if b_.dtype == torch.float32 else b_), \
                f"replay {rep}: {name} differs from eager"
