"""GPU: the library's launches captured in a HIP graph (torch.cuda.CUDAGraph)
and replayed.

A serving loop captures one prefill and one decode step and replays them on
new inputs. The entry points launch kernels only on the caller's stream and
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
