#!/usr/bin/env python3
"""Benchmark of libmiattn's hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
  * attn_fwd on the Llama-class causal prefill workload
    (B=2, Hq=Hkv=32, Sq=Sk=4096, d=128, bf16, N(0,1)*0.5), and
  * attn_fwd_decode on the batched decode workload (32 streams, Hq=32, Hkv=8,
    d=128, lengths U[1024, 8192], 16 splits; split kernel + combine kernel).

`value` is the prefill throughput in TFLOP/s (4*B*Hq*Sq*Sk*d, halved for
causal) from HIP events recorded around every prefill launch on its stream;
the decode HBM throughput and the long-context GQA workload (B=1, Hq=16,
Hkv=2, S=44032, d=256, causal) are reported beside it. Inputs are resident in
HBM before the timed region starts. The f64 oracle, timed on a bounded row
sample of the prefill workload on the host cores, is reported as a baseline.

    python bench.py [--steps K] [--warmup W] [--gpus 1]
    python bench.py --profile-pass   # every bench kernel a few times, for rocprofv3

Every rate is reported from the mean launch over three rounds, with the
median and the best round beside it. The machine probes (launch cost, DRAM
latency, the MFMA ceiling and its shader clock, the streaming-read ceiling)
come first; the decode's time floor is built from them.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOP/s (fraction of bf16 MFMA peak); decode HBM GB/s"
PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CU * 4096 flop/clk * 2.4 GHz
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
PREFILL_WID, LONG_WID, DECODE_WID = 3, 4, 5
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "prefill_b2_h32_s4096_d128_causal_traffic.txt")
KERNEL_SOURCES = ("online_softmax_monoid_amd/csrc/prefill_kernel.h",
                  "online_softmax_monoid_amd/csrc/prefill_d128.hip",
                  "online_softmax_monoid_amd/csrc/tile_order.h",
                  "online_softmax_monoid_amd/csrc/lds_copy.h",
                  "online_softmax_monoid_amd/csrc/resident.h",
                  "online_softmax_monoid_amd/csrc/launch.h")


def dev_bits(bits):
    """uint16 host bits -> int16 device tensor with the same bits."""
    import numpy as np
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per prefill launch from the committed counter summary, or None
    when it is missing or was taken on a different kernel source."""
    try:
        fields = {}
        with open(TRAFFIC_FILE) as f:
            for line in f:
                if ":" in line and not line.startswith("#"):
                    k, v = line.split(":", 1)
                    fields[k.strip()] = v.strip()
        if fields.get("kernel_source_sha256_16") != kernel_source_hash():
            return None
        return float(fields["hbm_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


class Prefill:
    def __init__(self, w, torch):
        from online_softmax_monoid_amd import inputs
        self.w = w
        q, k, v = inputs.prefill_inputs(w)
        self.q, self.k, self.v = dev_bits(q), dev_bits(k), dev_bits(v)
        n = w.B * w.Hq * w.Sq
        self.o = torch.empty(n * w.d, dtype=torch.int16, device="cuda")
        self.lse = torch.empty(n, dtype=torch.float32, device="cuda")
        self.causal = w.causal[0]
        self.flops = w.flops(self.causal)

    def __call__(self, stream):
        from online_softmax_monoid_amd import miattn
        w = self.w
        miattn.attn_fwd(self.q, self.k, self.v, self.o, self.lse, w.B, w.Hq, w.Hkv, w.Sq, w.Sk,
                        w.d, self.causal, w.scale, stream)


class Decode:
    """Two independent KV-cache copies, used alternately, so consecutive steps
    cannot serve K/V from the 256 MB last-level cache."""

    def __init__(self, w, torch):
        import numpy as np
        from online_softmax_monoid_amd import inputs, miattn
        self.w = w
        lens, q, kc, vc = inputs.decode_inputs(w)
        self.lens_host = lens
        self.q = dev_bits(q)
        self.caches = [(dev_bits(kc), dev_bits(vc))]
        self.caches.append((self.caches[0][0].clone(), self.caches[0][1].clone()))
        self.lens = torch.from_numpy(lens.astype(np.int32)).to("cuda")
        self.o = torch.empty(w.B * w.Hq * w.d, dtype=torch.int16, device="cuda")
        self.lse = torch.empty(w.B * w.Hq, dtype=torch.float32, device="cuda")
        self.ws_bytes = miattn.attn_fwd_decode_workspace_size(w.B, w.Hq, w.d, w.num_splits)
        self.ws = torch.empty(self.ws_bytes // 4, dtype=torch.float32, device="cuda")
        self.i = 0
        # algorithmic HBM bytes: every valid K and V row once, Q in, O and LSE out
        self.bytes = (2 * int(lens.sum()) * w.Hkv * w.d * 2 + 2 * w.B * w.Hq * w.d * 2
                      + 4 * w.B * w.Hq)

    def __call__(self, stream):
        from online_softmax_monoid_amd import miattn
        w = self.w
        kc, vc = self.caches[self.i & 1]
        self.i += 1
        miattn.attn_fwd_decode(self.q, kc, vc, self.lens, self.o, self.lse, w.B, w.Hq, w.Hkv,
                               w.S_cap, w.d, w.num_splits, w.scale, self.ws, self.ws_bytes,
                               stream)


class PrefillWindow:
    """Causal prefill with a sliding window of W keys before each row's own
    (attn_fwd_window), on seeded N(0, 1) draws."""

    def __init__(self, torch, seed, B, Hq, Hkv, S, d, W):
        from online_softmax_monoid_amd import inputs
        self.shape = (B, Hq, Hkv, S, d, W)
        q, k, v = inputs.draw_prefill_bits(seed, B, Hq, Hkv, S, S, d)
        self.q, self.k, self.v = dev_bits(q), dev_bits(k), dev_bits(v)
        n = B * Hq * S
        self.o = torch.empty(n * d, dtype=torch.int16, device="cuda")
        self.lse = torch.empty(n, dtype=torch.float32, device="cuda")
        # visible (query, key) pairs per head: row i sees min(i, W) + 1 keys
        pairs = W * (W + 1) // 2 + (S - W) * (W + 1) if S > W else S * (S + 1) // 2
        self.flops = 4.0 * d * pairs * B * Hq
        # Q, K, V read once, O and LSE written once
        self.bytes = 2 * d * 2 * (B * Hq * S + B * Hkv * S) + 4 * B * Hq * S
        self.scale = inputs.default_scale(d)

    def __call__(self, stream):
        from online_softmax_monoid_amd import miattn
        B, Hq, Hkv, S, d, W = self.shape
        miattn.attn_fwd_window(self.q, self.k, self.v, self.o, self.lse, B, Hq, Hkv, S, S, d,
                               True, W, self.scale, stream)


# Sliding-window workloads: the window row of the pages' variant table (window
# 128, forward, n = 8k, d = 64; batch and heads not stated there, 4 x 16 here)
# and a long window at d = 128 with GQA.
WINDOW_LEGS = (("window_d64_w128", dict(seed=7100, B=4, Hq=16, Hkv=16, S=8192, d=64, W=128)),
               ("window_d128_w4096", dict(seed=7200, B=1, Hq=32, Hkv=8, S=16384, d=128,
                                          W=4096)))


class PrefillScoreMod:
    """Non-causal prefill with a score modifier (attn_fwd_ext): a soft cap, or
    ALiBi with the geometric slopes 2^(-8 (h + 1) / Hq)."""

    def __init__(self, torch, seed, B, H, S, d, softcap=0.0, alibi=False):
        import numpy as np
        from online_softmax_monoid_amd import inputs
        self.shape = (B, H, S, d)
        q, k, v = inputs.draw_prefill_bits(seed, B, H, H, S, S, d)
        self.q, self.k, self.v = dev_bits(q), dev_bits(k), dev_bits(v)
        n = B * H * S
        self.o = torch.empty(n * d, dtype=torch.int16, device="cuda")
        self.lse = torch.empty(n, dtype=torch.float32, device="cuda")
        self.softcap = softcap
        self.alibi = None
        if alibi:
            sl = (2.0 ** (-8.0 * (np.arange(H) + 1) / H)).astype(np.float32)
            self.alibi = torch.from_numpy(sl).to("cuda")
        self.flops = 4.0 * d * S * S * B * H
        self.scale = inputs.default_scale(d)

    def __call__(self, stream):
        from online_softmax_monoid_amd import miattn
        B, H, S, d = self.shape
        miattn.attn_fwd_ext(self.q, self.k, self.v, self.o, self.lse, B, H, H, S, S, d, False,
                            -1, self.softcap, self.alibi, self.scale, stream)


# The score-variant rows of the pages' table (forward, n = 2k, d = 64; batch
# and heads not stated there, 4 x 16 here); cap 30
SCOREMOD_LEGS = (("softcap_d64_n2k", dict(seed=6200, B=4, H=16, S=2048, d=64, softcap=30.0)),
                 ("alibi_d64_n2k", dict(seed=6300, B=4, H=16, S=2048, d=64, alibi=True)))


class PrefillVarlen:
    """Chunked prefill of a packed batch (attn_fwd_varlen): 16 sequences of
    U[512, 4096] new queries, each against a cached prefix of U[0, 2048] keys
    plus itself, causal (bottom-right), Hq 32, Hkv 8, d 128."""

    def __init__(self, torch, seed=7300, n_seq=16, Hq=32, Hkv=8, d=128):
        import numpy as np
        from online_softmax_monoid_amd import inputs
        rng = np.random.Generator(np.random.PCG64(seed))
        lq = rng.integers(512, 4096, size=n_seq, endpoint=True)
        lk = lq + rng.integers(0, 2048, size=n_seq, endpoint=True)
        self.cu_q = torch.tensor(np.concatenate([[0], np.cumsum(lq)]), dtype=torch.int32,
                                 device="cuda")
        self.cu_k = torch.tensor(np.concatenate([[0], np.cumsum(lk)]), dtype=torch.int32,
                                 device="cuda")
        self.dims = (n_seq, int(lq.sum()), int(lk.sum()), int(lq.max()), int(lk.max()), Hq, Hkv, d)
        q, k, v = inputs.draw_prefill_bits(seed + 1, 1, Hq, Hkv, int(lq.sum()), int(lk.sum()), d)
        self.q, self.k, self.v = dev_bits(q), dev_bits(k), dev_bits(v)
        self.o = torch.empty(Hq * int(lq.sum()) * d, dtype=torch.int16, device="cuda")
        self.lse = torch.empty(Hq * int(lq.sum()), dtype=torch.float32, device="cuda")
        # causal pairs: row i of a sequence sees i + (Sk - Sq) + 1 keys
        pairs = sum(int(a) * (int(b) - int(a)) + int(a) * (int(a) + 1) // 2 for a, b in zip(lq, lk))
        self.flops = 4.0 * d * Hq * pairs
        self.scale = inputs.default_scale(d)
        self.shape = {"sequences": n_seq, "total_q": int(lq.sum()), "total_k": int(lk.sum()),
                      "Hq": Hq, "Hkv": Hkv, "d": d, "causal": True}

    def __call__(self, stream):
        from online_softmax_monoid_amd import miattn
        n, tq, tk, mq, mk, Hq, Hkv, d = self.dims
        miattn.attn_fwd_varlen(self.q, self.k, self.v, self.o, self.lse, self.cu_q, self.cu_k, n,
                               tq, tk, mq, mk, Hq, Hkv, d, True, self.scale, stream)


class Backward:
    """attn_bwd on the prefill workload (B2 H32 S4096 d128 causal), fed by the
    GPU forward's O and LSE and a seeded N(0, 1) upstream gradient.
    Algorithmic flops: five products of the forward's size (S, dP, dV, dK,
    dQ), 2.5 times the forward's."""

    def __init__(self, pre, torch):
        from online_softmax_monoid_amd import inputs
        w = pre.w
        self.pre = pre
        pre(torch.cuda.current_stream())
        (do,) = inputs.draw_prefill_bits(w.seed + 11, w.B, w.Hq, w.Hkv, w.Sq, w.Sk, w.d)[:1]
        self.do = dev_bits(do)
        nq, nk = w.B * w.Hq * w.Sq * w.d, w.B * w.Hkv * w.Sk * w.d
        self.dq = torch.empty(nq, dtype=torch.int16, device="cuda")
        self.dk = torch.empty(nk, dtype=torch.int16, device="cuda")
        self.dv = torch.empty(nk, dtype=torch.int16, device="cuda")
        from online_softmax_monoid_amd import miattn
        self.ws_bytes = miattn.attn_bwd_workspace_size(w.B, w.Hq, w.Sq)
        self.ws = torch.empty(self.ws_bytes // 4, dtype=torch.float32, device="cuda")
        self.flops = 2.5 * pre.flops

    def __call__(self, stream):
        from online_softmax_monoid_amd import miattn
        p, w = self.pre, self.pre.w
        miattn.attn_bwd(p.q, p.k, p.v, p.o, p.lse, self.do, self.dq, self.dk, self.dv, w.B, w.Hq,
                        w.Hkv, w.Sq, w.Sk, w.d, p.causal, w.scale, self.ws, self.ws_bytes, stream)


class BackwardShape:
    """attn_bwd on seeded N(0, 1) * 0.5 inputs of a given shape, fed by the GPU
    forward's O and LSE; the d = 256 leg takes the pages' backward regime
    (head dimension 256, B * H * N = 131072: B2 H16 N4096, causal)."""

    def __init__(self, torch, seed, B, H, S, d, causal):
        from online_softmax_monoid_amd import inputs, miattn
        q, k, v = inputs.draw_prefill_bits(seed, B, H, H, S, S, d, 0.5)
        (do,) = inputs.draw_prefill_bits(seed + 1, B, H, H, S, S, d)[:1]
        self.q, self.k, self.v, self.do = dev_bits(q), dev_bits(k), dev_bits(v), dev_bits(do)
        n = B * H * S
        self.o = torch.empty(n * d, dtype=torch.int16, device="cuda")
        self.lse = torch.empty(n, dtype=torch.float32, device="cuda")
        self.dq = torch.empty(n * d, dtype=torch.int16, device="cuda")
        self.dk = torch.empty(n * d, dtype=torch.int16, device="cuda")
        self.dv = torch.empty(n * d, dtype=torch.int16, device="cuda")
        self.ws_bytes = miattn.attn_bwd_workspace_size(B, H, S)
        self.ws = torch.empty(self.ws_bytes // 4, dtype=torch.float32, device="cuda")
        self.shape = (B, H, S, d, causal)
        self.scale = inputs.default_scale(d)
        miattn.attn_fwd(self.q, self.k, self.v, self.o, self.lse, B, H, H, S, S, d, causal,
                        self.scale, torch.cuda.current_stream())
        fwd = 4.0 * B * H * S * S * d / (2 if causal else 1)
        self.flops = 2.5 * fwd

    def __call__(self, stream):
        from online_softmax_monoid_amd import miattn
        B, H, S, d, causal = self.shape
        miattn.attn_bwd(self.q, self.k, self.v, self.o, self.lse, self.do, self.dq, self.dk,
                        self.dv, B, H, H, S, S, d, causal, self.scale, self.ws, self.ws_bytes,
                        stream)


class DecodePaged:
    """The decode workload with its cache in pages of ``page`` keys, pool
    pages in a seeded random order; two pool copies used alternately, as for
    Decode. The page size is fixed at construction: the pools are sized for
    it."""

    PAGE = 16  # page size the bench reports

    def __init__(self, w, torch, page=PAGE):
        import numpy as np
        from online_softmax_monoid_amd import inputs, miattn
        self.w = w
        lens, q, kc, vc = inputs.decode_inputs(w)
        P = self.page = int(page)
        table, self.num_pages = inputs.paged_layout(w.seed + 7, lens, P, w.S_cap // P,
                                                    spare_pages=64)
        kp = dev_bits(inputs.scatter_to_pages(kc, table, self.num_pages, P))
        vp = dev_bits(inputs.scatter_to_pages(vc, table, self.num_pages, P))
        del kc, vc
        self.pools = [(kp, vp), (kp.clone(), vp.clone())]
        self.max_pages = table.shape[1]
        assert kp.numel() == self.num_pages * w.Hkv * P * w.d
        self.table = torch.from_numpy(table).to("cuda")
        self.q = dev_bits(q)
        self.lens = torch.from_numpy(lens.astype(np.int32)).to("cuda")
        self.o = torch.empty(w.B * w.Hq * w.d, dtype=torch.int16, device="cuda")
        self.lse = torch.empty(w.B * w.Hq, dtype=torch.float32, device="cuda")
        self.ws_bytes = miattn.attn_fwd_decode_workspace_size(w.B, w.Hq, w.d, w.num_splits)
        self.ws = torch.empty(self.ws_bytes // 4, dtype=torch.float32, device="cuda")
        self.i = 0
        self.bytes = (2 * int(lens.sum()) * w.Hkv * w.d * 2 + 2 * w.B * w.Hq * w.d * 2
                      + 4 * w.B * w.Hq)

    def __call__(self, stream):
        from online_softmax_monoid_amd import miattn
        w = self.w
        kp, vp = self.pools[self.i & 1]
        self.i += 1
        miattn.attn_fwd_decode_paged(self.q, kp, vp, self.table, self.lens, self.o, self.lse,
                                     w.B, w.Hq, w.Hkv, self.num_pages, self.page, self.max_pages,
                                     w.d, w.num_splits, w.scale, self.ws, self.ws_bytes, stream)


def time_launches(fn, stream, torch, n):
    """Per-launch durations (ms) from HIP events recorded on the launch stream."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n)]
    with torch.cuda.stream(stream):
        for a, b in evs:
            a.record(stream)
            fn(stream)
            b.record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


ROUNDS = 3


def rounds_stats(rounds_ms):
    """Timing summary of ROUNDS rounds of launches (ms per launch): the mean
    over every launch, the median and the minimum of the round means, and the
    fastest single launch."""
    import statistics
    means = [sum(r) / len(r) for r in rounds_ms]
    allms = [x for r in rounds_ms for x in r]
    return {"mean": sum(allms) / len(allms), "median": statistics.median(means),
            "min": min(means), "min_launch": min(allms), "rounds": [round(m, 5) for m in means],
            "launches": len(allms)}


def measure(fn, stream, torch, per_round, warmup=10):
    """Launches of one leg after `warmup` untimed ones (the clock settles over
    the first few after a change of kernel), in ROUNDS rounds."""
    time_launches(fn, stream, torch, warmup)
    return rounds_stats([time_launches(fn, stream, torch, per_round) for _ in range(ROUNDS)])


def rate_entry(st, work, unit, peak, extra=None):
    """Rates of one leg from its timing summary: `value` from the mean launch,
    the median and best rounds beside it."""
    div = 1e12 if unit == "TFLOP/s" else 1e9
    v = work / (st["mean"] * 1e-3) / div
    e = {"value": round(v, 2), "unit": unit, "ms": round(st["mean"], 5),
         "ms_median_round": round(st["median"], 5), "ms_min_round": round(st["min"], 5),
         "ms_min_launch": round(st["min_launch"], 5), "rounds_ms": st["rounds"],
         "value_median_round": round(work / (st["median"] * 1e-3) / div, 2),
         "value_best_round": round(work / (st["min"] * 1e-3) / div, 2),
         "frac": round(v / peak, 4)}
    if extra:
        e.update(extra)
    return e


class Probes:
    """Machine probes (libmiprobe.so): launch cost, DRAM latency, the MFMA
    ceiling with its shader clock, and the streaming-read ceiling."""

    def __init__(self, torch):
        import ctypes
        from online_softmax_monoid_amd import build, miattn
        miattn.bind_to_torch_runtime()
        if not os.path.exists(build.PROBE_LIB):
            build._build_lib(build.PROBE_LIB, build.PROBE_SOURCES)
        L = ctypes.CDLL(build.PROBE_LIB)
        vp, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        L.probe_empty.argtypes = [i, vp]
        L.probe_chase.argtypes = [vp, sz, ctypes.c_uint32, i, vp, vp]
        L.probe_mfma.argtypes = [i, i, vp, vp, vp]
        L.probe_read.argtypes = [vp, sz, i, vp, vp]
        for f in (L.probe_empty, L.probe_chase, L.probe_mfma, L.probe_read):
            f.restype = i
        self.L, self.torch = L, torch

    def _ok(self, rc, what):
        if rc != 0:
            raise RuntimeError(f"{what}: probe status {rc}")

    def launch(self, stream):
        """One empty launch (events around it, median of 200), and 2000
        launches back to back (per launch)."""
        import statistics
        torch = self.torch
        s = stream.cuda_stream
        one = time_launches(lambda st: self._ok(self.L.probe_empty(1, s), "empty"), stream,
                            torch, 200)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        self._ok(self.L.probe_empty(2000, s), "empty")
        b.record(stream)
        torch.cuda.synchronize()
        return {"single_launch_us": round(statistics.median(one) * 1e3, 2),
                "back_to_back_us": round(a.elapsed_time(b) * 1e3 / 2000, 3)}

    def chase(self, stream, hops=20000):
        """DRAM latency: a random cycle through 2^20 nodes 4 KiB apart in a
        4 GiB buffer, built on the device; the last-level cache is flushed
        by a 2 GiB read first, and each hop then reaches a line not read
        before."""
        torch = self.torch
        n_elems = 1 << 30
        stride = 1024
        nodes = n_elems // stride
        buf = torch.empty(n_elems, dtype=torch.int32, device="cuda")
        g = torch.Generator().manual_seed(20261250)
        perm = torch.randperm(nodes, generator=g).to("cuda")
        idx = perm.to(torch.int64) * stride
        nxt = (torch.roll(perm, -1).to(torch.int64) * stride).to(torch.int32)
        buf[idx] = nxt
        assert int(nxt.max()) < n_elems and int(idx.max()) < n_elems
        out = torch.zeros(4, dtype=torch.int32, device="cuda")
        flush = torch.empty(1 << 29, dtype=torch.float32, device="cuda")
        sink = torch.empty(2048 * 4, dtype=torch.int32, device="cuda")
        s = stream.cuda_stream
        start = int(idx[0])
        res = []
        for _ in range(3):
            self._ok(self.L.probe_read(flush.data_ptr(), flush.numel() * 4, 2048, sink.data_ptr(),
                                       s), "read")
            ms = time_launches(lambda st: self._ok(
                self.L.probe_chase(buf.data_ptr(), n_elems, start, hops, out.data_ptr(), s),
                "chase"), stream, torch, 1)[0]
            res.append(ms * 1e6 / hops)
        del buf, flush
        torch.cuda.empty_cache()
        return {"dram_latency_ns": round(min(res), 1), "hops": hops,
                "runs_ns": [round(x, 1) for x in res]}

    def mfma(self, stream, blocks=512, iters=6000):
        """MFMA ceiling: 512 workgroups of four waves (two waves per SIMD on
        256 CUs), each wave iters * 32 independent 32x32x16 bf16 MFMAs; the
        shader clock from the cycle counter against the 100 MHz reference."""
        import statistics
        torch = self.torch
        sink = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
        clk = torch.zeros(blocks * 4, dtype=torch.int64, device="cuda")
        s = stream.cuda_stream
        fn = lambda st: self._ok(self.L.probe_mfma(blocks, iters, sink.data_ptr(), clk.data_ptr(),
                                                   s), "mfma")
        st = measure(fn, stream, torch, 3, warmup=1)
        c = clk.cpu().numpy().reshape(blocks, 4).astype("float64")
        ghz = (c[:, 1] - c[:, 0]) / ((c[:, 3] - c[:, 2]) / 1e8) / 1e9
        flops = blocks * 4 * iters * 32 * 32768.0
        return {"tflops": round(flops / (st["mean"] * 1e-3) / 1e12, 1),
                "tflops_best": round(flops / (st["min_launch"] * 1e-3) / 1e12, 1),
                "shader_clock_ghz": round(float(statistics.median(ghz)), 3),
                "frac_of_spec": round(flops / (st["mean"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}

    def read(self, stream, nbytes=2 << 30, blocks=2048):
        """Streaming-read ceiling over a 2 GiB buffer, and torch's device copy
        of 1 GiB (read + write) beside it."""
        torch = self.torch
        buf = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
        sink = torch.empty(blocks * 4, dtype=torch.int32, device="cuda")
        s = stream.cuda_stream
        st = measure(lambda x: self._ok(self.L.probe_read(buf.data_ptr(), nbytes, blocks,
                                                          sink.data_ptr(), s), "read"),
                     stream, torch, 5)
        half = nbytes // 2
        src = buf[:half // 4]
        dst = torch.empty_like(src)
        cst = measure(lambda x: dst.copy_(src), stream, torch, 5)
        del buf, dst
        torch.cuda.empty_cache()
        return {"read_GBs": round(nbytes / (st["mean"] * 1e-3) / 1e9, 1),
                "read_GBs_best": round(nbytes / (st["min_launch"] * 1e-3) / 1e9, 1),
                "copy_GBs": round(2 * half / (cst["mean"] * 1e-3) / 1e9, 1),
                "read_frac_of_spec": round(nbytes / (st["mean"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}


def cpu_baseline(target_seconds: float = 12.0):
    """The f64 oracle on a bounded random row sample of the prefill workload,
    on every host thread; then the tiny workload (B1 H2 S128 d64) on one
    thread."""
    import numpy as np
    import oracle
    from online_softmax_monoid_amd import inputs
    w = inputs.WORKLOADS[PREFILL_WID]
    q, k, v = inputs.prefill_inputs(w)
    causal = w.causal[0]
    total_rows = w.B * w.Hq * w.Sq
    rng = np.random.Generator(np.random.PCG64(w.seed + 7))
    threads = oracle.max_threads()

    def row_flops(rows):
        i = rows % w.Sq
        keys = np.minimum(w.Sk, i + (w.Sk - w.Sq) + 1) if causal else np.full(rows.shape, w.Sk)
        return float(np.sum(4.0 * w.d * keys))

    probe = np.sort(rng.choice(total_rows, size=2048, replace=False)).astype(np.int64)
    t0 = time.perf_counter()
    oracle.attn_fwd(q, k, v, causal, w.scale, rows=probe, nthreads=threads)
    dt = time.perf_counter() - t0
    rate = row_flops(probe) / dt
    n = int(min(total_rows, max(2048, target_seconds * rate / (row_flops(probe) / 2048))))
    rows = np.sort(rng.choice(total_rows, size=n, replace=False)).astype(np.int64)
    t0 = time.perf_counter()
    oracle.attn_fwd(q, k, v, causal, w.scale, rows=rows, nthreads=threads)
    dt = time.perf_counter() - t0
    fl = row_flops(rows)
    # the tiny workload, every row, on one thread
    w1 = inputs.WORKLOADS[1]
    q1, k1, v1 = inputs.prefill_inputs(w1)
    t0 = time.perf_counter()
    for _ in range(5):
        oracle.attn_fwd(q1, k1, v1, False, w1.scale, nthreads=1)
    dt1 = (time.perf_counter() - t0) / 5
    oracle.attn_fwd(q1, k1, v1, False, w1.scale, nthreads=threads)  # restore the thread count
    return {"value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} of {total_rows} query rows (uniform random, seed {w.seed + 7}) of "
                      f"the B2 H32 S4096 d128 causal prefill, f64 two-pass, {dt:.1f} s, "
                      f"{fl / 1e9:.1f} GFLOP",
            "one_thread_tiny": {"workload": "B1 H2 S128 d64 non-causal, all 256 rows",
                                "seconds": round(dt1, 5), "cores": 1,
                                "TFLOP/s": w1.flops(False) / dt1 / 1e12}}


class PrefillCfg:
    """A prefill workload at one causal setting (attn_fwd)."""

    def __init__(self, w, torch, causal):
        from online_softmax_monoid_amd import inputs
        self.w = w
        q, k, v = inputs.prefill_inputs(w)
        self.q, self.k, self.v = dev_bits(q), dev_bits(k), dev_bits(v)
        n = w.B * w.Hq * w.Sq
        self.o = torch.empty(n * w.d, dtype=torch.int16, device="cuda")
        self.lse = torch.empty(n, dtype=torch.float32, device="cuda")
        self.causal = causal
        self.flops = w.flops(causal)

    def __call__(self, stream):
        from online_softmax_monoid_amd import miattn
        w = self.w
        miattn.attn_fwd(self.q, self.k, self.v, self.o, self.lse, w.B, w.Hq, w.Hkv, w.Sq, w.Sk,
                        w.d, self.causal, w.scale, stream)


def profile_pass():
    """A short fixed sequence for rocprofv3 counter passes: a plain 1 GiB
    device copy (the counter calibration), then every kernel the bench times:
    3 launches each of the step's prefill and decode, the d = 64 workloads,
    the window, score-modifier, packed, paged-decode and backward legs, and
    one launch of the long-context d = 256 prefill."""
    import torch
    from online_softmax_monoid_amd import inputs
    stream = torch.cuda.current_stream()
    src = torch.empty(1 << 28, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    legs = [Prefill(inputs.WORKLOADS[PREFILL_WID], torch), Decode(inputs.WORKLOADS[DECODE_WID], torch),
            PrefillCfg(inputs.WORKLOADS[1], torch, False),
            PrefillCfg(inputs.WORKLOADS[2], torch, True), PrefillCfg(inputs.WORKLOADS[2], torch, False)]
    legs += [PrefillWindow(torch, **cfg) for _, cfg in WINDOW_LEGS]
    legs += [PrefillScoreMod(torch, **cfg) for _, cfg in SCOREMOD_LEGS]
    legs += [PrefillVarlen(torch), DecodePaged(inputs.WORKLOADS[DECODE_WID], torch)]
    legs.append(Backward(legs[0], torch))
    legs.append(BackwardShape(torch, 7400, 2, 16, 4096, 256, True))
    torch.cuda.synchronize()
    for leg in legs:
        for _ in range(3):
            leg(stream)
        torch.cuda.synchronize()
        log(f"profile pass: {type(leg).__name__} done")
    del legs
    torch.cuda.empty_cache()
    lng = Prefill(inputs.WORKLOADS[LONG_WID], torch)
    lng(stream)
    torch.cuda.synchronize()
    log("profile pass done")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=60,
                    help="timed steps, in three rounds (default 60: 3 x 20)")
    ap.add_argument("--warmup", type=int, default=50,
                    help="untimed steps first (the clock settles over the first tens of steps)")
    ap.add_argument("--long-steps", type=int, default=2, help="long-context launches per round")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-probes", action="store_true")
    ap.add_argument("--profile-pass", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus})", file=sys.stderr)
        sys.exit(2)
    if args.profile_pass:
        profile_pass()
        return

    import torch
    from online_softmax_monoid_amd import inputs, miattn
    miattn.load()
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()

    machine = None
    if not args.no_probes:
        log("bench: machine probes")
        pr = Probes(torch)
        machine = {"launch": pr.launch(stream), "mfma_ceiling": pr.mfma(stream),
                   "hbm": pr.read(stream), "latency": pr.chase(stream)}
        log(f"bench: machine {json.dumps(machine)}")
        del pr

    log("bench: drawing inputs")
    pre = Prefill(inputs.WORKLOADS[PREFILL_WID], torch)
    dec = Decode(inputs.WORKLOADS[DECODE_WID], torch)
    torch.cuda.synchronize()

    log(f"bench: warmup {args.warmup}")
    for _ in range(args.warmup):
        pre(stream)
        dec(stream)
    torch.cuda.synchronize()

    # the timed region: args.steps steps (prefill + decode) in three rounds,
    # each round bracketed by a device synchronisation
    per = [args.steps // ROUNDS + (1 if r < args.steps % ROUNDS else 0) for r in range(ROUNDS)]
    log(f"bench: timing {args.steps} steps in rounds of {per}")
    pre_rounds, dec_rounds, walls = [], [], []
    for n in per:
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for e in ev:
            e[0].record(stream)
            pre(stream)
            e[1].record(stream)
            dec(stream)
            e[2].record(stream)
        torch.cuda.synchronize()
        walls.append(time.perf_counter() - t0)
        pre_rounds.append([a.elapsed_time(b) for a, b, _ in ev])
        dec_rounds.append([b.elapsed_time(c) for _, b, c in ev])
    pst, dst_ = rounds_stats(pre_rounds), rounds_stats(dec_rounds)
    tflops = pre.flops / (pst["mean"] * 1e-3) / 1e12
    dec_gbs = dec.bytes / (dst_["mean"] * 1e-3) / 1e9
    log(f"bench: prefill {pst['mean']:.4f} ms ({tflops:.1f} TFLOP/s; rounds {pst['rounds']}), "
        f"decode {dst_['mean']:.4f} ms ({dec_gbs:.0f} GB/s; rounds {dst_['rounds']})")

    legs = {}
    bwd = Backward(pre, torch)
    legs["backward_d128"] = rate_entry(measure(bwd, stream, torch, 5), bwd.flops, "TFLOP/s",
                                       PEAK_BF16_TFLOPS,
                                       {"flops": "2.5 x the forward's (S, dP, dV, dK, dQ)"})
    log(f"bench: backward_d128 {legs['backward_d128']['ms']} ms")
    del bwd, pre
    torch.cuda.empty_cache()
    b256 = BackwardShape(torch, 7400, 2, 16, 4096, 256, True)
    legs["backward_d256"] = rate_entry(measure(b256, stream, torch, 5), b256.flops, "TFLOP/s",
                                       PEAK_BF16_TFLOPS,
                                       {"flops": "2.5 x the forward's (S, dP, dV, dK, dQ)",
                                        "shape": {"B": 2, "H": 16, "S": 4096, "d": 256,
                                                  "causal": True}})
    log(f"bench: backward_d256 {legs['backward_d256']['ms']} ms")
    del b256
    torch.cuda.empty_cache()

    for wid, causal, per_round in ((1, False, 50), (2, True, 20), (2, False, 20)):
        leg = PrefillCfg(inputs.WORKLOADS[wid], torch, causal)
        name = f"workload{wid}_d64_{'causal' if causal else 'noncausal'}"
        w = inputs.WORKLOADS[wid]
        legs[name] = rate_entry(measure(leg, stream, torch, per_round), leg.flops, "TFLOP/s",
                                PEAK_BF16_TFLOPS, {"shape": {"B": w.B, "Hq": w.Hq, "S": w.Sq,
                                                             "d": w.d, "causal": causal}})
        log(f"bench: {name} {legs[name]['ms']} ms ({legs[name]['value']} TFLOP/s)")
        del leg
    torch.cuda.empty_cache()

    log("bench: long-context GQA workload")
    lng = Prefill(inputs.WORKLOADS[LONG_WID], torch)
    legs["long_context_gqa_d256"] = rate_entry(measure(lng, stream, torch, args.long_steps, 1),
                                               lng.flops, "TFLOP/s", PEAK_BF16_TFLOPS)
    log(f"bench: long-context {legs['long_context_gqa_d256']['ms']} ms")
    del lng
    torch.cuda.empty_cache()

    for name, cfg in WINDOW_LEGS:
        wl = PrefillWindow(torch, **cfg)
        st = measure(wl, stream, torch, 10)
        legs[name] = rate_entry(st, wl.flops, "TFLOP/s", PEAK_BF16_TFLOPS,
                                {"GB/s": round(wl.bytes / (st["mean"] * 1e-3) / 1e9, 1),
                                 "hbm_frac": round(wl.bytes / (st["mean"] * 1e-3) / 1e9
                                                   / PEAK_HBM_GBS, 4),
                                 "shape": {k: v for k, v in cfg.items() if k != "seed"}})
        log(f"bench: {name} {legs[name]['ms']} ms")
        del wl
        torch.cuda.empty_cache()

    for name, cfg in SCOREMOD_LEGS:
        sm = PrefillScoreMod(torch, **cfg)
        legs[name] = rate_entry(measure(sm, stream, torch, 10), sm.flops, "TFLOP/s",
                                PEAK_BF16_TFLOPS,
                                {"shape": {k: v for k, v in cfg.items() if k != "seed"}})
        log(f"bench: {name} {legs[name]['ms']} ms")
        del sm
        torch.cuda.empty_cache()

    vl = PrefillVarlen(torch)
    legs["varlen_chunked_d128"] = rate_entry(measure(vl, stream, torch, 10), vl.flops, "TFLOP/s",
                                             PEAK_BF16_TFLOPS, {"shape": vl.shape})
    log(f"bench: varlen_chunked_d128 {legs['varlen_chunked_d128']['ms']} ms")
    del vl
    torch.cuda.empty_cache()

    log("bench: paged decode (16-key pages)")
    dp = DecodePaged(inputs.WORKLOADS[DECODE_WID], torch)
    legs["decode_paged"] = rate_entry(measure(dp, stream, torch, 20, args.warmup), dp.bytes,
                                      "GB/s", PEAK_HBM_GBS,
                                      {"bound": "hbm", "page_size": DecodePaged.PAGE})
    log(f"bench: paged decode {legs['decode_paged']['ms']} ms")
    del dp
    torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline:
        log("bench: cpu baseline (f64 oracle on a row sample)")
        cpu = cpu_baseline()

    # the decode's time floor (the tang paper, §9.2 "From traffic to time"):
    # two dependent launches, one DRAM round trip, and the bytes at the
    # bandwidth (the spec and the measured read ceiling)
    floor = None
    if machine is not None:
        lat_ms = machine["latency"]["dram_latency_ns"] * 1e-6
        launch_ms = machine["launch"]["back_to_back_us"] * 1e-3
        floor = {"launches": 2, "launch_ms": round(launch_ms, 5), "latency_ms": round(lat_ms, 5),
                 "bytes_ms_spec": round(dec.bytes / (PEAK_HBM_GBS * 1e6), 5),
                 "bytes_ms_measured_read": round(dec.bytes / (machine["hbm"]["read_GBs"] * 1e6), 5)}
        floor["floor_ms_spec"] = round(2 * launch_ms + lat_ms + floor["bytes_ms_spec"], 5)
        floor["floor_ms_measured"] = round(2 * launch_ms + lat_ms + floor["bytes_ms_measured_read"], 5)
        floor["decode_ms_over_floor_measured"] = round(dst_["mean"] / floor["floor_ms_measured"], 3)

    traffic = measured_traffic()
    pw, dw = inputs.WORKLOADS[PREFILL_WID], inputs.WORKLOADS[DECODE_WID]
    wall = sum(walls)
    out = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "Llama-class causal prefill B=2 Hq=Hkv=32 Sq=Sk=4096 d=128 bf16 "
                        "+ batched split-KV decode B=32 Hq=32 Hkv=8 d=128 len U[1024,8192] "
                        "16 splits",
            "prefill": {"B": pw.B, "Hq": pw.Hq, "Hkv": pw.Hkv, "Sq": pw.Sq, "Sk": pw.Sk,
                        "d": pw.d, "causal": True, "flops": pw.flops(True)},
            "decode": {"B": dw.B, "Hq": dw.Hq, "Hkv": dw.Hkv, "d": dw.d,
                       "kv_len_sum": int(dec.lens_host.sum()), "splits": dw.num_splits},
            "parallelism": "single GPU",
            "rounds": per,
            "seeds": {"prefill": inputs.WORKLOADS[PREFILL_WID].seed,
                      "decode": inputs.WORKLOADS[DECODE_WID].seed,
                      "long_context": inputs.WORKLOADS[LONG_WID].seed},
        },
        "roofline": {
            "bound": "mfma",
            "achieved": round(tflops, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
        },
        "prefill": rate_entry(pst, pre_flops(pw), "TFLOP/s", PEAK_BF16_TFLOPS),
        "decode": rate_entry(dst_, dec.bytes, "GB/s", PEAK_HBM_GBS,
                             {"bound": "hbm", "algorithmic_bytes": dec.bytes,
                              "floor": floor}),
        **legs,
        "machine": machine,
        "cpu_baseline": cpu,
    }
    # the same rates against the ceilings measured on this machine (the MFMA and
    # streaming-read probes), beside the spec peaks
    if machine is not None:
        mf, rd = machine["mfma_ceiling"]["tflops"], machine["hbm"]["read_GBs"]
        for key in ("prefill", "long_context_gqa_d256", "backward_d128", "backward_d256",
                    "window_d128_w4096", "varlen_chunked_d128"):
            if isinstance(out.get(key), dict) and mf > 0:
                out[key]["frac_of_measured_mfma"] = round(out[key]["value"] / mf, 4)
        for key in ("decode", "decode_paged"):
            if isinstance(out.get(key), dict) and rd > 0:
                out[key]["frac_of_measured_read"] = round(out[key]["value"] / rd, 4)
    print(json.dumps(out), flush=True)


def pre_flops(w):
    return w.flops(w.causal[0])


if __name__ == "__main__":
    main()
