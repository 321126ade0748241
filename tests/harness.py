"""Shared helpers for the GPU parity tests: upload bits, run through the C
ABI, compare with the oracle at the tolerances the operation is held to.

Tolerances for bf16 inputs with f32 accumulation:
  O   : max |O_gpu - O_ref| <= 1e-2 and ||O_gpu - O_ref||_2 / ||O_ref||_2 <= 4e-3
  LSE : max |LSE_gpu - LSE_ref| <= 1e-3 over rows with at least one key
  rows with no visible key: O == +0.0 bitwise and LSE == -inf, exactly.
"""
from __future__ import annotations

import numpy as np

from online_softmax_monoid_amd import inputs, miattn

O_MAX_ABS = 1e-2
O_REL_RMS = 4e-3
LSE_MAX_ABS = 1e-3
GUARD = 4096  # elements of guard region after each output buffer
NAN_BF16 = 0x7FC0


def torch_mod():
    import torch
    return torch


def dev_bits(bits: np.ndarray):
    """uint16 host bits -> int16 device tensor holding the same bits."""
    torch = torch_mod()
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda")


def nan_out(n_bf16: int, n_f32: int):
    """NaN-prefilled output buffers with a guard region after the logical part."""
    torch = torch_mod()
    o = torch.full((n_bf16 + GUARD,), NAN_BF16, dtype=torch.int32).to(torch.int16).to("cuda")
    lse = torch.full((n_f32 + GUARD,), float("nan"), dtype=torch.float32, device="cuda")
    return o, lse


def host_bits(t) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


def run_fwd(q, k, v, causal, scale, stream=None, window=-1):
    """Run attn_fwd (attn_fwd_window when window >= 0) on bit arrays; returns
    (o_bits [B,Hq,Sq,d], lse f32, guards_ok)."""
    torch = torch_mod()
    B, Hq, Sq, d = q.shape
    _, Hkv, Sk, _ = k.shape
    qd, kd, vd = dev_bits(q), dev_bits(k), dev_bits(v)
    n = B * Hq * Sq
    o, lse = nan_out(n * d, n)
    if window >= 0:
        miattn.attn_fwd_window(qd, kd, vd, o, lse, B, Hq, Hkv, Sq, Sk, d, causal, window, scale,
                               stream)
    else:
        miattn.attn_fwd(qd, kd, vd, o, lse, B, Hq, Hkv, Sq, Sk, d, causal, scale, stream)
    torch.cuda.synchronize()
    ob = host_bits(o)
    lh = lse.cpu().numpy()
    guards = bool(np.all(ob[n * d:] == NAN_BF16) and np.all(np.isnan(lh[n:])))
    return ob[:n * d].reshape(B, Hq, Sq, d), lh[:n].reshape(B, Hq, Sq), guards


def run_fwd_ext(q, k, v, causal, scale, window=-1, softcap=0.0, alibi=None):
    """Run attn_fwd_ext on bit arrays (alibi: float32 slopes [Hq] or None);
    returns (o_bits [B,Hq,Sq,d], lse f32, guards_ok)."""
    torch = torch_mod()
    B, Hq, Sq, d = q.shape
    _, Hkv, Sk, _ = k.shape
    qd, kd, vd = dev_bits(q), dev_bits(k), dev_bits(v)
    ad = None
    if alibi is not None:
        ad = torch.from_numpy(np.ascontiguousarray(alibi, dtype=np.float32)).to("cuda")
    n = B * Hq * Sq
    o, lse = nan_out(n * d, n)
    miattn.attn_fwd_ext(qd, kd, vd, o, lse, B, Hq, Hkv, Sq, Sk, d, causal, window, softcap, ad,
                        scale)
    torch.cuda.synchronize()
    ob = host_bits(o)
    lh = lse.cpu().numpy()
    guards = bool(np.all(ob[n * d:] == NAN_BF16) and np.all(np.isnan(lh[n:])))
    return ob[:n * d].reshape(B, Hq, Sq, d), lh[:n].reshape(B, Hq, Sq), guards


def run_bwd(q, k, v, o_bits, lse, do, causal, scale):
    """Run attn_bwd on bit arrays (o_bits bf16, lse f32 as the forward wrote
    them); returns (dq, dk, dv) bits and guards_ok."""
    torch = torch_mod()
    B, Hq, Sq, d = q.shape
    _, Hkv, Sk, _ = k.shape
    nq, nk = B * Hq * Sq * d, B * Hkv * Sk * d
    dq, _ = nan_out(nq, 1)
    dk, _ = nan_out(nk, 1)
    dv, _ = nan_out(nk, 1)
    ld = torch.from_numpy(np.ascontiguousarray(lse, dtype=np.float32).reshape(-1)).to("cuda")
    wsb = miattn.attn_bwd_workspace_size(B, Hq, Sq)
    ws = torch.full((max(wsb // 4, 1),), float("nan"), dtype=torch.float32, device="cuda")
    miattn.attn_bwd(dev_bits(q), dev_bits(k), dev_bits(v), dev_bits(o_bits), ld, dev_bits(do),
                    dq, dk, dv, B, Hq, Hkv, Sq, Sk, d, causal, scale, ws, wsb)
    torch.cuda.synchronize()
    out = []
    guards = True
    for t, n, shape in ((dq, nq, q.shape), (dk, nk, k.shape), (dv, nk, k.shape)):
        b = host_bits(t)
        guards &= bool(np.all(b[n:] == NAN_BF16))
        out.append(b[:n].reshape(shape))
    return out[0], out[1], out[2], guards


def grad_metrics(bits, ref):
    """rel-RMS and max-abs (relative to max |ref|) of bf16 gradient bits
    against the f64 reference."""
    g = inputs.bf16_to_f32(bits).astype(np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    scale = max(float(np.abs(ref).max()) if ref.size else 0.0, 1e-30)
    return {"finite": bool(np.all(np.isfinite(g))),
            "rel_rms": float(np.linalg.norm(g - ref) / max(np.linalg.norm(ref), 1e-30)),
            "max_abs_rel": float(np.abs(g - ref).max() / scale) if g.size else 0.0}


def run_decode(q, kc, vc, lens, scale, splits, ws_fill=float("nan")):
    torch = torch_mod()
    B, Hq, d = q.shape
    _, Hkv, S_cap, _ = kc.shape
    qd, kd, vd = dev_bits(q), dev_bits(kc), dev_bits(vc)
    ld = torch.from_numpy(np.ascontiguousarray(lens, dtype=np.int32)).to("cuda")
    n = B * Hq
    o, lse = nan_out(n * d, n)
    nbytes = miattn.attn_fwd_decode_workspace_size(B, Hq, d, splits)
    ws = torch.full((max(nbytes // 4, 4),), ws_fill, dtype=torch.float32, device="cuda")
    miattn.attn_fwd_decode(qd, kd, vd, ld, o, lse, B, Hq, Hkv, S_cap, d, splits, scale, ws,
                           nbytes)
    torch.cuda.synchronize()
    ob = host_bits(o)
    lh = lse.cpu().numpy()
    guards = bool(np.all(ob[n * d:] == NAN_BF16) and np.all(np.isnan(lh[n:])))
    return ob[:n * d].reshape(B, Hq, d), lh[:n].reshape(B, Hq), guards


def run_decode_paged(q, k_pool, v_pool, table, lens, page_size, scale, splits,
                     ws_fill=float("nan")):
    torch = torch_mod()
    B, Hq, d = q.shape
    num_pages, Hkv, P, _ = k_pool.shape
    assert P == page_size and v_pool.shape == k_pool.shape
    qd, kd, vd = dev_bits(q), dev_bits(k_pool), dev_bits(v_pool)
    td = torch.from_numpy(np.ascontiguousarray(table, dtype=np.int32)).to("cuda")
    ld = torch.from_numpy(np.ascontiguousarray(lens, dtype=np.int32)).to("cuda")
    n = B * Hq
    o, lse = nan_out(n * d, n)
    nbytes = miattn.attn_fwd_decode_workspace_size(B, Hq, d, splits)
    ws = torch.full((max(nbytes // 4, 4),), ws_fill, dtype=torch.float32, device="cuda")
    miattn.attn_fwd_decode_paged(qd, kd, vd, td, ld, o, lse, B, Hq, Hkv, num_pages, page_size,
                                 table.shape[1], d, splits, scale, ws, nbytes)
    torch.cuda.synchronize()
    ob = host_bits(o)
    lh = lse.cpu().numpy()
    guards = bool(np.all(ob[n * d:] == NAN_BF16) and np.all(np.isnan(lh[n:])))
    return ob[:n * d].reshape(B, Hq, d), lh[:n].reshape(B, Hq), guards


def metrics(o_bits, lse, o_ref, lse_ref):
    """Error metrics of GPU outputs against f64 references (same shapes)."""
    og = inputs.bf16_to_f32(o_bits).astype(np.float64)
    o_ref = np.asarray(o_ref, dtype=np.float64)
    lse = np.asarray(lse, dtype=np.float64)
    lse_ref = np.asarray(lse_ref, dtype=np.float64)
    empty = np.isneginf(lse_ref)
    full = ~empty
    diff = og - o_ref
    res = {
        "o_finite": bool(np.all(np.isfinite(og))),
        "o_max_abs": float(np.max(np.abs(diff))) if diff.size else 0.0,
        "o_rel_rms": float(np.linalg.norm(diff) / max(np.linalg.norm(o_ref), 1e-300))
        if diff.size else 0.0,
        "lse_max_abs": float(np.max(np.abs(lse[full] - lse_ref[full]))) if full.any() else 0.0,
        "empty_rows": int(empty.sum()),
        "empty_exact": bool(np.all(np.isneginf(lse[empty]))
                            and np.all(o_bits[empty] == 0)) if empty.any() else True,
        "lse_finite_where_expected": bool(np.all(np.isfinite(lse[full]))),
    }
    return res


def assert_parity(m, label=""):
    assert m["o_finite"], (label, m)
    assert m["lse_finite_where_expected"], (label, m)
    assert m["o_max_abs"] <= O_MAX_ABS, (label, m)
    assert m["o_rel_rms"] <= O_REL_RMS, (label, m)
    assert m["lse_max_abs"] <= LSE_MAX_ABS, (label, m)
    assert m["empty_exact"], (label, m)
