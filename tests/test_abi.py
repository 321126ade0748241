"""The C ABI on the host (no GPU needed): the library loads, exports every
entry point include/miattn.h declares, and rejects bad arguments with the
documented status before anything is launched."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

from online_softmax_monoid_amd import miattn as M

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    text = open(os.path.join(ROOT, "include", "miattn.h")).read()
    return sorted(set(re.findall(r"^MIATTN_API\s+[\w\s\*]*?\b(\w+)\s*\(", text, re.M)))


def test_header_declares_the_binding_names():
    assert _declared() == sorted(M.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(M.LIB_PATH if os.path.exists(M.LIB_PATH) else M.load()._name)
    for name in _declared():
        assert hasattr(lib, name), name


def test_probe_library_exports_every_declared_symbol():
    """libmiprobe.so (the bench's machine probes) exports what include/miprobe.h
    declares."""
    from online_softmax_monoid_amd import build
    text = open(os.path.join(ROOT, "include", "miprobe.h")).read()
    names = sorted(set(re.findall(r"^MIPROBE_API\s+[\w\s\*]*?\b(\w+)\s*\(", text, re.M)))
    assert names == ["probe_chase", "probe_empty", "probe_mfma", "probe_read"]
    if not os.path.exists(build.PROBE_LIB):
        build._build_lib(build.PROBE_LIB, build.PROBE_SOURCES)
    lib = ctypes.CDLL(build.PROBE_LIB)
    for name in names:
        assert hasattr(lib, name), name


def test_version_and_workspace_size():
    assert M.miattn_version() == 700
    assert M.attn_fwd_decode_workspace_size(32, 32, 128, 16) == 32 * 32 * 16 * 130 * 4
    assert M.attn_fwd_decode_workspace_size(0, 32, 128, 16) == 0
    assert M.attn_fwd_decode_workspace_size(1, 0, 128, 16) == 0
    assert M.attn_fwd_decode_workspace_size(1, 1, 128, 0) == 0


FAKE = 0x7F0000000000  # 16-byte aligned, never dereferenced: validation fails first


def _fwd(**kw):
    args = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=1, Hq=2, Hkv=2, Sq=8, Sk=8, d=64,
                causal=0, scale=0.125, stream=0)
    args.update(kw)
    return M.load().attn_fwd(args["q"], args["k"], args["v"], args["o"], args["lse"],
                             args["B"], args["Hq"], args["Hkv"], args["Sq"], args["Sk"],
                             args["d"], args["causal"], args["scale"], args["stream"])


@pytest.mark.parametrize("kw,status,needle", [
    (dict(q=0), M.MIATTN_ERR_INVALID_ARG, "q is NULL"),
    (dict(k=0), M.MIATTN_ERR_INVALID_ARG, "k is NULL"),
    (dict(v=0), M.MIATTN_ERR_INVALID_ARG, "v is NULL"),
    (dict(o=0), M.MIATTN_ERR_INVALID_ARG, "o is NULL"),
    (dict(lse=0), M.MIATTN_ERR_INVALID_ARG, "lse is NULL"),
    (dict(q=FAKE + 8), M.MIATTN_ERR_INVALID_ARG, "aligned"),
    (dict(lse=FAKE + 2), M.MIATTN_ERR_INVALID_ARG, "aligned"),
    (dict(Hq=3, Hkv=2), M.MIATTN_ERR_INVALID_ARG, "multiple"),
    (dict(Hkv=0), M.MIATTN_ERR_INVALID_ARG, "head counts"),
    (dict(B=-1), M.MIATTN_ERR_INVALID_ARG, "sizes"),
    (dict(Sk=-1), M.MIATTN_ERR_INVALID_ARG, "sizes"),
    (dict(d=96), M.MIATTN_ERR_UNSUPPORTED, "head dimension"),
    (dict(d=32), M.MIATTN_ERR_UNSUPPORTED, "head dimension"),
    (dict(Sq=1 << 23, d=128), M.MIATTN_ERR_UNSUPPORTED, "2 GiB"),
    (dict(Sk=1 << 22, d=256), M.MIATTN_ERR_UNSUPPORTED, "2 GiB"),
    (dict(scale=0.0), M.MIATTN_ERR_INVALID_ARG, "scale"),
    (dict(scale=-1.0), M.MIATTN_ERR_INVALID_ARG, "scale"),
    (dict(scale=float("inf")), M.MIATTN_ERR_INVALID_ARG, "scale"),
    (dict(scale=float("nan")), M.MIATTN_ERR_INVALID_ARG, "scale"),
])
def test_attn_fwd_rejects(kw, status, needle):
    assert _fwd(**kw) == status
    assert needle in M.miattn_last_error()


def test_attn_fwd_empty_is_a_no_op():
    assert _fwd(B=0, q=0, k=0, v=0, o=0, lse=0) == M.MIATTN_OK
    assert _fwd(Sq=0, q=0, k=0, v=0, o=0, lse=0) == M.MIATTN_OK


def test_binding_raises_with_message():
    with pytest.raises(M.MiattnError) as e:
        M.attn_fwd(0, FAKE, FAKE, FAKE, FAKE, 1, 2, 2, 8, 8, 64, False, 0.125, stream=0)
    assert e.value.status == M.MIATTN_ERR_INVALID_ARG and "q is NULL" in e.value.message


def test_attn_fwd_window_rejects_a_negative_window():
    L = M.load()
    assert L.attn_fwd_window(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 2, 2, 8, 8, 64, 1, -3, 0.125,
                             0) == M.MIATTN_ERR_INVALID_ARG
    assert "window_left" in M.miattn_last_error()
    # the other checks are attn_fwd's
    assert L.attn_fwd_window(0, FAKE, FAKE, FAKE, FAKE, 1, 2, 2, 8, 8, 64, 1, 4, 0.125,
                             0) == M.MIATTN_ERR_INVALID_ARG
    assert "q is NULL" in M.miattn_last_error()
    assert L.attn_fwd_window(0, 0, 0, 0, 0, 0, 2, 2, 8, 8, 64, 1, 4, 0.125, 0) == M.MIATTN_OK


@pytest.mark.parametrize("softcap,alibi,status,needle", [
    (-1.0, 0, M.MIATTN_ERR_INVALID_ARG, "softcap"),
    (float("nan"), 0, M.MIATTN_ERR_INVALID_ARG, "softcap"),
    (float("inf"), 0, M.MIATTN_ERR_INVALID_ARG, "softcap"),
    (5.0, FAKE + 2, M.MIATTN_ERR_INVALID_ARG, "alibi_slopes"),
    (0.0, FAKE + 2, M.MIATTN_ERR_INVALID_ARG, "alibi_slopes"),
])
def test_attn_fwd_ext_rejects(softcap, alibi, status, needle):
    L = M.load()
    assert L.attn_fwd_ext(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 2, 2, 8, 8, 64, 1, -1, softcap,
                          alibi, 0.125, 0) == status
    assert needle in M.miattn_last_error()


def test_attn_fwd_varlen_rejects():
    L = M.load()
    args = lambda **kw: [kw.get(n, dv) for n, dv in (
        ("q", FAKE), ("k", FAKE), ("v", FAKE), ("o", FAKE), ("lse", FAKE), ("cq", FAKE),
        ("ck", FAKE), ("B", 2), ("tq", 100), ("tk", 120), ("mq", 60), ("mk", 70), ("Hq", 4),
        ("Hkv", 2), ("d", 128), ("causal", 1), ("scale", 0.1), ("stream", 0))]
    for kw, status, needle in [
            (dict(d=96), M.MIATTN_ERR_UNSUPPORTED, "head dimension"),
            (dict(cq=0), M.MIATTN_ERR_INVALID_ARG, "cu_seqlens_q is NULL"),
            (dict(ck=FAKE + 2), M.MIATTN_ERR_INVALID_ARG, "aligned"),
            (dict(tq=-1), M.MIATTN_ERR_INVALID_ARG, "sizes"),
            (dict(mk=-3), M.MIATTN_ERR_INVALID_ARG, "sizes"),
            (dict(Hq=3), M.MIATTN_ERR_INVALID_ARG, "multiple"),
            (dict(tq=1 << 23), M.MIATTN_ERR_UNSUPPORTED, "2 GiB")]:
        assert L.attn_fwd_varlen(*args(**kw)) == status, kw
        assert needle in M.miattn_last_error()
    assert L.attn_fwd_varlen(*args(q=0, k=0, v=0, o=0, lse=0, cq=0, ck=0, B=0)) == M.MIATTN_OK


def test_attn_fwd_varlen_ext_rejects():
    """The packed batch with variants: attn_fwd_varlen's checks, plus the soft
    cap and ALiBi slope checks of attn_fwd_ext."""
    L = M.load()
    args = lambda **kw: [kw.get(n, dv) for n, dv in (
        ("q", FAKE), ("k", FAKE), ("v", FAKE), ("o", FAKE), ("lse", FAKE), ("cq", FAKE),
        ("ck", FAKE), ("B", 2), ("tq", 100), ("tk", 120), ("mq", 60), ("mk", 70), ("Hq", 4),
        ("Hkv", 2), ("d", 128), ("causal", 1), ("window", -1), ("softcap", 0.0),
        ("alibi", 0), ("scale", 0.1), ("stream", 0))]
    for kw, status, needle in [
            (dict(softcap=-1.0), M.MIATTN_ERR_INVALID_ARG, "softcap"),
            (dict(softcap=float("nan")), M.MIATTN_ERR_INVALID_ARG, "softcap"),
            (dict(alibi=FAKE + 2), M.MIATTN_ERR_INVALID_ARG, "alibi_slopes"),
            (dict(d=96), M.MIATTN_ERR_UNSUPPORTED, "head dimension"),
            (dict(cq=0), M.MIATTN_ERR_INVALID_ARG, "cu_seqlens_q is NULL"),
            (dict(tq=-1), M.MIATTN_ERR_INVALID_ARG, "sizes"),
            (dict(Hq=3), M.MIATTN_ERR_INVALID_ARG, "multiple")]:
        assert L.attn_fwd_varlen_ext(*args(**kw)) == status, kw
        assert needle in M.miattn_last_error()
    assert L.attn_fwd_varlen_ext(*args(q=0, k=0, v=0, o=0, lse=0, cq=0, ck=0, B=0)) == M.MIATTN_OK


def test_attn_bwd_rejects():
    L = M.load()
    wsb = M.attn_bwd_workspace_size(1, 2, 8)
    assert wsb == 1 * 2 * 8 * 8 and M.attn_bwd_workspace_size(-1, 2, 8) == 0
    base = [FAKE] * 9 + [1, 2, 2, 8, 8, 128, 1, 0.125, FAKE, wsb, 0]
    for idx, val, status, needle in [
            (14, 96, M.MIATTN_ERR_UNSUPPORTED, "head dimension"),
            (18, 16, M.MIATTN_ERR_INVALID_ARG, "workspace too small"),
            (17, 0, M.MIATTN_ERR_INVALID_ARG, "workspace is NULL"),
            (5, 0, M.MIATTN_ERR_INVALID_ARG, "dout is NULL"),
            (8, FAKE + 2, M.MIATTN_ERR_INVALID_ARG, "aligned"),
            (16, 0.0, M.MIATTN_ERR_INVALID_ARG, "scale")]:
        args = list(base)
        args[idx] = val
        assert L.attn_bwd(*args) == status, (idx, val)
        assert needle in M.miattn_last_error()


def _dec(**kw):
    args = dict(q=FAKE, k=FAKE, v=FAKE, lens=FAKE, o=FAKE, lse=FAKE, B=2, Hq=4, Hkv=2, S_cap=16,
                d=128, ns=4, scale=0.1, ws=FAKE, wsb=None, stream=0)
    args.update(kw)
    if args["wsb"] is None:
        args["wsb"] = M.attn_fwd_decode_workspace_size(args["B"], args["Hq"], args["d"],
                                                       max(args["ns"], 1))
    return M.load().attn_fwd_decode(args["q"], args["k"], args["v"], args["lens"], args["o"],
                                    args["lse"], args["B"], args["Hq"], args["Hkv"],
                                    args["S_cap"], args["d"], args["ns"], args["scale"],
                                    args["ws"], args["wsb"], args["stream"])


@pytest.mark.parametrize("kw,status,needle", [
    (dict(q=0), M.MIATTN_ERR_INVALID_ARG, "q is NULL"),
    (dict(lens=0), M.MIATTN_ERR_INVALID_ARG, "kv_lens is NULL"),
    (dict(k=0), M.MIATTN_ERR_INVALID_ARG, "k_cache is NULL"),
    (dict(ws=0), M.MIATTN_ERR_INVALID_ARG, "workspace is NULL"),
    (dict(ws=FAKE + 4), M.MIATTN_ERR_INVALID_ARG, "aligned"),
    (dict(wsb=100), M.MIATTN_ERR_INVALID_ARG, "workspace too small"),
    (dict(ns=0), M.MIATTN_ERR_INVALID_ARG, "num_splits"),
    (dict(Hq=5), M.MIATTN_ERR_INVALID_ARG, "multiple"),
    (dict(d=80), M.MIATTN_ERR_UNSUPPORTED, "head dimension"),
    (dict(scale=0.0), M.MIATTN_ERR_INVALID_ARG, "scale"),
    (dict(S_cap=-1), M.MIATTN_ERR_INVALID_ARG, "sizes"),
])
def test_attn_fwd_decode_rejects(kw, status, needle):
    assert _dec(**kw) == status
    assert needle in M.miattn_last_error()


def test_decode_empty_batch_is_a_no_op():
    assert _dec(B=0, q=0, k=0, v=0, lens=0, o=0, lse=0, ws=0, wsb=0) == M.MIATTN_OK


def _dec_noalloc(**kw):
    args = dict(q=FAKE, k=FAKE, v=FAKE, lens=FAKE, o=FAKE, lse=FAKE, B=2, Hq=4, Hkv=2, S_cap=16,
                d=128, ns=4, scale=0.1, stream=0)
    args.update(kw)
    return M.load().attn_fwd_decode_noalloc(args["q"], args["k"], args["v"], args["lens"],
                                            args["o"], args["lse"], args["B"], args["Hq"],
                                            args["Hkv"], args["S_cap"], args["d"], args["ns"],
                                            args["scale"], args["stream"])


@pytest.mark.parametrize("kw,status,needle", [
    (dict(q=0), M.MIATTN_ERR_INVALID_ARG, "q is NULL"),
    (dict(lens=0), M.MIATTN_ERR_INVALID_ARG, "kv_lens is NULL"),
    (dict(v=FAKE + 8), M.MIATTN_ERR_INVALID_ARG, "aligned"),
    (dict(ns=0), M.MIATTN_ERR_INVALID_ARG, "num_splits"),
    (dict(d=80), M.MIATTN_ERR_UNSUPPORTED, "head dimension"),
    # 64 * 64 * 16 * (256 + 2) * 4 bytes of partials: more than the 16 MiB scratch
    (dict(B=64, Hq=64, Hkv=8, d=256, ns=16), M.MIATTN_ERR_UNSUPPORTED, "scratch"),
])
def test_attn_fwd_decode_noalloc_rejects(kw, status, needle):
    assert _dec_noalloc(**kw) == status
    assert needle in M.miattn_last_error()


def test_decode_noalloc_empty_batch_is_a_no_op():
    assert _dec_noalloc(B=0, q=0, k=0, v=0, lens=0, o=0, lse=0) == M.MIATTN_OK


def _paged(**kw):
    args = dict(q=FAKE, k=FAKE, v=FAKE, table=FAKE, lens=FAKE, o=FAKE, lse=FAKE, B=2, Hq=4,
                Hkv=2, num_pages=8, page_size=16, max_pages=4, d=128, ns=4, scale=0.1, ws=FAKE,
                wsb=None, stream=0)
    args.update(kw)
    if args["wsb"] is None:
        args["wsb"] = M.attn_fwd_decode_workspace_size(args["B"], args["Hq"], args["d"],
                                                       max(args["ns"], 1))
    return M.load().attn_fwd_decode_paged(
        args["q"], args["k"], args["v"], args["table"], args["lens"], args["o"], args["lse"],
        args["B"], args["Hq"], args["Hkv"], args["num_pages"], args["page_size"],
        args["max_pages"], args["d"], args["ns"], args["scale"], args["ws"], args["wsb"],
        args["stream"])


@pytest.mark.parametrize("kw,status,needle", [
    (dict(q=0), M.MIATTN_ERR_INVALID_ARG, "q is NULL"),
    (dict(table=0), M.MIATTN_ERR_INVALID_ARG, "block_table is NULL"),
    (dict(table=FAKE + 2), M.MIATTN_ERR_INVALID_ARG, "aligned"),
    (dict(k=0), M.MIATTN_ERR_INVALID_ARG, "k_pages is NULL"),
    (dict(v=FAKE + 8), M.MIATTN_ERR_INVALID_ARG, "aligned"),
    (dict(lens=0), M.MIATTN_ERR_INVALID_ARG, "kv_lens is NULL"),
    (dict(ws=0), M.MIATTN_ERR_INVALID_ARG, "workspace is NULL"),
    (dict(wsb=100), M.MIATTN_ERR_INVALID_ARG, "workspace too small"),
    (dict(page_size=8), M.MIATTN_ERR_INVALID_ARG, "page_size"),
    (dict(page_size=48), M.MIATTN_ERR_INVALID_ARG, "page_size"),
    (dict(page_size=1 << 21), M.MIATTN_ERR_INVALID_ARG, "page_size"),
    (dict(max_pages=1 << 20, page_size=1 << 11), M.MIATTN_ERR_INVALID_ARG, "2^31"),
    (dict(num_pages=0), M.MIATTN_ERR_INVALID_ARG, "num_pages"),
    (dict(num_pages=-1), M.MIATTN_ERR_INVALID_ARG, "sizes"),
    (dict(max_pages=-1), M.MIATTN_ERR_INVALID_ARG, "sizes"),
    (dict(ns=0), M.MIATTN_ERR_INVALID_ARG, "num_splits"),
    (dict(Hq=5), M.MIATTN_ERR_INVALID_ARG, "multiple"),
    (dict(d=80), M.MIATTN_ERR_UNSUPPORTED, "head dimension"),
    (dict(scale=float("inf")), M.MIATTN_ERR_INVALID_ARG, "scale"),
])
def test_attn_fwd_decode_paged_rejects(kw, status, needle):
    assert _paged(**kw) == status
    assert needle in M.miattn_last_error()


def test_decode_paged_empty_batch_is_a_no_op():
    assert _paged(B=0, q=0, k=0, v=0, table=0, lens=0, o=0, lse=0, ws=0, wsb=0) == M.MIATTN_OK


def test_product_path_does_not_import_the_oracle():
    import subprocess
    import sys
    code = ("import sys; sys.path.insert(0, %r)\n"
            "from online_softmax_monoid_amd import miattn, inputs\n"
            "miattn.load()\n"
            "assert 'oracle' not in sys.modules, sorted(sys.modules)\n") % ROOT
    subprocess.run([sys.executable, "-c", code], check=True)
