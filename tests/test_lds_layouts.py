"""CPU model of the LDS tile layouts of the prefill and backward kernels.

Each layout is restated here from the kernels' offset functions (prefill:
`koff`/`voff`, `klane`/`vlane`, `vimm` in `prefill_kernel.h`; backward:
`off_ft`, `ft_frag_off`, `ft_tr_off`, `off_rm`, `rm_frag_off`, `rm_tr_off` in
`backward.hip`) and checked on two counts:

* every read returns what the MFMA operand needs: a copy instruction moves
  lane L's 16 bytes from its global offset to byte 16 L of its 1 KB block, and
  each fragment read (16 bytes per lane: row l % 32, dims 16 kk + 8 (l / 32)
  .. +7) and each transposing read (8 bytes per lane L = 16 m + 4 e + c: row
  16 ch + 8 hh + 4 (m / 2) + e, dims 32 db + 16 (m % 2) + 4 c .. +3) lands on
  those bytes;
* no read has a bank conflict under the way the LDS serves them, as measured
  with the bank-conflict counter: a 16-byte read in four passes of 16 lanes
  (lanes l % 16 < 8 of one 16-lane row with l % 16 >= 8 of its neighbour),
  each pass needing 16 different 16-byte bank groups; a transposing 8-byte
  read in two passes of 32 lanes, each needing 32 different 8-byte slots of a
  256-byte bank row.

The negative cases show that the model finds the conflicts a plain stride
would have.
"""
from __future__ import annotations

import itertools

import pytest


def _frag_passes():
    for lo, hi in ((0, 1), (1, 0), (2, 3), (3, 2)):
        yield [16 * lo + x for x in range(8)] + [16 * hi + 8 + x for x in range(8)]


def _frag_conflicts(addr):
    return sum(len({(addr[l] // 16) % 16 for l in p}) != 16 for p in _frag_passes())


def _tr_conflicts(addr):
    return sum(len({(addr[l] // 8) % 32 for l in range(32 * h, 32 * h + 32)}) != 32 for h in (0, 1))


def _stored(copies):
    """LDS 16-byte chunk address -> (row, global 16-byte chunk of the row)."""
    t = {}
    for block, row_bytes, offs in copies:
        for lane, off in enumerate(offs):
            assert off % 16 == 0
            t[block + 16 * lane] = (off // row_bytes, (off % row_bytes) // 16)
    return t


def _check_frag(t, addr_of, D, n_kk):
    conf = 0
    for kk in range(n_kk):
        addr = {l: addr_of(l, kk) for l in range(64)}
        for l, a in addr.items():
            assert a % 16 == 0
            assert t[a] == (l % 32, 2 * kk + l // 32), (D, kk, l)
        conf += _frag_conflicts(addr)
    return conf


def _check_tr(t, addr_of, D):
    conf = 0
    for db, ch, hh in itertools.product(range(D // 32), range(2), range(2)):
        addr = {l: addr_of(l, db, ch, hh) for l in range(64)}
        for l, a in addr.items():
            m, e, c = l >> 4, (l >> 2) & 3, l & 3
            row = 16 * ch + 8 * hh + 4 * (m >> 1) + e
            dim = 32 * db + 16 * (m & 1) + 4 * c
            r, chunk = t[(a // 16) * 16]
            assert r == row and 16 * chunk + a % 16 == 2 * dim, (D, db, ch, hh, l)
        conf += _tr_conflicts(addr)
    return conf


# ---- prefill: row copies of K and V (head dimensions 128 and 256) ------------------

def _prefill_rows(D, kpb, vpb, swap=True):
    nblk = 32 // (512 // D)      # blocks per tile
    cpr = D // 8                 # 16-byte chunks per row
    kswap = (lambda q: q & 1) if (D == 128 and swap) else (lambda q: 0)
    kc, vc = [], []
    for i in range(nblk):
        ko, vo = [], []
        for lane in range(64):
            q, chunk = lane // cpr, lane % cpr
            key = i + nblk * q
            ko.append(key * 2 * D + 16 * (chunk ^ kswap(q)))
            vo.append(key * 2 * D + 16 * chunk)
        kc.append((i * kpb, 2 * D, ko))
        vc.append((i * vpb, 2 * D, vo))
    tk, tv = _stored(kc), _stored(vc)

    def kread(l, kk):
        l32, g = l & 31, l >> 5
        q = l32 // nblk
        return (l32 % nblk) * kpb + 2 * D * q + 16 * (g ^ kswap(q)) + 32 * kk

    def vread(l, db, ch, hh):
        vlane = (4 * (l >> 5) + ((l & 15) >> 2)) * vpb + 32 * ((l >> 4) & 1) + 8 * (l & 3)
        vimm = 8 * hh * vpb + 512 * ch + 64 * db if D == 256 else 512 * ch + 256 * hh + 64 * db
        return vlane + vimm

    return _check_frag(tk, kread, D, D // 16), _check_tr(tv, vread, D)


@pytest.mark.parametrize("D,kpb,vpb", [(128, 1056, 1088), (256, 1040, 1088)])
def test_prefill_row_copies(D, kpb, vpb):
    assert _prefill_rows(D, kpb, vpb) == (0, 0)


def test_prefill_row_copies_model_finds_conflicts():
    # without the chunk swap (or at a 1040 stride) the d = 128 K reads conflict
    assert _prefill_rows(128, 1040, 1088, swap=False)[0] > 0
    assert _prefill_rows(128, 1056, 1088, swap=False)[0] > 0
    # a V stride that is a multiple of 256 puts a key quad on one bank row
    assert _prefill_rows(128, 1056, 1024)[1] > 0


# ---- backward: both-ways tiles (head dimension 128) -----------------------------

def _ft(pb):
    swz = lambda r: 2 * ((r & 7) >> 2) + ((r >> 3) & 1)
    copies = []
    for i in range(8):
        offs = []
        for lane in range(64):
            r, p = i + 8 * (lane >> 4), lane & 15
            offs.append(r * 256 + 16 * (p ^ swz(r)))
        copies.append((i * pb, 256, offs))
    t = _stored(copies)

    def frag_off(l, odd):
        r, g = l & 31, l >> 5
        sw = swz(r)
        flip = 32 * (sw >> 1)
        return (r & 7) * pb + 256 * (r >> 3) + 16 * (g ^ (sw & 1)) + (-flip if odd else flip)

    def tr_off(l, hh):
        m, e, c = l >> 4, (l >> 2) & 3, l & 3
        r = 8 * hh + 4 * (m >> 1) + e
        return (r & 7) * pb + 256 * hh + 16 * ((2 * (m & 1) + (c >> 1)) ^ swz(r)) + 8 * (c & 1)

    fr = _check_frag(t, lambda l, kk: frag_off(l, kk & 1) + 32 * kk, 128, 8)
    tr = _check_tr(t, lambda l, db, ch, hh: tr_off(l, hh) + 512 * ch + 64 * db, 128)
    return fr, tr


def test_backward_both_ways_tiles():
    assert _ft(1088) == (0, 0)


def test_backward_both_ways_model_finds_conflicts():
    fr, tr = _ft(1024)
    assert fr + tr > 0
    fr, tr = _ft(1056)
    assert fr + tr > 0


# ---- backward: row-major tiles (head dimension 256) ------------------------------

def test_backward_row_major_tiles_d256():
    D = 256
    swz = lambda r: 4 * (r & 3) | ((r >> 2) & 1) | 2 * ((r >> 4) & 1)
    cpr = D // 8
    copies = []
    for i in range(16):
        offs = []
        for lane in range(64):
            row, c = (64 // cpr) * i + lane // cpr, lane % cpr
            offs.append(row * 2 * D + 16 * (c ^ swz(row)))
        # a row-major tile is its rows of 2D bytes, copy i at byte 1024 i
        copies.append((1024 * i, 2 * D, offs))
    t = _stored(copies)

    def frag(l, kk):
        r, g = l & 31, l >> 5
        k8, h = kk % 8, kk // 8
        return r * 2 * D + 16 * ((2 * k8 + g) ^ swz(r)) + 256 * h

    def tr(l, db, ch, hh):
        G, jj, q = l >> 4, (l >> 2) & 3, l & 3
        R = 16 * ch + 4 * (G >> 1) + jj
        o = R * 2 * D + 64 * ((db % 4) ^ jj) + 16 * ((2 * (G & 1) + (q >> 1)) ^ ((G >> 1) + 2 * ch)) + 8 * (q & 1)
        return o + 256 * (db // 4) + 16 * D * hh

    assert _check_frag(t, frag, D, 16) == 0
    assert _check_tr(t, tr, D) == 0
