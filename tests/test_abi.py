"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, sizes its buffers, and rejects bad arguments before it
enqueues anything.  Every call below fails an argument check, so no kernel is
ever launched and no pointer is ever dereferenced.
"""
from __future__ import annotations

import ctypes

import pytest

import bwd_mamba2_scan_amd as m2


@pytest.fixture(scope="module")
def L():
    return m2.lib()


def test_exports_every_header_symbol(L):
    names = m2.header_functions()
    assert set(names) == {
        "mamba2_scan_saved_bytes", "mamba2_scan_bwd_workspace_bytes", "mamba2_scan_fwd",
        "mamba2_scan_bwd", "mamba2_scan_bwd_partials", "mamba2_scan_bwd_reduce", "mamba2_scan_bwd_input",
        "mamba2_scan_fwd_blend", "mamba2_scan_bwd_blend_workspace_bytes", "mamba2_scan_bwd_blend",
        "mamba2_scan_fwd_bf16", "mamba2_scan_bwd_bf16", "mamba2_scan_bwd_partials_bf16",
        "mamba2_scan_strerror", "mamba2_scan_fwd_plan", "mamba2_scan_bwd_noalloc",
        "mamba2_scan_bwd_full", "mamba2_scan_bwd_full_bf16",
    }
    for n in names:
        assert hasattr(L, n), n


def test_strerror_covers_codes():
    for code in (m2.OK, m2.EBADDIM, m2.EUNSUPPORTED, m2.ENULL, m2.ESIZE, m2.EALIGN, m2.EHIP, m2.ESCRATCH):
        assert m2.strerror(code) and m2.strerror(code) != "unknown status"
    assert m2.strerror(12345) == "unknown status"


def test_buffer_sizes():
    # saved: per 16-sample block and state group, 2K+1 planes of 16x16 floats,
    # plus one plane per 8-step round when K spans more than one round
    for B, K, SH2, D in ((64, 8, 256, 16), (8192, 8, 256, 16), (17, 3, 128, 32), (1, 1, 64, 64),
                         (100, 9, 256, 16), (8192, 64, 256, 16), (3, 100, 64, 32)):
        nb = (B + 15) // 16
        rounds = (K + 7) // 8
        planes = 2 * K + 1 + (rounds if rounds > 1 else 0)
        assert m2.saved_bytes(B, K, SH2, D) == nb * (D // 16) * planes * 256 * 4
        ws = m2.workspace_bytes(B, K, SH2, D)
        assert ws > 0 and ws % (SH2 * 48 * 4 * (D // 16)) == 0
    # workspace never shrinks as B grows
    for K, SH2, D in ((8, 256, 16), (64, 256, 16), (8, 512, 64), (3, 192, 32)):
        prev = 0
        for B in list(range(1, 3000)) + [8192, 32768, 100000]:
            ws = m2.workspace_bytes(B, K, SH2, D)
            assert ws >= prev, (B, K, SH2, D)
            prev = ws
    assert m2.workspace_bytes(8192, 8, 256, 16) == 64 * 256 * 48 * 4


@pytest.mark.parametrize("dims,code", [
    ((0, 8, 256, 16), m2.EBADDIM), ((8, 0, 256, 16), m2.EBADDIM), ((8, 8, 0, 16), m2.EBADDIM),
    ((8, 8, 256, 0), m2.EBADDIM), ((-1, 8, 256, 16), m2.EBADDIM),
    ((8, 8, 256, 8), m2.EUNSUPPORTED), ((8, 8, 256, 48), m2.EUNSUPPORTED),
    ((8, 8, 100, 16), m2.EUNSUPPORTED), ((8, 8, 1024, 16), m2.EUNSUPPORTED),
    ((2 ** 30, 2 ** 10, 512, 16), m2.EBADDIM),
])
def test_bad_dims(L, dims, code):
    assert m2.saved_bytes(*dims) == 0
    assert m2.workspace_bytes(*dims) == 0
    fake = ctypes.c_void_p(0x10000)
    assert L.mamba2_scan_fwd(*dims, fake, fake, fake, fake, fake, fake, fake, 1 << 40, None) == code
    assert L.mamba2_scan_bwd(*dims, fake, fake, fake, 1 << 40, fake, fake, fake, fake, None, None, None,
                             fake, 1 << 40, None) == code
    assert L.mamba2_scan_bwd_partials(*dims, fake, fake, fake, 1 << 40, fake, None, None, None,
                                      fake, 1 << 40, None) == code
    assert L.mamba2_scan_bwd_reduce(*dims, fake, 1 << 40, fake, fake, fake, None) == code
    assert L.mamba2_scan_bwd_input(*dims, fake, fake, fake, fake, 1 << 40, fake, fake, fake, None) == code
    assert m2.blend_workspace_bytes(*dims) == 0
    assert L.mamba2_scan_fwd_bf16(*dims, fake, fake, fake, fake, fake, fake, fake, 1 << 40, None) == code
    assert L.mamba2_scan_bwd_bf16(*dims, fake, fake, fake, 1 << 40, fake, fake, fake, fake, None, None, None,
                                  fake, 1 << 40, None) == code
    assert L.mamba2_scan_bwd_partials_bf16(*dims, fake, fake, fake, 1 << 40, fake, None, None, None,
                                           fake, 1 << 40, None) == code
    assert L.mamba2_scan_fwd_blend(*dims, fake, fake, fake, fake, fake, None, None, fake, fake, fake, 1 << 40,
                                   None) == code
    assert L.mamba2_scan_bwd_blend(*dims, fake, fake, fake, 1 << 40, None, fake, fake, fake, fake, fake, None,
                                   fake, 1 << 40, None) == code


def _fwd_args(dims, ptrs, saved_bytes):
    return (*dims, *ptrs, saved_bytes, None)


def test_fwd_argument_checks(L):
    dims = (64, 8, 256, 16)
    need = m2.saved_bytes(*dims)
    good = ctypes.c_void_p(0x10000)
    # a NULL in any required slot
    for i in range(7):
        ptrs = [good] * 7
        ptrs[i] = None
        assert L.mamba2_scan_fwd(*_fwd_args(dims, ptrs, need)) == m2.ENULL, i
    # saved too small
    assert L.mamba2_scan_fwd(*_fwd_args(dims, [good] * 7, need - 4)) == m2.ESIZE
    # misaligned: 16 bytes for h_history, h_s2, W_A/B/C, saved (slots 0-4, 6); 4 for context
    for i, off in ((0, 4), (1, 8), (6, 12), (2, 2), (3, 4), (4, 8), (5, 1)):
        ptrs = [good] * 7
        ptrs[i] = ctypes.c_void_p(0x10000 + off)
        assert L.mamba2_scan_fwd(*_fwd_args(dims, ptrs, need)) == m2.EALIGN, i


def test_bwd_argument_checks(L):
    dims = (100, 5, 192, 32)
    sv = m2.saved_bytes(*dims)
    ws = m2.workspace_bytes(*dims)
    g = ctypes.c_void_p(0x20000)

    def call(h=g, hs=g, saved=g, svb=sv, dctx=g, dwa=g, dwb=g, dwc=g, da=None, db=None, dc=None, w=g, wsb=ws):
        return L.mamba2_scan_bwd(*dims, h, hs, saved, svb, dctx, dwa, dwb, dwc, da, db, dc, w, wsb, None)

    for kw in ("h", "hs", "saved", "dctx", "dwa", "dwb", "dwc", "w"):
        assert call(**{kw: None}) == m2.ENULL, kw
    assert call(svb=sv - 1) == m2.ESIZE
    assert call(wsb=ws - 4) == m2.ESIZE
    for kw, off in (("h", 4), ("hs", 8), ("saved", 4), ("w", 8), ("dctx", 2), ("dwa", 1), ("da", 2)):
        assert call(**{kw: ctypes.c_void_p(0x20000 + off)}) == m2.EALIGN, kw

    assert L.mamba2_scan_bwd_partials(*dims, g, g, g, sv, g, None, None, None, None, ws, None) == m2.ENULL
    assert L.mamba2_scan_bwd_partials(*dims, g, g, g, sv, g, None, None, None, g, ws - 4, None) == m2.ESIZE
    assert L.mamba2_scan_bwd_reduce(*dims, g, ws, None, g, g, None) == m2.ENULL
    assert L.mamba2_scan_bwd_reduce(*dims, g, ws - 4, g, g, g, None) == m2.ESIZE
    assert L.mamba2_scan_bwd_reduce(*dims, ctypes.c_void_p(0x20004), ws, g, g, g, None) == m2.EALIGN


def test_bwd_row_span_limit(L):
    """With several state groups the backward addresses a block's rows with
    32-bit offsets: K * SH2 above 2^26 is refused before any other check, and
    only there (one state group has no such limit; a NULL pointer shows which
    check ran)."""
    big, edge = (16, 2 ** 18, 512, 32), (16, 2 ** 17, 512, 32)  # K * SH2 = 2^27, 2^26
    assert m2.workspace_bytes(*big) == 0 and m2.workspace_bytes(*edge) > 0
    assert m2.workspace_bytes(16, 2 ** 18, 512, 16) > 0
    for dims, code in ((big, m2.EUNSUPPORTED), (edge, m2.ENULL), ((16, 2 ** 18, 512, 16), m2.ENULL)):
        assert L.mamba2_scan_bwd(*dims, None, None, None, 0, None, None, None, None, None, None, None, None, 0,
                                 None) == code, dims
        assert L.mamba2_scan_bwd_noalloc(*dims, None, None, None, 0, None, None, None, None, None, None, None,
                                         None) == code, dims
        assert L.mamba2_scan_bwd_bf16(*dims, None, None, None, 0, None, None, None, None, None, None, None, None,
                                      0, None) == code, dims


def test_bwd_input_argument_checks(L):
    dims = (100, 5, 192, 32)
    sv = m2.saved_bytes(*dims)
    g = ctypes.c_void_p(0x30000)

    def call(wa=g, wb=g, wc=g, saved=g, svb=sv, dctx=g, dh=g, dhs=g):
        return L.mamba2_scan_bwd_input(*dims, wa, wb, wc, saved, svb, dctx, dh, dhs, None)

    for kw in ("wa", "wb", "wc", "saved", "dctx"):
        assert call(**{kw: None}) == m2.ENULL, kw
    assert call(dh=None, dhs=None) == m2.ENULL
    assert call(svb=sv - 4) == m2.ESIZE
    for kw, off in (("wa", 2), ("wb", 1), ("wc", 3), ("dctx", 2), ("saved", 4), ("dh", 8), ("dhs", 4)):
        assert call(**{kw: ctypes.c_void_p(0x30000 + off)}) == m2.EALIGN, kw
    # one output may be NULL (and then is not checked for alignment)
    assert call(dh=None, dhs=ctypes.c_void_p(0x30000 + 4)) == m2.EALIGN
    # a 16-sample block of d_h_history rows must stay under 4 GiB (K * SH2 <= 2^26)
    assert L.mamba2_scan_bwd_input(1, 1 << 18, 512, 16, g, g, g, g, 1 << 40, g, g, g, None) == m2.EUNSUPPORTED


def test_blend_workspace_covers_the_scan_backward():
    # the blend's workspace holds the scan backward's slices, then at most 256
    # d_temporal_weight slices of SH2 floats from a 256-byte boundary
    for B, K, SH2, D in ((64, 8, 256, 16), (8192, 8, 256, 16), (17, 3, 128, 32), (32768, 8, 512, 64)):
        ws = m2.workspace_bytes(B, K, SH2, D)
        assert m2.blend_workspace_bytes(B, K, SH2, D) == ((ws + 255) // 256) * 256 + 256 * SH2 * 4


def test_fwd_blend_argument_checks(L):
    dims = (64, 8, 256, 16)
    need = m2.saved_bytes(*dims)
    g = ctypes.c_void_p(0x40000)

    def call(h=g, hs=g, wa=g, wb=g, wc=g, stab=None, w=None, ctx=g, he=g, saved=g, svb=need):
        return L.mamba2_scan_fwd_blend(*dims, h, hs, wa, wb, wc, stab, w, ctx, he, saved, svb, None)

    for kw in ("h", "hs", "wa", "wb", "wc", "ctx", "saved"):
        assert call(**{kw: None}) == m2.ENULL, kw
    assert call(svb=need - 4) == m2.ESIZE
    for kw, off in (("stab", 2), ("w", 4), ("he", 8), ("h", 4)):
        assert call(**{kw: ctypes.c_void_p(0x40000 + off)}) == m2.EALIGN, kw


def test_bwd_blend_argument_checks(L):
    dims = (100, 5, 192, 32)
    sv = m2.saved_bytes(*dims)
    ws = m2.blend_workspace_bytes(*dims)
    g = ctypes.c_void_p(0x50000)

    def call(h=g, hs=g, saved=g, svb=sv, w=None, dhe=g, dctx=g, dwa=g, dwb=g, dwc=g, dw=None, wk=g, wsb=ws):
        return L.mamba2_scan_bwd_blend(*dims, h, hs, saved, svb, w, dhe, dctx, dwa, dwb, dwc, dw, wk, wsb, None)

    for kw in ("h", "hs", "saved", "dhe", "dctx", "dwa", "dwb", "dwc", "wk"):
        assert call(**{kw: None}) == m2.ENULL, kw
    assert call(svb=sv - 4) == m2.ESIZE
    assert call(wsb=ws - 4) == m2.ESIZE  # enough for the scan backward, short for the blend's slices
    assert call(wsb=m2.workspace_bytes(*dims)) == m2.ESIZE
    for kw, off in (("dhe", 4), ("w", 8), ("dw", 2), ("wk", 4)):
        assert call(**{kw: ctypes.c_void_p(0x50000 + off)}) == m2.EALIGN, kw


def test_bf16_entry_points_check_like_fp32(L):
    # same checks as the fp32 entry points: one defect per call, nothing launched
    dims = (64, 8, 256, 16)
    sv = m2.saved_bytes(*dims)
    ws = m2.workspace_bytes(*dims)
    g = ctypes.c_void_p(0x60000)
    assert L.mamba2_scan_fwd_bf16(*dims, None, g, g, g, g, g, g, sv, None) == m2.ENULL
    assert L.mamba2_scan_fwd_bf16(*dims, g, g, g, g, g, g, g, sv - 4, None) == m2.ESIZE
    assert L.mamba2_scan_fwd_bf16(*dims, ctypes.c_void_p(0x60008), g, g, g, g, g, g, sv, None) == m2.EALIGN
    assert L.mamba2_scan_bwd_bf16(*dims, g, None, g, sv, g, g, g, g, None, None, None, g, ws, None) == m2.ENULL
    assert L.mamba2_scan_bwd_bf16(*dims, g, g, g, sv, g, g, g, g, None, None, None, g, ws - 4, None) == m2.ESIZE
    assert L.mamba2_scan_bwd_partials_bf16(*dims, g, ctypes.c_void_p(0x60002), g, sv, g, None, None, None, g, ws,
                                           None) == m2.EALIGN


def test_noalloc_argument_checks(L):
    """The no-alloc backward runs every check before it looks up its buffer (no device needed here)."""
    dims = (100, 5, 192, 32)
    sv = m2.saved_bytes(*dims)
    g = ctypes.c_void_p(0x20000)

    def call(*, dims=dims, h=g, hs=g, saved=g, svb=sv, dctx=g, dwa=g, dwb=g, dwc=g, da=None, db=None, dc=None):
        return L.mamba2_scan_bwd_noalloc(*dims, h, hs, saved, svb, dctx, dwa, dwb, dwc, da, db, dc, None)

    L.mamba2_scan_bwd_noalloc.restype = ctypes.c_int
    assert call(dims=(0, 5, 192, 32)) == m2.EBADDIM
    assert call(dims=(100, 5, 100, 32)) == m2.EUNSUPPORTED
    for k in ("h", "hs", "saved", "dctx", "dwa", "dwb", "dwc"):
        assert call(**{k: None}) == m2.ENULL, k
    assert call(svb=sv - 4) == m2.ESIZE
    assert call(saved=ctypes.c_void_p(0x20004)) == m2.EALIGN
    assert call(dwb=ctypes.c_void_p(0x20002)) == m2.EALIGN
    assert call(da=ctypes.c_void_p(0x20001)) == m2.EALIGN
    assert m2.strerror(m2.ESCRATCH) != "unknown status"



def test_backward_workspace_follows_the_unit_plan():
    """The backward's split-K workspace is D/16 state groups x p0 slices x
    SH2 x 48 floats, with p0 = min(ceil(256 / V), ceil(units / waves)) and
    V = (SH2/64) * (D/16) work-group variants.  A sample block contributes
    K step units and its readout with one state group (12 waves), and
    ceil(K/2) step pairs and its readout with several (8 waves).  Checked
    against the library's own plan over a sweep of shapes (host only)."""
    for D in (16, 32, 64):
        NG = D // 16
        for SH2 in (64, 192, 256, 512):
            V = (SH2 // 64) * NG
            for K in (1, 2, 3, 8, 9, 64, 2048):
                for B in (1, 16, 17, 100, 1000, 8192, 32768):
                    NB = -(-B // 16)
                    units = NB * ((K + 1) // 2 + 1 if NG > 1 else K + 1)
                    waves = 8 if NG > 1 else 12
                    p0 = min(-(-256 // V), -(-units // waves))
                    assert m2.workspace_bytes(B, K, SH2, D) == NG * p0 * SH2 * 48 * 4, (B, K, SH2, D)


def test_noalloc_scratch_covers_every_shape():
    """The allocation-free backward's 4 MiB buffer holds the split-K slices of
    every supported shape: a sweep over sample counts, history lengths, trunk
    widths and state widths never asks for more."""
    limit = 4 << 20
    worst = (0, None)
    Bs = list(range(1, 65)) + [100, 255, 256, 257, 1000, 1024, 4096, 8192, 32768, 100000, 1 << 20]
    Ks = [1, 2, 3, 7, 8, 9, 15, 16, 17, 31, 32, 33, 64, 100, 1000, 2048, 8192, 65536]
    for D in (16, 32, 64):
        for SH2 in range(64, 513, 64):
            for K in Ks:
                for B in Bs:
                    if m2.saved_bytes(B, K, SH2, D) == 0:
                        continue  # beyond the supported sizes
                    ws = m2.workspace_bytes(B, K, SH2, D)
                    assert 0 < ws <= limit, (B, K, SH2, D, ws)
                    worst = max(worst, (ws, (B, K, SH2, D)))
    assert worst[0] > limit // 2, worst  # the sweep reaches the large-slice shapes


@pytest.mark.parametrize("fn", ["mamba2_scan_bwd_full", "mamba2_scan_bwd_full_bf16"])
def test_bwd_full_argument_checks(L, fn):
    dims = (100, 5, 192, 16)
    sv, ws = m2.saved_bytes(*dims), m2.workspace_bytes(*dims)
    g = ctypes.c_void_p(0x20000)
    f = getattr(L, fn)

    def call(*, dims=dims, h=g, hs=g, saved=g, svb=sv, dctx=g, wa=g, wb=g, wc=g, dwa=g, dwb=g, dwc=g, dh=g, dhs=g,
             w=g, wsb=ws):
        return f(*dims, h, hs, saved, svb, dctx, wa, wb, wc, dwa, dwb, dwc, dh, dhs, w, wsb, None)

    assert call(dims=(0, 5, 192, 16)) == m2.EBADDIM
    assert call(dims=(100, 5, 100, 16)) == m2.EUNSUPPORTED
    assert call(dims=(100, 2 ** 18, 512, 16)) == m2.EUNSUPPORTED  # K * SH2 > 2^26
    for k in ("h", "hs", "saved", "dctx", "wa", "wb", "wc", "dwa", "dwb", "dwc", "w"):
        assert call(**{k: None}) == m2.ENULL, k
    assert call(dh=None, dhs=None) == m2.ENULL
    assert call(svb=sv - 4) == m2.ESIZE
    assert call(wsb=ws - 4) == m2.ESIZE
    for k in ("wa", "dh", "dhs"):
        assert call(**{k: ctypes.c_void_p(0x20004)}) == m2.EALIGN, k
