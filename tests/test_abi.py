"""Host-side ABI checks of libgdn (CPU only: no kernel is launched).

The library must load, export every entry point include/gdn.h declares, and
reject bad arguments with its status codes before anything is enqueued (the
calls below all fail validation, so none reaches a launch).
"""

import ctypes
import subprocess

import pytest

from frame_wise_gated_amd import gdn


@pytest.fixture(scope="module")
def L():
    return gdn.lib()


def test_exports_every_declared_symbol(L):
    names = gdn.exported_names_in_header()
    assert set(names) == {"gdn_status_str", "gdn_workspace_bytes", "gdn_prepare", "gdn_frame_terms",
                          "gdn_scan_fwd", "gdn_scan_bidir_chunked", "gdn_compose", "gdn_readout",
                          "gdn_step", "gdn_scan_bwd", "gdn_bwd_workspace_bytes",
                          "gdn_scan_bidir_chunked_bwd", "gdn_bidir_bwd_workspace_bytes",
                          "gdn_trace_set", "gdn_step_noalloc"}
    out = subprocess.run(["nm", "-D", "--defined-only", gdn.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for n in names:
        assert n in exported, n
        getattr(L, n)
    # nothing but the ABI is exported from the library's own code
    assert {n for n in exported if n.startswith("gdn")} == set(names)


def test_status_strings():
    assert gdn.gdn_status_str(0) == "GDN_OK"
    for s in range(1, 5):
        assert gdn.gdn_status_str(s).startswith("GDN_E")
    assert "unknown" in gdn.gdn_status_str(99)


def _ws(d, P=1):
    return gdn.gdn_workspace_bytes(d, P)


def test_workspace_sizes():
    d = gdn.make_desc(1, 16, 121, 3600, 128, gdn.GDN_BF16)
    w1 = _ws(d, 1)
    w8 = _ws(d, 8)
    assert w8 > w1 > 0
    DD = 128 * 128 * 4
    fh = 16 * 121
    assert w1 >= fh * DD * 4  # terms (A and U) + forward and reverse state scratch
    assert w8 - w1 >= 3 * 16 * 7 * DD  # composites C, H and chunk starts for 7 more chunks
    # monotone in every dimension
    for field in ("B", "H", "T", "S"):
        d2 = gdn.make_desc(1, 16, 121, 3600, 128, gdn.GDN_BF16)
        setattr(d2, field, getattr(d2, field) * 2)
        assert _ws(d2, 1) >= w1, field
    # an empty problem needs almost nothing
    assert _ws(gdn.make_desc(1, 1, 0, 12, 16, gdn.GDN_F32)) < 4096


def test_shapes_whose_grids_exceed_a_dispatch_are_unsupported():
    """A dispatch holds fewer than 2^32 work-items; shapes that would need a
    larger grid are refused on the host (GDN_EUNSUPPORTED), before anything is
    enqueued, instead of launching a truncated grid."""
    n = ctypes.c_size_t(0)
    ws = lambda d, P=1: gdn.lib().gdn_workspace_bytes(ctypes.byref(d), P, ctypes.byref(n))
    # fp32 path: token-parallel kernels need about S * D work-items per frame-head
    assert ws(gdn.make_desc(1, 1, 20000, 3600, 128, gdn.GDN_F32)) == gdn.GDN_EUNSUPPORTED
    assert ws(gdn.make_desc(1, 1, 2000, 3600, 128, gdn.GDN_F32)) == gdn.GDN_OK
    # MFMA path: per-frame-head kernels, up to 4096 work-items each
    assert ws(gdn.make_desc(1, 1, 1000000, 16, 128, gdn.GDN_BF16)) == gdn.GDN_OK
    assert ws(gdn.make_desc(1, 2, 1000000, 16, 128, gdn.GDN_BF16)) == gdn.GDN_EUNSUPPORTED
    # scans: up to 32 blocks per (head, chunk) job, so the time-chunk count counts
    d = gdn.make_desc(1, 8000, 100, 16, 128, gdn.GDN_BF16)
    assert ws(d, 1) == gdn.GDN_OK
    assert ws(d, 100) == gdn.GDN_EUNSUPPORTED
    bb = ctypes.c_size_t(0)
    assert gdn.lib().gdn_bidir_bwd_workspace_bytes(ctypes.byref(d), 1, ctypes.byref(bb)) == \
        gdn.GDN_EUNSUPPORTED
    # and the entry points refuse them the same way, with nothing to enqueue
    fake = ctypes.c_void_p(256)
    assert gdn.lib().gdn_scan_fwd(ctypes.byref(d), fake, fake, fake, fake, fake, None, fake, None,
                                  None, 100, fake, 1 << 40, None) == gdn.GDN_EUNSUPPORTED


def test_reuse_flag_changes_no_workspace_size():
    """GDN_REUSE_FWD_TERMS only tells a backward call where A_t already is:
    every workspace query answers the same with or without it."""
    d = gdn.make_desc(1, 2, 5, 300, 128, gdn.GDN_BF16)
    r = gdn.make_desc(1, 2, 5, 300, 128, gdn.GDN_BF16, reuse_fwd_terms=True)
    assert r.flags == d.flags | gdn.GDN_REUSE_FWD_TERMS
    for P in (1, 3):
        assert gdn.gdn_workspace_bytes(r, P) == gdn.gdn_workspace_bytes(d, P)
    assert gdn.gdn_bwd_workspace_bytes(r) == gdn.gdn_bwd_workspace_bytes(d)
    assert gdn.gdn_bidir_bwd_workspace_bytes(r, 2) == gdn.gdn_bidir_bwd_workspace_bytes(d, 2)


@pytest.mark.parametrize("mutate,status", [
    (dict(D=48), gdn.GDN_EUNSUPPORTED),
    (dict(D=256), gdn.GDN_EUNSUPPORTED),
    (dict(S=0), gdn.GDN_EINVAL),
    (dict(T=-1), gdn.GDN_EINVAL),
    (dict(io_dtype=7), gdn.GDN_EINVAL),
    (dict(flags=8), gdn.GDN_EINVAL),
    (dict(flags=3), gdn.GDN_OK),
    (dict(flags=7), gdn.GDN_OK),
    (dict(key_scale=float("nan")), gdn.GDN_EINVAL),
])
def test_bad_descriptor(mutate, status):
    d = gdn.make_desc(1, 2, 3, 12, 16, gdn.GDN_F32)
    for kk, vv in mutate.items():
        setattr(d, kk, vv)
    n = ctypes.c_size_t(12345)
    assert gdn.lib().gdn_workspace_bytes(ctypes.byref(d), 1, ctypes.byref(n)) == status
    if status != gdn.GDN_OK:
        assert n.value == 12345  # left unchanged on error


def test_null_and_chunk_arguments(L):
    d = gdn.make_desc(1, 1, 4, 12, 16, gdn.GDN_F32)
    n = ctypes.c_size_t(0)
    assert L.gdn_workspace_bytes(None, 1, ctypes.byref(n)) == gdn.GDN_EINVAL
    assert L.gdn_workspace_bytes(ctypes.byref(d), 0, ctypes.byref(n)) == gdn.GDN_EINVAL
    assert L.gdn_workspace_bytes(ctypes.byref(d), 257, ctypes.byref(n)) == gdn.GDN_EINVAL
    fake = 0x100000  # never dereferenced: every call below fails validation first
    # n_time_chunks > T
    assert L.gdn_scan_fwd(ctypes.byref(d), fake, fake, fake, fake, fake, None, fake, None, None, 5,
                          fake, 1 << 30, None) == gdn.GDN_EINVAL
    # missing gamma
    assert L.gdn_scan_fwd(ctypes.byref(d), fake, fake, fake, fake, None, None, fake, None, None, 1,
                          fake, 1 << 30, None) == gdn.GDN_EINVAL
    # o requested without q
    assert L.gdn_scan_fwd(ctypes.byref(d), None, fake, fake, fake, fake, None, None, None, fake, 1,
                          fake, 1 << 30, None) == gdn.GDN_EINVAL
    # workspace too small
    assert L.gdn_scan_fwd(ctypes.byref(d), fake, fake, fake, fake, fake, None, fake, None, None, 1,
                          fake, 16, None) == gdn.GDN_EWORKSPACE
    # misaligned pointer
    assert L.gdn_scan_fwd(ctypes.byref(d), fake, fake + 2, fake, fake, fake, None, fake, None, None,
                          1, fake, 1 << 30, None) == gdn.GDN_EINVAL
    # bidirectional: chunk_len < 1
    assert L.gdn_scan_bidir_chunked(ctypes.byref(d), fake, fake, fake, fake, fake, None, 0, fake,
                                    None, None, None, 1, fake, 1 << 30, None) == gdn.GDN_EINVAL
    # compose: offsets must start at 0, end at T and not decrease
    for offs in ([1, 4], [0, 3], [0, 3, 2, 4]):
        arr = (ctypes.c_int32 * len(offs))(*offs)
        assert L.gdn_compose(ctypes.byref(d), fake, fake, fake, fake, arr, len(offs) - 1, fake,
                             None, None, None, fake, 1 << 30, None) == gdn.GDN_EINVAL
    # streaming step: NULL descriptor, missing gamma, workspace too small
    assert L.gdn_step(None, fake, fake, fake, fake, fake, None, fake, fake, None, None, fake,
                      1 << 30, None) == gdn.GDN_EINVAL
    assert L.gdn_step(ctypes.byref(d), fake, fake, fake, fake, None, None, fake, fake, None, None,
                      fake, 1 << 30, None) == gdn.GDN_EINVAL
    assert L.gdn_step(ctypes.byref(d), fake, fake, fake, fake, fake, None, fake, fake, None, None,
                      fake, 16, None) == gdn.GDN_EWORKSPACE
    # backward: RMSNorm unsupported, missing states, workspace too small
    dn = gdn.make_desc(1, 1, 4, 12, 16, gdn.GDN_F32, qk_rmsnorm=True)
    bwd = lambda dd, states, nb: L.gdn_scan_bwd(ctypes.byref(dd), fake, fake, fake, fake, fake, None,
                                                states, fake, None, fake, fake, fake, fake, fake,
                                                None, fake, nb, None)
    assert bwd(dn, fake, 16) == gdn.GDN_EWORKSPACE  # RMSNorm accepted
    assert bwd(d, None, 1 << 30) == gdn.GDN_EINVAL
    assert bwd(d, fake, 16) == gdn.GDN_EWORKSPACE
    nbw = ctypes.c_size_t(0)
    assert L.gdn_bwd_workspace_bytes(ctypes.byref(d), ctypes.byref(nbw)) == gdn.GDN_OK
    assert nbw.value > 0
    # bidirectional backward: chunk_len < 1, missing reverse states, RMSNorm,
    # workspace too small, more than 256 chunks; its workspace holds the causal one
    bbw = lambda dd, L_, rev, nb: L.gdn_scan_bidir_chunked_bwd(
        ctypes.byref(dd), L_, fake, fake, fake, fake, fake, None, fake, rev, fake, None, fake, fake,
        fake, fake, fake, None, fake, nb, None)
    assert bbw(d, 0, fake, 1 << 30) == gdn.GDN_EINVAL
    assert bbw(d, 2, None, 1 << 30) == gdn.GDN_EINVAL
    assert bbw(dn, 2, fake, 16) == gdn.GDN_EWORKSPACE  # RMSNorm accepted
    assert bbw(d, 2, fake, 16) == gdn.GDN_EWORKSPACE
    dlong = gdn.make_desc(1, 1, 300, 12, 16, gdn.GDN_F32)
    assert bbw(dlong, 1, fake, 1 << 30) == gdn.GDN_EUNSUPPORTED
    nbb = ctypes.c_size_t(0)
    assert L.gdn_bidir_bwd_workspace_bytes(ctypes.byref(d), 0, ctypes.byref(nbb)) == gdn.GDN_EINVAL
    assert L.gdn_bidir_bwd_workspace_bytes(ctypes.byref(dlong), 1, ctypes.byref(nbb)) == \
        gdn.GDN_EUNSUPPORTED
    assert L.gdn_bidir_bwd_workspace_bytes(ctypes.byref(d), 2, ctypes.byref(nbb)) == gdn.GDN_OK
    assert nbb.value > nbw.value
    # prepare refuses already-prepared keys
    dp = gdn.make_desc(1, 1, 4, 12, 16, gdn.GDN_F32, keys_prepared=True)
    assert L.gdn_prepare(ctypes.byref(dp), fake, fake, None) == gdn.GDN_EINVAL
    # nothing requested: a no-op that succeeds without touching the device
    assert L.gdn_scan_fwd(ctypes.byref(d), None, fake, fake, fake, fake, None, None, None, None, 1,
                          None, 0, None) == gdn.GDN_OK
    # B*H = 0: nothing to do
    d0 = gdn.make_desc(0, 4, 4, 12, 16, gdn.GDN_F32)
    assert L.gdn_scan_fwd(ctypes.byref(d0), None, None, None, None, None, None, None, None, None, 1,
                          None, 0, None) == gdn.GDN_OK


def test_trace_set_validates_and_clears(L):
    """gdn_trace_set refuses a trace with NULL arrays or negative sizes and
    accepts NULL (tracing off); with a trace set, a call that fails its
    argument checks records nothing."""
    ev = (ctypes.c_void_p * 4)()
    ph = (ctypes.c_int32 * 4)()
    assert L.gdn_trace_set(ctypes.byref(gdn.gdn_trace(None, ph, 4, 0))) == gdn.GDN_EINVAL
    assert L.gdn_trace_set(ctypes.byref(gdn.gdn_trace(ev, None, 4, 0))) == gdn.GDN_EINVAL
    assert L.gdn_trace_set(ctypes.byref(gdn.gdn_trace(ev, ph, -1, 0))) == gdn.GDN_EINVAL
    t = gdn.gdn_trace(ev, ph, 4, 0)
    assert L.gdn_trace_set(ctypes.byref(t)) == gdn.GDN_OK
    try:
        d = gdn.make_desc(1, 1, 2, 12, 16, gdn.GDN_F32)
        # NULL k with an output wanted (a host address that is never touched):
        # refused before anything is enqueued
        st = L.gdn_scan_fwd(ctypes.byref(d), None, None, None, None, None, None,
                            ctypes.c_void_p(0x1000), None, None, 1, None, 0, None)
        assert st == gdn.GDN_EINVAL
        assert t.count == 0
    finally:
        assert L.gdn_trace_set(None) == gdn.GDN_OK


def test_step_noalloc_refuses_shapes_beyond_its_scratch(L):
    """gdn_step_noalloc works in a fixed device array; a block whose workspace
    would not fit is refused with GDN_EWORKSPACE on the host, before any HIP
    call (the pointers below are never touched)."""
    big = gdn.make_desc(1, 16, 32, 3600, 128, gdn.GDN_BF16)
    assert gdn.gdn_workspace_bytes(big, 1) > gdn.GDN_NOALLOC_SCRATCH_BYTES
    fake = ctypes.c_void_p(0x1000)
    st = L.gdn_step_noalloc(ctypes.byref(big), fake, fake, fake, fake, fake, None, fake, fake,
                            None, None, None)
    assert st == gdn.GDN_EWORKSPACE
    # the 720p streaming block (16 heads, 1 to 6 frames) fits
    for T in range(1, 7):
        d = gdn.make_desc(1, 16, T, 3600, 128, gdn.GDN_BF16)
        assert gdn.gdn_workspace_bytes(d, 1) <= gdn.GDN_NOALLOC_SCRATCH_BYTES
    # a bad descriptor is still EINVAL
    bad = gdn.make_desc(1, 1, 1, 0, 128, gdn.GDN_BF16)
    assert L.gdn_step_noalloc(ctypes.byref(bad), fake, fake, fake, fake, fake, None, fake, fake,
                              None, None, None) == gdn.GDN_EINVAL


def test_binding_refuses_host_tensors():
    """The binding passes tensor addresses to the kernels as they are, so it
    refuses tensors that are not on the current GPU before calling the
    library (a host address would fault the device)."""
    import torch
    B, H, T, S, D = 1, 1, 2, 12, 16
    q = torch.zeros((B, H, T, S, D))
    st = torch.zeros((B, H, T, D, D))
    with pytest.raises(ValueError, match="current GPU"):
        gdn.gdn_readout(q, st, o=torch.zeros_like(q))
    with pytest.raises(ValueError, match="current GPU"):
        gdn.gdn_prepare(q, k_hat=torch.zeros_like(q))
