"""gdn_step_noalloc (the streaming step on the library's static device
scratch) against gdn_step (the same step on a caller-allocated workspace),
through the C ABI, on two calls in a row, the second with a smaller block.

Both run the same kernels on the same inputs, so the results must be
bitwise equal; the 720p block is also checked against the float64 oracle on
one head (the bf16 bar)."""

import numpy as np
import pytest
import torch

from frame_wise_gated_amd import gdn
from frame_wise_gated_amd import inputs as gi
from oracle import gdn_oracle as orc

from gpu_helpers import DEV, frame_errs, head_arrays, host, say, tol, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gdn.lib()
    yield
    torch.cuda.synchronize()


def _inputs(w, seed):
    x = gi.batch_inputs(w, seed)
    d = upload(x, w)
    rng = np.random.default_rng([55, seed])
    s0 = (0.5 * rng.standard_normal((w.B, w.H, w.D, w.D))).astype(np.float32)
    return x, d, s0


def test_step_noalloc_matches_step_on_two_calls():
    # a 720p streaming block of 16 heads, then a smaller ragged block
    cases = [gi.workload(5).with_shape(H=16, T=3), gi.workload(5).with_shape(H=2, T=2, S=500)]
    for i, w in enumerate(cases):
        x, d, s0 = _inputs(w, i)
        s0d = torch.from_numpy(s0).to(DEV)
        say("noalloc step", i, (w.B, w.H, w.T, w.S, w.D))
        ref = gdn.gdn_step(d["q"], d["k"], d["v"], d["beta"], d["gamma"], carry_in=s0d,
                           want_states=True)
        # every output given, so nothing is allocated around the call
        got = {"o": torch.full_like(ref["o"], float("nan")),
               "states_fwd": torch.full_like(ref["states_fwd"], float("nan")),
               "states_rev": torch.full_like(ref["states_rev"], float("nan")),
               "carry_out": torch.full_like(ref["carry_out"], float("nan"))}
        r = gdn.gdn_step_noalloc(d["q"], d["k"], d["v"], d["beta"], d["gamma"], carry_in=s0d,
                                 carry_out=got["carry_out"], o=got["o"],
                                 states_fwd=got["states_fwd"], states_rev=got["states_rev"])
        torch.cuda.synchronize()
        for n in ("o", "states_fwd", "states_rev", "carry_out"):
            assert r[n] is got[n]
            assert torch.equal(got[n], ref[n]), (i, n)
        if i == 0:
            a = head_arrays(x, 0, 7)
            oref = orc.scan_bidir_chunked(a["q"], a["k"], a["v"], a["beta"], a["gamma"], w.T,
                                          s0=s0[0, 7][None, None].astype(np.float64))
            for n in ("o", "states_fwd", "states_rev"):
                e = frame_errs(host(got[n][0, 7]), oref[n][0, 0]).max()
                say("noalloc vs oracle", n, f"{e:.2e}")
                assert e <= tol(w), (n, e)


def test_step_noalloc_in_place_carry_chain():
    """Blocks chained with the carry updated in place, as a serving loop runs
    them: the same outputs as gdn_step chained the same way."""
    w = gi.workload(5).with_shape(H=4, T=7, S=300)
    x, d, s0 = _inputs(w, 3)
    c_ref = torch.from_numpy(s0).to(DEV)
    c_got = c_ref.clone()
    for a in range(0, w.T, 3):
        b = min(a + 3, w.T)
        blk = {n: d[n][:, :, a:b].contiguous() for n in ("q", "k", "v", "beta", "gamma")}
        say("noalloc chain block", a, b)
        r1 = gdn.gdn_step(blk["q"], blk["k"], blk["v"], blk["beta"], blk["gamma"], carry_in=c_ref,
                          carry_out=c_ref)
        o2 = torch.empty_like(blk["q"])
        gdn.gdn_step_noalloc(blk["q"], blk["k"], blk["v"], blk["beta"], blk["gamma"],
                             carry_in=c_got, carry_out=c_got, o=o2)
        torch.cuda.synchronize()
        assert torch.equal(o2, r1["o"]), (a, b)
    assert torch.equal(c_got, c_ref)


def test_step_noalloc_refuses_oversized_block():
    w = gi.workload(5).with_shape(H=16, T=32, S=3600)
    z = torch.zeros((1, 1, 1, 1, 1), device=DEV)
    desc = gdn.make_desc(w.B, w.H, w.T, w.S, w.D, gdn.GDN_BF16)
    import ctypes
    st = gdn.lib().gdn_step_noalloc(ctypes.byref(desc), z.data_ptr(), z.data_ptr(), z.data_ptr(),
                                    z.data_ptr(), z.data_ptr(), None, z.data_ptr(), z.data_ptr(),
                                    None, None, None)
    assert st == gdn.GDN_EWORKSPACE
