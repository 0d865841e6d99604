"""Parity of the HIP library against the float64 oracle, element by element on
the same seeded inputs (run on an MI355X: ``pytest -m gpu``).

Bars: relative Frobenius error <= 1e-5 for fp32 workloads and <= 2e-2 for
bf16 workloads, on states and outputs separately, per head. Small cases cover
several tiles plus ragged tails; the five named workloads run at full size in
the launch configuration the benchmark times, checked on sampled heads.
"""

import ctypes

import numpy as np
import pytest
import torch

from frame_wise_gated_amd import gdn
from frame_wise_gated_amd import inputs as gi
from oracle import gdn_oracle as orc

from gpu_helpers import (DEV, bits_to_dev, frame_errs, head_arrays, host, rel_fro, rne_bf16_bits,
                         say, token_errs, tol, upload)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gdn.lib()  # loud failure if the library is missing
    yield
    torch.cuda.synchronize()


def _gen(w, seed=0):
    x = gi.batch_inputs(w, seed)
    return x, upload(x, w)


def _s0(w, seed=1, scale=0.5):
    rng = np.random.default_rng([99, seed])
    return (scale * rng.standard_normal((w.B, w.H, w.D, w.D))).astype(np.float32)


# ------------------------------------------------------------------ prepare
@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_prepare(io):
    """K_hat is the exact product ReLU(k) * c rounded once to the io dtype
    (round to nearest even), c being the library's fp32 key scale: bitwise
    equal to that rounding of the float64 product, which is exact for two
    fp32 factors."""
    w = gi.workload(2).with_shape(T=2, S=300, io=io)
    x, d = _gen(w)
    say("prepare", io)
    c32 = float(np.float32(1.0 / np.sqrt(float(w.D) * w.S)))
    for scale, kw in ((c32, {}), (0.25, {"key_scale": 0.25}), (0.3, {"key_scale": 0.3})):
        got = gdn.gdn_prepare(d["k"], **kw)
        torch.cuda.synchronize()
        exact = orc.prepare_keys(x["k"], key_scale=float(np.float32(scale)))
        if io == "bf16":
            got_bits = got.view(torch.int16).cpu().numpy().view(np.uint16)
            want = rne_bf16_bits(exact)
            n_bad = int((got_bits != want).sum())
            say("prepare", io, "scale", scale, "mismatches", n_bad)
            assert n_bad == 0
        else:
            want = exact.astype(np.float32)
            assert np.array_equal(got.cpu().numpy().view(np.uint32), want.view(np.uint32))


# ------------------------------------------------------------- frame terms
TERMS_CASES = {
    "bf16_D128_ragged_S1000": gi.workload(2).with_shape(H=2, T=3, S=1000),
    # calls with few frame-heads split each frame's tokens over up to five
    # workgroups, at most one per 512 tokens: 5, 3 and 2 splits (ragged tails)
    "bf16_D128_split5_S3600": gi.workload(2).with_shape(T=2),
    "bf16_D128_split3_S1700": gi.workload(2).with_shape(T=2, S=1700),
    "bf16_D128_split2_S1100": gi.workload(2).with_shape(T=2, S=1100),
    "bf16_D128_S5": gi.workload(2).with_shape(T=2, S=5),
    "bf16_D128_S1": gi.workload(2).with_shape(T=1, S=1),
    "f32_D16": gi.workload(1),
    "f32_D64_S50": gi.workload(1).with_shape(D=64, S=50, T=3),
    "f32_D128_S300": gi.workload(1).with_shape(D=128, S=300, T=2),
    "bf16_D32_S77": gi.workload(2).with_shape(D=32, S=77, T=2),
}


@pytest.mark.parametrize("name", sorted(TERMS_CASES))
def test_frame_terms(name):
    w = TERMS_CASES[name]
    x, d = _gen(w)
    say("frame_terms", name)
    A, U = gdn.gdn_frame_terms(d["k"], d["v"], d["beta"])
    A, U = host(A), host(U)
    for b in range(w.B):
        for h in range(w.H):
            kh = orc.prepare_keys(x["k"][b, h].astype(np.float64))
            for t in range(w.T):
                Ar, Ur = orc.frame_terms(kh[t], x["v"][b, h, t], x["beta"][b, h, t])
                assert rel_fro(A[b, h, t], Ar) <= tol(w), (b, h, t, rel_fro(A[b, h, t], Ar))
                assert rel_fro(U[b, h, t], Ur) <= tol(w), (b, h, t, rel_fro(U[b, h, t], Ur))


def test_frame_terms_prepared_keys():
    w = gi.workload(2).with_shape(T=2, S=700)
    x = gi.batch_inputs(w, 0)
    kh = orc.prepare_keys(x["k"].astype(np.float64))
    bits = gi.f32_to_bf16_bits(kh.astype(np.float32))
    kh_vals = gi.bf16_bits_to_f32(bits).astype(np.float64)
    from gpu_helpers import bits_to_dev
    d = upload(x, w)
    say("frame_terms prepared")
    A, U = gdn.gdn_frame_terms(bits_to_dev(bits), d["v"], d["beta"], keys_prepared=True)
    A, U = host(A), host(U)
    for t in range(w.T):
        Ar, Ur = orc.frame_terms(kh_vals[0, 0, t], x["v"][0, 0, t], x["beta"][0, 0, t])
        assert rel_fro(A[0, 0, t], Ar) <= tol(w)
        assert rel_fro(U[0, 0, t], Ur) <= tol(w)


# ------------------------------------------------------------ forward scan
SCAN_CASES = {
    "tiny_f32_seq": (gi.workload(1), 1, False),
    "tiny_f32_seq_s0": (gi.workload(1), 1, True),
    "tiny_f32_cp2_s0": (gi.workload(1), 2, True),
    "tiny_f32_cp8": (gi.workload(1), 8, False),
    "tiny_f32_B2H3": (gi.workload(1).with_shape(B=2, H=3), 3, True),
    "bf16_D128_seq": (gi.workload(2).with_shape(H=2, T=6, S=700), 1, False),
    "bf16_D128_cp3_s0": (gi.workload(2).with_shape(H=2, T=6, S=700), 3, True),
    # 64 (head, chunk) jobs: a compose launch that fills the chip, with 64-row blocks
    "bf16_D128_H16_cp4_s0": (gi.workload(2).with_shape(H=16, T=9, S=100), 4, True),
    "bf16_D64_seq": (gi.workload(2).with_shape(D=64, T=4, S=130), 1, True),
    "f32_D128_cp2": (gi.workload(1).with_shape(D=128, T=4, S=200), 2, True),
    # split phase 1 reduced straight into the scan's granule layout: 5, 3 and
    # 2 token splits per frame
    "bf16_D128_split5_S2600": (gi.workload(2).with_shape(T=2, S=2600), 1, False),
    # frames shorter than one stage of phase 1 and one tile of the readout
    "bf16_D128_S5_cp2_s0": (gi.workload(2).with_shape(H=2, T=4, S=5), 2, True),
    "bf16_D128_S1_s0": (gi.workload(2).with_shape(T=3, S=1), 1, True),
    "bf16_D128_split3_S1700_cp2": (gi.workload(2).with_shape(T=4, S=1700), 2, True),
    "bf16_D128_split2_S1100": (gi.workload(2).with_shape(H=2, T=3, S=1100), 1, True),
}


def _check_fwd(w, x, res, s0, heads, P=1, what=""):
    """States and outputs of the forward scan against the oracle: relative
    Frobenius error of every frame (states, o), of every token's output vector
    and of the final state, each within the bar."""
    for (b, h) in heads:
        a = head_arrays(x, b, h)
        ref = orc.scan_fwd(a["q"], a["k"], a["v"], a["beta"], a["gamma"],
                           s0=None if s0 is None else s0[b, h][None, None].astype(np.float64))
        e_st = frame_errs(host(res["states"][b, h]), ref["states"][0, 0]).max()
        o = host(res["o"][b, h])
        e_o = frame_errs(o, ref["o"][0, 0]).max()
        e_ot = token_errs(o, ref["o"][0, 0]).max()
        e_f = rel_fro(host(res["s_final"][b, h]), ref["s_final"][0, 0])
        say(what, f"head ({b},{h}) P={P}: max per frame: states {e_st:.2e} o {e_o:.2e}; "
                  f"max per token o {e_ot:.2e}; s_final {e_f:.2e}")
        assert max(e_st, e_o, e_ot, e_f) <= tol(w)


@pytest.mark.parametrize("name", sorted(SCAN_CASES))
def test_scan_fwd(name):
    w, P, with_s0 = SCAN_CASES[name]
    x, d = _gen(w)
    s0 = _s0(w) if with_s0 else None
    s0d = None if s0 is None else torch.from_numpy(s0).to(DEV)
    say("scan_fwd", name)
    res = gdn.gdn_scan_fwd(d["q"], d["k"], d["v"], d["beta"], d["gamma"], s0=s0d, n_time_chunks=P)
    torch.cuda.synchronize()
    _check_fwd(w, x, res, s0, [(b, h) for b in range(w.B) for h in range(w.H)], P, name)


def test_scan_fwd_optional_outputs():
    """NULL outputs are skipped; what is requested matches the full call bitwise."""
    w = gi.workload(2).with_shape(T=5, S=300)
    x, d = _gen(w)
    say("scan_fwd optional outputs")
    full = gdn.gdn_scan_fwd(d["q"], d["k"], d["v"], d["beta"], d["gamma"], n_time_chunks=2)
    only_o = gdn.gdn_scan_fwd(d["q"], d["k"], d["v"], d["beta"], d["gamma"], n_time_chunks=2,
                              want_states=False, want_s_final=False)
    only_fin = gdn.gdn_scan_fwd(None, d["k"], d["v"], d["beta"], d["gamma"], n_time_chunks=2,
                                want_states=False, want_o=False)
    assert only_o["states"] is None and only_o["s_final"] is None
    assert torch.equal(only_o["o"], full["o"])
    assert torch.equal(only_fin["s_final"], full["s_final"])


# ------------------------------------------------------ bidirectional scan
BIDIR_CASES = {
    "tiny_f32_L3": (gi.workload(1), 3, 1),
    "tiny_f32_L1": (gi.workload(1), 1, 1),
    "tiny_f32_L8_full": (gi.workload(1), 8, 2),
    "tiny_f32_L100": (gi.workload(1), 100, 1),
    "bf16_D128_L2_cp2": (gi.workload(5).with_shape(H=2, T=5, S=600), 2, 2),
}


@pytest.mark.parametrize("name", sorted(BIDIR_CASES))
def test_scan_bidir(name):
    w, L, P = BIDIR_CASES[name]
    x, d = _gen(w)
    s0 = _s0(w)
    say("scan_bidir", name)
    res = gdn.gdn_scan_bidir_chunked(d["q"], d["k"], d["v"], d["beta"], d["gamma"], L,
                                     s0=torch.from_numpy(s0).to(DEV), n_time_chunks=P)
    torch.cuda.synchronize()
    for b in range(w.B):
        for h in range(w.H):
            a = head_arrays(x, b, h)
            ref = orc.scan_bidir_chunked(a["q"], a["k"], a["v"], a["beta"], a["gamma"], L,
                                         s0=s0[b, h][None, None].astype(np.float64))
            o = host(res["o"][b, h])
            errs = {
                "fwd frame": frame_errs(host(res["states_fwd"][b, h]), ref["states_fwd"][0, 0]).max(),
                "rev frame": frame_errs(host(res["states_rev"][b, h]), ref["states_rev"][0, 0]).max(),
                "o frame": frame_errs(o, ref["o"][0, 0]).max(),
                "o token": token_errs(o, ref["o"][0, 0]).max(),
                "fin": rel_fro(host(res["s_final"][b, h]), ref["s_final"][0, 0]),
            }
            say(name, (b, h), errs)
            assert max(errs.values()) <= tol(w)


# --------------------------------------------------------------- compose
@pytest.mark.parametrize("name,w,offs", [
    ("tiny_f32_empty_chunk", gi.workload(1), [0, 3, 3, 8]),
    ("tiny_f32_one_chunk", gi.workload(1), [0, 8]),
    ("bf16_D128", gi.workload(4).with_shape(H=2, T=7, S=500), [0, 2, 5, 7]),
    # 64 (head, chunk) jobs: the compose launch with 64-row blocks, one chunk empty
    ("bf16_D128_H16_empty_chunk", gi.workload(4).with_shape(H=16, T=7, S=60), [0, 2, 2, 5, 7]),
])
def test_compose(name, w, offs):
    x, d = _gen(w)
    s0 = _s0(w)
    say("compose", name)
    res = gdn.gdn_compose(d["k"], d["v"], d["beta"], d["gamma"], offs, s0=torch.from_numpy(s0).to(DEV))
    torch.cuda.synchronize()
    for b in range(w.B):
        for h in range(w.H):
            a = head_arrays(x, b, h)
            C, Hc = orc.compose(a["k"], a["v"], a["beta"], a["gamma"], offs)
            st, _ = orc.combine(C, Hc, s0=s0[b, h][None, None].astype(np.float64))
            for p in range(len(offs) - 1):
                assert rel_fro(host(res["C"][b, h, p]), C[0, 0, p]) <= tol(w)
                if offs[p + 1] > offs[p]:
                    assert rel_fro(host(res["Hc"][b, h, p]), Hc[0, 0, p]) <= tol(w)
                else:
                    assert np.abs(host(res["Hc"][b, h, p])).max() == 0.0
                assert rel_fro(host(res["s_start"][b, h, p]), st[0, 0, p]) <= tol(w)


# ------------------------------------------------------------- edge cases
def test_no_frames_passes_state_through():
    w = gi.workload(1).with_shape(T=0, H=2)
    s0 = _s0(w)
    z = torch.zeros((1, 2, 0, 12, 16), device=DEV)
    say("T = 0")
    res = gdn.gdn_scan_fwd(z, z, z, torch.zeros((1, 2, 0, 12), device=DEV),
                           torch.zeros((1, 2, 0), device=DEV), s0=torch.from_numpy(s0).to(DEV))
    assert np.array_equal(host(res["s_final"]), s0.astype(np.float64))
    res0 = gdn.gdn_scan_fwd(z, z, z, torch.zeros((1, 2, 0, 12), device=DEV),
                            torch.zeros((1, 2, 0), device=DEV))
    assert host(res0["s_final"]).max() == 0.0 and host(res0["s_final"]).min() == 0.0


def test_single_frame_is_U():
    """T = 1 from zero: S_0 = U_0 and o = U_0 q, the same numbers gdn_frame_terms returns."""
    w = gi.workload(2).with_shape(T=1, S=900)
    x, d = _gen(w)
    say("T = 1")
    res = gdn.gdn_scan_fwd(d["q"], d["k"], d["v"], d["beta"], d["gamma"])
    _, U = gdn.gdn_frame_terms(d["k"], d["v"], d["beta"])
    assert torch.equal(res["states"][0, 0, 0], U[0, 0, 0])
    _check_fwd(w, x, res, None, [(0, 0)])


def test_deterministic():
    w = gi.workload(3).with_shape(H=4, T=4)
    x, d = _gen(w)
    say("determinism")
    r1 = gdn.gdn_scan_bidir_chunked(d["q"], d["k"], d["v"], d["beta"], d["gamma"], 2, n_time_chunks=2)
    r2 = gdn.gdn_scan_bidir_chunked(d["q"], d["k"], d["v"], d["beta"], d["gamma"], 2, n_time_chunks=2)
    for n in ("states_fwd", "states_rev", "s_final", "o"):
        assert torch.equal(r1[n], r2[n]), n


DEGENERATE_KINDS = ("beta_zero", "gates_off_on_odd_frames", "gamma_zero", "keys_nonpositive",
                    "beta_binary")


def _degenerate(x, w, kind):
    """One of the method's degenerate regimes, made in place from seeded inputs
    (float copies and, for bf16, the bit patterns the device gets)."""
    if kind == "beta_zero":                  # no writes: S_t = gamma_t S_{t-1}
        x["beta"][:] = 0.0
    elif kind == "gates_off_on_odd_frames":  # frames 1, 3, ... write nothing
        x["beta"][:, :, 1::2] = 0.0
    elif kind == "gamma_zero":               # no memory: S_t = U_t (R_t = U_t)
        x["gamma"][:] = 0.0
    elif kind == "keys_nonpositive":         # ReLU zeroes every key: A_t = U_t = 0
        x["k"][:] = -np.abs(x["k"])
        if w.io == "bf16":
            x["k_bits"] |= np.uint16(0x8000)
    elif kind == "beta_binary":              # every token written fully or not at all
        rng = np.random.default_rng([77, w.S])
        x["beta"][:] = (rng.random(x["beta"].shape) < 0.5).astype(np.float32)
    else:
        raise ValueError(kind)


@pytest.mark.parametrize("wname", ["bf16_D128", "f32_D16"])
@pytest.mark.parametrize("kind", DEGENERATE_KINDS)
def test_degenerate_inputs(kind, wname):
    """The degenerate regimes of the recurrence (P1 "混合线性注意力": M_t =
    gamma_t (I - A_t), U_t = V beta K_hat^T) on the MFMA path and on the fp32
    vector path: forward states and outputs (3 time chunks, with s0) and the
    chunk-causal scan (chunks of 2 frames) against the oracle at the usual bar;
    where the arithmetic makes them exact, A_t = U_t = 0 (no gate or no
    positive key) and S_t = R_t = U_t (gamma = 0), bit for bit."""
    w = (gi.workload(2).with_shape(H=2, T=6, S=300) if wname == "bf16_D128"
         else gi.workload(1).with_shape(T=6))
    x = gi.batch_inputs(w, 0)
    _degenerate(x, w, kind)
    d = upload(x, w)
    s0 = _s0(w)
    s0d = torch.from_numpy(s0).to(DEV)
    say("degenerate", kind, wname, "terms")
    A, U = gdn.gdn_frame_terms(d["k"], d["v"], d["beta"])
    say("degenerate", kind, wname, "forward, 3 time chunks")
    res = gdn.gdn_scan_fwd(d["q"], d["k"], d["v"], d["beta"], d["gamma"], s0=s0d, n_time_chunks=3)
    say("degenerate", kind, wname, "chunk-causal, chunks of 2")
    bid = gdn.gdn_scan_bidir_chunked(d["q"], d["k"], d["v"], d["beta"], d["gamma"], 2, s0=s0d,
                                     n_time_chunks=2)
    torch.cuda.synchronize()
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    _check_fwd(w, x, res, s0, heads, 3, f"degenerate {kind} {wname}")
    for (b, h) in heads:
        a = head_arrays(x, b, h)
        ref = orc.scan_bidir_chunked(a["q"], a["k"], a["v"], a["beta"], a["gamma"], 2,
                                     s0=s0[b, h][None, None].astype(np.float64))
        for n in ("states_fwd", "states_rev", "o"):
            assert frame_errs(host(bid[n][b, h]), ref[n][0, 0]).max() <= tol(w), n
    zero_frames = {"beta_zero": range(w.T), "keys_nonpositive": range(w.T),
                   "gates_off_on_odd_frames": range(1, w.T, 2)}.get(kind, ())
    for t in zero_frames:
        assert not A[:, :, t].any() and not U[:, :, t].any(), t
    if kind == "gamma_zero":
        assert torch.equal(res["states"], U)
        assert torch.equal(bid["states_fwd"], U) and torch.equal(bid["states_rev"], U)


@pytest.mark.parametrize("P", [1, 3])
def test_bidir_scans_sharing_a_launch_match_separate_scans(P):
    """The chunk-causal call runs its reverse scan in the same launch as the
    first forward one (the sequential scan, or the compose). Sharing the
    launch changes no arithmetic: the forward states equal gdn_scan_fwd's and
    the reverse states those of a call that wants only them (which runs the
    reverse scan alone), bit for bit."""
    w = gi.workload(5).with_shape(H=3, T=13, S=256)
    x, d = _gen(w)
    say("bidir with shared launch, P =", P)
    both = gdn.gdn_scan_bidir_chunked(d["q"], d["k"], d["v"], d["beta"], d["gamma"], 4,
                                      n_time_chunks=P)
    fwd = gdn.gdn_scan_fwd(d["q"], d["k"], d["v"], d["beta"], d["gamma"], n_time_chunks=P,
                           want_o=False)
    rev_only = gdn.gdn_scan_bidir_chunked(d["q"], d["k"], d["v"], d["beta"], d["gamma"], 4,
                                          n_time_chunks=P, want_o=False, want_s_final=False,
                                          want_states=False,
                                          states_rev=torch.empty_like(both["states_rev"]))
    assert rev_only["states_fwd"] is None
    torch.cuda.synchronize()
    assert torch.equal(both["states_fwd"], fwd["states"])
    assert torch.equal(both["s_final"], fwd["s_final"])
    assert torch.equal(both["states_rev"], rev_only["states_rev"])


# ------------------------------------------------------------ limits
def test_largest_chunk_counts():
    """The largest chunk counts the library takes, on one 720p-width head
    (D = 128, bf16) with 256 frames of 40 tokens: 256 composite time chunks of
    one frame each, a reverse scan restarted after every frame (256 chunks),
    explicit composites of 256 chunks, and the backward with 256 reverse
    chunks."""
    w = gi.workload(2).with_shape(T=256, S=40)
    x, d = _gen(w)
    say("256 time chunks")
    r256 = gdn.gdn_scan_fwd(d["q"], d["k"], d["v"], d["beta"], d["gamma"], n_time_chunks=256)
    seq = gdn.gdn_scan_fwd(d["q"], d["k"], d["v"], d["beta"], d["gamma"], n_time_chunks=1)
    torch.cuda.synchronize()
    _check_fwd(w, x, r256, None, [(0, 0)], P=256, what="P = 256")
    assert rel_fro(host(r256["states"]), host(seq["states"])) <= 1e-4
    say("reverse scan restarted after every frame")
    bid = gdn.gdn_scan_bidir_chunked(d["q"], d["k"], d["v"], d["beta"], d["gamma"], 1,
                                     n_time_chunks=256)
    _, U = gdn.gdn_frame_terms(d["k"], d["v"], d["beta"])
    torch.cuda.synchronize()
    assert torch.equal(bid["states_rev"], U)  # one frame from a zero state: R_t = U_t
    assert torch.equal(bid["states_fwd"], r256["states"])
    say("composites of 256 chunks")
    comp = gdn.gdn_compose(d["k"], d["v"], d["beta"], d["gamma"], list(range(257)))
    torch.cuda.synchronize()
    # chunk p is frame p alone: H_p = U_p, and s_start[p + 1] is the state after frame p
    assert torch.equal(comp["Hc"], U)
    assert rel_fro(host(comp["s_start"][0, 0, 1:]), host(seq["states"][0, 0, :-1])) <= 1e-4
    say("backward with 256 reverse chunks")
    do, do_d, s0, dsf = _bwd_inputs(w, x, d, True)
    dev = lambda a: torch.from_numpy(a).to(DEV)
    fb = gdn.gdn_scan_bidir_chunked(d["q"], d["k"], d["v"], d["beta"], d["gamma"], 1,
                                    s0=dev(s0), n_time_chunks=256, want_o=False)
    g = gdn.gdn_scan_bidir_chunked_bwd(d["q"], d["k"], d["v"], d["beta"], d["gamma"], 1,
                                       fb["states_fwd"], fb["states_rev"], do_d, s0=dev(s0),
                                       ds_final=dev(dsf))
    torch.cuda.synchronize()
    a = head_arrays(x, 0, 0)
    ref = orc.scan_bidir_bwd(a["q"], a["k"], a["v"], a["beta"], a["gamma"], 1,
                             do[0, 0][None, None].astype(np.float64),
                             ds_final=dsf[0, 0][None, None].astype(np.float64),
                             s0=s0[0, 0][None, None].astype(np.float64))
    _check_grads(w, g, ref, 0, 0, ("256 reverse chunks",))


def test_long_frame():
    """A frame of 40,000 tokens (11 times a 720p frame; 1250 token tiles of
    phase 1, ragged against the readout's tiles): frame terms, states and
    outputs of a 2-frame scan against the oracle."""
    w = gi.workload(2).with_shape(T=2, S=40000)
    x, d = _gen(w)
    say("S = 40000")
    res = gdn.gdn_scan_fwd(d["q"], d["k"], d["v"], d["beta"], d["gamma"])
    A, U = gdn.gdn_frame_terms(d["k"], d["v"], d["beta"])
    torch.cuda.synchronize()
    kh = orc.prepare_keys(x["k"][0, 0])
    for t in range(w.T):
        Ar, Ur = orc.frame_terms(kh[t], x["v"][0, 0, t], x["beta"][0, 0, t])
        assert rel_fro(host(A[0, 0, t]), Ar) <= tol(w)
        assert rel_fro(host(U[0, 0, t]), Ur) <= tol(w)
    _check_fwd(w, x, res, None, [(0, 0)], what="S = 40000")


@pytest.mark.parametrize("mode", ["causal", "chunk_causal"])
def test_offsets_beyond_32_bits(mode):
    """Three 60 s 720p layers in one call (B = 3, H = 16, T = 121, S = 3600,
    bf16; 2.68e9 elements per token tensor): the last batch's heads start
    beyond 2^31 elements and 2^32 bytes, where an offset held in 32 bits
    anywhere in a kernel would wrap. Forward in the benchmark's launch
    configuration (8 time chunks; chunk-causal: chunks of 10 frames) and the
    backward; states, outputs and every gradient of the first and the last
    head against the oracle. The two heads carry the workload's seeded
    inputs, the others seeded device draws."""
    w = gi.workload(4 if mode == "causal" else 5).with_shape(B=3)
    heads = [(0, 0), (w.B - 1, w.H - 1)]
    shp = (w.B, w.H, w.T, w.S, w.D)
    per_head = w.T * w.S * w.D
    assert (w.B * w.H - 1) * per_head > 2**31 and 2 * (w.B * w.H - 1) * per_head > 2**32
    gen = torch.Generator(device=DEV)
    gen.manual_seed(2024)
    say("generate", w.name, "B = 3")
    d = {}
    for n in ("q", "k", "v", "do"):
        d[n] = torch.empty(shp, dtype=torch.bfloat16, device=DEV)
        for b in range(w.B):
            d[n][b] = torch.randn(shp[1:], generator=gen, device=DEV)
    d["beta"] = torch.rand(shp[:4], generator=gen, device=DEV)
    d["gamma"] = w.gamma_lo + (1.0 - w.gamma_lo) * torch.rand(shp[:3], generator=gen, device=DEV)
    xs = {}
    for (b, h) in heads:
        xh = gi.head_inputs(w, 0, b, h)
        for n in ("q", "k", "v"):
            d[n][b, h] = bits_to_dev(xh[n + "_bits"])
        for n in ("beta", "gamma"):
            d[n][b, h] = torch.from_numpy(xh[n]).to(DEV)
        xs[(b, h)] = xh
    L = w.chunk_len
    args = (d["q"], d["k"], d["v"], d["beta"], d["gamma"])
    say("forward", w.name, "B = 3")
    if L:
        fwd = gdn.gdn_scan_bidir_chunked(*args, L, n_time_chunks=w.time_chunks)
        say("backward", w.name, "B = 3")
        g = gdn.gdn_scan_bidir_chunked_bwd(*args, L, fwd["states_fwd"], fwd["states_rev"], d["do"])
        names = ("states_fwd", "states_rev", "o")
    else:
        fwd = gdn.gdn_scan_fwd(*args, n_time_chunks=w.time_chunks)
        say("backward", w.name, "B = 3")
        g = gdn.gdn_scan_bwd(*args, fwd["states"], d["do"])
        names = ("states", "o")
    torch.cuda.synchronize()
    for (b, h) in heads:
        xh = xs[(b, h)]
        a = [np.asarray(xh[n], dtype=np.float64)[None, None] for n in ("q", "k", "v", "beta", "gamma")]
        dob = host(d["do"][b, h])[None, None]
        if L:
            ref = orc.scan_bidir_chunked(*a, L)
            gref = orc.scan_bidir_bwd(*a, L, dob)
        else:
            ref = orc.scan_fwd(*a)
            gref = orc.scan_fwd_bwd(*a, dob)
        errs = {n + " frame": float(frame_errs(host(fwd[n][b, h]), ref[n][0, 0]).max())
                for n in names}
        errs["o token"] = float(token_errs(host(fwd["o"][b, h]), ref["o"][0, 0]).max())
        errs["s_final"] = rel_fro(host(fwd["s_final"][b, h]), ref["s_final"][0, 0])
        errs.update(_grad_errs(g, gref, b, h))
        say(w.name, "B = 3", (b, h), {n: f"{e:.2e}" for n, e in errs.items()})
        assert max(errs.values()) <= tol(w), ((b, h), errs)
    del d, fwd, g
    torch.cuda.empty_cache()


# ---------------------------------------------------- readout alone, trace
READOUT_CASES = {
    # name: (workload, with a second state, RMSNorm of q)
    "bf16_D128_ragged_S1000": (gi.workload(2).with_shape(H=2, T=3, S=1000), False, False),
    "bf16_D128_two_states": (gi.workload(2).with_shape(H=2, T=3, S=1000), True, False),
    "bf16_D128_two_states_norm": (gi.workload(2).with_shape(H=2, T=3, S=1000), True, True),
    # two frame-heads: up to 16 workgroups per frame-head, ragged against their tiles
    "bf16_D128_two_frame_heads_S300": (gi.workload(2).with_shape(T=2, S=300), False, False),
    "bf16_D64_norm": (gi.workload(2).with_shape(D=64, T=2, S=130), False, True),
    "f32_D16_two_states": (gi.workload(1), True, False),
}


@pytest.mark.parametrize("name", sorted(READOUT_CASES))
def test_readout_alone(name):
    """gdn_readout (phase 3 alone) on given fp32 states against the oracle's
    readout o = (S_t [+ R_t]) q (with q RMS-normalised when flagged), per frame
    and per token; and bitwise the output gdn_scan_fwd forms from the same
    states."""
    w, two, norm = READOUT_CASES[name]
    x, d = _gen(w)
    rng = np.random.default_rng([66, w.S])
    shp = (w.B, w.H, w.T, w.D, w.D)
    st = (0.05 * rng.standard_normal(shp)).astype(np.float32)
    st2 = (0.05 * rng.standard_normal(shp)).astype(np.float32) if two else None
    dev = lambda a: None if a is None else torch.from_numpy(a).to(DEV)
    say("readout", name)
    o = gdn.gdn_readout(d["q"], dev(st), dev(st2), qk_rmsnorm=norm)
    torch.cuda.synchronize()
    for b in range(w.B):
        for h in range(w.H):
            qh = np.asarray(x["q"][b, h], dtype=np.float64)
            qn = orc.rms_norm(qh) if norm else qh
            ssum = st[b, h].astype(np.float64) + (0.0 if st2 is None else st2[b, h].astype(np.float64))
            ref = np.stack([orc.readout(ssum[t], qn[t]) for t in range(w.T)])
            got = host(o[b, h])
            e = max(frame_errs(got, ref).max(), token_errs(got, ref).max())
            say(name, (b, h), f"{e:.2e}")
            assert e <= tol(w), ((b, h), e)
    say("readout", name, "against the scan's own readout")
    res = gdn.gdn_scan_fwd(d["q"], d["k"], d["v"], d["beta"], d["gamma"], qk_rmsnorm=norm)
    o2 = gdn.gdn_readout(d["q"], res["states"], qk_rmsnorm=norm)
    torch.cuda.synchronize()
    assert torch.equal(o2, res["o"])


def test_phase_trace():
    """gdn_trace_set on the GPU: a traced forward call with composites records a
    call-begin event and one event per launch group (phase 1, composites,
    combine, replay, readout), whose device times add up to the call's total;
    a call that fails its argument checks records nothing; a full trace drops
    further marks and the call's results are unchanged; after the trace is
    cleared nothing is recorded."""
    w = gi.workload(2).with_shape(H=2, T=6, S=700)
    x, d = _gen(w)
    args = (d["q"], d["k"], d["v"], d["beta"], d["gamma"])
    say("trace: untraced reference call")
    ref = gdn.gdn_scan_fwd(*args, n_time_chunks=3)
    tr = gdn.PhaseTrace(64)
    with tr:
        say("trace: traced call")
        res = gdn.gdn_scan_fwd(*args, n_time_chunks=3)
        torch.cuda.synchronize()
        n = tr.count
        bad = gdn.make_desc(1, 2, 6, 700, 0, gdn.GDN_BF16)  # D = 0: rejected before any launch
        assert gdn.lib().gdn_readout(ctypes.byref(bad), d["q"].data_ptr(), res["states"].data_ptr(),
                                     None, res["o"].data_ptr(), None) == gdn.GDN_EINVAL
        assert tr.count == n
    calls = tr.calls()
    assert len(calls) == 1, calls
    c = calls[0]
    assert set(c) == {"terms", "scan", "combine", "replay", "readout", "total"}, c
    assert min(c.values()) >= 0.0 and c["total"] > 0.0, c
    parts = sum(v for k, v in c.items() if k != "total")
    assert abs(parts - c["total"]) <= 1e-3 * c["total"] + 1e-3, c
    for k in ("states", "s_final", "o"):
        assert torch.equal(res[k], ref[k]), k
    say("trace: a full trace")
    small = gdn.PhaseTrace(3)
    with small:
        res3 = gdn.gdn_scan_fwd(*args, n_time_chunks=3)
        torch.cuda.synchronize()
    assert small.count == 3 and small.full()
    assert torch.equal(res3["o"], ref["o"])
    say("trace: cleared")
    gdn.gdn_scan_fwd(*args, n_time_chunks=3)
    torch.cuda.synchronize()
    assert tr.count == n and small.count == 3
    tr.close()
    small.close()


# ---------------------------------------------- full-size named workloads
def _full(idx, seed=0):
    w = gi.workload(idx)
    say("generate", w.name, "seed", seed)
    x = gi.batch_inputs(w, seed, threads=16, keep_f32=False)
    return w, x, upload(x, w)


def _oracle_head(w, x, b, h):
    """The oracle on one head of a full-size workload (float64 inputs from the
    stored bf16 bit patterns)."""
    a = {n: gi.bf16_bits_to_f32(x[n + "_bits"][b, h]).astype(np.float64)[None, None]
         for n in ("q", "k", "v")}
    for n in ("beta", "gamma"):
        a[n] = np.asarray(x[n][b, h], dtype=np.float64)[None, None]
    if w.mode == "bidir":
        return orc.scan_bidir_chunked(a["q"], a["k"], a["v"], a["beta"], a["gamma"], w.chunk_len)
    return orc.scan_fwd(a["q"], a["k"], a["v"], a["beta"], a["gamma"])


def _run_workload(w, d):
    if w.mode == "bidir":
        return gdn.gdn_scan_bidir_chunked(d["q"], d["k"], d["v"], d["beta"], d["gamma"], w.chunk_len,
                                          n_time_chunks=w.time_chunks)
    return gdn.gdn_scan_fwd(d["q"], d["k"], d["v"], d["beta"], d["gamma"],
                            n_time_chunks=w.time_chunks)


@pytest.mark.parametrize("idx,seed", [(2, 0), (2, 1), (2, 2), (3, 0), (4, 0), (5, 0)])
def test_named_workload_full_size(idx, seed):
    """The named workloads at full size in the launch configuration the
    benchmark times, every head against the oracle: the relative Frobenius
    error of every frame of the states (both directions for the chunk-causal
    scan) and of the outputs, of every token's output vector and of the final
    state, each within the bar (seeds 1 and 2 as spot checks on the one-head
    workload)."""
    w, x, d = _full(idx, seed)
    say("run", w.name)
    res = _run_workload(w, d)
    torch.cuda.synchronize()
    if w.mode == "bidir":
        frames = [("states_fwd", "states_fwd"), ("states_rev", "states_rev"), ("o", "o")]
    else:
        frames = [("states", "states"), ("o", "o")]
    worst = {}
    for b in range(w.B):
        for h in range(w.H):
            ref = _oracle_head(w, x, b, h)
            errs = {}
            for g, r in frames:
                fe = frame_errs(host(res[g][b, h]), ref[r][0, 0])
                errs[g + " frame"] = (float(fe.max()), int(fe.argmax()))
            te = token_errs(host(res["o"][b, h]), ref["o"][0, 0])
            errs["o token"] = (float(te.max()), int(te.argmax()))
            errs["s_final"] = (rel_fro(host(res["s_final"][b, h]), ref["s_final"][0, 0]), 0)
            say(w.name, (b, h), {k: f"{v[0]:.2e}@{v[1]}" for k, v in errs.items()})
            for k, v in errs.items():
                if v[0] > worst.get(k, (-1.0,))[0]:
                    worst[k] = (v[0], (b, h, v[1]))
            assert max(v[0] for v in errs.values()) <= tol(w), ((b, h), errs)
    say(w.name, "seed", seed, "largest errors (value, (b, h, frame or flat token)):", worst)
    if w.time_chunks > 1:
        # composite route versus the sequential scan on every head (same terms)
        say("sequential vs composite", w.name)
        key = "states_fwd" if w.mode == "bidir" else "states"
        seq = _run_workload(w.with_shape(time_chunks=1), d)
        torch.cuda.synchronize()
        for h in range(w.H):
            e = frame_errs(host(res[key][0, h]), host(seq[key][0, h])).max()
            say(w.name, "composite vs sequential, max per frame", h, f"{e:.2e}")
            assert e <= 1e-4, (h, e)
            if w.mode == "bidir":
                assert torch.equal(res["states_rev"][0, h], seq["states_rev"][0, h])


# ------------------------------------------------------------ graph capture
def test_graph_capture_replays():
    """The library allocates nothing and clears memory with kernels, so its
    calls can be captured in a HIP graph: a captured forward scan (composites)
    and a captured backward, replayed several times with eager work and
    synchronisations in between, give bit-identical results to eager calls."""
    w = gi.workload(2).with_shape(H=2, T=9, S=300)
    x, d = _gen(w)
    dev = lambda a: torch.from_numpy(a).to(DEV)
    s0 = dev(_s0(w))
    do, do_d, _, dsf = _bwd_inputs(w, x, d, True)
    dsf = dev(dsf)
    B, H, T, S, D = w.B, w.H, w.T, w.S, w.D
    desc = gdn.make_desc(B, H, T, S, D, gdn.GDN_BF16)
    ws = gdn.workspace(desc, 3, DEV)
    bws = torch.empty(gdn.gdn_bwd_workspace_bytes(desc), dtype=torch.uint8, device=DEV)
    st = torch.empty((B, H, T, D, D), device=DEV)
    sf = torch.empty((B, H, D, D), device=DEV)
    o = torch.empty_like(d["q"])
    gout = {n: torch.empty_like(d["q"]) for n in ("dq", "dk", "dv")}
    gout["dbeta"] = torch.empty_like(d["beta"])
    gout["dgamma"] = torch.empty_like(d["gamma"])
    gout["ds0"] = torch.empty_like(sf)

    def call():
        gdn.gdn_scan_fwd(d["q"], d["k"], d["v"], d["beta"], d["gamma"], s0=s0, n_time_chunks=3,
                         states=st, s_final=sf, o=o, ws=ws)
        gdn.gdn_scan_bwd(d["q"], d["k"], d["v"], d["beta"], d["gamma"], st, do_d, s0=s0,
                         ds_final=dsf, out=gout, ws=bws)

    say("graph capture: eager reference")
    call()
    torch.cuda.synchronize()
    ref = {"states": st.clone(), "s_final": sf.clone(), "o": o.clone()}
    ref.update({n: t.clone() for n, t in gout.items()})
    say("graph capture: capture")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()
    outs = {"states": st, "s_final": sf, "o": o, **gout}
    for rep in range(3):
        for t in outs.values():  # eager work between the replays
            t.fill_(float("nan")) if t.dtype.is_floating_point else t.zero_()
        torch.cuda.synchronize()
        say("graph capture: replay", rep)
        graph.replay()
        torch.cuda.synchronize()
        for n, t in outs.items():
            assert torch.equal(t, ref[n]), (rep, n)


# ------------------------------------------------------- batch invariance
@pytest.mark.parametrize("mode", ["fwd", "bidir"])
def test_batch_invariance_bitwise(mode):
    """A head's results do not depend on the batch it is launched with: a
    large call (B=2, H=3, FH=1200) and calls on single heads sliced out of it
    give bit-identical states, final states and outputs; the large call also
    matches the oracle."""
    w = gi.workload(3).with_shape(B=2, H=3, T=200, S=64)
    x, d = _gen(w)
    s0 = _s0(w)
    s0d = torch.from_numpy(s0).to(DEV)

    def run(q, k, v, beta, gamma, s0_):
        if mode == "bidir":
            return gdn.gdn_scan_bidir_chunked(q, k, v, beta, gamma, 7, s0=s0_, n_time_chunks=3)
        return gdn.gdn_scan_fwd(q, k, v, beta, gamma, s0=s0_, n_time_chunks=4)

    say("batch invariance", mode, "full batch")
    full = run(d["q"], d["k"], d["v"], d["beta"], d["gamma"], s0d)
    torch.cuda.synchronize()
    for (b, h) in [(0, 0), (1, 2)]:
        say("batch invariance", mode, "head", (b, h))
        one = run(*(d[n][b:b + 1, h:h + 1].contiguous() for n in ("q", "k", "v", "beta", "gamma")),
                  s0d[b:b + 1, h:h + 1].contiguous())
        torch.cuda.synchronize()
        for n, t in one.items():
            assert torch.equal(t[0, 0], full[n][b, h]), (b, h, n)
    b, h = 1, 2
    a = head_arrays(x, b, h)
    s0h = s0[b, h][None, None].astype(np.float64)
    if mode == "bidir":
        ref = orc.scan_bidir_chunked(a["q"], a["k"], a["v"], a["beta"], a["gamma"], 7, s0=s0h)
        names = ("states_fwd", "states_rev", "s_final", "o")
    else:
        ref = orc.scan_fwd(a["q"], a["k"], a["v"], a["beta"], a["gamma"], s0=s0h)
        names = ("states", "s_final", "o")
    for n in names:
        e = rel_fro(host(full[n][b, h]), ref[n][0, 0])
        say(mode, n, f"{e:.2e}")
        assert e <= tol(w), (n, e)


# ------------------------------------------------------ streaming chunk step
def test_streaming_step_chain_equals_chunk_causal_scan():
    """gdn_step over consecutive 3-frame blocks (the last one short), with the
    forward state carried in place from block to block, reproduces the
    chunk-causal bidirectional scan with chunk_len = 3 bit for bit, and the
    oracle within the bf16 bar."""
    w = gi.workload(5).with_shape(H=2, T=31, S=200)
    x, d = _gen(w)
    L = 3
    say("step chain: one-shot chunk-causal scan")
    ref = gdn.gdn_scan_bidir_chunked(d["q"], d["k"], d["v"], d["beta"], d["gamma"], L)
    carry = torch.zeros((w.B, w.H, w.D, w.D), dtype=torch.float32, device=DEV)
    outs, fwd, rev = [], [], []
    for a in range(0, w.T, L):
        b = min(a + L, w.T)
        say("step chain: block", a, b)
        blk = {n: d[n][:, :, a:b].contiguous() for n in ("q", "k", "v", "beta", "gamma")}
        r = gdn.gdn_step(blk["q"], blk["k"], blk["v"], blk["beta"], blk["gamma"], carry_in=carry,
                         carry_out=carry, want_states=True)
        outs.append(r["o"])
        fwd.append(r["states_fwd"])
        rev.append(r["states_rev"])
    torch.cuda.synchronize()
    assert torch.equal(torch.cat(outs, dim=2), ref["o"])
    assert torch.equal(torch.cat(fwd, dim=2), ref["states_fwd"])
    assert torch.equal(torch.cat(rev, dim=2), ref["states_rev"])
    assert torch.equal(carry, ref["s_final"])
    a = head_arrays(x, 0, 1)
    orc_ref = orc.scan_bidir_chunked(a["q"], a["k"], a["v"], a["beta"], a["gamma"], L)
    for n in ("o", "states_fwd", "states_rev"):
        e = rel_fro(host(torch.cat({"o": outs, "states_fwd": fwd, "states_rev": rev}[n], dim=2)[0, 1]),
                    orc_ref[n][0, 0])
        say("step chain vs oracle", n, f"{e:.2e}")
        assert e <= tol(w), (n, e)


def test_streaming_step_full_size():
    """gdn_step as the benchmark streams the 60 s 720p layer (16 heads,
    S = 3600, 3-frame blocks; each block's phase 1 split over its tokens),
    chained over the first 4 blocks with the forward state carried in place:
    every head's outputs, forward and reverse states (per frame and per token)
    and the carry against the oracle's chunk-causal scan with chunk_len = 3."""
    L = 3
    w = gi.workload(4).with_shape(T=4 * L, time_chunks=1)
    x, d = _gen(w, seed=3)
    carry = torch.zeros((w.B, w.H, w.D, w.D), dtype=torch.float32, device=DEV)
    outs, fwd, rev = [], [], []
    for a in range(0, w.T, L):
        say("streaming full size: block", a, a + L)
        blk = {n: d[n][:, :, a:a + L].contiguous() for n in ("q", "k", "v", "beta", "gamma")}
        r = gdn.gdn_step(blk["q"], blk["k"], blk["v"], blk["beta"], blk["gamma"], carry_in=carry,
                         carry_out=carry, want_states=True)
        outs.append(r["o"])
        fwd.append(r["states_fwd"])
        rev.append(r["states_rev"])
    torch.cuda.synchronize()
    got = {"o": torch.cat(outs, dim=2), "states_fwd": torch.cat(fwd, dim=2),
           "states_rev": torch.cat(rev, dim=2)}
    for h in range(w.H):
        a = head_arrays(x, 0, h)
        ref = orc.scan_bidir_chunked(a["q"], a["k"], a["v"], a["beta"], a["gamma"], L)
        errs = {n: float(frame_errs(host(got[n][0, h]), ref[n][0, 0]).max())
                for n in ("o", "states_fwd", "states_rev")}
        errs["o token"] = float(token_errs(host(got["o"][0, h]), ref["o"][0, 0]).max())
        errs["carry"] = rel_fro(host(carry[0, h]), ref["s_final"][0, 0])
        say("streaming full size, head", h, {k: f"{v:.2e}" for k, v in errs.items()})
        assert max(errs.values()) <= tol(w), (h, errs)


# ------------------------------------------------------ fused q/k RMSNorm
def _gen_rescaled(w, seed=0):
    """Seeded inputs whose q and k tokens are rescaled by factors in
    [0.2, 5] (then rounded to the io dtype again), so that a missing or wrong
    per-token normalisation changes the result far beyond the bar."""
    x = gi.batch_inputs(w, seed)
    rng = np.random.default_rng([77, seed])
    for n in ("q", "k"):
        fac = rng.uniform(0.2, 5.0, x[n].shape[:-1] + (1,)).astype(np.float32)
        val = x[n] * fac
        if w.io == "bf16":
            x[n + "_bits"] = gi.f32_to_bf16_bits(val)
            x[n] = gi.bf16_bits_to_f32(x[n + "_bits"])
        else:
            x[n] = val.astype(np.float32)
    return x, upload(x, w)


@pytest.mark.parametrize("io,D", [("bf16", 16), ("bf16", 128), ("f32", 16), ("f32", 128)])
def test_prepare_rmsnorm(io, D):
    w = gi.workload(2).with_shape(T=2, S=77, D=D, io=io)
    x, d = _gen_rescaled(w)
    say("prepare rmsnorm", io, D)
    kh = host(gdn.gdn_prepare(d["k"], qk_rmsnorm=True))
    torch.cuda.synchronize()
    ref = orc.prepare_keys(x["k"], rmsnorm=True)
    assert (kh[ref == 0.0] == 0.0).all()
    rel = np.abs(kh - ref) / np.maximum(np.abs(ref), 1e-300)
    # bf16: one rounding of an fp32 value (2^-9) plus fp32 arithmetic; fp32: the
    # fp32 sum of squares (a few ulp), sqrt, reciprocal and two products
    bound = 2.0 ** -8 if io == "bf16" else 3e-6
    assert rel[ref != 0].max() <= bound * 1.01, rel[ref != 0].max()


RMS_CASES = {
    # name: (workload, mode, P or chunk_len, keys_prepared)
    "bf16_D128_fwd_P2": (gi.workload(2).with_shape(H=2, T=5, S=700), "fwd", 2, False),
    "bf16_D128_bidir_L2": (gi.workload(5).with_shape(H=2, T=5, S=600), "bidir", 2, False),
    "bf16_D128_split_S2100": (gi.workload(2).with_shape(T=2, S=2100), "fwd", 1, False),
    "bf16_D64_fwd": (gi.workload(2).with_shape(D=64, T=4, S=130), "fwd", 1, False),
    "f32_D16_fwd_P2": (gi.workload(1), "fwd", 2, False),
    "f32_D128_bidir_L3": (gi.workload(1).with_shape(D=128, S=60, T=4), "bidir", 3, False),
    "bf16_D128_prepared_keys": (gi.workload(2).with_shape(T=3, S=300), "fwd", 1, True),
}


@pytest.mark.parametrize("name", sorted(RMS_CASES))
def test_scan_rmsnorm(name):
    """GDN_QK_RMSNORM fused into phase 1 (keys) and the readout (queries)."""
    w, mode, par, prepared = RMS_CASES[name]
    x, d = _gen_rescaled(w)
    if prepared:
        # keys given as K_hat (normalised, ReLU'd and scaled by the oracle);
        # the flag then normalises q only
        kh = orc.prepare_keys(x["k"], rmsnorm=True)
        if w.io == "bf16":
            bits = gi.f32_to_bf16_bits(kh.astype(np.float32))
            x["k"] = gi.bf16_bits_to_f32(bits)
            d["k"] = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(DEV)
        else:
            x["k"] = kh.astype(np.float32)
            d["k"] = torch.from_numpy(x["k"]).to(DEV)
    say("scan rmsnorm", name)
    if mode == "bidir":
        res = gdn.gdn_scan_bidir_chunked(d["q"], d["k"], d["v"], d["beta"], d["gamma"], par,
                                         keys_prepared=prepared, qk_rmsnorm=True)
    else:
        res = gdn.gdn_scan_fwd(d["q"], d["k"], d["v"], d["beta"], d["gamma"], n_time_chunks=par,
                               keys_prepared=prepared, qk_rmsnorm=True)
    torch.cuda.synchronize()
    for (b, h) in [(0, w.H - 1)]:
        a = head_arrays(x, b, h)
        if mode == "bidir":
            ref = orc.scan_bidir_chunked(a["q"], a["k"], a["v"], a["beta"], a["gamma"], par,
                                         keys_prepared=prepared, qk_rmsnorm=True)
            names = ("states_fwd", "states_rev", "o")
        else:
            ref = orc.scan_fwd(a["q"], a["k"], a["v"], a["beta"], a["gamma"],
                               keys_prepared=prepared, qk_rmsnorm=True)
            names = ("states", "s_final", "o")
        for n in names:
            got = host(res[n][b, h])
            e = rel_fro(got, ref[n][0, 0]) if n == "s_final" else frame_errs(got, ref[n][0, 0]).max()
            if n == "o":
                e = max(e, token_errs(got, ref[n][0, 0]).max())
            say(name, n, f"{e:.2e}")
            assert e <= tol(w), (n, e)


def test_frame_terms_rmsnorm():
    w = gi.workload(2).with_shape(H=2, T=2, S=1000)
    x, d = _gen_rescaled(w)
    say("frame terms rmsnorm")
    A, U = gdn.gdn_frame_terms(d["k"], d["v"], d["beta"], qk_rmsnorm=True)
    torch.cuda.synchronize()
    kh = orc.prepare_keys(x["k"][0, 1], rmsnorm=True)
    for t in range(w.T):
        Ar, Ur = orc.frame_terms(kh[t], x["v"][0, 1, t], x["beta"][0, 1, t])
        assert rel_fro(host(A[0, 1, t]), Ar) <= tol(w)
        assert rel_fro(host(U[0, 1, t]), Ur) <= tol(w)


# --------------------------------------------------------------- backward
def _grad_errs(g, ref, b, h):
    """Errors of one head's gradients against the oracle's: dq, dk, dv per
    token (every token of every frame, the last token of each frame
    included) and per frame, dbeta per frame, dgamma and ds0 whole."""
    errs = {}
    for n in ("dq", "dk", "dv"):
        if g.get(n) is None:
            continue
        got = host(g[n][b, h])
        errs[n + " token"] = float(token_errs(got, ref[n][0, 0]).max())
        errs[n + " frame"] = float(frame_errs(got, ref[n][0, 0]).max())
    if g.get("dbeta") is not None:
        errs["dbeta frame"] = float(frame_errs(host(g["dbeta"][b, h]), ref["dbeta"][0, 0]).max())
    for n in ("dgamma", "ds0"):
        if g.get(n) is not None:
            errs[n] = rel_fro(host(g[n][b, h]), ref[n][0, 0])
    return errs


def _check_grads(w, g, ref, b, h, what):
    errs = _grad_errs(g, ref, b, h)
    say(what, (b, h), {k: f"{v:.2e}" for k, v in errs.items()})
    assert max(errs.values()) <= tol(w), ((b, h), errs)


BWD_CASES = {
    # name: (workload, with s0 / ds_final, keys_prepared)
    "f32_D16_s0_dsf": (gi.workload(1), True, False),
    "f32_D16_plain": (gi.workload(1).with_shape(B=2, H=2), False, False),
    "bf16_D128_s0_dsf": (gi.workload(2).with_shape(H=2, T=6, S=300), True, False),
    "bf16_D128_split_S2100": (gi.workload(2).with_shape(T=3, S=2100), True, False),
    "bf16_D64": (gi.workload(2).with_shape(D=64, T=5, S=130), True, False),
    "f32_D128_prepared": (gi.workload(1).with_shape(D=128, S=40, T=4), True, True),
    "bf16_D128_prepared": (gi.workload(2).with_shape(H=2, T=4, S=170), True, True),
    # frames shorter than one 32-token stage (every row past the end is a
    # clamped copy of the last one), a single frame, a single token
    "bf16_D128_S5": (gi.workload(2).with_shape(H=2, T=3, S=5), True, False),
    "bf16_D128_T1_S33": (gi.workload(2).with_shape(H=2, T=1, S=33), True, False),
    "bf16_D128_S1": (gi.workload(2).with_shape(T=2, S=1), True, False),
}


def _bwd_inputs(w, x, d, extras, seed=5):
    rng = np.random.default_rng([88, seed])
    do = rng.standard_normal((w.B, w.H, w.T, w.S, w.D)).astype(np.float32)
    if w.io == "bf16":
        do_bits = gi.f32_to_bf16_bits(do)
        do = gi.bf16_bits_to_f32(do_bits)
        do_d = torch.from_numpy(do_bits.view(np.int16)).view(torch.bfloat16).to(DEV)
    else:
        do_d = torch.from_numpy(do).to(DEV)
    s0 = dsf = None
    if extras:
        s0 = (0.5 * rng.standard_normal((w.B, w.H, w.D, w.D))).astype(np.float32)
        dsf = rng.standard_normal((w.B, w.H, w.D, w.D)).astype(np.float32)
    return do, do_d, s0, dsf


@pytest.mark.parametrize("name", sorted(BWD_CASES))
def test_scan_bwd(name):
    """Gradients of L = <do, o> + <ds_final, S_T-1> through the whole path
    (phase 1, adjoint scan, per-frame and per-token kernels) against the
    float64 oracle's reverse-mode gradients, per head."""
    w, extras, prepared = BWD_CASES[name]
    x, d = _gen(w)
    if prepared:
        kh = orc.prepare_keys(x["k"]).astype(np.float32)
        if w.io == "bf16":  # both sides take the bf16-rounded prepared keys
            bits = gi.f32_to_bf16_bits(kh)
            kh = gi.bf16_bits_to_f32(bits)
            d["k"] = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(DEV)
        else:
            d["k"] = torch.from_numpy(kh).to(DEV)
        x["k"] = kh
    do, do_d, s0, dsf = _bwd_inputs(w, x, d, extras)
    dev = lambda a: None if a is None else torch.from_numpy(a).to(DEV)
    say("scan_bwd", name, "forward")
    fwd = gdn.gdn_scan_fwd(d["q"], d["k"], d["v"], d["beta"], d["gamma"], s0=dev(s0),
                           keys_prepared=prepared, want_o=False)
    say("scan_bwd", name, "backward")
    g = gdn.gdn_scan_bwd(d["q"], d["k"], d["v"], d["beta"], d["gamma"], fwd["states"], do_d,
                         s0=dev(s0), ds_final=dev(dsf), keys_prepared=prepared)
    torch.cuda.synchronize()
    for (b, h) in [(0, 0), (w.B - 1, w.H - 1)]:
        a = head_arrays(x, b, h)
        ref = orc.scan_fwd_bwd(a["q"], a["k"], a["v"], a["beta"], a["gamma"],
                               do[b, h][None, None].astype(np.float64),
                               ds_final=None if dsf is None else dsf[b, h][None, None].astype(np.float64),
                               s0=None if s0 is None else s0[b, h][None, None].astype(np.float64),
                               keys_prepared=prepared)
        _check_grads(w, g, ref, b, h, (name,))


def test_scan_bwd_fused_dq_pass_matches_separate_passes():
    """With dq wanted, E_t and dq come from one pass over q and d_o; without
    it, E_t comes from the plain phase-1 pass. Both form E_t from the same
    bf16 operands in the same order, so every other gradient is bitwise
    equal; dq itself is checked against the oracle in test_scan_bwd."""
    w = gi.workload(2).with_shape(H=2, T=5, S=333)
    x, d = _gen(w)
    do, do_d, s0, dsf = _bwd_inputs(w, x, d, True)
    dev = lambda a: torch.from_numpy(a).to(DEV)
    say("scan_bwd fused vs separate E")
    fwd = gdn.gdn_scan_fwd(d["q"], d["k"], d["v"], d["beta"], d["gamma"], s0=dev(s0), want_o=False)
    full = gdn.gdn_scan_bwd(d["q"], d["k"], d["v"], d["beta"], d["gamma"], fwd["states"], do_d,
                            s0=dev(s0), ds_final=dev(dsf))
    part = gdn.gdn_scan_bwd(d["q"], d["k"], d["v"], d["beta"], d["gamma"], fwd["states"], do_d,
                            s0=dev(s0), ds_final=dev(dsf),
                            want=("dk", "dv", "dbeta", "dgamma", "ds0"))
    torch.cuda.synchronize()
    for n in ("dk", "dv", "dbeta", "dgamma", "ds0"):
        assert torch.equal(full[n], part[n]), n
    assert part["dq"] is None


def test_scan_bwd_subsets_of_outputs():
    """Any subset of the gradients may be requested; each requested one is
    bitwise equal to the same gradient of a call that wants all of them."""
    w = gi.workload(2).with_shape(H=2, T=4, S=200)
    x, d = _gen(w)
    do, do_d, s0, dsf = _bwd_inputs(w, x, d, True)
    dev = lambda a: torch.from_numpy(a).to(DEV)
    fwd = gdn.gdn_scan_fwd(d["q"], d["k"], d["v"], d["beta"], d["gamma"], s0=dev(s0), want_o=False)
    say("scan_bwd all outputs")
    full = gdn.gdn_scan_bwd(d["q"], d["k"], d["v"], d["beta"], d["gamma"], fwd["states"], do_d,
                            s0=dev(s0), ds_final=dev(dsf))
    for want in (("dbeta",), ("dv", "ds0"), ("dk", "dgamma"), ("dq", "dv")):
        say("scan_bwd outputs", want)
        g = gdn.gdn_scan_bwd(d["q"], d["k"], d["v"], d["beta"], d["gamma"], fwd["states"], do_d,
                             s0=dev(s0), ds_final=dev(dsf), want=want)
        torch.cuda.synchronize()
        for n in ("dq", "dk", "dv", "dbeta", "dgamma", "ds0"):
            if n in want:
                assert torch.equal(g[n], full[n]), (want, n)
            else:
                assert g[n] is None


def test_scan_bwd_layer_60s_fused_dq():
    """The 60 s 720p layer (T = 121, S = 3600, 16 heads) in the launch
    configuration the benchmark times. The oracle is too slow at this size, so
    the fused E_t + dq pass is checked by properties that hold at any size:
    the other gradients are bitwise equal to those of the unfused E pass
    (which the oracle checks at smaller sizes), and dq of sampled tokens
    equals S_t^T do computed on the host from the same fp32 states."""
    w = gi.workload(4)
    say("generate", w.name)
    x = gi.batch_inputs(w, 0, threads=16, keep_f32=False)
    d = upload(x, w)
    del x
    gen = torch.Generator(device=DEV)
    gen.manual_seed(1234)
    do_d = torch.randn(d["q"].shape, generator=gen, device=DEV).to(torch.bfloat16)
    say("forward", w.name)
    fwd = gdn.gdn_scan_fwd(d["q"], d["k"], d["v"], d["beta"], d["gamma"],
                           n_time_chunks=w.time_chunks, want_o=False)
    say("backward with dq (fused E pass)", w.name)
    full = gdn.gdn_scan_bwd(d["q"], d["k"], d["v"], d["beta"], d["gamma"], fwd["states"], do_d)
    torch.cuda.synchronize()
    say("backward without dq", w.name)
    part = gdn.gdn_scan_bwd(d["q"], d["k"], d["v"], d["beta"], d["gamma"], fwd["states"], do_d,
                            want=("dk", "dv", "dbeta", "dgamma", "ds0"))
    torch.cuda.synchronize()
    for n in ("dk", "dv", "dbeta", "dgamma", "ds0"):
        assert torch.equal(full[n], part[n]), n
    del part
    rng = np.random.default_rng(77)
    for _ in range(24):
        h, t = int(rng.integers(w.H)), int(rng.integers(w.T))
        s = int(rng.integers(w.S)) if rng.random() < 0.75 else w.S - 1 - int(rng.integers(20))
        St = host(fwd["states"][0, h, t])
        ref = St.T @ host(do_d[0, h, t, s])
        e = rel_fro(host(full["dq"][0, h, t, s]), ref)
        assert e <= tol(w), ((h, t, s), e)


BIDIR_BWD_CASES = {
    # name: (workload, chunk_len, with s0 / ds_final, keys_prepared)
    "f32_D16_L2_s0_dsf": (gi.workload(1), 2, True, False),
    "f32_D16_L3_plain": (gi.workload(1).with_shape(B=2, H=2), 3, False, False),
    "f32_D16_L1": (gi.workload(1), 1, True, False),
    "f32_D16_L_ge_T": (gi.workload(1), 20, True, False),
    "f32_D128_L2_prepared": (gi.workload(1).with_shape(D=128, S=40, T=4), 2, True, True),
    "bf16_D128_L3_s0_dsf": (gi.workload(2).with_shape(H=2, T=7, S=300), 3, True, False),
    "bf16_D128_L2_split_S2100": (gi.workload(2).with_shape(T=3, S=2100), 2, True, False),
    "bf16_D64_L2": (gi.workload(2).with_shape(D=64, T=5, S=130), 2, True, False),
    "bf16_D128_L3_prepared": (gi.workload(2).with_shape(H=2, T=5, S=170), 3, True, True),
    "bf16_D128_L2_S5": (gi.workload(2).with_shape(H=2, T=3, S=5), 2, True, False),
    "bf16_D128_L1_S1": (gi.workload(2).with_shape(T=2, S=1), 1, True, False),
}


@pytest.mark.parametrize("name", sorted(BIDIR_BWD_CASES))
def test_scan_bidir_bwd(name):
    """Gradients of L = <do, o> + <ds_final, S_T-1> for the chunk-causal
    bidirectional scan (o = (S_t + R_t) q) against the float64 oracle."""
    w, L, extras, prepared = BIDIR_BWD_CASES[name]
    x, d = _gen(w)
    if prepared:
        kh = orc.prepare_keys(x["k"]).astype(np.float32)
        if w.io == "bf16":
            bits = gi.f32_to_bf16_bits(kh)
            kh = gi.bf16_bits_to_f32(bits)
            d["k"] = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(DEV)
        else:
            d["k"] = torch.from_numpy(kh).to(DEV)
        x["k"] = kh
    do, do_d, s0, dsf = _bwd_inputs(w, x, d, extras)
    dev = lambda a: None if a is None else torch.from_numpy(a).to(DEV)
    say("scan_bidir_bwd", name, "forward")
    fwd = gdn.gdn_scan_bidir_chunked(d["q"], d["k"], d["v"], d["beta"], d["gamma"], L,
                                     s0=dev(s0), keys_prepared=prepared, want_o=False)
    say("scan_bidir_bwd", name, "backward")
    g = gdn.gdn_scan_bidir_chunked_bwd(d["q"], d["k"], d["v"], d["beta"], d["gamma"], L,
                                       fwd["states_fwd"], fwd["states_rev"], do_d, s0=dev(s0),
                                       ds_final=dev(dsf), keys_prepared=prepared)
    torch.cuda.synchronize()
    for (b, h) in [(0, 0), (w.B - 1, w.H - 1)]:
        a = head_arrays(x, b, h)
        ref = orc.scan_bidir_bwd(a["q"], a["k"], a["v"], a["beta"], a["gamma"], L,
                                 do[b, h][None, None].astype(np.float64),
                                 ds_final=None if dsf is None else dsf[b, h][None, None].astype(np.float64),
                                 s0=None if s0 is None else s0[b, h][None, None].astype(np.float64),
                                 keys_prepared=prepared)
        _check_grads(w, g, ref, b, h, (name,))


@pytest.mark.parametrize("wname", ["bf16_D128", "f32_D16"])
@pytest.mark.parametrize("kind", DEGENERATE_KINDS)
def test_degenerate_inputs_backward(kind, wname):
    """Gradients of both scans (causal; chunk-causal in chunks of 2 frames) in
    the recurrence's degenerate regimes against the oracle's, every head;
    and the gradients the arithmetic makes exactly zero: dk and dv where the
    gate is 0 (dk = beta c [k > 0] Z, dv = beta c Y), dk, dv and dbeta when
    ReLU zeroes every key, ds0 = G_0 M_0 when gamma = 0."""
    w = (gi.workload(2).with_shape(H=2, T=6, S=300) if wname == "bf16_D128"
         else gi.workload(1).with_shape(T=6))
    x = gi.batch_inputs(w, 0)
    _degenerate(x, w, kind)
    d = upload(x, w)
    do, do_d, s0, dsf = _bwd_inputs(w, x, d, True)
    dev = lambda a: torch.from_numpy(a).to(DEV)
    say("degenerate backward", kind, wname, "causal")
    fwd = gdn.gdn_scan_fwd(d["q"], d["k"], d["v"], d["beta"], d["gamma"], s0=dev(s0), want_o=False)
    g = gdn.gdn_scan_bwd(d["q"], d["k"], d["v"], d["beta"], d["gamma"], fwd["states"], do_d,
                         s0=dev(s0), ds_final=dev(dsf))
    say("degenerate backward", kind, wname, "chunk-causal")
    fb = gdn.gdn_scan_bidir_chunked(d["q"], d["k"], d["v"], d["beta"], d["gamma"], 2, s0=dev(s0),
                                    want_o=False)
    gb = gdn.gdn_scan_bidir_chunked_bwd(d["q"], d["k"], d["v"], d["beta"], d["gamma"], 2,
                                        fb["states_fwd"], fb["states_rev"], do_d, s0=dev(s0),
                                        ds_final=dev(dsf))
    torch.cuda.synchronize()
    for (b, h) in [(b, h) for b in range(w.B) for h in range(w.H)]:
        a = head_arrays(x, b, h)
        args = (a["q"], a["k"], a["v"], a["beta"], a["gamma"])
        kw = dict(ds_final=dsf[b, h][None, None].astype(np.float64),
                  s0=s0[b, h][None, None].astype(np.float64))
        dob = do[b, h][None, None].astype(np.float64)
        _check_grads(w, g, orc.scan_fwd_bwd(*args, dob, **kw), b, h, (kind, wname, "causal"))
        _check_grads(w, gb, orc.scan_bidir_bwd(*args, 2, dob, **kw), b, h,
                     (kind, wname, "chunk-causal"))
    gate_off = {"beta_zero": slice(None), "gates_off_on_odd_frames": slice(1, None, 2)}.get(kind)
    for grads in (g, gb):
        if gate_off is not None:
            assert not grads["dk"][:, :, gate_off].any() and not grads["dv"][:, :, gate_off].any()
        if kind == "keys_nonpositive":
            for n in ("dk", "dv", "dbeta"):
                assert not grads[n].any(), n
        if kind == "gamma_zero":
            assert not grads["ds0"].any()


@pytest.mark.parametrize("wname", ["bf16_D128", "f32_D16"])
def test_explicit_key_scale(wname):
    """A key scale given by the caller instead of 1/sqrt(D S) (phase 1 applies
    c^2 to A_t and c to U_t; the backward carries c into dk and dbeta):
    forward (2 time chunks) and chunk-causal scans and both backward passes
    against the oracle with the same scale, every head. The scale is chosen
    larger than the default but with tr(A_t) < 1, so that the recurrence stays
    contractive."""
    w = (gi.workload(2).with_shape(H=2, T=5, S=300) if wname == "bf16_D128"
         else gi.workload(1).with_shape(T=5))
    c = 1.6 / np.sqrt(w.D * w.S)
    c32 = float(np.float32(c))  # what the descriptor carries
    x, d = _gen(w)
    do, do_d, s0, dsf = _bwd_inputs(w, x, d, True)
    dev = lambda a: torch.from_numpy(a).to(DEV)
    args = (d["q"], d["k"], d["v"], d["beta"], d["gamma"])
    say("explicit key scale", wname)
    fwd = gdn.gdn_scan_fwd(*args, s0=dev(s0), n_time_chunks=2, key_scale=c32)
    g = gdn.gdn_scan_bwd(*args, fwd["states"], do_d, s0=dev(s0), ds_final=dev(dsf), key_scale=c32)
    bid = gdn.gdn_scan_bidir_chunked(*args, 2, s0=dev(s0), key_scale=c32)
    gb = gdn.gdn_scan_bidir_chunked_bwd(*args, 2, bid["states_fwd"], bid["states_rev"], do_d,
                                        s0=dev(s0), ds_final=dev(dsf), key_scale=c32)
    torch.cuda.synchronize()
    for (b, h) in [(b, h) for b in range(w.B) for h in range(w.H)]:
        a = [np.asarray(x[n][b, h], dtype=np.float64)[None, None] for n in ("q", "k", "v", "beta", "gamma")]
        kw = dict(s0=s0[b, h][None, None].astype(np.float64), key_scale=c32)
        dob = do[b, h][None, None].astype(np.float64)
        dsb = dsf[b, h][None, None].astype(np.float64)
        ref = orc.scan_fwd(*a, **kw)
        refb = orc.scan_bidir_chunked(*a, 2, **kw)
        for n in ("states", "o"):
            assert frame_errs(host(fwd[n][b, h]), ref[n][0, 0]).max() <= tol(w), n
        for n in ("states_fwd", "states_rev", "o"):
            assert frame_errs(host(bid[n][b, h]), refb[n][0, 0]).max() <= tol(w), n
        _check_grads(w, g, orc.scan_fwd_bwd(*a, dob, ds_final=dsb, **kw), b, h,
                     ("key scale", wname, "causal"))
        _check_grads(w, gb, orc.scan_bidir_bwd(*a, 2, dob, ds_final=dsb, **kw), b, h,
                     ("key scale", wname, "chunk-causal"))


def test_scan_bidir_bwd_layer_full_size():
    """Backward of the chunk-causal 16-head 720p layer (T = 11, S = 3600,
    chunks of 3 frames) at full size in the MFMA configuration, sampled heads."""
    w = gi.workload(3)
    L = 3
    heads = [(0, 5), (0, 11)]
    say("generate", w.name)
    x = gi.batch_inputs(w, 0, keep_f32=False)
    d = upload(x, w)
    rng = np.random.default_rng([88, 10])
    do_bits = gi.f32_to_bf16_bits(rng.standard_normal((w.B, w.H, w.T, w.S, w.D)).astype(np.float32))
    do_d = torch.from_numpy(do_bits.view(np.int16)).view(torch.bfloat16).to(DEV)
    say("forward + backward (bidirectional)", w.name)
    fwd = gdn.gdn_scan_bidir_chunked(d["q"], d["k"], d["v"], d["beta"], d["gamma"], L, want_o=False)
    g = gdn.gdn_scan_bidir_chunked_bwd(d["q"], d["k"], d["v"], d["beta"], d["gamma"], L,
                                       fwd["states_fwd"], fwd["states_rev"], do_d)
    torch.cuda.synchronize()
    for (b, h) in heads:
        s = gi.head_inputs(w, 0, b, h)
        a = {n: np.asarray(s[n], dtype=np.float64)[None, None] for n in ("q", "k", "v", "beta", "gamma")}
        dof = gi.bf16_bits_to_f32(do_bits[b, h]).astype(np.float64)[None, None]
        ref = orc.scan_bidir_bwd(a["q"], a["k"], a["v"], a["beta"], a["gamma"], L, dof)
        _check_grads(w, g, ref, b, h, (w.name, "bidir",))


RMS_BWD_CASES = {
    # name: (workload, chunk_len (0: causal), keys_prepared)
    "f32_D16": (gi.workload(1), 0, False),
    "f32_D64": (gi.workload(1).with_shape(D=64, S=40, T=4), 0, False),
    "f32_D16_bidir_L3": (gi.workload(1), 3, False),
    "bf16_D128": (gi.workload(2).with_shape(H=2, T=5, S=300), 0, False),
    "bf16_D128_split_S2100": (gi.workload(2).with_shape(T=3, S=2100), 0, False),
    "bf16_D128_bidir_L2": (gi.workload(2).with_shape(H=2, T=5, S=170), 2, False),
    "bf16_D128_prepared": (gi.workload(2).with_shape(H=2, T=4, S=170), 0, True),
    "bf16_D64": (gi.workload(2).with_shape(D=64, T=4, S=130), 0, False),
}


@pytest.mark.parametrize("name", sorted(RMS_BWD_CASES))
def test_scan_bwd_rmsnorm(name):
    """Backward with the RMSNorm of q and k (raw keys; prepared keys are used
    as given) against the float64 oracle, on inputs whose tokens are
    rescaled so that a missing or wrong norm would show."""
    w, L, prepared = RMS_BWD_CASES[name]
    x, d = _gen_rescaled(w)
    if prepared:
        kh = orc.prepare_keys(x["k"]).astype(np.float32)
        bits = gi.f32_to_bf16_bits(kh)
        kh = gi.bf16_bits_to_f32(bits)
        d["k"] = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(DEV)
        x["k"] = kh
    do, do_d, s0, dsf = _bwd_inputs(w, x, d, True)
    dev = lambda a: None if a is None else torch.from_numpy(a).to(DEV)
    say("scan_bwd rmsnorm", name, "forward")
    if L:
        fwd = gdn.gdn_scan_bidir_chunked(d["q"], d["k"], d["v"], d["beta"], d["gamma"], L,
                                         s0=dev(s0), keys_prepared=prepared, want_o=False,
                                         qk_rmsnorm=True)
        say("scan_bwd rmsnorm", name, "backward")
        g = gdn.gdn_scan_bidir_chunked_bwd(d["q"], d["k"], d["v"], d["beta"], d["gamma"], L,
                                           fwd["states_fwd"], fwd["states_rev"], do_d, s0=dev(s0),
                                           ds_final=dev(dsf), keys_prepared=prepared,
                                           qk_rmsnorm=True)
    else:
        fwd = gdn.gdn_scan_fwd(d["q"], d["k"], d["v"], d["beta"], d["gamma"], s0=dev(s0),
                               keys_prepared=prepared, want_o=False, qk_rmsnorm=True)
        say("scan_bwd rmsnorm", name, "backward")
        g = gdn.gdn_scan_bwd(d["q"], d["k"], d["v"], d["beta"], d["gamma"], fwd["states"], do_d,
                             s0=dev(s0), ds_final=dev(dsf), keys_prepared=prepared,
                             qk_rmsnorm=True)
    torch.cuda.synchronize()
    for (b, h) in [(0, 0), (w.B - 1, w.H - 1)]:
        a = head_arrays(x, b, h)
        kw = dict(ds_final=dsf[b, h][None, None].astype(np.float64),
                  s0=s0[b, h][None, None].astype(np.float64), keys_prepared=prepared,
                  qk_rmsnorm=True)
        dof = do[b, h][None, None].astype(np.float64)
        if L:
            ref = orc.scan_bidir_bwd(a["q"], a["k"], a["v"], a["beta"], a["gamma"], L, dof, **kw)
        else:
            ref = orc.scan_fwd_bwd(a["q"], a["k"], a["v"], a["beta"], a["gamma"], dof, **kw)
        _check_grads(w, g, ref, b, h, (name,))


@pytest.mark.parametrize("S", [300, 3600, 3599])
def test_scan_bwd_rmsnorm_last_token_dq(S):
    """Regression: with the RMSNorm of q, the fused E_t/dq pass must store the
    last token of a frame from its own row only (a ragged last stage once
    overwrote row S - 1 with the value of a zero-padded row, which lacks the
    norm's projection term). dq of the last tokens of every frame against the
    oracle, token by token."""
    w = gi.workload(2).with_shape(T=3, S=S)
    x, d = _gen_rescaled(w)
    do, do_d, s0, dsf = _bwd_inputs(w, x, d, False)
    say("scan_bwd rmsnorm last-token dq, S =", S)
    fwd = gdn.gdn_scan_fwd(d["q"], d["k"], d["v"], d["beta"], d["gamma"], want_o=False,
                           qk_rmsnorm=True)
    g = gdn.gdn_scan_bwd(d["q"], d["k"], d["v"], d["beta"], d["gamma"], fwd["states"], do_d,
                         qk_rmsnorm=True, want=("dq",))
    torch.cuda.synchronize()
    a = head_arrays(x, 0, 0)
    ref = orc.scan_fwd_bwd(a["q"], a["k"], a["v"], a["beta"], a["gamma"],
                           do[0, 0][None, None].astype(np.float64), qk_rmsnorm=True)
    got = host(g["dq"][0, 0])
    te = token_errs(got, ref["dq"][0, 0])
    say("last tokens", te[:, -4:].tolist())
    assert te[:, -40:].max() <= tol(w), te[:, -40:].max()
    assert te.max() <= tol(w), te.max()


@pytest.mark.parametrize("wname", ["bf16_D128", "f32_D16"])
def test_rmsnorm_zero_tokens(wname):
    """Tokens whose q and k are exactly zero under GDN_QK_RMSNORM. The norm's
    epsilon keeps 1 / rms finite, so such a key adds nothing to A_t and U_t,
    such a query gives an output of exactly zero, and every gradient stays
    finite (the norm's backward scales the incoming gradient by 1 / sqrt(eps)
    there). Forward with 2 time chunks and backward against the oracle."""
    w = (gi.workload(2).with_shape(H=2, T=4, S=300) if wname == "bf16_D128"
         else gi.workload(1).with_shape(T=4))
    x = gi.batch_inputs(w, 0)
    zero = np.zeros(w.S, dtype=bool)
    zero[::5] = True
    for n in ("q", "k"):
        x[n][:, :, :, zero] = 0.0
        if w.io == "bf16":
            x[n + "_bits"][:, :, :, zero] = 0
    d = upload(x, w)
    do, do_d, s0, dsf = _bwd_inputs(w, x, d, True)
    dev = lambda a: torch.from_numpy(a).to(DEV)
    say("rmsnorm zero tokens", wname, "forward")
    fwd = gdn.gdn_scan_fwd(d["q"], d["k"], d["v"], d["beta"], d["gamma"], s0=dev(s0),
                           n_time_chunks=2, qk_rmsnorm=True)
    say("rmsnorm zero tokens", wname, "backward")
    g = gdn.gdn_scan_bwd(d["q"], d["k"], d["v"], d["beta"], d["gamma"], fwd["states"], do_d,
                         s0=dev(s0), ds_final=dev(dsf), qk_rmsnorm=True)
    torch.cuda.synchronize()
    assert not fwd["o"][:, :, :, torch.from_numpy(zero).to(DEV)].any()
    for n in ("dq", "dk", "dv", "dbeta", "dgamma", "ds0"):
        assert torch.isfinite(g[n].float()).all(), n
    for (b, h) in [(b, h) for b in range(w.B) for h in range(w.H)]:
        a = head_arrays(x, b, h)
        args = (a["q"], a["k"], a["v"], a["beta"], a["gamma"])
        s0h = s0[b, h][None, None].astype(np.float64)
        ref = orc.scan_fwd(*args, s0=s0h, qk_rmsnorm=True)
        for n in ("states", "o"):
            got = host(fwd[n][b, h])
            e = frame_errs(got, ref[n][0, 0]).max()
            if n == "o":
                e = max(e, token_errs(got, ref[n][0, 0]).max())
            assert e <= tol(w), (n, e)
        refg = orc.scan_fwd_bwd(*args, do[b, h][None, None].astype(np.float64),
                                ds_final=dsf[b, h][None, None].astype(np.float64), s0=s0h,
                                qk_rmsnorm=True)
        _check_grads(w, g, refg, b, h, ("rmsnorm zero tokens", wname))


def test_scan_bwd_rmsnorm_without_dq():
    """With the RMSNorm of q, E_t still comes from the fused pass when dq is
    not wanted; the other gradients are bitwise those of the full call."""
    w = gi.workload(2).with_shape(H=2, T=4, S=200)
    x, d = _gen_rescaled(w)
    do, do_d, s0, dsf = _bwd_inputs(w, x, d, True)
    dev = lambda a: torch.from_numpy(a).to(DEV)
    fwd = gdn.gdn_scan_fwd(d["q"], d["k"], d["v"], d["beta"], d["gamma"], s0=dev(s0), want_o=False,
                           qk_rmsnorm=True)
    say("scan_bwd rmsnorm without dq")
    full = gdn.gdn_scan_bwd(d["q"], d["k"], d["v"], d["beta"], d["gamma"], fwd["states"], do_d,
                            s0=dev(s0), ds_final=dev(dsf), qk_rmsnorm=True)
    part = gdn.gdn_scan_bwd(d["q"], d["k"], d["v"], d["beta"], d["gamma"], fwd["states"], do_d,
                            s0=dev(s0), ds_final=dev(dsf), qk_rmsnorm=True,
                            want=("dk", "dv", "dbeta", "dgamma", "ds0"))
    torch.cuda.synchronize()
    for n in ("dk", "dv", "dbeta", "dgamma", "ds0"):
        assert torch.equal(full[n], part[n]), n


REUSE_CASES = {
    # name: (workload, chunk_len (0: causal, -1: one gdn_step block), P, rmsnorm, keys_prepared)
    "bf16_D128_P3": (gi.workload(2).with_shape(H=2, T=6, S=300), 0, 3, False, False),
    "bf16_D128_split_S2100": (gi.workload(2).with_shape(T=3, S=2100), 0, 1, False, False),
    "bf16_D128_bidir_L2_norm": (gi.workload(2).with_shape(H=2, T=5, S=170), 2, 2, True, False),
    "bf16_D128_step_prepared": (gi.workload(2).with_shape(H=2, T=3, S=170), -1, 1, False, True),
    # 90 tokens: the last 32-token stage of the recompute holds 26 tokens
    "bf16_D128_S90": (gi.workload(2).with_shape(H=2, T=3, S=90), 0, 1, False, False),
    "bf16_D128_S90_norm": (gi.workload(2).with_shape(H=2, T=3, S=90), 0, 2, True, False),
    "bf16_D64_norm": (gi.workload(2).with_shape(D=64, T=4, S=130), 0, 2, True, False),
    "f32_D16_bidir_L3": (gi.workload(1), 3, 1, False, False),
}


@pytest.mark.parametrize("name", sorted(REUSE_CASES))
def test_scan_bwd_reuses_forward_terms(name):
    """GDN_REUSE_FWD_TERMS: a backward call on the workspace of its forward
    call reads A_t from there instead of recomputing it. Both passes form
    every entry of A_t from the same operands in the same order, so all
    gradients are bitwise those of the recomputing call; a second backward on
    the same workspace shows that the first left the terms in place."""
    w, L, P, norm, prepared = REUSE_CASES[name]
    x, d = (_gen_rescaled if norm else _gen)(w)
    if prepared:
        kh = orc.prepare_keys(x["k"]).astype(np.float32)
        bits = gi.f32_to_bf16_bits(kh)
        d["k"] = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(DEV)
    do, do_d, s0, dsf = _bwd_inputs(w, x, d, True)
    dev = lambda a: torch.from_numpy(a).to(DEV)
    desc = gdn._desc_from(d["k"], 0.0, prepared, norm)
    chunk = w.T if L < 0 else L
    bwd_bytes = (gdn.gdn_bidir_bwd_workspace_bytes(desc, chunk) if L
                 else gdn.gdn_bwd_workspace_bytes(desc))
    ws = torch.empty(max(gdn.gdn_workspace_bytes(desc, P), bwd_bytes), dtype=torch.uint8,
                     device=DEV)
    say("reuse terms", name, "forward")
    kw = dict(keys_prepared=prepared, qk_rmsnorm=norm)
    if L < 0:
        fwd = gdn.gdn_step(d["q"], d["k"], d["v"], d["beta"], d["gamma"], carry_in=dev(s0),
                           want_o=False, want_states=True, ws=ws, **kw)
    elif L:
        fwd = gdn.gdn_scan_bidir_chunked(d["q"], d["k"], d["v"], d["beta"], d["gamma"], L,
                                         s0=dev(s0), n_time_chunks=P, want_o=False, ws=ws, **kw)
    else:
        fwd = gdn.gdn_scan_fwd(d["q"], d["k"], d["v"], d["beta"], d["gamma"], s0=dev(s0),
                               n_time_chunks=P, want_o=False, ws=ws, **kw)

    def bwd(reuse):
        args = (d["q"], d["k"], d["v"], d["beta"], d["gamma"])
        extra = dict(s0=dev(s0), ds_final=dev(dsf), reuse_fwd_terms=reuse,
                     ws=ws if reuse else None, **kw)
        if L:
            return gdn.gdn_scan_bidir_chunked_bwd(*args, chunk, fwd["states_fwd"],
                                                  fwd["states_rev"], do_d, **extra)
        return gdn.gdn_scan_bwd(*args, fwd["states"], do_d, **extra)

    say("reuse terms", name, "backward, reusing")
    g1 = bwd(True)
    torch.cuda.synchronize()
    g1 = {n: t.clone() for n, t in g1.items()}
    say("reuse terms", name, "backward, reusing again")
    g2 = bwd(True)
    say("reuse terms", name, "backward, recomputing")
    ref = bwd(False)
    torch.cuda.synchronize()
    for n in ("dq", "dk", "dv", "dbeta", "dgamma", "ds0"):
        assert torch.equal(g1[n], ref[n]), n
        assert torch.equal(g2[n], ref[n]), n


def test_scan_bwd_reuse_needs_workspace():
    w = gi.workload(2).with_shape(T=2, S=64)
    x, d = _gen(w)
    with pytest.raises(ValueError):
        gdn.gdn_scan_bwd(d["q"], d["k"], d["v"], d["beta"], d["gamma"],
                         torch.zeros((1, 1, 2, 128, 128), device=DEV), d["q"],
                         reuse_fwd_terms=True)


def test_rmsnorm_layer_60s_forward_and_backward():
    """The 60 s 720p layer (T = 121, S = 3600, 16 heads) with the RMSNorm of q
    and k, in the benchmark's launch configuration (8 time chunks; the
    backward reading A_t from the forward's workspace), on tokens whose q and
    k are rescaled per token by factors in [0.2, 5] (a missing norm would be
    far off): states, outputs and every gradient of two sampled heads against
    the oracle."""
    w = gi.workload(4)
    heads = [(0, 4), (0, 11)]
    say("generate", w.name)
    x = gi.batch_inputs(w, 0, keep_f32=False)
    for h in range(w.H):  # per-token rescaling, per head to bound host memory
        rng = np.random.default_rng([77, 4, h])
        for n in ("q", "k"):
            bits = x[n + "_bits"][0, h]
            fac = rng.uniform(0.2, 5.0, bits.shape[:-1] + (1,)).astype(np.float32)
            bits[...] = gi.f32_to_bf16_bits(gi.bf16_bits_to_f32(bits) * fac)
    d = upload(x, w)
    rng = np.random.default_rng([88, 12])
    do_bits = gi.f32_to_bf16_bits(rng.standard_normal((w.B, w.H, w.T, w.S, w.D)).astype(np.float32))
    do_d = bits_to_dev(do_bits)
    desc = gdn._desc_from(d["k"], 0.0, False, True)
    ws = torch.empty(max(gdn.gdn_workspace_bytes(desc, w.time_chunks), gdn.gdn_bwd_workspace_bytes(desc)),
                     dtype=torch.uint8, device=DEV)
    say("forward + backward with the RMSNorm", w.name)
    fwd = gdn.gdn_scan_fwd(d["q"], d["k"], d["v"], d["beta"], d["gamma"], n_time_chunks=w.time_chunks,
                           ws=ws, qk_rmsnorm=True)
    g = gdn.gdn_scan_bwd(d["q"], d["k"], d["v"], d["beta"], d["gamma"], fwd["states"], do_d, ws=ws,
                         qk_rmsnorm=True, reuse_fwd_terms=True)
    torch.cuda.synchronize()
    for (b, h) in heads:
        a = {n: gi.bf16_bits_to_f32(x[n + "_bits"][b, h]).astype(np.float64)[None, None]
             for n in ("q", "k", "v")}
        for n in ("beta", "gamma"):
            a[n] = np.asarray(x[n][b, h], dtype=np.float64)[None, None]
        ref = orc.scan_fwd(a["q"], a["k"], a["v"], a["beta"], a["gamma"], qk_rmsnorm=True)
        errs = {n + " frame": float(frame_errs(host(fwd[n][b, h]), ref[n][0, 0]).max())
                for n in ("states", "o")}
        errs["o token"] = float(token_errs(host(fwd["o"][b, h]), ref["o"][0, 0]).max())
        errs["s_final"] = rel_fro(host(fwd["s_final"][b, h]), ref["s_final"][0, 0])
        dof = gi.bf16_bits_to_f32(do_bits[b, h]).astype(np.float64)[None, None]
        gref = orc.scan_fwd_bwd(a["q"], a["k"], a["v"], a["beta"], a["gamma"], dof, qk_rmsnorm=True)
        errs.update(_grad_errs(g, gref, b, h))
        say(w.name, "rmsnorm", (b, h), {n: f"{e:.2e}" for n, e in errs.items()})
        assert max(errs.values()) <= tol(w), errs


def test_scan_bwd_no_frames():
    w = gi.workload(1).with_shape(T=0)
    x, d = _gen(w)
    dsf = torch.randn((w.B, w.H, w.D, w.D), device=DEV)
    states = torch.empty((w.B, w.H, 0, w.D, w.D), device=DEV)
    say("scan_bwd T=0")
    g = gdn.gdn_scan_bwd(d["q"], d["k"], d["v"], d["beta"], d["gamma"], states, d["q"],
                         ds_final=dsf, want=("ds0",))
    torch.cuda.synchronize()
    assert torch.equal(g["ds0"], dsf)


def test_scan_bwd_layer_full_size():
    """Backward of the 16-head 720p layer (T = 11, S = 3600) at full size in
    the MFMA configuration, checked on two sampled heads."""
    w = gi.workload(3)
    heads = [(0, 2), (0, 13)]
    say("generate", w.name)
    x = gi.batch_inputs(w, 0, keep_f32=False)
    d = upload(x, w)
    rng = np.random.default_rng([88, 9])
    do_bits = gi.f32_to_bf16_bits(rng.standard_normal((w.B, w.H, w.T, w.S, w.D)).astype(np.float32))
    do_d = torch.from_numpy(do_bits.view(np.int16)).view(torch.bfloat16).to(DEV)
    say("forward + backward", w.name)
    fwd = gdn.gdn_scan_fwd(d["q"], d["k"], d["v"], d["beta"], d["gamma"], want_o=False)
    g = gdn.gdn_scan_bwd(d["q"], d["k"], d["v"], d["beta"], d["gamma"], fwd["states"], do_d)
    torch.cuda.synchronize()
    for (b, h) in heads:
        s = gi.head_inputs(w, 0, b, h)
        a = {n: np.asarray(s[n], dtype=np.float64)[None, None] for n in ("q", "k", "v", "beta", "gamma")}
        dof = gi.bf16_bits_to_f32(do_bits[b, h]).astype(np.float64)[None, None]
        ref = orc.scan_fwd_bwd(a["q"], a["k"], a["v"], a["beta"], a["gamma"], dof)
        _check_grads(w, g, ref, b, h, (w.name,))
