"""Pins of the float64 oracle against facts fixed by the pages and by mathematics.

Each ``pin_*`` function takes the oracle module and raises AssertionError when
the oracle disagrees with an independent fact: a hand-derived worked example,
exact rational arithmetic of an unrolled closed form, a special case that
reduces to the token-level Gated DeltaNet, an exact-write property, the
non-expansiveness bound, or an algebraic identity between two routes. None of
them calls the oracle to produce its own expected value, except where the
fact is a relation between two different oracle routes (composite versus
sequential, reverse versus forward on reversed time).

Sources: blog.hotdry.top SANA-WM post, sections "混合线性注意力" (the three GDN
equations and the key scaling) and "显存分片: Context-Parallel 的工程实现"
(composites); xiejiayun.github.io "好文共赏 | SANA-WM", section 2.1 (token-level
GDN, trace inequality); hyper.ai page 2605.15178, method section (reverse scan
reset at chunk boundaries).
"""

from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _frac_arr(x):
    return np.array([[float(Fraction(str(e))) for e in row] for row in x])


def _frac_arr3(x):
    return np.stack([_frac_arr(m) for m in x])


def _close(a, b, tol=1e-12, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    err = np.max(np.abs(a - b)) if a.size else 0.0
    scale = max(1.0, float(np.max(np.abs(b))) if b.size else 1.0)
    assert err <= tol * scale, f"{what}: max abs err {err} (scale {scale})"


def _rand_case(rng, B=1, H=1, T=5, S=6, D=4, beta=(0.0, 1.0), gamma=(0.8, 1.0)):
    q = rng.standard_normal((B, H, T, S, D))
    k = rng.standard_normal((B, H, T, S, D))
    v = rng.standard_normal((B, H, T, S, D))
    b = rng.uniform(beta[0], beta[1], (B, H, T, S))
    g = rng.uniform(gamma[0], gamma[1], (B, H, T))
    return q, k, v, b, g


# ---------------------------------------------------------------- a1 prepare
def pin_prepare_closed_form(orc):
    """K_hat = max(k, 0) / sqrt(D S); ReLU commutes with a positive scale."""
    k = np.array([[[-2.0, -0.0, 0.0, 3.0], [1.5, -1e-300, 7.0, -4.0]]])  # [1, S=2, D=4]
    got = orc.prepare_keys(k)
    c = 1.0 / math.sqrt(4 * 2)
    exp = np.array([[[0.0, 0.0, 0.0, 3.0 * c], [1.5 * c, 0.0, 7.0 * c, 0.0]]])
    _close(got, exp, 0.0, "prepare default scale")
    assert not np.any(np.signbit(got[got == 0.0])), "ReLU must give +0"
    got2 = orc.prepare_keys(k, key_scale=0.25)
    _close(got2, np.maximum(k * 0.25, 0.0), 0.0, "relu(c k) == c relu(k)")
    assert abs(orc.default_key_scale(16, 12) - 1.0 / math.sqrt(192.0)) < 1e-16
    assert abs(orc.default_key_scale(128, 3600) - 1.0 / 678.8225099390856) < 1e-15


# ------------------------------------------------------- hand worked example
def load_hand_example():
    with open(os.path.join(GOLDEN, "hand_example_D2.json")) as f:
        g = json.load(f)
    ex = {
        "k_hat": np.array(g["k_hat"], dtype=np.float64)[None, None],
        "v": np.array(g["v"], dtype=np.float64)[None, None],
        "q": np.array(g["q"], dtype=np.float64)[None, None],
        "beta": np.array([[float(Fraction(e)) for e in r] for r in g["beta"]])[None, None],
        "gamma": np.array([float(Fraction(e)) for e in g["gamma"]])[None, None],
        "s0": _frac_arr(g["s0"])[None, None],
        "A": _frac_arr3(g["A"]),
        "U": _frac_arr3(g["U"]),
        "states": _frac_arr3(g["states"]),
        "o": _frac_arr3(g["o"]),
        "states_rev": _frac_arr3(g["chunk_len_2"]["states_rev"]),
        "o_bidir": _frac_arr3(g["chunk_len_2"]["o_bidir"]),
        "C": _frac_arr(g["composite_one_chunk"]["C"]),
        "H": _frac_arr(g["composite_one_chunk"]["H"]),
    }
    return ex


def pin_hand_example(orc):
    """Two-frame example worked by hand (tests/golden/hand_example_D2.json)."""
    ex = load_hand_example()
    for t in range(2):
        A, U = orc.frame_terms(ex["k_hat"][0, 0, t], ex["v"][0, 0, t], ex["beta"][0, 0, t])
        _close(A, ex["A"][t], 1e-15, f"A_{t}")
        _close(U, ex["U"][t], 1e-15, f"U_{t}")
    r = orc.scan_fwd(ex["q"], ex["k_hat"], ex["v"], ex["beta"], ex["gamma"], s0=ex["s0"],
                     keys_prepared=True)
    _close(r["states"][0, 0], ex["states"], 1e-15, "states")
    _close(r["s_final"][0, 0], ex["states"][-1], 1e-15, "s_final")
    _close(r["o"][0, 0], ex["o"], 1e-15, "o")
    rb = orc.scan_bidir_chunked(ex["q"], ex["k_hat"], ex["v"], ex["beta"], ex["gamma"], 2,
                                s0=ex["s0"], keys_prepared=True)
    _close(rb["states_rev"][0, 0], ex["states_rev"], 1e-15, "states_rev")
    _close(rb["o"][0, 0], ex["o_bidir"], 1e-15, "o_bidir")
    C, Hc = orc.compose(ex["k_hat"], ex["v"], ex["beta"], ex["gamma"], [0, 2], keys_prepared=True)
    _close(C[0, 0, 0], ex["C"], 1e-15, "C")
    _close(Hc[0, 0, 0], ex["H"], 1e-15, "H")


# --------------------------------------------- exact rationals, unrolled form
def _fr_mat(D, val=0):
    return [[Fraction(val) for _ in range(D)] for _ in range(D)]


def _fr_mm(a, b):
    n, m, p = len(a), len(b), len(b[0])
    return [[sum((a[i][r] * b[r][j] for r in range(m)), Fraction(0)) for j in range(p)]
            for i in range(n)]


def _fr_add(a, b):
    return [[x + y for x, y in zip(ra, rb)] for ra, rb in zip(a, b)]


def pin_exact_rational_unrolled(orc):
    """Unrolled closed form in exact rationals with raw keys and c = 1/6.

    With D = 4 and S = 9, 1/sqrt(D S) = 1/6 exactly. The state after frame t
    is S0 P(0..t) + sum_tau U_tau P(tau+1..t), P the ordered product of M;
    this route never forms the recurrence.
    """
    rng = np.random.default_rng(11)
    D, S, T = 4, 9, 3
    k = rng.integers(-3, 4, (T, S, D)).astype(np.float64)
    v = rng.integers(-3, 4, (T, S, D)).astype(np.float64)
    q = rng.integers(-2, 3, (T, S, D)).astype(np.float64)
    bnum = rng.integers(0, 5, (T, S))
    beta = bnum / 4.0
    gam_num = rng.integers(5, 9, T)
    gamma = gam_num / 8.0
    s0 = rng.integers(-2, 3, (D, D)).astype(np.float64)
    c = Fraction(1, 6)
    Ms, Us = [], []
    for t in range(T):
        A = _fr_mat(D)
        U = _fr_mat(D)
        for s in range(S):
            kh = [Fraction(max(int(k[t, s, i]), 0)) * c for i in range(D)]
            bs = Fraction(int(bnum[t, s]), 4)
            for i in range(D):
                for j in range(D):
                    A[i][j] += bs * kh[i] * kh[j]
                    U[i][j] += bs * Fraction(int(v[t, s, i])) * kh[j]
        g = Fraction(int(gam_num[t]), 8)
        M = [[g * ((1 if i == j else 0) - A[i][j]) for j in range(D)] for i in range(D)]
        Ms.append(M)
        Us.append(U)
    S0 = [[Fraction(int(x)) for x in row] for row in s0]
    exp_states = []
    for t in range(T):
        P = [[Fraction(1 if i == j else 0) for j in range(D)] for i in range(D)]
        for tau in range(0, t + 1):
            P = _fr_mm(P, Ms[tau])
        acc = _fr_mm(S0, P)
        for tau in range(t + 1):
            Pt = [[Fraction(1 if i == j else 0) for j in range(D)] for i in range(D)]
            for r in range(tau + 1, t + 1):
                Pt = _fr_mm(Pt, Ms[r])
            acc = _fr_add(acc, _fr_mm(Us[tau], Pt))
        exp_states.append(np.array([[float(x) for x in row] for row in acc]))
    exp_states = np.stack(exp_states)
    r = orc.scan_fwd(q[None, None], k[None, None], v[None, None], beta[None, None],
                     gamma[None, None], s0=s0[None, None])
    _close(r["states"][0, 0], exp_states, 1e-12, "exact unrolled states")
    # readout: o_{t,s,i} = sum_j S_t[i, j] q_{t,s,j}, as explicit sums
    for t in range(T):
        for s in range(S):
            for i in range(D):
                e = sum(exp_states[t, i, j] * q[t, s, j] for j in range(D))
                assert abs(r["o"][0, 0, t, s, i] - e) <= 1e-11 * max(1.0, abs(e)), (t, s, i)


# ------------------------------------------------------------- closed forms
def pin_pure_decay(orc):
    """beta = 0: no write and no correction, S_t = (prod gamma) S0."""
    rng = np.random.default_rng(3)
    q, k, v, b, g = _rand_case(rng, T=6)
    b[:] = 0.0
    s0 = rng.standard_normal((1, 1, 4, 4))
    r = orc.scan_fwd(q, k, v, b, g, s0=s0)
    for t in range(6):
        _close(r["states"][0, 0, t], np.prod(g[0, 0, : t + 1]) * s0[0, 0], 1e-14, f"decay t={t}")


def pin_constant_state(orc):
    """gamma = 1 and beta = 0: the state never changes."""
    rng = np.random.default_rng(4)
    q, k, v, b, g = _rand_case(rng, T=5)
    b[:] = 0.0
    g[:] = 1.0
    s0 = rng.standard_normal((1, 1, 4, 4))
    r = orc.scan_fwd(q, k, v, b, g, s0=s0)
    for t in range(5):
        _close(r["states"][0, 0, t], s0[0, 0], 0.0, "constant state")
    _close(r["o"][0, 0], q[0, 0] @ s0[0, 0].T, 1e-14, "constant-state readout")


def pin_single_frame_from_zero(orc):
    """T = 1 from a zero state: S_0 = U_0, written out as explicit sums."""
    rng = np.random.default_rng(5)
    q, k, v, b, g = _rand_case(rng, T=1, S=7, D=5)
    r = orc.scan_fwd(q, k, v, b, g)
    c = 1.0 / math.sqrt(5 * 7)
    U = np.zeros((5, 5))
    for s in range(7):
        kh = [max(x, 0.0) * c for x in k[0, 0, 0, s]]
        for i in range(5):
            for j in range(5):
                U[i, j] += b[0, 0, 0, s] * v[0, 0, 0, s, i] * kh[j]
    _close(r["states"][0, 0, 0], U, 1e-13, "U_0")
    for s in range(7):
        e = [sum(U[i, j] * q[0, 0, 0, s, j] for j in range(5)) for i in range(5)]
        _close(r["o"][0, 0, 0, s], e, 1e-13, "o = U_0 q")


def pin_token_level_special_case(orc):
    """One token per frame reduces to token-level Gated DeltaNet.

    Token form (xiejiayun.github.io, section 2.1): S_i = g S_{i-1} +
    (v_i - g S_{i-1} k_i) b_i k_i^T, evaluated in that unrearranged form.
    """
    rng = np.random.default_rng(6)
    D, T = 8, 20
    kh = np.abs(rng.standard_normal((T, 1, D))) / math.sqrt(D)
    v = rng.standard_normal((T, 1, D))
    q = rng.standard_normal((T, 1, D))
    b = rng.uniform(0, 1, (T, 1))
    g = rng.uniform(0.7, 1.0, T)
    S = rng.standard_normal((D, D))
    s0 = S.copy()
    exp = []
    for i in range(T):
        kk = kh[i, 0][:, None]
        vv = v[i, 0][:, None]
        S = g[i] * S + (vv - g[i] * S @ kk) * b[i, 0] @ kk.T
        exp.append(S.copy())
    r = orc.scan_fwd(q[None, None], kh[None, None], v[None, None], b[None, None], g[None, None],
                     s0=s0[None, None], keys_prepared=True)
    _close(r["states"][0, 0], np.stack(exp), 1e-12, "token-level GDN")


def pin_exact_write(orc):
    """beta = 1 with unit keys writes values exactly: S_t k_s = v_s.

    One token: S k = g S k (1 - |k|^2) + v |k|^2 = v for any gamma and any
    prior state. With several nonnegative keys of disjoint support (so
    orthonormal), every token of the frame is written exactly.
    """
    rng = np.random.default_rng(7)
    D, T = 6, 5
    kh = np.abs(rng.standard_normal((T, 1, D)))
    kh /= np.linalg.norm(kh, axis=-1, keepdims=True)
    v = rng.standard_normal((T, 1, D))
    q = rng.standard_normal((T, 1, D))
    b = np.ones((T, 1))
    g = rng.uniform(0.5, 1.0, T)
    s0 = rng.standard_normal((1, 1, D, D))
    r = orc.scan_fwd(q[None, None], kh[None, None], v[None, None], b[None, None], g[None, None],
                     s0=s0, keys_prepared=True)
    for t in range(T):
        _close(r["states"][0, 0, t] @ kh[t, 0], v[t, 0], 1e-12, f"exact write t={t}")
    # several tokens with disjoint supports
    S_tok, D2 = 3, 7
    kh2 = np.zeros((2, S_tok, D2))
    supports = [[0, 3], [1, 4, 6], [2, 5]]
    for t in range(2):
        for s, sup in enumerate(supports):
            x = rng.uniform(0.2, 1.0, len(sup))
            kh2[t, s, sup] = x / np.linalg.norm(x)
    v2 = rng.standard_normal((2, S_tok, D2))
    r2 = orc.scan_fwd(v2[None, None], kh2[None, None], v2[None, None], np.ones((1, 1, 2, S_tok)),
                      np.array([[[0.9, 0.6]]]), s0=rng.standard_normal((1, 1, D2, D2)),
                      keys_prepared=True)
    for t in range(2):
        for s in range(S_tok):
            _close(r2["states"][0, 0, t] @ kh2[t, s], v2[t, s], 1e-12, "orthonormal write")


def pin_affine_in_s0(orc):
    """The state is affine in S0: S_t(S0) - S_t(0) = S0 P(0..t), P the ordered
    product of M formed here from its own definition."""
    rng = np.random.default_rng(8)
    q, k, v, b, g = _rand_case(rng, T=4, S=5, D=3)
    s0 = rng.standard_normal((1, 1, 3, 3))
    r1 = orc.scan_fwd(q, k, v, b, g, s0=s0)
    r0 = orc.scan_fwd(q, k, v, b, g)
    c = 1.0 / math.sqrt(3 * 5)
    P = np.eye(3)
    for t in range(4):
        kh = np.maximum(k[0, 0, t], 0) * c
        A = np.einsum("s,si,sj->ij", b[0, 0, t], kh, kh)
        P = P @ (g[0, 0, t] * (np.eye(3) - A))
        _close(r1["states"][0, 0, t] - r0["states"][0, 0, t], s0[0, 0] @ P, 1e-12, "affine")


def pin_non_expansive(orc):
    """tr(K beta K^T) <= 1 implies ||M_t||_2 <= gamma_t <= 1 (xiejiayun.github.io,
    section 2.1), so two scans from different S0 draw together geometrically."""
    rng = np.random.default_rng(9)
    for (D, S) in ((16, 12), (8, 40)):
        q, k, v, b, g = _rand_case(rng, T=12, S=S, D=D, gamma=(0.9, 1.0))
        kh = orc.prepare_keys(k[0, 0])
        for t in range(12):
            A, _ = orc.frame_terms(kh[t], v[0, 0, t], b[0, 0, t])
            tr = np.trace(A)
            assert tr <= 1.0 + 1e-12
            ev = np.linalg.eigvalsh(A)
            assert ev.min() >= -1e-12 and ev.max() <= tr + 1e-12
            M = orc.transition(A, g[0, 0, t])
            assert np.linalg.norm(M, 2) <= g[0, 0, t] + 1e-12
        s0a = rng.standard_normal((1, 1, D, D))
        s0b = rng.standard_normal((1, 1, D, D))
        ra = orc.scan_fwd(q, k, v, b, g, s0=s0a)
        rb = orc.scan_fwd(q, k, v, b, g, s0=s0b)
        d0 = np.linalg.norm(s0a - s0b)
        for t in range(12):
            dt = np.linalg.norm(ra["states"][0, 0, t] - rb["states"][0, 0, t])
            assert dt <= np.prod(g[0, 0, : t + 1]) * d0 * (1 + 1e-12)


def pin_unscaled_keys_expand(orc):
    """Without the 1/sqrt(S) part of the key scale, a 720p frame (S = 3600)
    has tr(A) far above 1 and ||M||_2 > 1: the state grows instead of decaying
    (the instability the key scaling prevents)."""
    rng = np.random.default_rng(10)
    D, S = 128, 3600
    k = rng.standard_normal((S, D)).astype(np.float32).astype(np.float64)
    b = rng.uniform(0, 1, S)
    good = orc.prepare_keys(k)
    A, _ = orc.frame_terms(good, np.zeros((S, D)), b)
    assert np.trace(A) <= 1.0
    assert np.linalg.norm(orc.transition(A, 1.0), 2) <= 1.0 + 1e-12
    bad = orc.prepare_keys(k, key_scale=1.0 / math.sqrt(D))
    Ab, _ = orc.frame_terms(bad, np.zeros((S, D)), b)
    assert np.trace(Ab) > 100.0
    assert np.linalg.norm(orc.transition(Ab, 1.0), 2) > 100.0


# ------------------------------------------------------------ a4 composites
def pin_composite_equals_sequential(orc):
    """Composite route reaches the sequential states exactly (up to rounding):
    S_start(p+1) = S_start(p) C_p + H_p, from the context-parallel section."""
    rng = np.random.default_rng(12)
    q, k, v, b, g = _rand_case(rng, B=2, H=2, T=11, S=5, D=4)
    s0 = rng.standard_normal((2, 2, 4, 4))
    seq = orc.scan_fwd(q, k, v, b, g, s0=s0)
    for offs in ([0, 11], [0, 3, 7, 11], [0, 1, 2, 5, 9, 10, 11]):
        C, Hc = orc.compose(k, v, b, g, offs)
        s_start, s_end = orc.combine(C, Hc, s0=s0)
        _close(s_end, seq["s_final"], 1e-12, "composite end state")
        for p in range(1, len(offs) - 1):
            _close(s_start[:, :, p], seq["states"][:, :, offs[p] - 1], 1e-12, "chunk start")
        _close(s_start[:, :, 0], s0, 0.0, "first chunk start")
        # H_p is the chunk scanned from a zero state
        for p in range(len(offs) - 1):
            a, e = offs[p], offs[p + 1]
            part = orc.scan_fwd(q[:, :, a:e], k[:, :, a:e], v[:, :, a:e], b[:, :, a:e],
                                g[:, :, a:e], key_scale=1.0 / math.sqrt(4 * 5))
            _close(Hc[:, :, p], part["s_final"], 1e-13, "H_p")


def pin_composite_pure_decay(orc):
    """beta = 0: C_p = (prod gamma) I and H_p = 0."""
    rng = np.random.default_rng(13)
    q, k, v, b, g = _rand_case(rng, T=7)
    b[:] = 0.0
    C, Hc = orc.compose(k, v, b, g, [0, 4, 7])
    _close(C[0, 0, 0], np.prod(g[0, 0, :4]) * np.eye(4), 1e-15, "C_0")
    _close(C[0, 0, 1], np.prod(g[0, 0, 4:]) * np.eye(4), 1e-15, "C_1")
    _close(Hc, np.zeros_like(Hc), 0.0, "H")


def pin_resume(orc):
    """scan(0..tau) then scan(tau..T) from its final state equals scan(0..T)."""
    rng = np.random.default_rng(14)
    q, k, v, b, g = _rand_case(rng, T=9, S=6, D=4)
    c = 1.0 / math.sqrt(4 * 6)
    full = orc.scan_fwd(q, k, v, b, g, key_scale=c)
    first = orc.scan_fwd(q[:, :, :4], k[:, :, :4], v[:, :, :4], b[:, :, :4], g[:, :, :4], key_scale=c)
    rest = orc.scan_fwd(q[:, :, 4:], k[:, :, 4:], v[:, :, 4:], b[:, :, 4:], g[:, :, 4:],
                        s0=first["s_final"], key_scale=c)
    _close(rest["states"], full["states"][:, :, 4:], 1e-13, "resume states")
    _close(rest["o"], full["o"][:, :, 4:], 1e-13, "resume outputs")


# --------------------------------------------------------- a5 reverse scans
def pin_reverse_is_forward_on_reversed_chunk(orc):
    """Inside each chunk the reverse scan is the forward scan of the time-reversed
    chunk from zero; chunks never see each other (reset at boundaries)."""
    rng = np.random.default_rng(15)
    q, k, v, b, g = _rand_case(rng, B=1, H=2, T=10, S=5, D=4)
    c = 1.0 / math.sqrt(4 * 5)
    for L in (1, 3, 4, 10, 25):
        rev = orc.scan_reverse_chunked(k, v, b, g, L, key_scale=c)
        for a in range(0, 10, L):
            e = min(a + L, 10)
            sl = slice(e - 1, a - 1 if a > 0 else None, -1)
            f = orc.scan_fwd(q[:, :, sl], k[:, :, sl], v[:, :, sl], b[:, :, sl], g[:, :, sl],
                             key_scale=c)
            _close(rev[:, :, a:e], f["states"][:, :, ::-1], 1e-13, f"reverse L={L}")
    # chunk_len = 1: R_t = U_t, so bidirectional o = (S_t + U_t) q
    rb = orc.scan_bidir_chunked(q, k, v, b, g, 1, key_scale=c)
    zero = orc.scan_fwd(q, k, v, b, np.zeros_like(g), key_scale=c)  # gamma = 0: S_t = U_t
    _close(rb["states_rev"], zero["states"], 1e-14, "R_t = U_t")
    _close(rb["o"], np.einsum("bhtsj,bhtij->bhtsi", q, rb["states_fwd"] + zero["states"]), 1e-12,
           "bidir readout sums both states")


def pin_readout_linear(orc):
    """Bidirectional readout equals the sum of the two separate readouts."""
    rng = np.random.default_rng(16)
    q, k, v, b, g = _rand_case(rng, T=6, S=5, D=4)
    rb = orc.scan_bidir_chunked(q, k, v, b, g, 4)
    o1 = np.einsum("tsj,tij->tsi", q[0, 0], rb["states_fwd"][0, 0])
    o2 = np.einsum("tsj,tij->tsi", q[0, 0], rb["states_rev"][0, 0])
    _close(rb["o"][0, 0], o1 + o2, 1e-13, "linearity")
    fwd = orc.scan_fwd(q, k, v, b, g)
    _close(fwd["o"][0, 0], o1, 1e-13, "forward readout")


def pin_rmsnorm_values(orc):
    """Per-token RMSNorm over the head dimension (reading of the fused
    operator's RMSNorm, blog.hotdry.top SANA-WM post, section
    "显存分片: Context-Parallel 的工程实现"): hand values on tokens of
    different size, unit mean square up to epsilon, odd symmetry."""
    eps = orc.RMS_EPS
    x = np.array([[3.0, -4.0, 0.0, 0.0],      # mean square 25/4
                  [1.0, 1.0, 1.0, 1.0],       # mean square 1
                  [0.0, 0.0, 0.0, 2.0]])      # mean square 1
    want = np.array([[3.0 / math.sqrt(6.25 + eps), -4.0 / math.sqrt(6.25 + eps), 0.0, 0.0],
                     [1.0 / math.sqrt(1.0 + eps)] * 4,
                     [0.0, 0.0, 0.0, 2.0 / math.sqrt(1.0 + eps)]])
    _close(orc.rms_norm(x), want, 1e-15, "rms_norm hand values")
    rng = np.random.default_rng(21)
    y = rng.standard_normal((7, 16)) * rng.uniform(0.5, 50.0, (7, 1))
    z = orc.rms_norm(y)
    ms = np.mean(y * y, axis=-1)
    _close(np.mean(z * z, axis=-1), ms / (ms + eps), 1e-13, "unit mean square")
    _close(orc.rms_norm(-y), -z, 0.0, "odd symmetry")


def pin_rmsnorm_in_the_scan(orc):
    """With qk_rmsnorm, tokens whose entries are all +-a (mean square a^2)
    are normalised to +-a/sqrt(a^2 + eps): the flag must equal the plain scan
    on those hand-normalised q and k, on every route (forward, bidirectional,
    composites), and per-token rescaling of q and k must not change the result
    (far above epsilon), while without the flag it does."""
    rng = np.random.default_rng(22)
    B, H, T, S, D = 1, 2, 5, 6, 4
    eps = orc.RMS_EPS
    aq = rng.uniform(0.5, 2.0, (B, H, T, S, 1))
    ak = rng.uniform(0.5, 2.0, (B, H, T, S, 1))
    sq = rng.choice([-1.0, 1.0], (B, H, T, S, D))
    sk = rng.choice([-1.0, 1.0], (B, H, T, S, D))
    q, k = sq * aq, sk * ak
    qn, kn = sq * aq / np.sqrt(aq * aq + eps), sk * ak / np.sqrt(ak * ak + eps)
    v = rng.standard_normal((B, H, T, S, D))
    b = rng.uniform(0, 1, (B, H, T, S))
    g = rng.uniform(0.8, 1.0, (B, H, T))
    s0 = rng.standard_normal((B, H, D, D))
    r1 = orc.scan_fwd(q, k, v, b, g, s0=s0, qk_rmsnorm=True)
    r0 = orc.scan_fwd(qn, kn, v, b, g, s0=s0)
    for n in ("states", "s_final", "o"):
        _close(r1[n], r0[n], 1e-12, "rmsnorm forward " + n)
    r1 = orc.scan_bidir_chunked(q, k, v, b, g, 2, s0=s0, qk_rmsnorm=True)
    r0 = orc.scan_bidir_chunked(qn, kn, v, b, g, 2, s0=s0)
    for n in ("states_fwd", "states_rev", "o"):
        _close(r1[n], r0[n], 1e-12, "rmsnorm bidirectional " + n)
    c1 = orc.compose(k, v, b, g, [0, 2, 5], qk_rmsnorm=True)
    c0 = orc.compose(kn, v, b, g, [0, 2, 5])
    _close(c1[0], c0[0], 1e-12, "rmsnorm composite C")
    _close(c1[1], c0[1], 1e-12, "rmsnorm composite H")
    # scale invariance on generic tokens: two independent per-token rescalings
    # by 100..1000 (epsilon then moves the result by < 1e-7 relative)
    q, k, v, b, g = _rand_case(rng, T=4, S=5, D=4)
    sc = [rng.uniform(100.0, 1000.0, x.shape[:-1] + (1,)) for x in (q, k, q, k)]
    ra = orc.scan_fwd(q * sc[0], k * sc[1], v, b, g, qk_rmsnorm=True)
    rb = orc.scan_fwd(q * sc[2], k * sc[3], v, b, g, qk_rmsnorm=True)
    _close(ra["o"], rb["o"], 1e-6, "rmsnorm scale invariance")
    rc = orc.scan_fwd(q * sc[2], k * sc[3], v, b, g)
    assert np.linalg.norm(rc["o"] - rb["o"]) > 1e-3 * np.linalg.norm(rb["o"]), \
        "without the flag, rescaled tokens must change the output"


def _loss(orc, q, k, v, b, g, s0, do, dsf, qk_rmsnorm=False):
    r = orc.scan_fwd(q, k, v, b, g, s0=s0, qk_rmsnorm=qk_rmsnorm)
    return float(np.sum(r["o"] * do) + np.sum(r["s_final"] * dsf))


def pin_backward_finite_differences(orc):
    """Every gradient of L = <do, o> + <ds_final, S_{T-1}> matches a central
    finite difference of the forward oracle, element by element (no use of
    the chain-rule formulas). Keys are kept away from the ReLU kink."""
    rng = np.random.default_rng(31)
    B, H, T, S, D = 1, 2, 3, 4, 3
    q = rng.standard_normal((B, H, T, S, D))
    k = rng.standard_normal((B, H, T, S, D))
    k = np.where(np.abs(k) < 0.1, 0.1 * np.sign(k + 1e-30) + k, k)
    v = rng.standard_normal((B, H, T, S, D))
    b = rng.uniform(0.1, 1.0, (B, H, T, S))
    g = rng.uniform(0.8, 1.0, (B, H, T))
    s0 = rng.standard_normal((B, H, D, D))
    do = rng.standard_normal((B, H, T, S, D))
    dsf = rng.standard_normal((B, H, D, D))
    grads = orc.scan_fwd_bwd(q, k, v, b, g, do, ds_final=dsf, s0=s0)
    args = {"q": q, "k": k, "v": v, "beta": b, "gamma": g, "s0": s0}
    names = {"q": "dq", "k": "dk", "v": "dv", "beta": "dbeta", "gamma": "dgamma", "s0": "ds0"}
    h = 1e-6
    for name, arr in args.items():
        fd = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            old = arr[idx]
            arr[idx] = old + h
            lp = _loss(orc, q, k, v, b, g, s0, do, dsf)
            arr[idx] = old - h
            lm = _loss(orc, q, k, v, b, g, s0, do, dsf)
            arr[idx] = old
            fd[idx] = (lp - lm) / (2 * h)
        got = grads[names[name]]
        err = np.max(np.abs(got - fd)) / max(1.0, np.max(np.abs(fd)))
        assert err < 1e-6, f"backward {names[name]}: finite-difference mismatch {err:.3e}"


def pin_backward_pure_decay(orc):
    """beta = 0: S_t = (prod_{tau<=t} gamma_tau) S0, so the gradient reaching S0
    is sum_t (prod_{tau<=t} gamma_tau) E_t with E_t = sum_s do_{t,s} q_{t,s}^T,
    and dgamma_t = sum_{t'>=t} (prod_{tau<=t'} gamma_tau / gamma_t) <E_t', S0>;
    v and the gates get zero gradient."""
    rng = np.random.default_rng(32)
    q, k, v, b, g = _rand_case(rng, T=4, S=5, D=3)
    b[:] = 0.0
    B, H, T, S, D = q.shape
    s0 = rng.standard_normal((B, H, D, D))
    do = rng.standard_normal(q.shape)
    r = orc.scan_fwd_bwd(q, k, v, b, g, do, s0=s0)
    E = np.einsum("tsi,tsj->tij", do[0, 0], q[0, 0])
    pg = np.cumprod(g[0, 0])
    want_ds0 = sum(pg[t] * E[t] for t in range(T))
    _close(r["ds0"][0, 0], want_ds0, 1e-12, "beta = 0: ds0")
    for t in range(T):
        want = sum(pg[u] / g[0, 0, t] * np.sum(E[u] * s0[0, 0]) for u in range(t, T))
        _close(r["dgamma"][0, 0, t], want, 1e-12, "beta = 0: dgamma")
    _close(r["dv"], np.zeros_like(v), 0.0, "beta = 0: dv")
    _close(r["dk"], np.zeros_like(k), 0.0, "beta = 0: dk")


def _loss_bidir(orc, q, k, v, b, g, s0, do, dsf, L, qk_rmsnorm=False):
    r = orc.scan_bidir_chunked(q, k, v, b, g, L, s0=s0, qk_rmsnorm=qk_rmsnorm)
    return float(np.sum(r["o"] * do) + np.sum(r["s_final"] * dsf))


def _fd_check(grads, args, loss, what, h=1e-6, tol=1e-6):
    names = {"q": "dq", "k": "dk", "v": "dv", "beta": "dbeta", "gamma": "dgamma", "s0": "ds0"}
    for name, arr in args.items():
        fd = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            old = arr[idx]
            arr[idx] = old + h
            lp = loss()
            arr[idx] = old - h
            lm = loss()
            arr[idx] = old
            fd[idx] = (lp - lm) / (2 * h)
        got = grads[names[name]]
        err = np.max(np.abs(got - fd)) / max(1.0, np.max(np.abs(fd)))
        assert err < tol, f"{what} {names[name]}: finite-difference mismatch {err:.3e}"


def _fd_case(rng, B, H, T, S, D):
    q = rng.standard_normal((B, H, T, S, D))
    k = rng.standard_normal((B, H, T, S, D))
    k = np.where(np.abs(k) < 0.1, 0.1 * np.sign(k + 1e-30) + k, k)
    v = rng.standard_normal((B, H, T, S, D))
    b = rng.uniform(0.1, 1.0, (B, H, T, S))
    g = rng.uniform(0.8, 1.0, (B, H, T))
    s0 = rng.standard_normal((B, H, D, D))
    do = rng.standard_normal((B, H, T, S, D))
    dsf = rng.standard_normal((B, H, D, D))
    return q, k, v, b, g, s0, do, dsf


def pin_rms_norm_bwd_finite_differences(orc):
    """rms_norm_bwd(x, dy) is the gradient of <dy, rms_norm(x)>: central
    finite differences element by element, including a token of tiny norm
    (where eps matters)."""
    rng = np.random.default_rng(35)
    x = rng.standard_normal((3, 5))
    x[2] *= 1e-3
    dy = rng.standard_normal((3, 5))
    got = orc.rms_norm_bwd(x, dy)
    h = 1e-7
    fd = np.zeros_like(x)
    for idx in np.ndindex(x.shape):
        old = x[idx]
        x[idx] = old + h
        lp = float(np.sum(orc.rms_norm(x) * dy))
        x[idx] = old - h
        lm = float(np.sum(orc.rms_norm(x) * dy))
        x[idx] = old
        fd[idx] = (lp - lm) / (2 * h)
    err = np.max(np.abs(got - fd)) / max(1.0, np.max(np.abs(fd)))
    assert err < 1e-6, f"rms_norm_bwd: finite-difference mismatch {err:.3e}"


def pin_backward_rmsnorm_finite_differences(orc):
    """The causal and the chunk-causal backward with the RMSNorm of q and k:
    every gradient against central finite differences of the forward oracle
    with the same flag."""
    rng = np.random.default_rng(36)
    q, k, v, b, g, s0, do, dsf = _fd_case(rng, 1, 1, 3, 3, 3)
    args = {"q": q, "k": k, "v": v, "beta": b, "gamma": g, "s0": s0}
    grads = orc.scan_fwd_bwd(q, k, v, b, g, do, ds_final=dsf, s0=s0, qk_rmsnorm=True)
    _fd_check(grads, args, lambda: _loss(orc, q, k, v, b, g, s0, do, dsf, True),
              "backward with RMSNorm")
    grads = orc.scan_bidir_bwd(q, k, v, b, g, 2, do, ds_final=dsf, s0=s0, qk_rmsnorm=True)
    _fd_check(grads, args, lambda: _loss_bidir(orc, q, k, v, b, g, s0, do, dsf, 2, True),
              "bidirectional backward with RMSNorm")


def pin_bidir_backward_finite_differences(orc):
    """Every gradient of L = <do, o> + <ds_final, S_{T-1}> for the chunk-causal
    bidirectional scan (o = (S_t + R_t) q) matches a central finite difference
    of the forward oracle, element by element. T = 5 with chunk length 2 has
    two full chunks and a one-frame chunk."""
    rng = np.random.default_rng(33)
    B, H, T, S, D, L = 1, 1, 5, 3, 3, 2
    q = rng.standard_normal((B, H, T, S, D))
    k = rng.standard_normal((B, H, T, S, D))
    k = np.where(np.abs(k) < 0.1, 0.1 * np.sign(k + 1e-30) + k, k)
    v = rng.standard_normal((B, H, T, S, D))
    b = rng.uniform(0.1, 1.0, (B, H, T, S))
    g = rng.uniform(0.8, 1.0, (B, H, T))
    s0 = rng.standard_normal((B, H, D, D))
    do = rng.standard_normal((B, H, T, S, D))
    dsf = rng.standard_normal((B, H, D, D))
    grads = orc.scan_bidir_bwd(q, k, v, b, g, L, do, ds_final=dsf, s0=s0)
    args = {"q": q, "k": k, "v": v, "beta": b, "gamma": g, "s0": s0}
    names = {"q": "dq", "k": "dk", "v": "dv", "beta": "dbeta", "gamma": "dgamma", "s0": "ds0"}
    h = 1e-6
    for name, arr in args.items():
        fd = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            old = arr[idx]
            arr[idx] = old + h
            lp = _loss_bidir(orc, q, k, v, b, g, s0, do, dsf, L)
            arr[idx] = old - h
            lm = _loss_bidir(orc, q, k, v, b, g, s0, do, dsf, L)
            arr[idx] = old
            fd[idx] = (lp - lm) / (2 * h)
        got = grads[names[name]]
        err = np.max(np.abs(got - fd)) / max(1.0, np.max(np.abs(fd)))
        assert err < 1e-6, f"bidirectional backward {names[name]}: finite-difference mismatch {err:.3e}"


def pin_bidir_backward_without_readout(orc):
    """With do = 0 only <ds_final, S_{T-1}> remains, which the reverse states
    do not reach: the bidirectional gradients equal the causal ones."""
    rng = np.random.default_rng(34)
    q, k, v, b, g = _rand_case(rng, T=4, S=5, D=3)
    B, H, T, S, D = q.shape
    s0 = rng.standard_normal((B, H, D, D))
    dsf = rng.standard_normal((B, H, D, D))
    do = np.zeros(q.shape)
    bi = orc.scan_bidir_bwd(q, k, v, b, g, 2, do, ds_final=dsf, s0=s0)
    ca = orc.scan_fwd_bwd(q, k, v, b, g, do, ds_final=dsf, s0=s0)
    for n in ("dq", "dk", "dv", "dbeta", "dgamma", "ds0"):
        _close(bi[n], ca[n], 1e-12, f"do = 0: {n}")


ALL_PINS = [
    pin_prepare_closed_form,
    pin_hand_example,
    pin_exact_rational_unrolled,
    pin_pure_decay,
    pin_constant_state,
    pin_single_frame_from_zero,
    pin_token_level_special_case,
    pin_exact_write,
    pin_affine_in_s0,
    pin_non_expansive,
    pin_unscaled_keys_expand,
    pin_composite_equals_sequential,
    pin_composite_pure_decay,
    pin_resume,
    pin_reverse_is_forward_on_reversed_chunk,
    pin_readout_linear,
    pin_rmsnorm_values,
    pin_rmsnorm_in_the_scan,
    pin_backward_finite_differences,
    pin_backward_pure_decay,
    pin_bidir_backward_finite_differences,
    pin_bidir_backward_without_readout,
    pin_rms_norm_bwd_finite_differences,
    pin_backward_rmsnorm_finite_differences,
]
