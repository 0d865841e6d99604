"""Plant plausible mistakes in the oracle (on the CPU) and check that the pins
catch every one of them. A mutant that no pin rejects would mean the oracle is
not pinned against that class of error."""

import math

import numpy as np
import pytest

from oracle import gdn_oracle as orc

import oracle_pins as pins


def _head_fwd_variant(kind):
    def f(q, kh, v, beta, gamma, s0, t0, t1):
        D = kh.shape[-1]
        S_state = np.zeros((D, D)) if s0 is None else np.array(s0, dtype=np.float64)
        states, outs = [], []
        for t in range(t0, t1):
            A, U = orc.frame_terms(kh[t], v[t], beta[t])
            M = orc.transition(A, gamma[t])
            prev = S_state
            if kind == "left_multiply":
                S_state = M @ S_state + U
            elif kind == "gamma_on_U":
                S_state = gamma[t] * (S_state @ (np.eye(D) - A) + U)
            elif kind == "no_delta":
                S_state = gamma[t] * S_state + U
            else:
                S_state = S_state @ M + U
            states.append(S_state.copy())
            if q is not None:
                src = prev if kind == "readout_prev_state" else S_state
                outs.append(orc.readout(src, q[t]))
        return S_state, states, outs
    return f


def _frame_terms_variant(kind):
    good = orc.frame_terms

    def f(k_hat_t, v_t, beta_t):
        A, U = good(k_hat_t, v_t, beta_t)
        Kp = np.asarray(k_hat_t, dtype=np.float64).T
        Vp = np.asarray(v_t, dtype=np.float64).T
        if kind == "U_transposed":
            return A, U.T
        if kind == "U_no_beta":
            return A, Vp @ Kp.T
        if kind == "A_no_beta":
            return Kp @ Kp.T, U
        if kind == "beta_squared":
            b = np.asarray(beta_t, dtype=np.float64)
            return (Kp * b * b) @ Kp.T, U
        raise AssertionError(kind)
    return f


def _compose_reversed(k, v, beta, gamma, offsets, key_scale=None, keys_prepared=False,
                      qk_rmsnorm=False):
    k = np.asarray(k)
    B, H, T, S, D = k.shape
    P = len(offsets) - 1
    C = np.zeros((B, H, P, D, D))
    Hc = np.zeros((B, H, P, D, D))
    for b in range(B):
        for h in range(H):
            kh = orc._keys(k[b, h], key_scale, keys_prepared, qk_rmsnorm)
            for p in range(P):
                Cp, Hp = np.eye(D), np.zeros((D, D))
                for t in range(offsets[p], offsets[p + 1]):
                    A, U = orc.frame_terms(kh[t], v[b, h, t], beta[b, h, t])
                    M = orc.transition(A, gamma[b, h, t])
                    Cp = M @ Cp
                    Hp = Hp @ M + U
                C[b, h, p], Hc[b, h, p] = Cp, Hp
    return C, Hc


def _combine_swapped(C, Hc, s0=None):
    B, H, P, D, _ = C.shape
    s_start = np.zeros((B, H, P, D, D))
    s_end = np.zeros((B, H, D, D))
    for b in range(B):
        for h in range(H):
            X = np.zeros((D, D)) if s0 is None else np.array(s0[b, h], dtype=np.float64)
            for p in range(P):
                s_start[b, h, p] = X
                X = C[b, h, p] @ X + Hc[b, h, p]
            s_end[b, h] = X
    return s_start, s_end


def _reverse_off_by_one(k, v, beta, gamma, chunk_len, key_scale=None, keys_prepared=False,
                        qk_rmsnorm=False):
    k = np.asarray(k)
    B, H, T, S, D = k.shape
    rev = np.zeros((B, H, T, D, D))
    for b in range(B):
        for h in range(H):
            kh = orc._keys(k[b, h], key_scale, keys_prepared, qk_rmsnorm)
            for (a, e) in orc.chunk_bounds(T, chunk_len):
                R = np.zeros((D, D))
                for t in range(e - 1, a - 1, -1):
                    tt = min(t + 1, e - 1)  # gates of the wrong frame
                    A, _ = orc.frame_terms(kh[tt], v[b, h, tt], beta[b, h, tt])
                    _, U = orc.frame_terms(kh[t], v[b, h, t], beta[b, h, t])
                    R = R @ orc.transition(A, gamma[b, h, tt]) + U
                    rev[b, h, t] = R
    return rev


def _bwd_variant(kind):
    """scan_fwd_bwd with one planted mistake."""
    def f(q, k, v, beta, gamma, do, ds_final=None, s0=None, key_scale=None, keys_prepared=False,
          qk_rmsnorm=False):
        q, k, v, beta, gamma, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, beta, gamma, do))
        B, H, T, S, D = k.shape
        out = {n: np.zeros_like(x) for n, x in (("dq", q), ("dk", k), ("dv", v), ("dbeta", beta),
                                                  ("dgamma", gamma))}
        out["ds0"] = np.zeros((B, H, D, D))
        c = orc.default_key_scale(D, S)
        for b in range(B):
            for h in range(H):
                kh = orc._keys(k[b, h], key_scale, keys_prepared)
                sinit = None if s0 is None else s0[b, h]
                _, states, _ = orc._head_fwd(None, kh, v[b, h], beta[b, h], gamma[b, h], sinit, 0, T)
                G = np.zeros((D, D))
                if ds_final is not None and kind != "no_ds_final":
                    G = np.array(ds_final[b, h], dtype=np.float64)
                for t in range(T - 1, -1, -1):
                    St = states[t]
                    Sp = states[t - 1] if t > 0 else (np.zeros((D, D)) if sinit is None else sinit)
                    if kind == "dM_uses_S_t":
                        Sp = St
                    G = G + do[b, h, t].T @ q[b, h, t]
                    out["dq"][b, h, t] = do[b, h, t] @ (Sp if kind == "dq_uses_prev" else St)
                    A, _ = orc.frame_terms(kh[t], v[b, h, t], beta[b, h, t])
                    dM = Sp.T @ G
                    out["dgamma"][b, h, t] = np.sum(dM * (np.eye(D) - A))
                    dA = -gamma[b, h, t] * dM
                    Ksym = dA if kind == "dk_not_symmetrised" else dA + dA.T
                    kt, vt, bt = kh[t], v[b, h, t], beta[b, h, t]
                    out["dv"][b, h, t] = bt[:, None] * (kt @ G.T)
                    db = np.einsum("si,ij,sj->s", kt, dA, kt)
                    if kind != "dbeta_no_U_term":
                        db = db + np.einsum("si,ij,sj->s", vt, G, kt)
                    out["dbeta"][b, h, t] = db
                    out["dk"][b, h, t] = bt[:, None] * (kt @ Ksym.T + vt @ G) * c * (k[b, h, t] > 0)
                    if kind != "G_not_propagated":
                        G = G @ orc.transition(A, gamma[b, h, t]).T
                out["ds0"][b, h] = G
        return out
    return f


def _bidir_bwd_variant(kind):
    """scan_bidir_bwd with one planted mistake."""
    def f(q, k, v, beta, gamma, chunk_len, do, ds_final=None, s0=None, key_scale=None,
          keys_prepared=False, qk_rmsnorm=False):
        q, k, v, beta, gamma, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, beta, gamma, do))
        B, H, T, S, D = k.shape
        fwd = orc.scan_fwd(None, k, v, beta, gamma, s0=s0, key_scale=key_scale,
                           keys_prepared=keys_prepared, with_output=False)
        rev = orc.scan_reverse_chunked(k, v, beta, gamma, chunk_len, key_scale=key_scale,
                                       keys_prepared=keys_prepared)
        out = {n: np.zeros_like(x) for n, x in (("dq", q), ("dk", k), ("dv", v), ("dbeta", beta),
                                                  ("dgamma", gamma))}
        out["ds0"] = np.zeros((B, H, D, D))
        c = orc.default_key_scale(D, S)
        for b in range(B):
            for h in range(H):
                kh = orc._keys(k[b, h], key_scale, keys_prepared)
                St, Rt = fwd["states"][b, h], rev[b, h]
                sinit = np.zeros((D, D)) if s0 is None else np.asarray(s0[b, h], dtype=np.float64)
                A = [orc.frame_terms(kh[t], v[b, h, t], beta[b, h, t])[0] for t in range(T)]
                M = [orc.transition(A[t], gamma[b, h, t]) for t in range(T)]
                E = [do[b, h, t].T @ q[b, h, t] for t in range(T)]
                dU = [np.zeros((D, D)) for _ in range(T)]
                dM = [np.zeros((D, D)) for _ in range(T)]
                G = np.zeros((D, D)) if ds_final is None else np.array(ds_final[b, h], dtype=np.float64)
                for t in range(T - 1, -1, -1):
                    G = G + E[t]
                    dU[t] += G
                    dM[t] += (St[t - 1] if t > 0 else sinit).T @ G
                    G = G @ M[t].T
                out["ds0"][b, h] = G
                F = np.zeros((D, D))
                for (a, e) in orc.chunk_bounds(T, chunk_len):
                    for t in range(a, e):
                        if t == a and kind != "F_not_reset":
                            F = E[t]
                        elif t == 0:
                            F = E[t]
                        else:
                            F = E[t] + F @ M[t if kind == "F_same_frame_M" else t - 1].T
                        if kind != "dU_no_F":
                            dU[t] += F
                        if t + 1 < e and kind != "dM_no_R_term":
                            dM[t] += Rt[t + 1].T @ F
                for t in range(T):
                    Sq = St[t] if kind == "dq_causal_only" else St[t] + Rt[t]
                    out["dq"][b, h, t] = do[b, h, t] @ Sq
                    out["dgamma"][b, h, t] = np.sum(dM[t] * (np.eye(D) - A[t]))
                    dA = -gamma[b, h, t] * dM[t]
                    kt, vt, bt = kh[t], v[b, h, t], beta[b, h, t]
                    dkh = bt[:, None] * (kt @ (dA + dA.T).T + vt @ dU[t])
                    out["dv"][b, h, t] = bt[:, None] * (kt @ dU[t].T)
                    out["dbeta"][b, h, t] = (np.einsum("si,ij,sj->s", kt, dA, kt)
                                             + np.einsum("si,ij,sj->s", vt, dU[t], kt))
                    out["dk"][b, h, t] = dkh if keys_prepared else dkh * c * (k[b, h, t] > 0)
        return out
    return f


def _rms_bwd_flipped(x, dy, eps):
    """rms_norm_bwd with the sign of the projection term flipped."""
    x = np.asarray(x, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    D = x.shape[-1]
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    return r * dy + r ** 3 * np.sum(x * dy, axis=-1, keepdims=True) * x / D


MUTANTS = {
    "U_transposed": ("frame_terms", _frame_terms_variant("U_transposed")),
    "U_no_beta": ("frame_terms", _frame_terms_variant("U_no_beta")),
    "A_no_beta": ("frame_terms", _frame_terms_variant("A_no_beta")),
    "beta_squared": ("frame_terms", _frame_terms_variant("beta_squared")),
    "M_plus_A": ("transition", lambda A, g: float(g) * (np.eye(A.shape[0]) + A)),
    "M_no_gamma": ("transition", lambda A, g: np.eye(A.shape[0]) - A),
    "left_multiply": ("_head_fwd", _head_fwd_variant("left_multiply")),
    "gamma_on_U": ("_head_fwd", _head_fwd_variant("gamma_on_U")),
    "no_delta": ("_head_fwd", _head_fwd_variant("no_delta")),
    "readout_prev_state": ("_head_fwd", _head_fwd_variant("readout_prev_state")),
    "readout_transposed": ("readout", lambda st, q: np.asarray(q, dtype=np.float64) @ st),
    "scale_1_over_sqrt_S": ("default_key_scale", lambda D, S: 1.0 / math.sqrt(S)),
    "scale_1_over_D": ("default_key_scale", lambda D, S: 1.0 / D / math.sqrt(S)),
    "no_relu": ("prepare_keys", lambda k, key_scale=None, rmsnorm=False:
                np.asarray(orc.rms_norm(k) if rmsnorm else k, dtype=np.float64)
                * (key_scale if key_scale and key_scale > 0
                   else 1.0 / math.sqrt(np.shape(k)[-1] * np.shape(k)[-2]))),
    "reverse_not_reset": ("chunk_bounds", lambda T, L: [(0, T)]),
    "reverse_wrong_gates": ("scan_reverse_chunked", _reverse_off_by_one),
    "compose_reversed_product": ("compose", _compose_reversed),
    "bwd_dM_uses_S_t": ("scan_fwd_bwd", _bwd_variant("dM_uses_S_t")),
    "bwd_dq_uses_prev": ("scan_fwd_bwd", _bwd_variant("dq_uses_prev")),
    "bwd_dk_not_symmetrised": ("scan_fwd_bwd", _bwd_variant("dk_not_symmetrised")),
    "bwd_dbeta_no_U_term": ("scan_fwd_bwd", _bwd_variant("dbeta_no_U_term")),
    "bwd_G_not_propagated": ("scan_fwd_bwd", _bwd_variant("G_not_propagated")),
    "bwd_no_ds_final": ("scan_fwd_bwd", _bwd_variant("no_ds_final")),
    "rms_over_tokens": ("rms_norm", lambda x, eps=orc.RMS_EPS: np.asarray(x, dtype=np.float64)
                        / np.sqrt(np.mean(np.asarray(x, dtype=np.float64) ** 2, axis=-2,
                                          keepdims=True) + eps)),
    "rms_sum_not_mean": ("rms_norm", lambda x, eps=orc.RMS_EPS: np.asarray(x, dtype=np.float64)
                         / np.sqrt(np.sum(np.asarray(x, dtype=np.float64) ** 2, axis=-1,
                                          keepdims=True) + eps)),
    "rms_no_sqrt": ("rms_norm", lambda x, eps=orc.RMS_EPS: np.asarray(x, dtype=np.float64)
                    / (np.mean(np.asarray(x, dtype=np.float64) ** 2, axis=-1, keepdims=True) + eps)),
    "rms_q_ignored": ("_queries", lambda q, rmsnorm: None if q is None
                      else np.asarray(q, dtype=np.float64)),
    "combine_left_multiply": ("combine", _combine_swapped),
    "rms_bwd_no_projection": ("rms_norm_bwd", lambda x, dy, eps=orc.RMS_EPS:
                              np.asarray(dy, dtype=np.float64)
                              / np.sqrt(np.mean(np.asarray(x, dtype=np.float64) ** 2, axis=-1,
                                                keepdims=True) + eps)),
    "rms_bwd_plus_projection": ("rms_norm_bwd", lambda x, dy, eps=orc.RMS_EPS:
                                _rms_bwd_flipped(x, dy, eps)),
    "bidir_bwd_F_not_reset": ("scan_bidir_bwd", _bidir_bwd_variant("F_not_reset")),
    "bidir_bwd_F_same_frame_M": ("scan_bidir_bwd", _bidir_bwd_variant("F_same_frame_M")),
    "bidir_bwd_dM_no_R_term": ("scan_bidir_bwd", _bidir_bwd_variant("dM_no_R_term")),
    "bidir_bwd_dq_causal_only": ("scan_bidir_bwd", _bidir_bwd_variant("dq_causal_only")),
    "bidir_bwd_dU_no_F": ("scan_bidir_bwd", _bidir_bwd_variant("dU_no_F")),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(orc, attr, fn)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(orc)
        except (AssertionError, ValueError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"no pin rejects the mutant {name}"
