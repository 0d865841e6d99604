"""Float64 CPU oracle for the frame-wise Gated DeltaNet (GDN) frame scan.

TEST INFRASTRUCTURE. This module is the correctness reference for the HIP
library in ``frame_wise_gated_amd``. Only the test suite, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may import or
call it. The product path never routes through it, and it imports nothing from
the product package (the two share no code).

It is the plain definition written out, one frame at a time, in float64, with
the pages' notation. Sources (web pages, cited by title and section):

* [P1] blog.hotdry.top, "SANA-WM: 2.6B 参数分布式 Diffusion Transformer 实现消费级
  GPU 分钟级 720p 视频生成" -- section "混合线性注意力" (the three equations for
  S_t, M_t, U_t and the paragraph on the 1/sqrt(D*S) key scaling) and section
  "显存分片: Context-Parallel 的工程实现" (the composite identity
  S_end = S_start * C_p + H_p).
* [P2] xiejiayun.github.io, "好文共赏 | SANA-WM" -- section 2.1 "Frame-wise GDN"
  (token-level GDN equation, frame-wise equation, trace inequality).
* [P3] hyper.ai paper page 2605.15178 -- "方法" (method) section: the
  chunk-causal variant restarts its reverse temporal scan at every chunk
  boundary.

Array conventions (per batch b and head h, frames t = 0..T-1, tokens s):
q, k, v are [B, H, T, S, D]; beta is [B, H, T, S]; gamma is [B, H, T];
states are [B, H, T, D, D] with entry (i, j) = (value dim, key dim).
The pages write K_t, V_t as D x S matrices whose columns are tokens, so the
page's K_t is ``k[t].T`` here.

Readings where the pages are silent (each also listed in the design notes):
* the readout of token s in frame t uses the state after frame t: o = S_t q;
* q is used as given (no ReLU, no scaling);
* the reverse scan of the chunk-causal variant is R_t = R_{t+1} M_t + U_t,
  started from zero after the last frame of each chunk, and the
  bidirectional readout is o = (S_t + R_t) q;
* chunks of the reverse scan are [0, L), [L, 2L), ...; the last may be short;
* the optional RMSNorm that [P1] lists inside its fused kernel (section
  "显存分片: Context-Parallel 的工程实现", the paragraph on the fused Triton
  kernel: RMSNorm, ReLU, key scaling and the scan in one operator) normalises
  each token of q and of k over the head dimension, before the key's ReLU and
  scale, with epsilon 1e-6 and unit weight (the pages give neither).

Every function here is pinned by tests under ``tests/`` (closed forms, brute
force, exact rational arithmetic, invariants, and for the two backward
functions central finite differences of the forward definitions); none is
"parity unpinned".
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "RMS_EPS",
    "rms_norm",
    "rms_norm_bwd",
    "default_key_scale",
    "prepare_keys",
    "frame_terms",
    "transition",
    "scan_fwd",
    "scan_reverse_chunked",
    "scan_bidir_chunked",
    "compose",
    "combine",
    "readout",
    "scan_fwd_bwd",
    "scan_bidir_bwd",
]


def default_key_scale(D: int, S: int) -> float:
    """c = 1/sqrt(D*S): [P1] "混合线性注意力" key-scaling paragraph; [P2] 2.1."""
    return 1.0 / math.sqrt(float(D) * float(S))


RMS_EPS = 1e-6


def rms_norm(x, eps: float = RMS_EPS):
    """Per-token RMS normalisation over the last axis (the head dimension):
    x / sqrt(mean(x^2) + eps), unit weight. The RMSNorm step of the fused
    operator in [P1] "显存分片: Context-Parallel 的工程实现"; axis, epsilon and
    weight are this module's reading (see the module docstring)."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def rms_norm_bwd(x, dy, eps: float = RMS_EPS):
    """Gradient through y = rms_norm(x) per token: with r = (mean(x^2) +
    eps)^(-1/2), dy_i/dx_j = r delta_ij - r^3 x_i x_j / D, so
    dx = r dy - r^3 (x . dy) x / D (the derivative of the definition above)."""
    x = np.asarray(x, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    D = x.shape[-1]
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    return r * dy - r ** 3 * np.sum(x * dy, axis=-1, keepdims=True) * x / D


def prepare_keys(k, key_scale: float | None = None, rmsnorm: bool = False):
    """K_hat = ReLU(k) * c (with ``rmsnorm``: ReLU(rms_norm(k)) * c),
    elementwise per token, in float64.

    [P1] "混合线性注意力": keys are scaled by 1/sqrt(D*S); [P2] 2.1 states the
    trace bound that this scaling buys. ``key_scale`` <= 0 or None selects the
    default c for the array's own D (last axis) and S (second-to-last axis).
    """
    k = np.asarray(k, dtype=np.float64)
    if key_scale is None or key_scale <= 0:
        key_scale = default_key_scale(k.shape[-1], k.shape[-2])
    if rmsnorm:
        k = rms_norm(k)
    return np.maximum(k, 0.0) * float(key_scale)


def frame_terms(k_hat_t, v_t, beta_t):
    """A_t = K_t beta_t K_t^T and U_t = V_t beta_t K_t^T for one frame.

    [P1] "混合线性注意力", the M_t and U_t equations; beta_t is the diagonal
    matrix of per-token gates. Inputs are [S, D] (tokens as rows), so the
    page's D x S matrices are the transposes.
    """
    Kp = np.asarray(k_hat_t, dtype=np.float64).T  # D x S, columns are tokens
    Vp = np.asarray(v_t, dtype=np.float64).T
    b = np.asarray(beta_t, dtype=np.float64)
    KB = Kp * b[None, :]  # K_t beta_t
    A = KB @ Kp.T
    U = Vp @ (b[:, None] * Kp.T)
    return A, U


def transition(A_t, gamma_t):
    """M_t = gamma_t (I - A_t): [P1] "混合线性注意力", the M_t equation."""
    D = A_t.shape[0]
    return float(gamma_t) * (np.eye(D) - A_t)


def readout(state, q_t):
    """o_{t,s} = state q_{t,s} for every token: rows of the result are tokens."""
    return np.asarray(q_t, dtype=np.float64) @ state.T


def _keys(k, key_scale, keys_prepared, rmsnorm=False):
    if keys_prepared:
        return np.asarray(k, dtype=np.float64)
    return prepare_keys(k, key_scale, rmsnorm)


def _queries(q, rmsnorm):
    if q is None:
        return None
    return rms_norm(q) if rmsnorm else np.asarray(q, dtype=np.float64)


def _head_fwd(q, kh, v, beta, gamma, s0, t0, t1):
    """Forward frame loop over frames [t0, t1) of one head from state s0."""
    D = kh.shape[-1]
    S_state = np.zeros((D, D)) if s0 is None else np.array(s0, dtype=np.float64)
    states = []
    outs = []
    for t in range(t0, t1):
        A, U = frame_terms(kh[t], v[t], beta[t])
        M = transition(A, gamma[t])
        S_state = S_state @ M + U  # [P1] the S_t equation
        states.append(S_state.copy())
        if q is not None:
            outs.append(readout(S_state, q[t]))
    return S_state, states, outs


def scan_fwd(q, k, v, beta, gamma, s0=None, key_scale=None, keys_prepared=False,
             with_output=True, qk_rmsnorm=False):
    """Causal frame scan S_t = S_{t-1} M_t + U_t with per-token readout.

    Inputs as in the module docstring; ``s0`` is [B, H, D, D] or None (zero).
    ``qk_rmsnorm`` applies rms_norm to q and (unless ``keys_prepared``) to k.
    Returns a dict with ``states`` [B,H,T,D,D], ``s_final`` [B,H,D,D] and
    ``o`` [B,H,T,S,D] (absent when ``with_output`` is False or q is None).
    """
    k = np.asarray(k)
    B, H, T, S, D = k.shape
    states = np.zeros((B, H, T, D, D))
    s_final = np.zeros((B, H, D, D))
    o = np.zeros((B, H, T, S, D)) if (with_output and q is not None) else None
    for b in range(B):
        for h in range(H):
            kh = _keys(k[b, h], key_scale, keys_prepared, qk_rmsnorm)
            qh = None if o is None else _queries(q[b, h], qk_rmsnorm)
            sinit = None if s0 is None else s0[b, h]
            fin, st, outs = _head_fwd(qh, kh, v[b, h], beta[b, h], gamma[b, h],
                                      sinit, 0, T)
            s_final[b, h] = fin
            if T:
                states[b, h] = np.stack(st)
            if o is not None and T:
                o[b, h] = np.stack(outs)
    out = {"states": states, "s_final": s_final}
    if o is not None:
        out["o"] = o
    return out


def chunk_bounds(T: int, chunk_len: int):
    """Uniform chunks [0, L), [L, 2L), ... of the chunk-causal reverse scan."""
    return [(a, min(a + chunk_len, T)) for a in range(0, T, chunk_len)]


def scan_reverse_chunked(k, v, beta, gamma, chunk_len, key_scale=None,
                         keys_prepared=False, qk_rmsnorm=False):
    """Reverse temporal scan restarted at every chunk boundary ([P3], method).

    Inside chunk [a, b): R_{b-1} = U_{b-1} (zero state after the chunk's last
    frame) and R_t = R_{t+1} M_t + U_t for t = b-2 down to a, with each frame's
    own M_t, U_t. Returns ``states_rev`` [B,H,T,D,D].
    """
    k = np.asarray(k)
    B, H, T, S, D = k.shape
    rev = np.zeros((B, H, T, D, D))
    for b in range(B):
        for h in range(H):
            kh = _keys(k[b, h], key_scale, keys_prepared, qk_rmsnorm)
            for (a, e) in chunk_bounds(T, chunk_len):
                R = np.zeros((D, D))
                for t in range(e - 1, a - 1, -1):
                    A, U = frame_terms(kh[t], v[b, h, t], beta[b, h, t])
                    R = R @ transition(A, gamma[b, h, t]) + U
                    rev[b, h, t] = R
    return rev


def scan_bidir_chunked(q, k, v, beta, gamma, chunk_len, s0=None, key_scale=None,
                       keys_prepared=False, qk_rmsnorm=False):
    """Chunk-causal bidirectional scan: causal forward states plus the reverse
    chunk scan, read out together as o = (S_t + R_t) q.

    ``chunk_len`` >= T gives the full-sequence bidirectional variant.
    """
    fwd = scan_fwd(q, k, v, beta, gamma, s0=s0, key_scale=key_scale,
                   keys_prepared=keys_prepared, with_output=False, qk_rmsnorm=qk_rmsnorm)
    rev = scan_reverse_chunked(k, v, beta, gamma, chunk_len, key_scale=key_scale,
                               keys_prepared=keys_prepared, qk_rmsnorm=qk_rmsnorm)
    B, H, T, S, D = np.asarray(k).shape
    o = np.zeros((B, H, T, S, D))
    for b in range(B):
        for h in range(H):
            for t in range(T):
                o[b, h, t] = readout(fwd["states"][b, h, t] + rev[b, h, t],
                                     _queries(q[b, h, t], qk_rmsnorm))
    return {"states_fwd": fwd["states"], "states_rev": rev,
            "s_final": fwd["s_final"], "o": o}


def compose(k, v, beta, gamma, offsets, key_scale=None, keys_prepared=False,
            qk_rmsnorm=False):
    """Per-chunk affine composites (C_p, H_p) with S_end = S_start C_p + H_p.

    [P1] "显存分片: Context-Parallel 的工程实现": C_p is the ordered product of
    the chunk's transitions and H_p the chunk's scan from a zero state.
    ``offsets`` holds P+1 ascending frame indices, offsets[0] = 0 and
    offsets[P] = T. Returns C, Hc as [B, H, P, D, D].
    """
    k = np.asarray(k)
    B, H, T, S, D = k.shape
    P = len(offsets) - 1
    C = np.zeros((B, H, P, D, D))
    Hc = np.zeros((B, H, P, D, D))
    for b in range(B):
        for h in range(H):
            kh = _keys(k[b, h], key_scale, keys_prepared, qk_rmsnorm)
            for p in range(P):
                Cp = np.eye(D)
                Hp = np.zeros((D, D))
                for t in range(offsets[p], offsets[p + 1]):
                    A, U = frame_terms(kh[t], v[b, h, t], beta[b, h, t])
                    M = transition(A, gamma[b, h, t])
                    Cp = Cp @ M
                    Hp = Hp @ M + U
                C[b, h, p] = Cp
                Hc[b, h, p] = Hp
    return C, Hc


def combine(C, Hc, s0=None):
    """Exact chunk start states from the composites, left to right.

    s_start[0] = S0 and s_start[p+1] = s_start[p] C_p + H_p ([P1], the
    composite identity applied chunk after chunk). Returns s_start
    [B, H, P, D, D] and the state after the last chunk [B, H, D, D].
    """
    B, H, P, D, _ = C.shape
    s_start = np.zeros((B, H, P, D, D))
    s_end = np.zeros((B, H, D, D))
    for b in range(B):
        for h in range(H):
            X = np.zeros((D, D)) if s0 is None else np.array(s0[b, h], dtype=np.float64)
            for p in range(P):
                s_start[b, h, p] = X
                X = X @ C[b, h, p] + Hc[b, h, p]
            s_end[b, h] = X
    return s_start, s_end


def scan_fwd_bwd(q, k, v, beta, gamma, do, ds_final=None, s0=None, key_scale=None,
                 keys_prepared=False, qk_rmsnorm=False):
    """Reverse-mode gradients of the causal frame scan.

    The scalar is L = sum_{t,s} <do_{t,s}, o_{t,s}> + <ds_final, S_{T-1}>,
    with o_{t,s} = S_t q_{t,s} and S_t = S_{t-1} M_t + U_t as in scan_fwd
    ([P1] "混合线性注意力"). The chain rule is taken step by step through the
    forward definition, frames in reverse order. With G the gradient of L with
    respect to S_t:

        G      += sum_s do_{t,s} q_{t,s}^T            (readout of frame t)
        dq_t,s  = S_t^T do_{t,s}
        dU_t    = G
        dM_t    = S_{t-1}^T G                        (S_t = S_{t-1} M_t + U_t)
        dgamma_t = <dM_t, I - A_t>,   dA_t = -gamma_t dM_t
        G       = G M_t^T                            (gradient reaching S_{t-1})

    and, through A_t = sum_s beta_s k_s k_s^T and U_t = sum_s beta_s v_s k_s^T
    (k the prepared keys), dk_s = beta_s (dA + dA^T) k_s + beta_s G^T v_s,
    dbeta_s = k_s^T dA k_s + v_s^T G k_s, dv_s = beta_s G k_s; raw keys then
    pass through the key scale and the ReLU (gradient zero where k <= 0).
    With ``qk_rmsnorm`` the readout and E use the normalised queries and the
    keys are normalised before the ReLU (scan_fwd); dq and dk then pass back
    through rms_norm_bwd.
    Returns dq, dk, dv [B,H,T,S,D], dbeta [B,H,T,S], dgamma [B,H,T] and
    ds0 [B,H,D,D] (the gradient reaching the initial state).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    gamma = np.asarray(gamma, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    B, H, T, S, D = k.shape
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    dbeta = np.zeros_like(beta)
    dgamma = np.zeros_like(gamma)
    ds0 = np.zeros((B, H, D, D))
    c = None
    if not keys_prepared:
        c = key_scale if (key_scale is not None and key_scale > 0) else default_key_scale(D, S)
    for b in range(B):
        for h in range(H):
            kh = _keys(k[b, h], key_scale, keys_prepared, qk_rmsnorm)
            qh = _queries(q[b, h], qk_rmsnorm)
            kt_pre = rms_norm(k[b, h]) if qk_rmsnorm else k[b, h]  # keys before the ReLU
            sinit = None if s0 is None else s0[b, h]
            _, states, _ = _head_fwd(None, kh, v[b, h], beta[b, h], gamma[b, h], sinit, 0, T)
            G = np.zeros((D, D)) if ds_final is None else np.array(ds_final[b, h], dtype=np.float64)
            for t in range(T - 1, -1, -1):
                St = states[t]
                if t > 0:
                    Sp = states[t - 1]
                else:
                    Sp = np.zeros((D, D)) if sinit is None else np.asarray(sinit, dtype=np.float64)
                G = G + do[b, h, t].T @ qh[t]
                dqh = do[b, h, t] @ St
                dq[b, h, t] = rms_norm_bwd(q[b, h, t], dqh) if qk_rmsnorm else dqh
                A, _ = frame_terms(kh[t], v[b, h, t], beta[b, h, t])
                dM = Sp.T @ G
                dgamma[b, h, t] = np.sum(dM * (np.eye(D) - A))
                dA = -gamma[b, h, t] * dM
                Ksym = dA + dA.T
                kt, vt, bt = kh[t], v[b, h, t], beta[b, h, t]
                dkh = bt[:, None] * (kt @ Ksym.T + vt @ G)
                dv[b, h, t] = bt[:, None] * (kt @ G.T)
                dbeta[b, h, t] = np.einsum("si,ij,sj->s", kt, dA, kt) + np.einsum("si,ij,sj->s", vt, G, kt)
                if keys_prepared:
                    dk[b, h, t] = dkh
                else:
                    dpre = dkh * c * (kt_pre[t] > 0)
                    dk[b, h, t] = rms_norm_bwd(k[b, h, t], dpre) if qk_rmsnorm else dpre
                G = G @ transition(A, gamma[b, h, t]).T
            ds0[b, h] = G
    return {"dq": dq, "dk": dk, "dv": dv, "dbeta": dbeta, "dgamma": dgamma, "ds0": ds0}


def scan_bidir_bwd(q, k, v, beta, gamma, chunk_len, do, ds_final=None, s0=None,
                   key_scale=None, keys_prepared=False, qk_rmsnorm=False):
    """Reverse-mode gradients of the chunk-causal bidirectional scan.

    The scalar is L = sum_{t,s} <do_{t,s}, o_{t,s}> + <ds_final, S_{T-1}> with
    o_{t,s} = (S_t + R_t) q_{t,s} (scan_bidir_chunked: the causal states S_t
    and the reverse states R_t of the chunk holding t, [P3] method). The chain
    rule runs through both recurrences of the definition:

    * causal part, frames in reverse order (as in scan_fwd_bwd): G_t, the
      gradient of L with respect to S_t, is E_t + G_{t+1} M_{t+1}^T (plus
      ds_final at t = T-1), E_t = sum_s do_{t,s} q_{t,s}^T; S_t = S_{t-1} M_t
      + U_t adds G_t to dU_t and S_{t-1}^T G_t to dM_t;
    * reverse part, inside each chunk [a, e) in forward order: R_t feeds o_t
      and R_{t-1} = R_t M_{t-1} + U_{t-1}, so its gradient is F_a = E_a and
      F_t = E_t + F_{t-1} M_{t-1}^T; R_t = R_{t+1} M_t + U_t adds F_t to dU_t
      and, when t + 1 < e, R_{t+1}^T F_t to dM_t (the chunk's last frame starts
      from a zero state).

    Then per frame and token exactly as in scan_fwd_bwd with dU_t in place of
    G: dgamma_t = <dM_t, I - A_t>, dA_t = -gamma_t dM_t, dk_s = beta_s (dA +
    dA^T) k_s + beta_s dU^T v_s, dbeta_s = k_s^T dA k_s + v_s^T dU k_s,
    dv_s = beta_s dU k_s, and dq_{t,s} = (S_t + R_t)^T do_{t,s}. Raw keys pass
    through the key scale and the ReLU; ``qk_rmsnorm`` as in scan_fwd_bwd.
    Returns the same dict as scan_fwd_bwd.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    gamma = np.asarray(gamma, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    B, H, T, S, D = k.shape
    fwd = scan_fwd(None, k, v, beta, gamma, s0=s0, key_scale=key_scale,
                   keys_prepared=keys_prepared, with_output=False, qk_rmsnorm=qk_rmsnorm)
    rev = scan_reverse_chunked(k, v, beta, gamma, chunk_len, key_scale=key_scale,
                               keys_prepared=keys_prepared, qk_rmsnorm=qk_rmsnorm)
    out = {n: np.zeros_like(x) for n, x in (("dq", q), ("dk", k), ("dv", v), ("dbeta", beta),
                                              ("dgamma", gamma))}
    out["ds0"] = np.zeros((B, H, D, D))
    c = None
    if not keys_prepared:
        c = key_scale if (key_scale is not None and key_scale > 0) else default_key_scale(D, S)
    for b in range(B):
        for h in range(H):
            kh = _keys(k[b, h], key_scale, keys_prepared, qk_rmsnorm)
            qh = _queries(q[b, h], qk_rmsnorm)
            k_pre = rms_norm(k[b, h]) if qk_rmsnorm else k[b, h]  # keys before the ReLU
            St = fwd["states"][b, h]
            Rt = rev[b, h]
            sinit = np.zeros((D, D)) if s0 is None else np.asarray(s0[b, h], dtype=np.float64)
            A = [frame_terms(kh[t], v[b, h, t], beta[b, h, t])[0] for t in range(T)]
            M = [transition(A[t], gamma[b, h, t]) for t in range(T)]
            E = [do[b, h, t].T @ qh[t] for t in range(T)]
            dU = [np.zeros((D, D)) for _ in range(T)]
            dM = [np.zeros((D, D)) for _ in range(T)]
            # causal part
            G = np.zeros((D, D)) if ds_final is None else np.array(ds_final[b, h], dtype=np.float64)
            for t in range(T - 1, -1, -1):
                G = G + E[t]
                Sp = St[t - 1] if t > 0 else sinit
                dU[t] += G
                dM[t] += Sp.T @ G
                G = G @ M[t].T
            out["ds0"][b, h] = G
            # reverse part, chunk by chunk
            for (a, e) in chunk_bounds(T, chunk_len):
                F = np.zeros((D, D))
                for t in range(a, e):
                    F = E[t] if t == a else E[t] + F @ M[t - 1].T
                    dU[t] += F
                    if t + 1 < e:
                        dM[t] += Rt[t + 1].T @ F
            for t in range(T):
                dqh = do[b, h, t] @ (St[t] + Rt[t])
                out["dq"][b, h, t] = rms_norm_bwd(q[b, h, t], dqh) if qk_rmsnorm else dqh
                out["dgamma"][b, h, t] = np.sum(dM[t] * (np.eye(D) - A[t]))
                dA = -gamma[b, h, t] * dM[t]
                kt, vt, bt = kh[t], v[b, h, t], beta[b, h, t]
                dkh = bt[:, None] * (kt @ (dA + dA.T).T + vt @ dU[t])
                out["dv"][b, h, t] = bt[:, None] * (kt @ dU[t].T)
                out["dbeta"][b, h, t] = (np.einsum("si,ij,sj->s", kt, dA, kt)
                                         + np.einsum("si,ij,sj->s", vt, dU[t], kt))
                if keys_prepared:
                    out["dk"][b, h, t] = dkh
                else:
                    dpre = dkh * c * (k_pre[t] > 0)
                    out["dk"][b, h, t] = rms_norm_bwd(k[b, h, t], dpre) if qk_rmsnorm else dpre
    return out
