"""Shared helpers of the GPU parity tests: device upload of seeded inputs and
relative Frobenius errors. Expected values always come from the float64 oracle."""

from __future__ import annotations

import sys

import numpy as np
import torch

from frame_wise_gated_amd import inputs as gi

DEV = "cuda:0"
TOL_F32 = 1e-5   # relative Frobenius error bound for fp32 workloads
TOL_BF16 = 2e-2  # relative Frobenius error bound for bf16 workloads


def say(*a):
    """Name the case before each GPU step (flushed, so it survives a crash)."""
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def tol(w: gi.Workload) -> float:
    return TOL_F32 if w.io == "f32" else TOL_BF16


def bits_to_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def upload(x: dict, w: gi.Workload) -> dict:
    """Device tensors of a batch_inputs() result."""
    out = {}
    for n in ("q", "k", "v"):
        if w.io == "bf16":
            out[n] = bits_to_dev(x[n + "_bits"])
        else:
            out[n] = torch.from_numpy(np.ascontiguousarray(x[n])).to(DEV)
    out["beta"] = torch.from_numpy(np.ascontiguousarray(x["beta"])).to(DEV)
    out["gamma"] = torch.from_numpy(np.ascontiguousarray(x["gamma"])).to(DEV)
    return out


def head_arrays(x: dict, b: int, h: int) -> dict:
    """One (b, h) slice as float64 arrays with [1, 1, ...] leading dims (oracle input)."""
    return {n: np.asarray(x[n][b, h], dtype=np.float64)[None, None] for n in ("q", "k", "v", "beta", "gamma")}


def rel_fro(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    num = np.linalg.norm(got - ref)
    if den == 0.0:
        return float(num)
    return float(num / den)


def host(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def rne_bf16_bits(x) -> np.ndarray:
    """bf16 bit patterns of float64 values rounded ONCE to nearest even (8
    significant bits); finite values in the normal range of bf16."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                      # x = m 2^e, 0.5 <= |m| < 1
    r = np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)  # np.rint rounds half to even
    return (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def frame_errs(got, ref) -> np.ndarray:
    """Relative Frobenius error of every frame: arrays [T, ...] (one head)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    T = ref.shape[0]
    g = got.reshape(T, -1)
    r = ref.reshape(T, -1)
    den = np.linalg.norm(r, axis=1)
    num = np.linalg.norm(g - r, axis=1)
    return num / np.where(den > 0, den, 1.0)


def token_errs(got, ref, floor: float = 1e-3) -> np.ndarray:
    """Relative error of every token vector (last axis), arrays [T, S, D]:
    |g_s - r_s| / max(|r_s|, floor * rms_s'|r_s'|) with the rms over the
    frame's tokens, so that a token whose reference is (near) zero is measured
    against the frame's typical token norm."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rn = np.linalg.norm(ref, axis=-1)
    typ = np.sqrt(np.mean(rn * rn, axis=-1, keepdims=True))
    den = np.maximum(rn, floor * typ)
    num = np.linalg.norm(got - ref, axis=-1)
    return num / np.where(den > 0, den, 1.0)
