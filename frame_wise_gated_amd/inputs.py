"""Seeded synthetic inputs for the frame-wise GDN scan.

This module only draws random numbers and rounds them to the storage type.
It holds none of the method's arithmetic (no ReLU, no key scaling, no
recurrence), so both the HIP path and the float64 oracle may consume what it
produces.

Workload shapes follow the pages: S = 80 x 45 = 3600 latent tokens per 720p
frame (xiejiayun.github.io "好文共赏 | SANA-WM", section 2.1), 121 latent frames
for a 961-raw-frame (60 s at 16 fps) clip and T = 11 for a 5 s clip
(trdm.cn SANA-WM guide, section 七), chunk length 10 for the chunk-causal
stress case. Head count H = 16 and head dim D = 128 are the layer geometry
the scan is measured on.

Draw order per (config tag, seed, b, h) slice, with
``numpy.random.default_rng([tag, seed, b, h])``: q, k, v as [T, S, D]
float32 N(0, 1); then beta [T, S]; then gamma [T]. For bf16 workloads q, k, v
are rounded to bfloat16 with round-to-nearest-even, and those rounded values
are what every consumer sees.
"""

from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "workload",
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
    "head_inputs",
    "batch_inputs",
]


@dataclass(frozen=True)
class Workload:
    tag: int            # seeds the generator together with (seed, b, h)
    name: str
    B: int
    H: int
    T: int
    S: int
    D: int
    io: str             # "f32" or "bf16"
    beta: str           # "uniform" (U[0,1)) or "beta05" (Beta(0.5, 0.5))
    gamma_lo: float     # gamma ~ U[gamma_lo, 1)
    mode: str           # "fwd" or "bidir"
    time_chunks: int = 1    # composite time chunks of the forward scan
    chunk_len: int = 0      # reverse-scan chunk length (bidir only)

    def with_shape(self, **kw) -> "Workload":
        return replace(self, **kw)

    @property
    def frame_heads(self) -> int:
        return self.B * self.H * self.T


WORKLOADS = {
    1: Workload(1, "tiny_f32_causal_D16_S12_T8", 1, 1, 8, 12, 16, "f32", "uniform", 0.9, "fwd"),
    2: Workload(2, "head_720p_5s_H1_T11", 1, 1, 11, 3600, 128, "bf16", "uniform", 0.95, "fwd"),
    3: Workload(3, "layer_720p_5s_H16_T11", 1, 16, 11, 3600, 128, "bf16", "uniform", 0.95, "fwd"),
    4: Workload(4, "layer_720p_60s_H16_T121_cp8", 1, 16, 121, 3600, 128, "bf16", "uniform", 0.98,
                "fwd", time_chunks=8),
    5: Workload(5, "layer_720p_60s_H16_T121_bidir10", 1, 16, 121, 3600, 128, "bf16", "beta05",
                0.999, "bidir", time_chunks=8, chunk_len=10),
}


def workload(idx: int) -> Workload:
    return WORKLOADS[idx]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16, nearest-even; returns the uint16 bit patterns.

    Inputs are finite (normal draws), so no NaN handling is needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def head_inputs(w: Workload, seed: int, b: int, h: int) -> dict:
    """One (b, h) slice. Returns q, k, v as float32 arrays holding exactly the
    values consumers see (bf16-representable for bf16 workloads), plus the
    uint16 bit patterns under ``*_bits`` for bf16 workloads, beta and gamma."""
    rng = np.random.default_rng([w.tag, seed, b, h])
    shp = (w.T, w.S, w.D)
    out = {}
    for name in ("q", "k", "v"):
        x = rng.standard_normal(shp, dtype=np.float32)
        if w.io == "bf16":
            bits = f32_to_bf16_bits(x)
            out[name + "_bits"] = bits
            out[name] = bf16_bits_to_f32(bits)
        else:
            out[name] = x
    if w.beta == "uniform":
        out["beta"] = rng.random((w.T, w.S), dtype=np.float32)
    elif w.beta == "beta05":
        out["beta"] = rng.beta(0.5, 0.5, (w.T, w.S)).astype(np.float32)
    else:
        raise ValueError(w.beta)
    lo = float(w.gamma_lo)
    out["gamma"] = (lo + (1.0 - lo) * rng.random(w.T)).astype(np.float32)
    return out


def batch_inputs(w: Workload, seed: int = 0, threads: int = 8, keep_f32: bool = True) -> dict:
    """All (b, h) slices stacked into [B, H, ...] arrays.

    For bf16 workloads ``q_bits``/``k_bits``/``v_bits`` hold uint16 patterns;
    the float32 copies are kept only when ``keep_f32`` is set (they double the
    host memory of large workloads).
    """
    B, H = w.B, w.H
    bf = w.io == "bf16"
    names = ("q_bits", "k_bits", "v_bits") if bf else ("q", "k", "v")
    dt = np.uint16 if bf else np.float32
    out = {n: np.empty((B, H, w.T, w.S, w.D), dtype=dt) for n in names}
    if bf and keep_f32:
        for n in ("q", "k", "v"):
            out[n] = np.empty((B, H, w.T, w.S, w.D), dtype=np.float32)
    out["beta"] = np.empty((B, H, w.T, w.S), dtype=np.float32)
    out["gamma"] = np.empty((B, H, w.T), dtype=np.float32)

    def fill(bh):
        b, h = bh
        x = head_inputs(w, seed, b, h)
        for n in list(out.keys()):
            if n in x:
                out[n][b, h] = x[n]

    pairs = [(b, h) for b in range(B) for h in range(H)]
    if threads > 1 and len(pairs) > 1:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(fill, pairs))
    else:
        for bh in pairs:
            fill(bh)
    return out
