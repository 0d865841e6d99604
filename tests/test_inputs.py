"""Seeded input generator: determinism, bf16 rounding, and the key-energy
bound tr(A_t) <= 1 on the workloads' own distributions (CPU only)."""

import numpy as np
import torch

from frame_wise_gated_amd import inputs as gi
from oracle import gdn_oracle as orc


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10.0 ** rng.integers(-30, 30, 100000),
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 0.0, -0.0], np.float32)])
    x = x.astype(np.float32)
    ours = gi.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = gi.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_generator_is_deterministic_and_sliced():
    w = gi.workload(1)
    a = gi.head_inputs(w, 0, 0, 0)
    b = gi.head_inputs(w, 0, 0, 0)
    for n in ("q", "k", "v", "beta", "gamma"):
        assert np.array_equal(a[n], b[n])
    full = gi.batch_inputs(w.with_shape(H=3), seed=0)
    assert full["q"].shape == (1, 3, 8, 12, 16)
    assert np.array_equal(full["k"][0, 0], a["k"])
    c = gi.head_inputs(w, 1, 0, 0)
    assert not np.array_equal(a["k"], c["k"])
    assert (a["gamma"] >= 0.9).all() and (a["gamma"] <= 1.0).all()
    assert (a["beta"] >= 0).all() and (a["beta"] <= 1).all()


def test_bf16_workload_values_are_bf16():
    w = gi.workload(2).with_shape(T=2, S=64)
    x = gi.head_inputs(w, 0, 0, 0)
    assert x["k_bits"].dtype == np.uint16
    assert np.array_equal(gi.bf16_bits_to_f32(x["k_bits"]), x["k"])
    w5 = gi.workload(5).with_shape(T=3, S=500)
    y = gi.head_inputs(w5, 0, 0, 0)
    assert (y["gamma"] >= 0.999).all()
    # Beta(0.5, 0.5) piles mass at both ends
    assert (y["beta"] < 0.05).mean() > 0.1 and (y["beta"] > 0.95).mean() > 0.1


def test_trace_bound_holds_on_workload_distributions():
    """The non-expansiveness argument needs tr(K beta K^T) <= 1; check it on the
    workloads' draws (tiny case: every frame; 720p shape: two frames)."""
    w = gi.workload(1)
    x = gi.head_inputs(w, 0, 0, 0)
    kh = orc.prepare_keys(x["k"])
    for t in range(w.T):
        A, _ = orc.frame_terms(kh[t], x["v"][t], x["beta"][t])
        assert np.trace(A) <= 1.0
    for idx in (2, 5):
        w = gi.workload(idx).with_shape(T=2)
        x = gi.head_inputs(w, 0, 0, 0)
        kh = orc.prepare_keys(x["k"])
        for t in range(2):
            A, _ = orc.frame_terms(kh[t], x["v"][t], x["beta"][t])
            assert np.trace(A) <= 1.0
