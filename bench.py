#!/usr/bin/env python3
"""Benchmark: frame-wise GDN layer scan on one MI355X.

One step is one call of the library over the whole workload: phase 1 (A_t,
U_t), the affine scan (composite chunks when the workload asks for them) and
the per-token readout, for all heads and frames. Inputs are generated with the
seeded generator and are resident in HBM before timing starts. Default
workload: H = 16 heads, D = 128, S = 3600 tokens (80 x 45 latent grid of a
720p frame), T = 121 latent frames (a 60 s clip), causal scan split into 8
time chunks combined by affine composites.

Prints ONE JSON line (rank 0, N = 1). Phase kernels are also timed on their
own with HIP events on the library's stream; the slowest gives the
``roofline`` object. The ``cpu_baseline`` leg times the float64 oracle on a
bounded sample of the same workload on the host cores.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
BF16_PEAK_TFLOPS = 2516.6    # MI355X dense bf16 MFMA (256 CU x 2.4 GHz x 4096 flop/clk)


def per_frame_head(w):
    """Algorithmic flops and HBM bytes per frame-head of each phase."""
    S, D = w.S, w.D
    io = 2 if w.io == "bf16" else 4
    terms_flop = 4 * D * D * S
    terms_bytes = 2 * S * D * io + 4 * S + 2 * D * D * 4          # k, v, beta in; A, U out
    readout_flop = 2 * D * D * S
    nstate = 2 if w.mode == "bidir" else 1
    readout_bytes = 2 * S * D * io + nstate * 4 * D * D            # q in, o out, state(s) in
    scan_flop = 2 * D * D * D * nstate
    step_flop = terms_flop + readout_flop + scan_flop
    # whole path: q, k, v, beta, gamma in; o and every state out
    step_bytes = 3 * S * D * io + 4 * S + 4 + S * D * io + nstate * 4 * D * D
    return dict(terms_flop=terms_flop, terms_bytes=terms_bytes, readout_flop=readout_flop,
                readout_bytes=readout_bytes, step_flop=step_flop, step_bytes=step_bytes)


def kernel_names(w, norm):
    """(name, template arguments, source) of the phase-1 and readout kernels
    that gdn_frame_terms and gdn_readout launch for w, as rocprofv3 names them."""
    if w.io == "bf16" and w.D == 128:
        n = "true" if norm else "false"
        return {"terms": ("terms_dma_bf16_d128", f"<false, false, {n}, false, false>", "k_terms.hip"),
                "readout": ("readout_mfma_bf16_d128", f"<{n}>", "k_readout.hip")}
    return {"terms": ("terms_generic", "", "k_terms.hip"),
            "readout": ("readout_generic", "", "k_readout.hip")}


def recorded_traffic(kernel, variant, source, workload):
    """HBM bytes per launch of `kernel` (template arguments `variant`) on
    `workload` from the committed rocprofv3 counter summary (FETCH_SIZE and
    WRITE_SIZE, scaled by the plain-copy calibration), or None when there is
    none, it covers another instance of the kernel, or the kernel's source has
    changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"{kernel}__{workload}__hbm_traffic.txt")
    src = os.path.join(ROOT, "frame_wise_gated_amd", "csrc", source)
    if not (os.path.exists(path) and os.path.exists(src)):
        return None
    fields = {}
    for line in open(path):
        key, _, val = line.strip().partition(" ")
        if key in ("source_sha256", "hbm_bytes_per_launch", "kernel_instance"):
            fields.setdefault(key, val.strip())  # the first occurrence is the field
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    if (fields.get("source_sha256") != sha or "hbm_bytes_per_launch" not in fields
            or fields.get("kernel_instance") != kernel + variant):
        return None
    return int(fields["hbm_bytes_per_launch"])


def cpu_baseline(w, seed, budget_s):
    """Time the float64 oracle on whole heads of the workload until the budget
    is spent (at least one head). Returns the baseline dict."""
    import numpy as np

    import oracle
    from frame_wise_gated_amd import inputs as gi

    threads = None
    try:
        from threadpoolctl import threadpool_info
        info = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if info:
            threads = int(info[0]["num_threads"])
    except Exception:
        threads = None
    heads = 0
    spent = 0.0
    while heads < w.B * w.H and (heads == 0 or spent < budget_s):
        b, h = divmod(heads, w.H)
        x = gi.head_inputs(w, seed, b, h)
        a = {n: np.asarray(x[n], dtype=np.float32)[None, None] for n in ("q", "k", "v", "beta", "gamma")}
        t0 = time.perf_counter()
        if w.mode == "bidir":
            oracle.scan_bidir_chunked(a["q"], a["k"], a["v"], a["beta"], a["gamma"], w.chunk_len)
        else:
            oracle.scan_fwd(a["q"], a["k"], a["v"], a["beta"], a["gamma"])
        spent += time.perf_counter() - t0
        heads += 1
    layer_frames = heads * w.T / w.H
    return {
        "value": layer_frames / spent,
        "unit": "layer frames/s",
        "cores": threads if threads else os.cpu_count(),
        "kind": "oracle",
        "sample": f"{heads} of {w.B * w.H} heads x {w.T} frames of {w.name}, sequential float64 "
                  f"frame loop ({spent:.1f} s)",
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=4, help="named workload 2..5 (default 4)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--qk-rmsnorm", action="store_true",
                    help="fuse the per-token RMSNorm of q and k (GDN_QK_RMSNORM)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-phases", action="store_true", help="skip the per-phase timing loops")
    ap.add_argument("--no-streaming", action="store_true",
                    help="skip the streaming leg (the layer stepped in blocks of frames)")
    ap.add_argument("--stream-block", type=int, default=3,
                    help="latent frames per streaming block (default 3)")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip timing the backward pass")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy (reference for HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the scan would "
              f"shard over heads and time chunks, but no multi-GPU path is implemented)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np  # noqa: F401
    import torch

    from frame_wise_gated_amd import gdn
    from frame_wise_gated_amd import inputs as gi

    w = gi.workload(args.workload)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.calibrate_copy:
        nbytes = 1 << 30
        src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "launches": 3}))
        return
    print(f"[bench] generating {w.name}", file=sys.stderr, flush=True)
    x = gi.batch_inputs(w, args.seed, threads=min(16, os.cpu_count() or 1), keep_f32=False)

    def up(a, bf):
        t = torch.from_numpy(np.ascontiguousarray(a))
        if bf:
            t = t.view(torch.int16).view(torch.bfloat16)
        return t.to(dev)

    bf = w.io == "bf16"
    names = ("q_bits", "k_bits", "v_bits") if bf else ("q", "k", "v")
    q, k, v = (up(x[n].view(np.int16) if bf else x[n], bf) for n in names)
    beta = up(x["beta"], False)
    gamma = up(x["gamma"], False)
    del x
    B, H, T, S, D = w.B, w.H, w.T, w.S, w.D
    st_fwd = torch.empty((B, H, T, D, D), dtype=torch.float32, device=dev)
    st_rev = torch.empty_like(st_fwd) if w.mode == "bidir" else None
    s_fin = torch.empty((B, H, D, D), dtype=torch.float32, device=dev)
    o = torch.empty_like(q)
    norm = bool(args.qk_rmsnorm)
    desc = gdn.make_desc(B, H, T, S, D, gdn.GDN_BF16 if bf else gdn.GDN_F32, qk_rmsnorm=norm)
    ws = gdn.workspace(desc, w.time_chunks, dev)
    stream = torch.cuda.current_stream()

    def step(ws_=None):
        ws_ = ws if ws_ is None else ws_
        if w.mode == "bidir":
            gdn.gdn_scan_bidir_chunked(q, k, v, beta, gamma, w.chunk_len, n_time_chunks=w.time_chunks,
                                       states_fwd=st_fwd, states_rev=st_rev, s_final=s_fin, o=o,
                                       ws=ws_, stream=stream, qk_rmsnorm=norm)
        else:
            gdn.gdn_scan_fwd(q, k, v, beta, gamma, n_time_chunks=w.time_chunks, states=st_fwd,
                             s_final=s_fin, o=o, ws=ws_, stream=stream, qk_rmsnorm=norm)

    def timed(fn, reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        e1.synchronize()
        return e0.elapsed_time(e1) / reps

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ms = timed(step, args.steps)
    wall = (time.perf_counter() - wall0) / args.steps * 1e3
    print(f"[bench] {args.steps} steps: {ms:.3f} ms/step (event), {wall:.3f} ms/step (wall)",
          file=sys.stderr, flush=True)

    pf = per_frame_head(w)
    fh = B * H * T
    out = {
        "metric": "GDN layer latent frames/s (H=16,D=128,S=3600) + % of bf16 MFMA peak",
        "value": T / (ms / 1e3),
        "unit": "layer frames/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if bf else "f32",
        "data": "synthetic",
        "config": {"workload": w.name + ("_qk_rmsnorm" if norm else ""), "B": B, "H": H, "T": T,
                   "S": S, "D": D,
                   "scan": w.mode, "time_chunks": w.time_chunks, "chunk_len": w.chunk_len,
                   "parallelism": "single GPU"},
    }
    eff_tf = pf["step_flop"] * fh / (ms / 1e3) / 1e12
    out["effective_tflops"] = eff_tf
    out["mfma_peak_frac"] = eff_tf / BF16_PEAK_TFLOPS
    out["hbm_frac_step"] = pf["step_bytes"] * fh / (ms / 1e3) / 1e9 / HBM_PEAK_GBS

    if not args.no_phases:
        A = torch.empty((B, H, T, D, D), dtype=torch.float32, device=dev)
        U = torch.empty_like(A)
        reps = max(args.steps, 5)
        t_terms = timed(lambda: gdn.gdn_frame_terms(k, v, beta, A=A, U=U, ws=ws, stream=stream,
                                                    qk_rmsnorm=norm), reps)
        t_read = timed(lambda: gdn.gdn_readout(q, st_fwd, st_rev, o=o, stream=stream,
                                               qk_rmsnorm=norm), reps)
        phases = {
            "terms": (t_terms, pf["terms_bytes"] * fh, pf["terms_flop"] * fh),
            "readout": (t_read, pf["readout_bytes"] * fh, pf["readout_flop"] * fh),
        }
        out["phase_ms"] = {"terms": t_terms, "readout": t_read, "scan_and_rest": ms - t_terms - t_read}
        name = max(phases, key=lambda n: phases[n][0])
        t, nbytes, nflop = phases[name]
        achieved = nbytes / (t / 1e3) / 1e9
        kname, kvar, ksrc = kernel_names(w, norm)[name]
        out["roofline"] = {
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": recorded_traffic(kname, kvar, ksrc, out["config"]["workload"]),
            "kernel": kname,
            "algorithmic_bytes_per_launch": nbytes,
            "ms_per_launch": t,
            "mfma_tflops": nflop / (t / 1e3) / 1e12,
            "mfma_frac": nflop / (t / 1e3) / 1e12 / BF16_PEAK_TFLOPS,
        }
        # a plain device copy of q (the readout's input) on the same stream, as
        # the mixed read + write stream this box sustains next to the readout
        qc = torch.empty_like(q)
        t_copy = timed(lambda: qc.copy_(q), reps)
        copy_gbs = 2 * q.numel() * q.element_size() / (t_copy / 1e3) / 1e9
        out["roofline"]["copy_reference_GBps"] = copy_gbs
        out["roofline"]["achieved_over_copy"] = achieved / copy_gbs
        del A, U, qc

    if not args.no_streaming:
        # streaming: the same layer stepped through blocks of a few latent
        # frames with gdn_step (bidirectional inside a block, the forward state
        # carried in place from block to block), as a chunk-causal model runs
        # it; the inputs are cut into contiguous per-block tensors beforehand
        print("[bench] streaming", file=sys.stderr, flush=True)
        L = max(1, min(args.stream_block, T))
        cuts = [(a, min(a + L, T)) for a in range(0, T, L)]
        blk = [{n: t[:, :, a:b].contiguous() for n, t in (("q", q), ("k", k), ("v", v),
                                                          ("beta", beta), ("gamma", gamma))}
               for a, b in cuts]
        blk_o = [torch.empty_like(b["q"]) for b in blk]
        carry = torch.empty((B, H, D, D), dtype=torch.float32, device=dev)
        bws_s = gdn.workspace(gdn.make_desc(B, H, L, S, D, gdn.GDN_BF16 if bf else gdn.GDN_F32,
                                            qk_rmsnorm=norm), 1, dev)

        def stream_pass():
            cin = None  # the first block starts from the zero state
            for b, ob in zip(blk, blk_o):
                gdn.gdn_step(b["q"], b["k"], b["v"], b["beta"], b["gamma"], carry_in=cin,
                             carry_out=carry, o=ob, ws=bws_s, stream=stream, qk_rmsnorm=norm)
                cin = carry

        stream_pass()
        t_stream = timed(stream_pass, max(args.steps // 4, 3))
        out["streaming"] = {
            "block_frames": L,
            "blocks": len(cuts),
            "ms_per_layer": t_stream,
            "ms_per_block": t_stream / len(cuts),
            "layer_frames_per_s": T / (t_stream / 1e3),
        }
        del blk, blk_o, carry, bws_s

    if not args.no_backward:
        # backward of the same layer: gradients of <d_o, o> for a random d_o
        # (the chunk-causal backward for the bidirectional workload)
        print("[bench] backward", file=sys.stderr, flush=True)
        gen = torch.Generator(device=dev).manual_seed(args.seed + 1)
        d_o = torch.randn(q.shape, device=dev, dtype=torch.float32, generator=gen).to(q.dtype)
        grads = {n: torch.empty_like(q) for n in ("dq", "dk", "dv")}
        grads["dbeta"] = torch.empty_like(beta)
        grads["dgamma"] = torch.empty_like(gamma)
        grads["ds0"] = torch.empty_like(s_fin)
        if w.mode == "bidir":
            bws = torch.empty(gdn.gdn_bidir_bwd_workspace_bytes(desc, w.chunk_len), dtype=torch.uint8,
                              device=dev)
            bcall = lambda ws_, reuse: gdn.gdn_scan_bidir_chunked_bwd(
                q, k, v, beta, gamma, w.chunk_len, st_fwd, st_rev, d_o, out=grads, ws=ws_,
                stream=stream, qk_rmsnorm=norm, reuse_fwd_terms=reuse)
        else:
            bws = torch.empty(gdn.gdn_bwd_workspace_bytes(desc), dtype=torch.uint8, device=dev)
            bcall = lambda ws_, reuse: gdn.gdn_scan_bwd(
                q, k, v, beta, gamma, st_fwd, d_o, out=grads, ws=ws_, stream=stream,
                qk_rmsnorm=norm, reuse_fwd_terms=reuse)
        bstep = lambda: bcall(bws, False)
        for _ in range(2):
            bstep()
        t_bwd = timed(bstep, max(args.steps // 2, 3))
        # the same backward reading A_t from the workspace of its forward call
        # (GDN_REUSE_FWD_TERMS): one forward call into a workspace sized for
        # both, then the timed backward calls on it
        fws = torch.empty(max(ws.numel(), bws.numel()), dtype=torch.uint8, device=dev)
        step(fws)
        rstep = lambda: bcall(fws, True)
        for _ in range(2):
            rstep()
        t_bwd_r = timed(rstep, max(args.steps // 2, 3))
        del fws
        # algorithmic bytes: q, k, v, d_o, beta, gamma and the forward states
        # (both directions for the bidirectional scan) in; dq, dk, dv, dbeta,
        # dgamma out
        n_states = 2 if w.mode == "bidir" else 1
        bw_bytes = fh * (4 * S * D * (2 if bf else 4) + 4 * S + 4 + n_states * 4 * D * D
                         + 3 * S * D * (2 if bf else 4) + 4 * S + 4)
        out["backward"] = {
            "ms_per_call": t_bwd,
            "layer_frames_per_s": T / (t_bwd / 1e3),
            "algorithmic_bytes": bw_bytes,
            "hbm_frac": bw_bytes / (t_bwd / 1e3) / 1e9 / HBM_PEAK_GBS,
            "reusing_fwd_terms": {
                "ms_per_call": t_bwd_r,
                "layer_frames_per_s": T / (t_bwd_r / 1e3),
                "hbm_frac": bw_bytes / (t_bwd_r / 1e3) / 1e9 / HBM_PEAK_GBS,
            },
        }
        del grads, bws, d_o

    if not args.no_cpu_baseline and not norm:
        print("[bench] cpu baseline (float64 oracle)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(w, args.seed, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
