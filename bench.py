#!/usr/bin/env python3
"""Benchmark: frame-wise GDN layer scan on one MI355X.

One step is one call of the library over the whole workload: phase 1 (A_t,
U_t), the affine scan (composite chunks when the workload asks for them) and
the per-token readout, for all heads and frames. Inputs are generated with the
seeded generator and are resident in HBM before timing starts. Default
workload: H = 16 heads, D = 128, S = 3600 tokens (80 x 45 latent grid of a
720p frame), T = 121 latent frames (a 60 s clip), causal scan split into 8
time chunks combined by affine composites.

Prints ONE JSON line (rank 0, N = 1). ``value`` and ``ms_per_step`` come from
exactly K steps between two events with nothing else enqueued. The same K
steps are then run twice more: with an event between consecutive steps (the
per-step median and min), and with the library's phase trace on
(gdn_trace_set: HIP events recorded on the library's stream at the start of
each call and after each launch group), which gives the device time of every
phase of the step itself; the dominant kernel's time gives the ``roofline``
object. (The trace's events cost a few microseconds each, which is why the
headline figure comes from the untraced steps.) Sub-objects: the
other named workloads (``configs``), a cache-resident phase-1 leg
(``warm``), the streaming step, the backward, and the float64 oracle timed
on the host cores on a bounded sample (``cpu_baseline``).
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
BF16_PEAK_TFLOPS = 2516.6    # MI355X dense bf16 MFMA (256 CU x 2.4 GHz x 4096 flop/clk)

# the pages' own figures, for context only (other hardware, other scope)
PAGES_CONTEXT = {
    "fused_kernel_speedup": "1.5-2x from the fused GDN kernel (RMSNorm + ReLU + key scaling + "
                            "RoPE prep + scan) during 64xH100 training (blog.hotdry.top SANA-WM "
                            "post, section on context-parallel sharding)",
    "whole_model_60s_720p": "34 s whole-model denoising of a 60 s 720p video on an RTX 5090 with "
                            "NVFP4, 4-step distilled (xiejiayun.github.io review, section 2.6)",
    "comparable": False,
}


def per_frame_head(w):
    """Algorithmic flops and HBM bytes per frame-head of each phase, as the
    step's kernel instances need them (phase 1 writes bf16 A_t and fp32 U_t on
    the MFMA path, fp32 A_t and U_t on the fp32 path)."""
    S, D = w.S, w.D
    io = 2 if w.io == "bf16" else 4
    mfma = w.io == "bf16" and D == 128
    terms_flop = 4 * D * D * S
    terms_out = (2 + 4) * D * D if mfma else 8 * D * D
    terms_bytes = 2 * S * D * io + 4 * S + terms_out              # k, v, beta in; A, U out
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
    """(name, template arguments, source) of the phase-1 and readout kernel
    instances that a forward call (gdn_scan_fwd, gdn_scan_bidir_chunked) on
    w launches, as rocprofv3 names them."""
    n = "true" if norm else "false"
    if w.io == "bf16" and w.D == 128:
        return {"terms": ("terms_dma_bf16_d128", f"<true, false, {n}, false, false>", "k_terms.hip"),
                "readout": ("readout_mfma_bf16_d128", f"<{n}>", "k_readout.hip")}
    return {"terms": ("terms_generic", "", "k_terms.hip"),
            "readout": ("readout_generic", "", "k_readout.hip")}


class Roctx:
    """Named host-side ranges around the benchmark's legs, one open at a time,
    for `rocprofv3 --marker-trace` (roctx, which ROCm ships with its profiler
    SDK); every call is a no-op when no roctx library can be loaded."""

    def __init__(self):
        self._lib = None
        self._open = False
        for name in ("librocprofiler-sdk-roctx.so.1", "libroctx64.so.4"):
            try:
                lib = ctypes.CDLL(name)
            except OSError:
                continue
            lib.roctxRangePushA.argtypes = [ctypes.c_char_p]
            lib.roctxRangePushA.restype = ctypes.c_int
            lib.roctxRangePop.argtypes = []
            lib.roctxRangePop.restype = ctypes.c_int
            self._lib = lib
            break

    def begin(self, name: str) -> None:
        """Close the open range (if any) and open one called `name`."""
        self.end()
        if self._lib is not None:
            self._lib.roctxRangePushA(name.encode())
            self._open = True

    def end(self) -> None:
        if self._open:
            self._lib.roctxRangePop()
            self._open = False


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


def summarize_calls(calls):
    """Per-call totals and per-phase device times (ms) of traced calls:
    mean / median / min of the call, and the median and mean of each phase."""
    tot = [c["total"] for c in calls]
    phases = sorted({k for c in calls for k in c if k != "total"})
    med = {p: statistics.median([c.get(p, 0.0) for c in calls]) for p in phases}
    mean = {p: sum(c.get(p, 0.0) for c in calls) / len(calls) for p in phases}
    return {"mean": sum(tot) / len(tot), "median": statistics.median(tot), "min": min(tot),
            "phase_median": med, "phase_mean": mean}


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


def calibrate_hbm(dev, reps=10):
    """Plain HBM streams over 1 GiB (read-only, write-only, copy) with the
    probe library's kernels, the best over a few grid sizes, and torch's
    device copy: the ceilings the phase kernels are compared with."""
    import ctypes

    import torch

    probe = ctypes.CDLL(os.path.join(ROOT, "frame_wise_gated_amd", "libhbm_probe.so"))
    probe.hbm_probe.restype = ctypes.c_int
    probe.hbm_probe.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    nbytes = 1 << 30
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    sink = torch.zeros(64, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream

    def timed(fn):
        fn()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        e1.synchronize()
        return e0.elapsed_time(e1) / reps

    out = {"bytes": nbytes, "reps": reps,
           "kernels": "libhbm_probe.so (16-byte accesses, grid-stride, 8 loads in flight per "
                      "thread, plain or non-temporal; read_span: one contiguous span per "
                      "workgroup, 32 KB steps, non-temporal register loads; read_span_lds: the "
                      "same spans as global -> LDS copies into a two-step ring; copy_span: "
                      "one contiguous span copied per workgroup, plain or non-temporal stores)",
           "GBps": {}, "best_config": {}, "sweep": {}}
    for kind, name, moved in ((0, "read_only", nbytes), (1, "write_only", nbytes),
                              (2, "copy", 2 * nbytes), (3, "read_span", nbytes),
                              (4, "read_span_lds", nbytes), (5, "copy_span", 2 * nbytes)):
        best, cfg = 0.0, None
        for nt in ((0, 1) if kind in (0, 1, 2, 5) else (1,)):
            for blocks in (1024, 2048, 4096, 8192, 16384, 32768):
                s_ = src.data_ptr() if kind != 1 else None
                d_ = sink.data_ptr() if kind in (0, 3, 4) else dst.data_ptr()

                def fn(kind=kind, s_=s_, d_=d_, blocks=blocks, nt=nt):
                    rc = probe.hbm_probe(kind, s_, d_, nbytes, blocks, nt, sp)
                    if rc != 0:
                        raise RuntimeError(f"hbm_probe({kind}) returned {rc}")

                gbs = moved / (timed(fn) / 1e3) / 1e9
                out["sweep"][f"{name}_{'nt' if nt else 'plain'}_{blocks}"] = round(gbs, 1)
                if gbs > best:
                    best, cfg = gbs, {"nontemporal": bool(nt), "blocks": blocks}
        out["GBps"][name] = best
        out["best_config"][name] = cfg
    out["GBps"]["torch_copy"] = 2 * nbytes / (timed(lambda: dst.copy_(src)) / 1e3) / 1e9
    return out


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
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other named workloads (configs sub-object)")
    ap.add_argument("--no-warm", action="store_true", help="skip the cache-resident phase-1 leg")
    ap.add_argument("--no-streaming", action="store_true",
                    help="skip the streaming leg (the layer stepped in blocks of frames)")
    ap.add_argument("--stream-block", type=int, default=3,
                    help="latent frames per streaming block (default 3)")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip timing the backward pass")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy (reference for HBM byte counters)")
    ap.add_argument("--calibrate-hbm", action="store_true",
                    help="only time plain read-only, write-only and copy streams over 1 GiB")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the scan would "
              f"shard over heads and time chunks, but no multi-GPU path is implemented)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from frame_wise_gated_amd import gdn
    from frame_wise_gated_amd import inputs as gi

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
    if args.calibrate_hbm:
        print(json.dumps(calibrate_hbm(dev)), flush=True)
        return

    stream = torch.cuda.current_stream()
    norm = bool(args.qk_rmsnorm)

    ranges = Roctx()

    def log(*a, leg=False):
        """Progress on stderr; leg=True also starts a roctx range of that name
        (the legs run one after another, so each range ends where the next
        begins)."""
        print("[bench]", *a, file=sys.stderr, flush=True)
        if leg:
            ranges.begin(" ".join(str(x) for x in a))

    def load(w):
        """Seeded inputs of workload w on the device, with output buffers."""
        x = gi.batch_inputs(w, args.seed, threads=min(16, os.cpu_count() or 1), keep_f32=False)
        bf = w.io == "bf16"

        def up(a, as_bf16):
            t = torch.from_numpy(np.ascontiguousarray(a))
            if as_bf16:
                t = t.view(torch.int16).view(torch.bfloat16)
            return t.to(dev)

        names = ("q_bits", "k_bits", "v_bits") if bf else ("q", "k", "v")
        q, k, v = (up(x[n].view(np.int16) if bf else x[n], bf) for n in names)
        d = {"q": q, "k": k, "v": v, "beta": up(x["beta"], False), "gamma": up(x["gamma"], False)}
        del x
        B, H, T, S, D = w.B, w.H, w.T, w.S, w.D
        d["st_fwd"] = torch.empty((B, H, T, D, D), dtype=torch.float32, device=dev)
        d["st_rev"] = torch.empty_like(d["st_fwd"]) if w.mode == "bidir" else None
        d["s_fin"] = torch.empty((B, H, D, D), dtype=torch.float32, device=dev)
        d["o"] = torch.empty_like(q)
        desc = gdn.make_desc(B, H, T, S, D, gdn.GDN_BF16 if bf else gdn.GDN_F32, qk_rmsnorm=norm)
        d["desc"] = desc
        d["ws"] = gdn.workspace(desc, w.time_chunks, dev)
        return d

    def step_fn(w, d, ws_=None):
        ws_ = d["ws"] if ws_ is None else ws_

        def step():
            if w.mode == "bidir":
                gdn.gdn_scan_bidir_chunked(d["q"], d["k"], d["v"], d["beta"], d["gamma"], w.chunk_len,
                                           n_time_chunks=w.time_chunks, states_fwd=d["st_fwd"],
                                           states_rev=d["st_rev"], s_final=d["s_fin"], o=d["o"],
                                           ws=ws_, stream=stream, qk_rmsnorm=norm)
            else:
                gdn.gdn_scan_fwd(d["q"], d["k"], d["v"], d["beta"], d["gamma"],
                                 n_time_chunks=w.time_chunks, states=d["st_fwd"], s_final=d["s_fin"],
                                 o=d["o"], ws=ws_, stream=stream, qk_rmsnorm=norm)
        return step

    def timed(fn, reps, traced=True, events_per_call=24):
        """reps calls of fn between two events (synchronised on both sides);
        with traced, the library's phase trace is on for exactly these calls.
        Returns (ms per call over the bracket, traced-call summary or None)."""
        tr = gdn.PhaseTrace(reps * events_per_call) if traced else None
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        if traced:
            with tr:
                for _ in range(reps):
                    fn()
        else:
            for _ in range(reps):
                fn()
        e1.record(stream)
        e1.synchronize()
        ms = e0.elapsed_time(e1) / reps
        if not traced:
            return ms, None
        if tr.full():
            raise RuntimeError("phase trace capacity exhausted")
        calls = tr.calls()
        return ms, summarize_calls(calls)

    def per_step(fn, reps):
        """reps calls of fn with one event between consecutive calls (and one
        before the first, one after the last): the device time of every call,
        as (median, min) in ms."""
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        torch.cuda.synchronize()
        ev[0].record(stream)
        for i in range(reps):
            fn()
            ev[i + 1].record(stream)
        ev[-1].synchronize()
        t = [ev[i].elapsed_time(ev[i + 1]) for i in range(reps)]
        return statistics.median(t), min(t)

    w = gi.workload(args.workload)
    log("generating", w.name, leg=True)
    d = load(w)
    B, H, T, S, D = w.B, w.H, w.T, w.S, w.D
    bf = w.io == "bf16"
    step = step_fn(w, d)
    pf = per_frame_head(w)
    fh = B * H * T
    # Order: the streaming leg, the forward step's per-step pass and its
    # phase-traced pass (K steps each), then the W warm-up steps and the K
    # timed steps of the headline. The first ~40 ms of back-to-back forward
    # steps run 2-3 % slower than the rest (20 steps after a 5-step warm-up:
    # 1.539 ms/step, every later block of 20 1.489-1.493), and the headline
    # is meant as the steady rate of back-to-back steps, so it comes last.
    streaming_out = None
    if not args.no_streaming:
        # streaming: the same layer stepped through blocks of a few latent
        # frames with gdn_step (bidirectional inside a block, the forward state
        # carried in place from block to block), as a chunk-causal model runs
        # it; the inputs are cut into contiguous per-block tensors beforehand
        log("streaming", leg=True)
        L = max(1, min(args.stream_block, T))
        cuts = [(a, min(a + L, T)) for a in range(0, T, L)]
        blk = [{n: d[n][:, :, a:b].contiguous() for n in ("q", "k", "v", "beta", "gamma")}
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
        reps = max(args.steps // 2, 10)
        t_stream, _ = timed(stream_pass, reps, traced=False)
        _, ss = timed(stream_pass, reps, events_per_call=24 * len(cuts))
        full_blocks = [c for c in range(len(cuts)) if cuts[c][1] - cuts[c][0] == L]
        streaming_out = {
            "block_frames": L,
            "blocks": len(cuts),
            "ms_per_layer": t_stream,
            "ms_per_block": t_stream / len(cuts),
            "layer_frames_per_s": T / (t_stream / 1e3),
            "block_ms_median": ss["median"],
            "block_phase_ms_median": ss["phase_median"],
            "hbm_frac_block": pf["step_bytes"] * B * H * L / (ss["median"] / 1e3) / 1e9 / HBM_PEAK_GBS,
        }
        del blk, blk_o, carry, bws_s, full_blocks

    # K steps with an event between consecutive steps (the first steps of the
    # call on this device), K steps with the phase trace on (per-phase device
    # times), K steps with per-step events again (per-step median and min)
    log("per-step and phase-traced passes", leg=True)
    med_first, _ = per_step(step, args.steps)
    ms_traced, summ = timed(step, args.steps)
    med, mn = per_step(step, args.steps)
    log(f"per step: median {med:.3f} (first pass {med_first:.3f}), min {mn:.3f}; "
        f"phase-traced steps: {ms_traced:.3f} ms/step")
    log("warmup", args.warmup, leg=True)
    for _ in range(args.warmup):
        step()
    log("timed steps", args.steps, leg=True)
    # the timed region: exactly K steps between two events, nothing else
    # enqueued in between
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ms, _ = timed(step, args.steps, traced=False)
    wall = (time.perf_counter() - wall0) / args.steps * 1e3
    log(f"{args.steps} steps: {ms:.3f} ms/step (events), {wall:.3f} ms/step (wall)")

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
        "ms_step_median": med,
        "ms_step_min": mn,
        "ms_step_median_first_pass": med_first,
        "ms_per_step_phase_traced": ms_traced,
    }
    eff_tf = pf["step_flop"] * fh / (ms / 1e3) / 1e12
    out["effective_tflops"] = eff_tf
    out["mfma_peak_frac"] = eff_tf / BF16_PEAK_TFLOPS
    out["hbm_frac_step"] = pf["step_bytes"] * fh / (ms / 1e3) / 1e9 / HBM_PEAK_GBS
    out["phase_ms"] = {"median": summ["phase_median"], "mean": summ["phase_mean"]}

    # dominant kernel of the step: the longer of phase 1 and the readout, timed
    # by the trace events around its own launch inside the timed steps
    kn = kernel_names(w, norm)
    cand = {"terms": (pf["terms_bytes"], pf["terms_flop"]),
            "readout": (pf["readout_bytes"], pf["readout_flop"])}
    name = max(cand, key=lambda n: summ["phase_mean"].get(n, 0.0))
    t = summ["phase_mean"][name]
    nbytes, nflop = cand[name][0] * fh, cand[name][1] * fh
    achieved = nbytes / (t / 1e3) / 1e9
    kname, kvar, ksrc = kn[name]
    out["roofline"] = {
        "bound": "hbm",
        "achieved": achieved,
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": achieved / HBM_PEAK_GBS,
        "traffic": recorded_traffic(kname, kvar, ksrc, out["config"]["workload"]),
        "kernel": kname + kvar,
        "phase": name,
        "algorithmic_bytes_per_launch": nbytes,
        "ms_per_launch": t,
        "ms_per_launch_median": summ["phase_median"][name],
        "mfma_tflops": nflop / (t / 1e3) / 1e12,
        "mfma_frac": nflop / (t / 1e3) / 1e12 / BF16_PEAK_TFLOPS,
    }
    # the other contraction phase beside it
    other = "readout" if name == "terms" else "terms"
    if other in summ["phase_mean"]:
        to = summ["phase_mean"][other]
        ob = cand[other][0] * fh
        out["roofline"]["other_phase"] = {
            "phase": other, "kernel": "".join(kn[other][:2]), "ms_per_launch": to,
            "achieved": ob / (to / 1e3) / 1e9, "frac": ob / (to / 1e3) / 1e9 / HBM_PEAK_GBS,
            "traffic": recorded_traffic(kn[other][0], kn[other][1], kn[other][2],
                                        out["config"]["workload"]),
            "mfma_frac": cand[other][1] * fh / (to / 1e3) / 1e12 / BF16_PEAK_TFLOPS}
    # a plain device copy of q (the readout's input) on the same stream: the
    # mixed read + write stream this box sustains next to the readout
    qc = torch.empty_like(d["q"])
    for _ in range(3):  # a fresh allocation: its first copies run slower
        qc.copy_(d["q"])
    t_copy, _ = timed(lambda: qc.copy_(d["q"]), max(args.steps // 2, 5), traced=False)
    copy_gbs = 2 * d["q"].numel() * d["q"].element_size() / (t_copy / 1e3) / 1e9
    out["roofline"]["copy_reference_GBps"] = copy_gbs
    del qc
    out["pages_context"] = PAGES_CONTEXT

    if streaming_out is not None:
        out["streaming"] = streaming_out

    if not args.no_backward:
        # backward of the same layer: gradients of <d_o, o> for a random d_o
        # (the chunk-causal backward for the bidirectional workload)
        log("backward", leg=True)
        gen = torch.Generator(device=dev).manual_seed(args.seed + 1)
        q = d["q"]
        d_o = torch.randn(q.shape, device=dev, dtype=torch.float32, generator=gen).to(q.dtype)
        grads = {n: torch.empty_like(q) for n in ("dq", "dk", "dv")}
        grads["dbeta"] = torch.empty_like(d["beta"])
        grads["dgamma"] = torch.empty_like(d["gamma"])
        grads["ds0"] = torch.empty_like(d["s_fin"])
        desc = d["desc"]
        if w.mode == "bidir":
            bws = torch.empty(gdn.gdn_bidir_bwd_workspace_bytes(desc, w.chunk_len), dtype=torch.uint8,
                              device=dev)
            bcall = lambda ws_, reuse: gdn.gdn_scan_bidir_chunked_bwd(
                d["q"], d["k"], d["v"], d["beta"], d["gamma"], w.chunk_len, d["st_fwd"], d["st_rev"],
                d_o, out=grads, ws=ws_, stream=stream, qk_rmsnorm=norm, reuse_fwd_terms=reuse)
        else:
            bws = torch.empty(gdn.gdn_bwd_workspace_bytes(desc), dtype=torch.uint8, device=dev)
            bcall = lambda ws_, reuse: gdn.gdn_scan_bwd(
                d["q"], d["k"], d["v"], d["beta"], d["gamma"], d["st_fwd"], d_o, out=grads, ws=ws_,
                stream=stream, qk_rmsnorm=norm, reuse_fwd_terms=reuse)
        bstep = lambda: bcall(bws, False)
        for _ in range(2):
            bstep()
        t_bwd, _ = timed(bstep, max(args.steps // 2, 3), traced=False)
        _, bs = timed(bstep, max(args.steps // 2, 3))
        # the same backward reading A_t from the workspace of its forward call
        # (GDN_REUSE_FWD_TERMS): one forward call into a workspace sized for
        # both, then the timed backward calls on it
        fws = torch.empty(max(d["ws"].numel(), bws.numel()), dtype=torch.uint8, device=dev)
        step_fn(w, d, fws)()
        rstep = lambda: bcall(fws, True)
        for _ in range(2):
            rstep()
        t_bwd_r, _ = timed(rstep, max(args.steps // 2, 3), traced=False)
        _, rs = timed(rstep, max(args.steps // 2, 3))
        del fws
        # algorithmic bytes: q, k, v, d_o, beta, gamma and the forward states
        # (both directions for the bidirectional scan) in; dq, dk, dv, dbeta,
        # dgamma out
        n_states = 2 if w.mode == "bidir" else 1
        io = 2 if bf else 4
        bw_bytes = fh * (4 * S * D * io + 4 * S + 4 + n_states * 4 * D * D + 3 * S * D * io + 4 * S + 4)
        out["backward"] = {
            "ms_per_call": t_bwd,
            "ms_median": bs["median"],
            "layer_frames_per_s": T / (t_bwd / 1e3),
            "algorithmic_bytes": bw_bytes,
            "hbm_frac": bw_bytes / (t_bwd / 1e3) / 1e9 / HBM_PEAK_GBS,
            "phase_ms_median": bs["phase_median"],
            "reusing_fwd_terms": {
                "ms_per_call": t_bwd_r,
                "ms_median": rs["median"],
                "layer_frames_per_s": T / (t_bwd_r / 1e3),
                "hbm_frac": bw_bytes / (t_bwd_r / 1e3) / 1e9 / HBM_PEAK_GBS,
            },
        }
        del grads, bws, d_o

    if not args.no_warm and bf and D == 128:
        # phase 1 on an input set that stays in the 256 MB last-level cache
        # (MALL) between back-to-back calls, run the way the step runs it
        # (whole frame-heads, two workgroups per CU, one round): 512
        # frame-heads of 448 tokens (16 heads x 32 frames, the first 448
        # tokens of each), k + v = 117 MB. The phase-1 time comes from the
        # same trace events as in the step.
        log("warm phase-1 leg", leg=True)
        TW, SW = 32, 448
        ww = w.with_shape(T=TW, S=SW, time_chunks=1, chunk_len=0, mode="fwd")
        dw = {n: d[n][:, :, :TW, :SW].contiguous() for n in ("q", "k", "v", "beta")}
        dw["gamma"] = d["gamma"][:, :, :TW].contiguous()
        sf = torch.empty((B, H, D, D), dtype=torch.float32, device=dev)
        wsw = gdn.workspace(gdn.make_desc(B, H, TW, SW, D, gdn.GDN_BF16, qk_rmsnorm=norm), 1, dev)
        wcall = lambda: gdn.gdn_scan_fwd(dw["q"], dw["k"], dw["v"], dw["beta"], dw["gamma"],
                                         want_states=False, want_o=False, s_final=sf, ws=wsw,
                                         stream=stream, qk_rmsnorm=norm)
        for _ in range(5):
            wcall()
        _, wsum = timed(wcall, 50)
        pw = per_frame_head(ww)
        fhw = B * H * TW
        tw = wsum["phase_median"].get("terms", 0.0) + wsum["phase_median"].get("terms_reduce", 0.0)
        out["warm"] = {
            "label": "warm (cache-resident operands, not an HBM figure)",
            "config": {"workload": f"H{H}_T{TW}_S{SW}", "B": B, "H": H, "T": TW, "S": SW, "D": D,
                       "k_plus_v_MB": 2 * fhw * SW * D * 2 / 1e6},
            "reps": 50,
            "terms_ms_median": tw,
            "terms_phases": {k: v for k, v in wsum["phase_median"].items() if k.startswith("terms")},
            "tflops": pw["terms_flop"] * fhw / (tw / 1e3) / 1e12,
            "mfma_frac": pw["terms_flop"] * fhw / (tw / 1e3) / 1e12 / BF16_PEAK_TFLOPS,
            "operand_GBps": pw["terms_bytes"] * fhw / (tw / 1e3) / 1e9,
        }
        del dw, sf, wsw

    if not args.no_configs:
        # the other named workloads as sub-objects of the one line, each timed
        # in the headline's order (per-step and traced passes, then the
        # warm-up and the timed steps)
        del d, step
        torch.cuda.empty_cache()
        out["configs"] = {}
        for idx in (2, 3, 5, 4) if args.workload != 4 else (2, 3, 5):
            if idx == args.workload:
                continue
            wc = gi.workload(idx)
            log("config", wc.name, leg=True)
            dc = load(wc)
            sc = step_fn(wc, dc)
            medc_first, _ = per_step(sc, args.steps)
            _, sm = timed(sc, args.steps)
            medc, mnc = per_step(sc, args.steps)
            for _ in range(args.warmup):
                sc()
            msc, _ = timed(sc, args.steps, traced=False)
            pc = per_frame_head(wc)
            fhc = wc.B * wc.H * wc.T
            out["configs"][wc.name] = {
                "ms_per_step": msc, "ms_step_median": medc, "ms_step_min": mnc,
                "ms_step_median_first_pass": medc_first,
                "layer_frames_per_s": wc.T / (msc / 1e3),
                "hbm_frac_step": pc["step_bytes"] * fhc / (msc / 1e3) / 1e9 / HBM_PEAK_GBS,
                "effective_tflops": pc["step_flop"] * fhc / (msc / 1e3) / 1e12,
                "phase_ms_median": sm["phase_median"],
                "shape": {"B": wc.B, "H": wc.H, "T": wc.T, "S": wc.S, "D": wc.D, "scan": wc.mode,
                          "time_chunks": wc.time_chunks, "chunk_len": wc.chunk_len},
            }
            del dc, sc
            torch.cuda.empty_cache()

    if not args.no_cpu_baseline and not norm:
        log("cpu baseline (float64 oracle)", leg=True)
        out["cpu_baseline"] = cpu_baseline(w, args.seed, args.cpu_seconds)
    ranges.end()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
