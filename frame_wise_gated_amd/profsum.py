"""Summaries of rocprofv3 CSV output (kernel traces and PMC counters).

    python -m frame_wise_gated_amd.profsum trace DIR [--skip N]
        per-kernel dispatch count, mean / min / max duration (us) from
        DIR/*kernel_trace.csv; --skip drops each kernel's first N dispatches
        (warm-up launches).
    python -m frame_wise_gated_amd.profsum pmc DIR [--scale F]
        per-kernel mean counter value per dispatch (KiB for FETCH_SIZE and
        WRITE_SIZE) from DIR/*counter_collection.csv, also multiplied by F
        and shown in MB.
    python -m frame_wise_gated_amd.profsum mfma DIR [--simds N] [--clock-ghz F]
        per-kernel MFMA utilisation from a counter run that collected
        SQ_INSTS_MFMA and SQ_VALU_MFMA_BUSY_CYCLES: the busy cycles summed over
        all SIMDs, divided by SIMDs x clock x the dispatch's duration (its start
        and end timestamps in the same CSV). The defaults are MI355X's 1024
        SIMDs (256 CUs x 4) at its 2.4 GHz peak engine clock, the clock of the
        published dense MFMA peak.
    python -m frame_wise_gated_amd.profsum markers DIR
        the roctx ranges of a run traced with --marker-trace and --kernel-trace
        (bench.py opens one per leg), in order: each range's host duration,
        the kernel dispatches that started inside it and their summed device
        time (ms).

Kernels are keyed by name and grid size, so launches of one kernel with
different shapes stay apart.
"""

from __future__ import annotations

import argparse
import collections
import csv
import glob
import os
import sys


def _one(pattern: str) -> str:
    hits = sorted(glob.glob(pattern))
    if not hits:
        raise SystemExit(f"no file matches {pattern}")
    return hits[0]


def _short(name: str) -> str:
    """Kernel base name, with its template arguments when the trace kept them
    (rocprofv3 without -T), e.g. terms_dma_bf16_d128<true, false>."""
    keys = ("terms_dma_bf16_d128", "terms_generic", "reduce_partials", "scan_mfma_d128",
            "scan_rows_kernel", "combine_rows_kernel", "combine_mfma_d128", "readout_mfma_bf16_d128",
            "readout_generic", "prepare_bf16_kernel", "prepare_f32_kernel",
            "copy_f32_kernel", "zero_f32_kernel", "fill_f32_kernel", "grad_init_kernel",
            "frame_grad_mfma_d128", "frame_grad_kernel", "token_grad_mfma_bf16_d128",
            "token_grad_ws_bf16_d128", "chunk_init_kernel",
            "token_grad_generic", "prepare_norm_kernel")
    for key in keys:
        at = name.find(key)
        if at < 0:
            continue
        rest = name[at + len(key):]
        if rest.startswith("<"):
            depth = 0
            for i, ch in enumerate(rest):
                depth += ch == "<"
                depth -= ch == ">"
                if depth == 0:
                    return key + rest[:i + 1]
        return key
    return name.split("(")[0][:48]


def trace(d: str, skip: int) -> list[str]:
    rows = list(csv.DictReader(open(_one(os.path.join(d, "*kernel_trace.csv")))))
    agg = collections.defaultdict(list)
    for r in rows:
        key = (_short(r["Kernel_Name"]), int(r["Grid_Size_X"]) if "Grid_Size_X" in r else int(r["Grid_Size"]))
        agg[key].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    out = [f"{'kernel':40s} {'grid':>9s} {'calls':>5s} {'mean_us':>9s} {'min_us':>9s} {'max_us':>9s}"]
    for (name, grid), v in sorted(agg.items()):
        v = v[skip:] if len(v) > skip else v
        out.append(f"{name:40s} {grid:9d} {len(v):5d} {sum(v) / len(v):9.1f} {min(v):9.1f} {max(v):9.1f}")
    return out


def pmc(d: str, scale: float) -> list[str]:
    rows = list(csv.DictReader(open(_one(os.path.join(d, "*counter_collection.csv")))))
    agg = collections.defaultdict(list)
    for r in rows:
        agg[(_short(r["Kernel_Name"]), int(r["Grid_Size"]), r["Counter_Name"])].append(
            float(r["Counter_Value"]))
    out = [f"{'kernel':40s} {'grid':>9s} {'counter':>11s} {'calls':>5s} {'mean_KiB':>12s} "
           f"{'x' + format(scale, 'g'):>5s} {'MB':>10s}"]
    for (name, grid, ctr), v in sorted(agg.items()):
        m = sum(v) / len(v)
        out.append(f"{name:40s} {grid:9d} {ctr:>11s} {len(v):5d} {m:12.1f} {'':>5s} "
                   f"{m * 1024 * scale / 1e6:10.2f}")
    return out


def mfma(d: str, simds: int, clock_ghz: float) -> list[str]:
    rows = list(csv.DictReader(open(_one(os.path.join(d, "*counter_collection.csv")))))
    agg = collections.defaultdict(lambda: collections.defaultdict(list))
    for r in rows:
        key = (_short(r["Kernel_Name"]), int(r["Grid_Size"]))
        dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
        agg[key][r["Counter_Name"]].append((float(r["Counter_Value"]), dur))
    out = [f"{'kernel':54s} {'grid':>9s} {'calls':>5s} {'mean_us':>9s} {'mfma_insts':>11s} "
           f"{'busy/inst':>9s} {'mfma_util':>9s}"]
    for (name, grid), ctr in sorted(agg.items()):
        busy, insts = ctr.get("SQ_VALU_MFMA_BUSY_CYCLES"), ctr.get("SQ_INSTS_MFMA")
        if not busy or not insts:
            continue
        n = len(busy)
        b = sum(x for x, _ in busy) / n
        t = sum(x for _, x in busy) / n
        m = sum(x for x, _ in insts) / len(insts)
        if m == 0 or t <= 0:
            continue
        out.append(f"{name:54s} {grid:9d} {n:5d} {t * 1e6:9.1f} {m:11.0f} {b / m:9.1f} "
                   f"{b / (simds * clock_ghz * 1e9 * t):9.3f}")
    return out


def markers(d: str) -> list[str]:
    ranges = list(csv.DictReader(open(_one(os.path.join(d, "*marker_api_trace.csv")))))
    kt = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"]))
                for r in csv.DictReader(open(_one(os.path.join(d, "*kernel_trace.csv")))))
    out = [f"{'range':48s} {'host_ms':>10s} {'kernels':>8s} {'kernel_ms':>10s}"]
    for r in sorted(ranges, key=lambda r: int(r["Start_Timestamp"])):
        a, b = int(r["Start_Timestamp"]), int(r["End_Timestamp"])
        inside = [(s, e) for s, e in kt if a <= s < b]
        out.append(f"{r['Function'][:48]:48s} {(b - a) / 1e6:10.3f} {len(inside):8d} "
                   f"{sum(e - s for s, e in inside) / 1e6:10.3f}")
    return out


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("kind", choices=("trace", "pmc", "mfma", "markers"))
    ap.add_argument("dir")
    ap.add_argument("--skip", type=int, default=0)
    ap.add_argument("--scale", type=float, default=1.0)
    ap.add_argument("--simds", type=int, default=1024)
    ap.add_argument("--clock-ghz", type=float, default=2.4)
    a = ap.parse_args(argv)
    if a.kind == "trace":
        lines = trace(a.dir, a.skip)
    elif a.kind == "pmc":
        lines = pmc(a.dir, a.scale)
    elif a.kind == "markers":
        lines = markers(a.dir)
    else:
        lines = mfma(a.dir, a.simds, a.clock_ghz)
    print("\n".join(lines))
    return 0


if __name__ == "__main__":
    sys.exit(main())
