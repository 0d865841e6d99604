"""Summaries of rocprofv3 CSV output (kernel traces and PMC counters).

    python -m frame_wise_gated_amd.profsum trace DIR [--skip N]
        per-kernel dispatch count, mean / min / max duration (us) from
        DIR/*kernel_trace.csv; --skip drops each kernel's first N dispatches
        (warm-up launches).
    python -m frame_wise_gated_amd.profsum pmc DIR [--scale F]
        per-kernel mean counter value per dispatch (KiB for FETCH_SIZE and
        WRITE_SIZE) from DIR/*counter_collection.csv, also multiplied by F
        and shown in MB.

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


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("kind", choices=("trace", "pmc"))
    ap.add_argument("dir")
    ap.add_argument("--skip", type=int, default=0)
    ap.add_argument("--scale", type=float, default=1.0)
    a = ap.parse_args(argv)
    lines = trace(a.dir, a.skip) if a.kind == "trace" else pmc(a.dir, a.scale)
    print("\n".join(lines))
    return 0


if __name__ == "__main__":
    sys.exit(main())
