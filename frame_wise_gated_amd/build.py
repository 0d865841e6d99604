"""Build libgdn.so (the HIP/gfx950 C-ABI library) in-tree with hipcc, and
libhbm_probe.so (the plain HBM streams the benchmark's calibration mode times).

Usage: python -m frame_wise_gated_amd.build   (or call build()).
Every call recompiles; the shared objects land next to this file.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(HERE, "libgdn.so")
SOURCES = ["gdn_api.hip", "k_misc.hip", "k_terms.hip", "k_scan.hip", "k_readout.hip", "k_bwd.hip"]
PROBE_OUT = os.path.join(HERE, "libhbm_probe.so")
PROBE_SOURCES = ["hbm_probe.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fvisibility=hidden",
    "-Wall",
    "-Wno-unused-function",
    # packed fp32 vector ops stay disabled in all device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE,
    "-I", CSRC,
]


# Host-only sanitizers for the C-ABI layer (argument checks, workspace layout,
# launch sequencing): each -fsanitize applies to the host pass alone, the
# device code is built as usual.
SANITIZE_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def _compile(src: str, obj_dir: str, extra=()) -> str:
    obj = os.path.join(obj_dir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    noise = "is not a recognized feature for this target"
    warn = "\n".join(l for l in (r.stderr or "").splitlines() if noise not in l)
    if warn.strip():
        sys.stderr.write(warn + "\n")
    return obj


def _link(objs: list[str], out: str, extra=()) -> None:
    tmp = out + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *extra, *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = True) -> str:
    obj_dir = os.path.join(HERE, "_build")
    os.makedirs(obj_dir, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    with ThreadPoolExecutor(max_workers=min(len(srcs), 8)) as ex:
        objs = list(ex.map(lambda s: _compile(s, obj_dir), srcs))
    _link(objs[:len(SOURCES)], OUT)
    _link(objs[len(SOURCES):], PROBE_OUT)
    shutil.rmtree(obj_dir, ignore_errors=True)
    if verbose:
        print(f"built {OUT} and {PROBE_OUT}")
    return OUT


def build_sanitized(out_dir: str) -> str:
    """libgdn.so with its C-ABI layer (gdn_api.hip) built under host-only
    AddressSanitizer and UndefinedBehaviorSanitizer, into out_dir. Load it
    into a process that preloads the ASan runtime (sanitizer_runtime())."""
    obj_dir = os.path.join(out_dir, "obj")
    os.makedirs(obj_dir, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), 8)) as ex:
        objs = list(ex.map(lambda s: _compile(s, obj_dir, SANITIZE_HOST if s == "gdn_api.hip" else ()),
                           SOURCES))
    out = os.path.join(out_dir, "libgdn.so")
    # the sanitizer entry points stay undefined in the library and resolve
    # against the preloaded runtime
    _link(objs, out)
    return out


def sanitizer_runtime() -> str:
    """Path of the clang ASan runtime that a sanitized libgdn.so needs preloaded."""
    clang = os.path.join(os.path.dirname(os.path.realpath(HIPCC)), "..", "lib", "llvm", "bin", "clang")
    if not os.path.exists(clang):
        clang = "/opt/rocm/llvm/bin/clang"
    r = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                       text=True, check=True)
    return r.stdout.strip()


if __name__ == "__main__":
    build()
