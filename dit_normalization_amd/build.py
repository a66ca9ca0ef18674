"""Build the gfx950 HIP library ``libdnorm.so`` in-tree with hipcc.

    python -m dit_normalization_amd.build [--jobs N] [--verbose]

Each ``csrc/*.hip`` unit is compiled to an object (in parallel) under ``_build/`` at the
repository root, then the objects are linked into ``dit_normalization_amd/libdnorm.so``.
The library exposes only the C ABI declared in ``include/dnorm.h``.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libdnorm.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")

COMPILE_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fno-gpu-flush-denormals-to-zero",   # IEEE FP32 denormals on the device
    "-fno-fast-math",
    # Keep the compiler from emitting packed FP32 arithmetic (v_pk_*_f32).
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str, verbose: bool, extra=(), objdir: str = BUILD) -> str:
    obj = os.path.join(objdir, os.path.basename(src).replace(".hip", ".o"))
    cmd = [HIPCC, *COMPILE_FLAGS, *extra, "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so; drop that line.
    noise = "is not a recognized feature for this target"
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {os.path.basename(src)}:\n{msg}")
    if msg.strip() and verbose:
        print(msg, flush=True)
    return obj


def build(jobs: int | None = None, verbose: bool = False, extra=(), out: str = LIB) -> str:
    """Compile every HIP unit for gfx950 and link libdnorm.so (or `out`); returns its path.
    `extra` adds compiler flags (tuning builds); objects then go to a separate folder."""
    tag = "".join(c if c.isalnum() else "_" for c in "".join(extra))
    objdir = BUILD if not extra else os.path.join(BUILD, "variant" + tag)
    os.makedirs(objdir, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), max(1, (os.cpu_count() or 4)))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, extra, objdir), srcs))
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, out)
    return out


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("--verbose", action="store_true")
    a = ap.parse_args(argv)
    path = build(a.jobs, a.verbose)
    print(path)
    return 0


if __name__ == "__main__":
    sys.exit(main())
