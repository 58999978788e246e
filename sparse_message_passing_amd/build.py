"""Build libgnnmp.so (the C-ABI library) for gfx950 with hipcc.

    python -m sparse_message_passing_amd.build [--jobs N]

Every source under ``csrc/`` becomes an object in ``_build/`` (compiled in
parallel); the objects are linked into ``libgnnmp.so`` next to this file.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libgnnmp.so")
CALIB_LIB = os.path.join(HERE, "libgnnmp_calib.so")
ARCH = os.environ.get("GNNMP_ARCH", "gfx950")

COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # packed fp32 instructions stay off (hipcc still forms ordinary fp32 code)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-Wall", "-Wno-unused-result",
]


def hipcc() -> str:
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(p):
        raise RuntimeError("hipcc not found: the HIP toolchain (ROCm) is required to build libgnnmp.so")
    return p


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


# Per-file flags.  The quantiser's codes must match any faithful binary32
# evaluation bit for bit, so nothing in it may be fused into an FMA (the
# backend contracts across statements under the default fp-contract=fast).
PER_FILE = {"quant.hip": ["-ffp-contract=off"]}


def _headers_mtime() -> float:
    hs = [os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".h")]
    hs += [os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))]
    return max(os.path.getmtime(h) for h in hs)


def _compile(src: str, incremental: bool = False) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    if incremental and os.path.exists(obj) and \
            os.path.getmtime(obj) > max(os.path.getmtime(src), _headers_mtime(), os.path.getmtime(__file__)):
        return obj
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [hipcc(), *COMMON, *PER_FILE.get(os.path.basename(src), []), *lang, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    # the host pass does not know the gfx feature name; that warning is expected
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l).strip()
    if err:
        sys.stderr.write(err + "\n")
    return obj


def build(jobs: int | None = None, verbose: bool = True, incremental: bool = False) -> str:
    """Compile every source (incremental: only those whose object is older
    than the source, a header or this script) and link the library."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), max(1, (os.cpu_count() or 4)), 16)
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, incremental), srcs))
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp, "-lpthread"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    build_calib()
    if verbose:
        print(f"built {LIB} and {CALIB_LIB}")
    return LIB


def build_calib() -> str:
    """The reference kernels of known traffic and flops (calib/calib.hip) the
    bench's --calibrate mode runs; a library of their own."""
    src = os.path.join(HERE, "calib", "calib.hip")
    tmp = CALIB_LIB + f".tmp{os.getpid()}"
    cmd = [hipcc(), *COMMON, "-x", "hip", "-shared", src, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, CALIB_LIB)
    return CALIB_LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("--incremental", action="store_true")
    a = ap.parse_args()
    build(a.jobs, incremental=a.incremental)
