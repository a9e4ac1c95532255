"""Build libssd.so (HIP, gfx950) in-tree with hipcc.

Usage: python -m mamba_ssd_chunked_scan_amd.build   (or build() from Python)

Every source under csrc/ is compiled to an object in _build/ (in parallel),
then linked into mamba_ssd_chunked_scan_amd/libssd.so.  The device code targets
gfx950 only.  Packed fp32 VALU instructions are disabled for the device pass
(-packed-fp32-ops); the host pass warns that it does not know the feature,
which is harmless.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libssd.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    "-Wall", "-Wno-unused-function",
]


def sources():
    return sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def _compile(src: str, bdir: str = BUILD, extra=()) -> str:
    obj = os.path.join(bdir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *CFLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    noise = "not a recognized feature for this target"
    msgs = [ln for ln in r.stderr.splitlines() if noise not in ln and ln.strip()]
    if msgs:
        sys.stderr.write(f"[{src}]\n" + "\n".join(msgs) + "\n")
    return obj


def build(jobs: int | None = None, variant: str = "") -> str:
    """Compile all HIP sources for gfx950 and link libssd.so; returns its path.

    ``variant="trace"`` builds the profiling library libssd_trace.so instead:
    the same sources with -DSSD_FUSED_TRACE (the fused forward stores per-item
    phase timestamps at the end of its workspace; see fused_trace.py).
    """
    bdir = BUILD if not variant else BUILD + "_" + variant
    lib = LIB if not variant else os.path.join(HERE, f"libssd_{variant}.so")
    extra = [] if not variant else ["-DSSD_FUSED_TRACE"]
    os.makedirs(bdir, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(8, os.cpu_count() or 1)
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda f: _compile(f, bdir, extra), srcs))
    tmp = lib + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(variant=sys.argv[1] if len(sys.argv) > 1 else ""))
