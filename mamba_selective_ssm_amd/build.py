"""Build libm3scan.so (HIP, gfx950 only) in-tree.

    python -m mamba_selective_ssm_amd.build             # compile every unit, link
    python -m mamba_selective_ssm_amd.build --timeline  # the instrumented copy

Each .hip unit under csrc/ is compiled by hipcc for --offload-arch=gfx950 in
parallel into _build/, then linked into mamba_selective_ssm_amd/libm3scan.so.
Packed fp32 instructions are disabled for all device code.  --timeline builds
a separate library, libm3scan_timeline.so, whose scan kernels stamp each
wave's phase boundaries (M3_TIMELINE=1; read by the timeline module).
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libm3scan.so")
LIB_TIMELINE = os.path.join(PKG, "libm3scan_timeline.so")
ARCH = "gfx950"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else (shutil.which("hipcc") or "hipcc")


def compile_flags():
    return ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-I" + INCLUDE,
            "-I" + CSRC, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wno-unused-result"]


def _compile(src: str, bdir: str = BUILD, extra=()) -> str:
    obj = os.path.join(bdir, os.path.basename(src) + ".o")
    cmd = [hipcc()] + compile_flags() + list(extra) + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, r.stdout))
    return obj


def build(jobs: int | None = None, verbose: bool = False, timeline: bool = False) -> str:
    """Compile all units and link libm3scan.so (timeline: the instrumented
    libm3scan_timeline.so); returns the library path."""
    bdir = os.path.join(BUILD, "timeline") if timeline else BUILD
    lib = LIB_TIMELINE if timeline else LIB
    extra = ("-DM3_TIMELINE=1",) if timeline else ()
    os.makedirs(bdir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    jobs = jobs or min(len(srcs), max(1, (os.cpu_count() or 2)))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda f: _compile(f, bdir, extra), srcs))
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s" % r.stdout)
    os.replace(tmp, lib)
    if verbose:
        print("built", lib)
    return lib


if __name__ == "__main__":
    build(verbose=True, timeline="--timeline" in sys.argv[1:])
    sys.exit(0)
