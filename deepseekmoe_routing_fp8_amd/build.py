"""Build libmoe_fp8.so (gfx950 only) from csrc/*.hip with hipcc.

Usage: python deepseekmoe_routing_fp8_amd/build.py [--tools]  (run as a file: importing
the package would first load the library being built).
Objects go to <repo>/_build/, the library next to this file. ``--tools`` (build_tools())
also builds the measurement drivers: bench/moe_counters, a native driver of one layer
step for profiler counter runs, bench/hbm_read, the plain streaming read that the HBM
rooflines are compared with, and bench/hbm_write, the store patterns that the
write-bound weight gradients are compared with.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libmoe_fp8.so")
COUNTERS = os.path.join(PKG, "bench", "moe_counters")
HBM_READ = os.path.join(PKG, "bench", "hbm_read")
HBM_WRITE = os.path.join(PKG, "bench", "hbm_write")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
    # no packed-FP32 (v_pk_*_f32) instructions anywhere
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed: {' '.join(cmd)}\n{err}")
    return err


def build(verbose: bool = False) -> str:
    srcs = sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))
    bdir = os.path.join(ROOT, "_build")
    os.makedirs(bdir, exist_ok=True)
    objs = [os.path.join(bdir, os.path.basename(s)[:-4] + ".o") for s in srcs]
    jobs = [[HIPCC, *FLAGS, "-c", s, "-o", o] for s, o in zip(srcs, objs)]
    with ThreadPoolExecutor(min(8, len(jobs))) as ex:
        for msg in ex.map(_run, jobs):
            if verbose and msg.strip():
                print(msg)
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


def build_tools() -> None:
    """The measurement drivers (not part of the library): moe_counters links the library."""
    if not os.path.exists(LIB):
        build()
    tmp = COUNTERS + ".tmp"
    _run([HIPCC, *FLAGS, COUNTERS + ".hip", "-L" + PKG, "-lmoe_fp8", "-Wl,-rpath,$ORIGIN/..",
          "-o", tmp])
    os.replace(tmp, COUNTERS)
    for tool in (HBM_READ, HBM_WRITE):
        tmp = tool + ".tmp"
        _run([HIPCC, *FLAGS, tool + ".hip", "-o", tmp])
        os.replace(tmp, tool)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
    if "--tools" in sys.argv:
        build_tools()
