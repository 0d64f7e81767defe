"""Builds libfibattn.so in-tree for gfx950 with hipcc (cross-compiles without a GPU).

    python fibonacci_offset_sparse_amd/build.py      (or __graft_entry__.build())

Run it as a script (not with -m): importing the package loads the library being rebuilt.

Objects go to _build/ at the repository root; the library lands next to this file.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(PKG, "libfibattn.so")
# the streaming-bandwidth probe the benchmark reads the kernels' bandwidth against (not part of the
# attention library)
PROBE_SRC = "stream_probe.hip"
PROBE_OUT = os.path.join(PKG, "libstreamprobe.so")
# the same library with the forward attention kernel's phase trace compiled in (FIBATTN_PHASE_TRACE:
# per-workgroup stamps read back by fibattn_phase_trace_read; `bench.py --phase-trace` loads it)
TRACE_SRC = "fibattn_fwd_mfma.hip"
TRACE_OUT = os.path.join(PKG, "libfibattn_trace.so")
BUILD_DIR = os.path.join(ROOT, "_build")

ARCH = "gfx950"
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", f"-I{INCLUDE}", f"-I{CSRC}"]
# Packed fp32 VALU instructions stay off: kernels use scalar fp32 FMA only.
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]

SOURCES = ["fibattn_api.cpp", "fibattn_fwd.hip", "fibattn_fwd_mfma.hip", "fibattn_bwd.hip", "fibattn_bwd_mfma.hip",
           "fibattn_decode.hip", "fibattn_noalloc.hip"]


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found (ROCm is required to build libfibattn.so)")
    return exe


def _compile(src: str, defines=()) -> str:
    tag = "".join("_" + d.lower() for d in defines)
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + tag + ".o")
    cmd = [hipcc(), *COMMON, *(f"-D{d}" for d in defines), "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".hip"):
        cmd[1:1] = DEVICE
    else:
        cmd[1:1] = ["-x", "c++", "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def _link(objs, out):
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"linking failed:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES) + 2) as ex:
        jobs = [ex.submit(_compile, s) for s in SOURCES + [PROBE_SRC]]
        trace_job = ex.submit(_compile, TRACE_SRC, ("FIBATTN_PHASE_TRACE",))
        objs = [j.result() for j in jobs]
        trace_obj = trace_job.result()
    _link(objs[:-1], OUT)
    _link(objs[-1:], PROBE_OUT)
    _link([trace_obj if s == TRACE_SRC else o for s, o in zip(SOURCES, objs[:-1])], TRACE_OUT)
    if verbose:
        print(f"built {OUT}, {PROBE_OUT} and {TRACE_OUT}")
    return OUT


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
