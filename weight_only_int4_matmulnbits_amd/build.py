"""Build libmnb.so in-tree with hipcc for gfx950.

Every HIP source is compiled with packed-FP32 instructions disabled
(``-target-feature -packed-fp32-ops``): the kernels rely on ordinary scalar
float32 arithmetic only.  The library links the HIP runtime by soname, so in a
process that imported torch first it shares torch's runtime.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmnb.so")
# the benchmark's bandwidth control arm, a separate library (include/mnb_probe.h)
PROBE_LIB = os.path.join(PKG, "libmnb_probe.so")
PROBE_SOURCE = "mnb_probe.hip"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# the longest compiles first (the GEMV instances of each activation type and
# the prefill GEMM), so that they start at once
SOURCES = ["mnb_gemv_f32.hip", "mnb_gemv_bf16.hip", "mnb_gemm.hip", "mnb_gemv.hip", "mnb_api.hip", "mnb_pack.hip",
           "mnb_smallm.hip", "mnb_aux.hip", "mnb_step.hip"]

CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-mcode-object-version=5",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so;
    # that warning is expected and dropped from the log
    err = "\n".join(l for l in r.stderr.splitlines()
                    if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed: {' '.join(cmd)}\n{r.stdout}\n{err}")
    return err


def build(verbose: bool = False) -> str:
    """Compile every source and link libmnb.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES + [PROBE_SOURCE]:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        if src != PROBE_SOURCE:
            objs.append(obj)
        cmds.append([HIPCC, *CFLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    with cf.ThreadPoolExecutor(max_workers=min(len(cmds), os.cpu_count() or 4, 8)) as ex:
        for log in ex.map(_run, cmds):
            if verbose and log.strip():
                print(log, file=sys.stderr)
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    tmp = PROBE_LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp,
          os.path.join(BUILD, PROBE_SOURCE.replace(".hip", ".o"))])
    os.replace(tmp, PROBE_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
