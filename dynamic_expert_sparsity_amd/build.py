"""Build libbeam_moe.so (HIP, gfx950) in-tree with hipcc.

    python -m dynamic_expert_sparsity_amd.build

Compiles the layer's csrc/*.hip translation units to objects under _build/
(in parallel), links them into dynamic_expert_sparsity_amd/libbeam_moe.so and
replaces the previous library atomically; the measurement kernels
(csrc/peak.hip) become libbeam_peak.so the same way.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libbeam_moe.so")
SOURCES = ["router.hip", "compact.hip", "experts.hip", "small.hip", "gemm.hip", "stats.hip",
           "backward.hip", "api.hip"]
PEAK_LIB = os.path.join(PKG, "libbeam_peak.so")
PEAK_SOURCES = ["peak.hip"]

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
CFLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # no packed-fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
]


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the device-only feature: drop that notice
    out = "\n".join(l for l in p.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if p.returncode != 0:
        raise RuntimeError(f"command failed ({p.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    libs = [(LIB, SOURCES), (PEAK_LIB, PEAK_SOURCES)]
    units = [s for _, srcs in libs for s in srcs]
    objs = {s: os.path.join(BUILD, s.replace(".hip", ".o")) for s in units}
    cmds = [[HIPCC, *CFLAGS, "-c", os.path.join(CSRC, s), "-o", objs[s]] for s in units]
    with cf.ThreadPoolExecutor(max_workers=min(len(cmds), 8)) as ex:
        for out in ex.map(_run, cmds):
            if verbose and out.strip():
                print(out)
    for lib, srcs in libs:
        tmp = lib + ".tmp"
        out = _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp,
                    *[objs[s] for s in srcs]])
        if verbose and out.strip():
            print(out)
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
