"""Compile the HIP library ``libdg.so`` for gfx950 in-tree with hipcc.

Used by ``__graft_entry__.build()``; also runnable as ``python -m
fp8_block_scaled_scales_amd.build``. Always recompiles.
"""

from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libdg.so")
SOURCES = ["dg_host.hip", "gemm_fp8_nt.hip", "gemm_fp8_nt_big.hip", "gemm_fp8_stream.hip", "gemm_fp8_layouts.hip",
           "gemm_fp8_big_layouts.hip", "gemm_fp8_layouts_rowa.hip", "gemm_fp8_big_layouts_rowa.hip", "quant_fp8.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # no packed FP32 VALU instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results land in ordinary VGPRs, so the FP32 promotion reads them directly
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wno-unused-command-line-argument",
]


def build(verbose: bool = False) -> str:
    """Compile every source to an object at once (one hipcc per source), then link."""
    tag = "%d" % os.getpid()
    objs, procs = [], []
    for src in SOURCES:
        obj = os.path.join(CSRC, src + ".tmp%s.o" % tag)
        cmd = [HIPCC] + [f for f in FLAGS if f != "-shared"] + ["-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        objs.append(obj)
        procs.append(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True))
    failed = False
    for p in procs:
        out, err = p.communicate()
        if p.returncode != 0:
            sys.stderr.write(out + err)
            failed = True
    try:
        if failed:
            raise RuntimeError("hipcc failed compiling libdg.so's sources")
        tmp = LIB + ".tmp" + tag
        cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            sys.stderr.write(res.stdout + res.stderr)
            raise RuntimeError("hipcc failed linking libdg.so")
        os.replace(tmp, LIB)
    finally:
        for obj in objs:
            if os.path.exists(obj):
                os.remove(obj)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
