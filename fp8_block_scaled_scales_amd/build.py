"""Compile the HIP library ``libdg.so`` for gfx950 in-tree with hipcc.

Used by ``__graft_entry__.build()``; also runnable as ``python -m
fp8_block_scaled_scales_amd.build``. Always recompiles.
"""

from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libdg.so")
# Longest compiles first, so the parallel build's slowest jobs start at once.
SOURCES = ["gemm_fp8_big_layouts_rowa.hip", "gemm_fp8_big_layouts.hip", "gemm_fp8_stream.hip",
           "gemm_fp8_layouts_rowa.hip", "gemm_fp8_layouts.hip", "gemm_fp8_nt_big.hip", "gemm_fp8_nt.hip",
           "quant_fp8.hip", "dg_host.hip"]

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


# Libraries built from the same sources: the release build, and the race
# check build with an extra full wait and workgroup barrier after every
# pipeline step (DG_EXTRA_SYNC in gemm_common.h), whose results must equal the
# release build's bit for bit.
VARIANTS = {"libdg.so": [], "libdg_sync.so": ["-DDG_EXTRA_SYNC"]}
LINK = ["--offload-arch=gfx950", "-shared", "-fPIC", "-Wl,-Bsymbolic"]


def build(verbose: bool = False, variants=None) -> str:
    """Compile every source of every variant to an object (at most one hipcc
    per CPU at a time), then link each library. Returns the release library's
    path."""
    names = list(VARIANTS) if variants is None else list(variants)
    tag = "%d" % os.getpid()
    jobs = []
    for src in SOURCES:
        for name in names:
            obj = os.path.join(CSRC, "%s.%s.tmp%s.o" % (src, name.split(".")[0], tag))
            cmd = [HIPCC] + [f for f in FLAGS if f != "-shared"] + VARIANTS[name] + \
                ["-c", os.path.join(CSRC, src), "-o", obj]
            jobs.append((name, obj, cmd))

    def compile_one(cmd):
        if verbose:
            print(" ".join(cmd), flush=True)
        return subprocess.run(cmd, capture_output=True, text=True)

    width = max(1, min(len(jobs), os.cpu_count() or 1))
    try:
        with concurrent.futures.ThreadPoolExecutor(max_workers=width) as pool:
            results = list(pool.map(compile_one, [cmd for _, _, cmd in jobs]))
        failed = [r for r in results if r.returncode != 0]
        for r in failed:
            sys.stderr.write(r.stdout + r.stderr)
        if failed:
            raise RuntimeError("hipcc failed compiling the library sources")
        for name in names:
            lib = os.path.join(HERE, name)
            tmp = lib + ".tmp" + tag
            cmd = [HIPCC] + LINK + [obj for n, obj, _ in jobs if n == name] + ["-o", tmp]
            if verbose:
                print(" ".join(cmd), flush=True)
            res = subprocess.run(cmd, capture_output=True, text=True)
            if res.returncode != 0:
                sys.stderr.write(res.stdout + res.stderr)
                raise RuntimeError("hipcc failed linking " + name)
            os.replace(tmp, lib)
    finally:
        for _, obj, _ in jobs:
            if os.path.exists(obj):
                os.remove(obj)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
