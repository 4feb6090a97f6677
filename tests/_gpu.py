"""GPU-side helpers for the parity tests: quantised workloads (CPU oracle) and
calls through the C ABI binding."""

from __future__ import annotations

import sys

import numpy as np

import oracle
import synth

_WL = {}


def say(msg: str) -> None:
    """Print and flush before a GPU step, so a crash log names the case."""
    print(msg, flush=True)
    sys.stdout.flush()


def workload(c: int):
    """(w, a8, sa, b8, sb) of workload c, quantised by the oracle on the CPU."""
    if c not in _WL:
        w = synth.WORKLOADS[c]
        a8, sa = oracle.quantize_blocks(synth.make_a(c), w["g"])
        b8, sb = oracle.quantize_blocks(synth.make_b(c), w["g"])
        _WL[c] = (w, a8, sa, b8, sb)
    return _WL[c]


def device_inputs(a8, sa, b8, sb, dev="cuda:0"):
    import torch

    return (torch.from_numpy(np.ascontiguousarray(a8)).to(dev), torch.from_numpy(np.ascontiguousarray(sa)).to(dev),
            torch.from_numpy(np.ascontiguousarray(b8)).to(dev), torch.from_numpy(np.ascontiguousarray(sb)).to(dev))


def gemm(a8, sa, b8, sb, g, dev="cuda:0"):
    """Run dg_gemm_fp8_nt; returns (float64 values, uint16 bf16 bits) on the host."""
    import torch

    import fp8_block_scaled_scales_amd as dg

    ta, tsa, tb, tsb = device_inputs(a8, sa, b8, sb, dev)
    out = dg.dg_gemm_fp8_nt(ta, tb, tsa, tsb, gran=g)
    torch.cuda.synchronize()
    bits = out.view(torch.int16).cpu().numpy().view(np.uint16)
    return out.float().cpu().numpy().astype(np.float64), bits
