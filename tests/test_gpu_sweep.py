"""A seeded sweep over combinations of the call's options.

The other GPU tests take the options one or two at a time on chosen shapes.
Here each case draws, from a fixed seed, a shape from edge sizes (1-3, one
under/over a tile edge, ragged), a granularity, formats for A and B, block or
per-row A factors, an epilogue, and whether a workspace is given (then the
split-K class runs, through the tile override, and splits K over
workgroups), and runs it in all four layouts. Every output element is
compared with the oracle (tolerance as everywhere), and the three transposed
layouts must give the NT layout's bits (the same K order inside every
product).
"""

from __future__ import annotations

import contextlib

import numpy as np
import pytest

import oracle
import synth
from tests import _common
from tests._gpu import say

pytestmark = pytest.mark.gpu

SIZES = [1, 2, 3, 15, 17, 31, 33, 63, 64, 65, 97, 127, 128, 129, 200, 255, 257, 300]


def _case(i):
    rng = np.random.default_rng(70000 + i)
    g = int(rng.choice([64, 128, 256]))
    M = int(rng.choice(SIZES))
    N = int(rng.choice(SIZES + [513, 1000]))
    K = g * int(rng.integers(1, 10 if g < 256 else 5))
    fa, fb = int(rng.integers(0, 2)), int(rng.integers(0, 2))
    rowa = bool(rng.integers(0, 2))
    epi = int(rng.integers(0, 4))  # none, bias, bias + ReLU, GELU
    ws = bool(rng.integers(0, 2))
    return M, N, K, g, fa, fb, rowa, epi, ws


CASES = [_case(i) for i in range(96)]


@pytest.mark.parametrize("i", range(len(CASES)))
def test_option_sweep(i):
    import torch

    import fp8_block_scaled_scales_amd as dg

    M, N, K, g, fa, fb, rowa, epi, ws = CASES[i]
    x = synth.normal(71000 + i, (M, K))
    if rowa:
        x = (x * np.exp(np.random.default_rng(i).uniform(-3, 3, size=(M, 1)))).astype(np.float32)
        a8, sa = oracle.quantize_rows_fmt(x, g, fa)
    else:
        a8, sa = oracle.quantize_blocks_fmt(x, g, fa)
    b8, sb = oracle.quantize_blocks_fmt(synth.normal(72000 + i, (N, K), sigma=0.02), g, fb)
    bias = synth.normal(73000 + i, (N,), sigma=0.5).astype(np.float32) if epi in (1, 2) else None
    act = {0: 0, 1: 0, 2: 1, 3: 2}[epi]
    ref = oracle.gemm_ref_rowa(a8, b8, sa, sb, g, fa, fb) if rowa else oracle.gemm_ref_fmt(a8, b8, sa, sb, g, fa, fb)
    if bias is not None or act:
        ref = oracle.epilogue(ref, bias, act)
    dev = "cuda:0"
    tsa, tsb = torch.from_numpy(sa).to(dev), torch.from_numpy(sb).to(dev)
    tbias = None if bias is None else torch.from_numpy(bias).to(dev)
    bits = {}
    with _common.forced_split(g) if ws else contextlib.nullcontext():
        for layout in range(4):
            a_st = np.ascontiguousarray(a8.T) if layout & 2 else a8
            b_st = np.ascontiguousarray(b8.T) if layout & 1 else b8
            plan = dg.dg_query_tile(M, N, K, g, layout, workspace=ws)
            say("sweep %d: %dx%dx%d g=%d fmt %d,%d rowa=%d epi=%d ws=%d layout %d -> %dx%d ksplit %d" % (
                i, M, N, K, g, fa, fb, rowa, epi, ws, layout, plan["bm"], plan["bn"], plan["ksplit"]))
            out = dg.dg_gemm_fp8_ws(torch.from_numpy(a_st).to(dev), torch.from_numpy(b_st).to(dev), tsa, tsb, gran=g,
                                    layout=layout, sa_rows=1 if rowa else None, fmt_a=fa, fmt_b=fb, bias=tbias, act=act,
                                    workspace=dg.dg_workspace(M, N, K, g, layout, device=dev) if ws else None)
            torch.cuda.synchronize()
            bits[layout] = out.view(torch.int16).cpu().numpy().view(np.uint16)
            got = _common.bf16_bits_to_f64(bits[layout])
            ok, rms = _common.within_tolerance(got, ref)
            assert ok.all(), "case %d layout %d: %d of %d outside tolerance (first at %s)" % (
                i, layout, int((~ok).sum()), ok.size, np.argwhere(~ok)[0])
    for layout in (1, 2, 3):
        assert np.array_equal(bits[layout], bits[0]), "case %d: layout %d differs from NT" % (i, layout)


def _large_case(i):
    rng = np.random.default_rng(80000 + i)
    g = int(rng.choice([64, 128, 256]))
    M = int(rng.integers(1800, 4200))
    N = int(rng.integers(3300, 4200))
    K = g * int(rng.integers(2, 9 if g < 256 else 5))
    fa, fb = int(rng.integers(0, 2)), int(rng.integers(0, 2))
    rowa = bool(rng.integers(0, 2))
    epi = int(rng.integers(0, 4))
    return M, N, K, g, fa, fb, rowa, epi


LARGE = [_large_case(i) for i in range(16)]


@pytest.mark.parametrize("i", range(len(LARGE)))
def test_option_sweep_large(i):
    """The same on the 256-row (and 128x128) tiles: ragged M and N in the
    thousands, sampled rows and columns against the oracle (every tile edge
    included), every layout against NT bit for bit."""
    import torch

    import fp8_block_scaled_scales_amd as dg

    M, N, K, g, fa, fb, rowa, epi = LARGE[i]
    x = synth.normal(81000 + i, (M, K))
    if rowa:
        x = (x * np.exp(np.random.default_rng(i).uniform(-3, 3, size=(M, 1)))).astype(np.float32)
        a8, sa = oracle.quantize_rows_fmt(x, g, fa)
    else:
        a8, sa = oracle.quantize_blocks_fmt(x, g, fa)
    b8, sb = oracle.quantize_blocks_fmt(synth.normal(82000 + i, (N, K), sigma=0.02), g, fb)
    bias = synth.normal(83000 + i, (N,), sigma=0.5).astype(np.float32) if epi in (1, 2) else None
    act = {0: 0, 1: 0, 2: 1, 3: 2}[epi]
    plan = dg.dg_query_tile(M, N, K, g)
    bm, bn = plan["bm"], plan["bn"]
    rows = np.unique(np.concatenate([_common.sample_indices(M, 48, seed=i), np.arange(0, M, bm),
                                     np.arange(bm - 1, M, bm), [M - 1]]))
    cols = np.unique(np.concatenate([_common.sample_indices(N, 96, seed=i + 1), np.arange(0, N, bn),
                                     np.arange(bn - 1, N, bn), [N - 1]]))
    if rowa:
        ref = oracle.gemm_ref_rowa(a8, b8, sa, sb, g, fa, fb, rows=rows, cols=cols)
    else:
        ref = oracle.gemm_ref_fmt(a8, b8, sa, sb, g, fa, fb, rows=rows, cols=cols)
    if bias is not None or act:
        ref = oracle.epilogue(ref, bias, act, cols=cols)
    dev = "cuda:0"
    tsa, tsb = torch.from_numpy(sa).to(dev), torch.from_numpy(sb).to(dev)
    tbias = None if bias is None else torch.from_numpy(bias).to(dev)
    bits = {}
    for layout in range(4):
        a_st = np.ascontiguousarray(a8.T) if layout & 2 else a8
        b_st = np.ascontiguousarray(b8.T) if layout & 1 else b8
        say("large sweep %d: %dx%dx%d g=%d fmt %d,%d rowa=%d epi=%d layout %d -> %dx%d" % (
            i, M, N, K, g, fa, fb, rowa, epi, layout, bm, bn))
        out = dg.dg_gemm_fp8_ws(torch.from_numpy(a_st).to(dev), torch.from_numpy(b_st).to(dev), tsa, tsb, gran=g,
                                layout=layout, sa_rows=1 if rowa else None, fmt_a=fa, fmt_b=fb, bias=tbias, act=act)
        torch.cuda.synchronize()
        bits[layout] = out.view(torch.int16).cpu().numpy().view(np.uint16)
        if layout == 0:
            got = _common.bf16_bits_to_f64(bits[0])[np.ix_(rows, cols)]
            ok, _ = _common.within_tolerance(got, ref)
            assert ok.all(), "large case %d: %d of %d outside tolerance (first at %s)" % (
                i, int((~ok).sum()), ok.size, np.argwhere(~ok)[0])
        else:
            assert np.array_equal(bits[layout], bits[0]), "large case %d: layout %d differs from NT" % (i, layout)
