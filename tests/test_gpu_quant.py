"""The GPU block quantiser (dg_quantize_e4m3_blocks) against the CPU oracle's.

Both take scale = amax/448 per g x g block (1.0 for an all-zero block) and
code = E4M3FN(x / scale) with a correctly rounded FP32 divide and
round-to-nearest-even, so codes and scales must agree bit for bit.
"""

import numpy as np
import pytest

import oracle
import synth
from tests._gpu import say

pytestmark = pytest.mark.gpu


def _gpu_quant(x, g):
    import torch

    import fp8_block_scaled_scales_amd as dg

    tx = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda:0")
    q, s = dg.dg_quantize_e4m3_blocks(tx, gran=g)
    torch.cuda.synchronize()
    return q.cpu().numpy(), s.cpu().numpy()


def _check(x, g, label):
    say("quantise %s %s g=%d" % (label, x.shape, g))
    q, s = _gpu_quant(x, g)
    rq, rs = oracle.quantize_blocks(x, g)
    assert np.array_equal(s.view(np.uint32), rs.view(np.uint32)), "scales differ"
    bad = q != rq
    assert not bad.any(), "%d codes differ, first at %s" % (int(bad.sum()), np.argwhere(bad)[0])


@pytest.mark.parametrize("c", [1, 2, 3, 5])
def test_workload_operands_bitwise(c):
    w = synth.WORKLOADS[c]
    M = min(w["M"], 1000)
    N = min(w["N"], 1000)
    _check(synth.make_a(c, M=M), w["g"], "A of workload %d" % c)
    _check(synth.make_b(c, N=N), w["g"], "B of workload %d" % c)


@pytest.mark.parametrize("rows,cols,g", [(1, 64, 64), (1, 128, 128), (17, 192, 64), (129, 256, 128),
                                         (200, 640, 64), (1023, 384, 128)])
def test_ragged_rows_bitwise(rows, cols, g):
    _check(synth.normal(900 + rows, (rows, cols)), g, "ragged")


def test_special_blocks_bitwise():
    g = 64
    x = synth.normal(77, (192, 256)) * np.float32(3.0)
    x[0:64, 0:64] = 0.0                      # all-zero block: scale 1.0, codes 0
    x[64:128, 64:128] = np.float32(1e-30)    # tiny constant block
    x[128:192, 128:192] *= np.float32(1e6)   # wide range
    x[0, 200] = np.float32(-7.5)             # negative extreme of its block
    _check(x, g, "special blocks")


# --- quotients next to a rounding midpoint of the FP8 format ----------------
# The kernels divide by a block's scale through its reciprocal and two FMA
# corrections, which must give the correctly rounded FP32 quotient the oracle
# takes (its FP32 divide), because the code is that quotient rounded again to
# FP8: where the quotient sits within a few FP32 ulps of a midpoint between
# two FP8 values, one ulp decides the code. These inputs put x / scale there
# on purpose: x = RN(t * scale) moved by -3..3 ulps, t a midpoint of the format
# (normal and subnormal), in blocks whose largest element fixes scale.

def _midpoints(fmt):
    if fmt == 0:  # E4M3FN: 3 mantissa bits, exponents -6..8, subnormal step 2^-9
        normal = [(1 + (2 * m + 1) / 16.0) * 2.0 ** e for e in range(-6, 9) for m in range(8)]
        sub = [(2 * j + 1) * 2.0 ** -10 for j in range(8)]
        fmax = 448.0
    else:  # E5M2: 2 mantissa bits, exponents -14..15, subnormal step 2^-16
        normal = [(1 + (2 * m + 1) / 8.0) * 2.0 ** e for e in range(-14, 16) for m in range(4)]
        sub = [(2 * j + 1) * 2.0 ** -17 for j in range(4)]
        fmax = 57344.0
    t = np.array([v for v in normal + sub if v < 0.99 * fmax], dtype=np.float64)
    return t, np.float32(fmax)


def _near_midpoints(seed, rows, cols, brows, g, fmt):
    """rows x cols FP32 whose blocks (brows x g) each hold one element that
    sets amax and quotients near FP8 midpoints everywhere else."""
    rng = np.random.default_rng(seed)
    t, fmax = _midpoints(fmt)
    x = np.empty((rows, cols), np.float32)
    for r0 in range(0, rows, brows):
        for c0 in range(0, cols, g):
            blk = x[r0:r0 + brows, c0:c0 + g]
            amax = np.float32(fmax * np.float32(2.0 ** rng.uniform(-30, 30)))
            scale = np.float32(amax / fmax)  # FP32 divide, as both sides take it
            tv = t[rng.integers(0, t.size, size=blk.shape)] * rng.choice([-1.0, 1.0], size=blk.shape)
            v = (tv.astype(np.float32) * scale).astype(np.float32)
            for _ in range(3):  # move each value by k ulps, k in -3..3
                step = rng.integers(-1, 2, size=blk.shape)
                v = np.where(step > 0, np.nextafter(v, np.float32(np.inf)),
                             np.where(step < 0, np.nextafter(v, np.float32(-np.inf)), v)).astype(np.float32)
            v = np.clip(v, -amax, amax)
            blk[...] = v
            i, j = rng.integers(0, blk.shape[0]), rng.integers(0, blk.shape[1])
            blk[i, j] = amax * np.float32(rng.choice([-1.0, 1.0]))
    return x


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("rows,cols,g", [(256, 512, 128), (192, 256, 64), (512, 512, 256), (130, 384, 64)])
def test_blocks_near_midpoints_bitwise(fmt, rows, cols, g):
    import torch

    import fp8_block_scaled_scales_amd as dg

    x = _near_midpoints(3000 + rows + fmt, rows, cols, g, g, fmt)
    say("quantise near midpoints fmt=%d %dx%d g=%d" % (fmt, rows, cols, g))
    q, s = dg.dg_quantize_fp8_blocks(torch.from_numpy(x).to("cuda:0"), gran=g, fmt=fmt)
    torch.cuda.synchronize()
    rq, rs = oracle.quantize_blocks_fmt(x, g, fmt)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), rs.view(np.uint32)), "scales differ"
    bad = q.cpu().numpy() != rq
    assert not bad.any(), "%d codes differ, first at %s" % (int(bad.sum()), np.argwhere(bad)[0])


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("rows,cols,g", [(64, 512, 128), (33, 256, 64), (16, 512, 256)])
def test_rows_near_midpoints_bitwise(fmt, rows, cols, g):
    import torch

    import fp8_block_scaled_scales_amd as dg

    x = _near_midpoints(4000 + rows + fmt, rows, cols, 1, g, fmt)
    say("quantise rows near midpoints fmt=%d %dx%d g=%d" % (fmt, rows, cols, g))
    q, s = dg.dg_quantize_fp8_rows(torch.from_numpy(x).to("cuda:0"), gran=g, fmt=fmt)
    torch.cuda.synchronize()
    rq, rs = oracle.quantize_rows_fmt(x, g, fmt)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), rs.view(np.uint32)), "scales differ"
    bad = q.cpu().numpy() != rq
    assert not bad.any(), "%d codes differ, first at %s" % (int(bad.sum()), np.argwhere(bad)[0])


@pytest.mark.parametrize("per_row", [False, True])
def test_extreme_scales_bitwise(per_row):
    """Blocks whose scale or its reciprocal leaves the normal range (the
    kernels then divide per element), blocks just inside that range, tiny
    and huge magnitudes, signed zeros."""
    import torch

    import fp8_block_scaled_scales_amd as dg

    g = 64
    rng = np.random.default_rng(55 + per_row)
    # 1e-44 and 1e-42: amax / fmax underflows (E4M3, resp. E5M2), scale 1.0
    mags = [1e-44, 1e-42, 3e-39, 448.0 * 2.0 ** -121, 448.0 * 2.0 ** -119, 1e-30, 1.0, 1e30, 3e38]
    x = np.zeros((64 * len(mags), 128), np.float32)
    for i, m in enumerate(mags):
        blk = (rng.uniform(-1.0, 1.0, (64, 128)) * m).astype(np.float32)  # finite, as the quantiser requires
        blk[0, 0] = np.float32(-0.0)
        blk[1, 1] = np.float32(0.0)
        x[64 * i:64 * i + 64] = blk
    say("quantise extreme scales per_row=%d" % per_row)
    for fmt in (0, 1):
        tx = torch.from_numpy(x).to("cuda:0")
        if per_row:
            q, s = dg.dg_quantize_fp8_rows(tx, gran=g, fmt=fmt)
            rq, rs = oracle.quantize_rows_fmt(x, g, fmt)
        else:
            q, s = dg.dg_quantize_fp8_blocks(tx, gran=g, fmt=fmt)
            rq, rs = oracle.quantize_blocks_fmt(x, g, fmt)
        torch.cuda.synchronize()
        assert np.array_equal(s.cpu().numpy().view(np.uint32), rs.view(np.uint32)), ("scales differ", fmt)
        bad = q.cpu().numpy() != rq
        assert not bad.any(), "fmt %d: %d codes differ, first at %s" % (fmt, int(bad.sum()), np.argwhere(bad)[0])
