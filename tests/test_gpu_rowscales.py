"""Per-row A scales on the GPU (through the C ABI) against the CPU oracle.

A carries one FP32 factor per row and g-wide K segment (1 x g blocks, the
per-channel factors of the template article, §3.4), B keeps its g x g blocks.
Each kernel class is hit by a shape the tile planner sends to it; the tile is
asserted. Bars: the elementwise tolerance |gpu - ref| <= 1e-2*|ref| +
1e-2*rms(ref); bit for bit for closed forms whose FP32 accumulation is exact,
against the block-scaled call when each row's factors repeat its block's, and
for the 1 x g quantiser.
"""

import numpy as np
import pytest

import oracle
import synth
from tests import _common
from tests._gpu import device_inputs, gemm, say

pytestmark = pytest.mark.gpu

E4, E5 = 0, 1

# (M, N, K, g, expected (bm, bn)): one shape per kernel class, ragged edges,
# K % 128 == 64 at g = 64, g = 256 on the G = 128 kernels.
SHAPES = [
    (64, 4096, 1024, 128, (32, 32)),     # streaming
    (100, 4096, 1088, 64, (64, 64)),     # M <= 128, many tiles: 64x64
    (64, 4096, 1536, 256, (32, 32)),
    (64, 520, 2048, 128, (32, 32)),      # streaming, few tiles
    (100, 520, 1088, 64, (32, 32)),
    (250, 1000, 2048, 128, (32, 32)),    # streaming, M > 128 with few tiles
    (300, 1031, 1024, 64, (64, 64)),     # 64x64 over the whole K
    (257, 3000, 1024, 128, (64, 64)),
    (777, 3333, 2048, 128, (128, 128)),  # tiled
    (1000, 3000, 576, 64, (128, 128)),
    (4000, 4000, 768, 128, (256, 256)),  # 256-row tiles
    (4000, 4000, 704, 64, (256, 256)),
    (3583, 3585, 512, 256, (256, 256)),
    (2000, 4000, 1024, 128, (256, 128)),
    (2000, 4000, 704, 64, (256, 128)),
]


def _run(a8, sa, b8, sb, g, sa_rows, fa=E4, fb=E4, bias=None, act=0):
    import torch

    import fp8_block_scaled_scales_amd as dg

    ta, tsa, tb, tsb = device_inputs(a8, sa, b8, sb)
    tbias = None if bias is None else torch.from_numpy(bias).to("cuda:0")
    out = dg.dg_gemm_fp8_nt_ex(ta, tb, tsa, tsb, gran=g, sa_rows=sa_rows, fmt_a=fa, fmt_b=fb, bias=tbias, act=act)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), out.view(torch.int16).cpu().numpy().view(np.uint16)


def _operands(M, N, K, g, fa, fb, seed):
    # rows of very different magnitudes: what per-row factors are for
    x = synth.normal(seed, (M, K)) * np.exp(np.random.default_rng(seed).uniform(-4, 4, size=(M, 1)))
    y = synth.normal(seed + 1, (N, K), sigma=0.02)
    a8, sa = oracle.quantize_rows_fmt(x.astype(np.float32), g, fa)
    b8, sb = oracle.quantize_blocks_fmt(y, g, fb)
    return a8, sa, b8, sb


def _sample(M, N, tile, seed):
    rows = np.unique(np.concatenate([_common.sample_indices(M, 150, seed=seed), np.arange(0, M, tile[0]),
                                     np.arange(tile[0] - 1, M, tile[0]), [M - 1]]))
    cols = np.unique(np.concatenate([_common.sample_indices(N, 150, seed=seed + 1), np.arange(0, N, tile[1]),
                                     np.arange(tile[1] - 1, N, tile[1]), [N - 1]]))
    return rows, cols


def _assert_parity(got, ref, label):
    ok, rms = _common.within_tolerance(got, ref)
    if not ok.all():
        idx = np.argwhere(~ok)[:5]
        detail = ", ".join("(%d,%d) got %.6g ref %.6g" % (i, j, got[i, j], ref[i, j]) for i, j in idx)
        raise AssertionError("%s: %d of %d outside tolerance: %s" % (label, int((~ok).sum()), ok.size, detail))
    say("%s: max|err|/rms = %.3g" % (label, np.max(np.abs(got - ref)) / rms))


@pytest.mark.parametrize("M,N,K,g,tile", SHAPES)
def test_rowa_parity(M, N, K, g, tile):
    import fp8_block_scaled_scales_amd as dg

    t = dg.dg_query_tile(M, N, K, g)
    assert (t["bm"], t["bn"]) == tile, t
    a8, sa, b8, sb = _operands(M, N, K, g, E4, E4, seed=9000 + M + K)
    say("per-row A M=%d N=%d K=%d g=%d tile %s" % (M, N, K, g, tile))
    got, _ = _run(a8, sa, b8, sb, g, 1)
    rows, cols = _sample(M, N, tile, M + N)
    ref = oracle.gemm_ref_rowa(a8, b8, sa, sb, g, 0, 0, rows, cols)
    _assert_parity(got[np.ix_(rows, cols)], ref, "rowa %dx%dx%d g=%d" % (M, N, K, g))


@pytest.mark.parametrize("fa,fb,act,with_bias", [(E5, E4, 0, False), (E4, E5, 2, True), (E4, E4, 1, True)])
@pytest.mark.parametrize("M,N,K,g,tile", [SHAPES[0], SHAPES[4], SHAPES[5], SHAPES[8], SHAPES[9]])
def test_rowa_with_formats_and_epilogue(M, N, K, g, tile, fa, fb, act, with_bias):
    a8, sa, b8, sb = _operands(M, N, K, g, fa, fb, seed=9500 + M + 10 * fa + 20 * fb + act)
    bias = synth.normal(9600 + N, (N,), sigma=0.5).astype(np.float32) if with_bias else None
    say("per-row A fmt %d,%d act=%d bias=%d M=%d N=%d K=%d g=%d" % (fa, fb, act, with_bias, M, N, K, g))
    got, _ = _run(a8, sa, b8, sb, g, 1, fa, fb, bias, act)
    rows, cols = _sample(M, N, tile, M + 2 * N)
    ref = oracle.epilogue(oracle.gemm_ref_rowa(a8, b8, sa, sb, g, fa, fb, rows, cols), bias, act, cols)
    _assert_parity(got[np.ix_(rows, cols)], ref, "rowa fmt %d,%d act %d" % (fa, fb, act))


@pytest.mark.parametrize("M,N,K,g,tile", SHAPES)
def test_repeated_block_factors_equal_the_block_call_bitwise(M, N, K, g, tile):
    # per-row factors that repeat each row's block factor: the kernels form
    # the same FP32 product sa*sb and the same FMAs, so the bits agree
    rng = np.random.default_rng(M * 7 + N)
    a8 = rng.integers(0, 0x7F, size=(M, K), dtype=np.uint8)
    b8 = rng.integers(0, 0x7F, size=(N, K), dtype=np.uint8) | (rng.integers(0, 2, size=(N, K), dtype=np.uint8) << 7)
    sa_blk = rng.uniform(0.01, 2.0, size=((M + g - 1) // g, K // g)).astype(np.float32)
    sb = rng.uniform(0.01, 2.0, size=((N + g - 1) // g, K // g)).astype(np.float32)
    sa_row = np.ascontiguousarray(sa_blk[np.arange(M) // g])
    say("repeated factors M=%d N=%d K=%d g=%d" % (M, N, K, g))
    _, bits_row = _run(a8, sa_row, b8, sb, g, 1)
    _, bits_blk = gemm(a8, sa_blk, b8, sb, g)
    assert np.array_equal(bits_row, bits_blk)


@pytest.mark.parametrize("M,N,K,g,tile", SHAPES)
def test_rowa_closed_form_all_ones_bitwise(M, N, K, g, tile):
    # all-ones operands, power-of-two factors differing per row and segment:
    # C[i,j] = g * sum_kb 2^(p(i,kb) + q(j/g,kb)), exact in FP32 and in BF16
    a8 = np.full((M, K), 0x38, np.uint8)
    b8 = np.full((N, K), 0x38, np.uint8)
    nkb = K // g
    sa = (2.0 ** ((np.arange(M)[:, None] * 5 + np.arange(nkb)[None, :]) % 9 - 4)).astype(np.float32)
    sb = (2.0 ** ((np.arange((N + g - 1) // g)[:, None] + 2 * np.arange(nkb)[None, :]) % 3)).astype(np.float32)
    say("per-row closed form M=%d N=%d K=%d g=%d" % (M, N, K, g))
    _, bits = _run(a8, sa, b8, sb, g, 1)
    rows = np.unique(np.concatenate([np.arange(0, M, 7), [M - 1]]))
    cols = np.unique(np.concatenate([np.arange(0, N, 41), [N - 1]]))
    ref = oracle.gemm_ref_rowa(a8, b8, sa, sb, g, 0, 0, rows, cols)
    assert np.array_equal(bits[np.ix_(rows, cols)], _common.f32_to_bf16_bits(ref.astype(np.float32)))


def test_sa_rows_gran_is_the_epilogue_call_bitwise():
    import torch

    import fp8_block_scaled_scales_amd as dg

    M, N, K, g = 1000, 3000, 512, 128
    a8, sa = oracle.quantize_blocks(synth.normal(9700, (M, K)), g)
    b8, sb = oracle.quantize_blocks(synth.normal(9701, (N, K), sigma=0.02), g)
    ta, tsa, tb, tsb = device_inputs(a8, sa, b8, sb)
    bias = torch.from_numpy(synth.normal(9702, (N,)).astype(np.float32)).to("cuda:0")
    say("sa_rows = gran through the extended call")
    o1 = dg.dg_gemm_fp8_nt_ex(ta, tb, tsa, tsb, gran=g, sa_rows=g, bias=bias, act=1)
    o2 = dg.dg_gemm_fp8_nt_epi(ta, tb, tsa, tsb, gran=g, bias=bias, act=1)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


# ------------------------------------------------------------ quantiser

@pytest.mark.parametrize("fmt,g", [(E4, 64), (E4, 128), (E4, 256), (E5, 128), (E5, 256)])
@pytest.mark.parametrize("rows,cols", [(2000, 1024), (64, 7168), (3, 512), (257, 256)])
def test_rows_quantiser_bitwise(fmt, g, rows, cols):
    import torch

    import fp8_block_scaled_scales_amd as dg

    x = synth.student_t3(9800 + rows, (rows, cols))
    x[:, :g] *= 1e-30  # tiny segments: tiny factors
    x[::3, g:2 * g] *= 1e-9
    x[-1, -g:] = 0.0  # an all-zero segment: factor 1
    say("quantise rows fmt %d g=%d %dx%d" % (fmt, g, rows, cols))
    tx = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda:0")
    q, s = dg.dg_quantize_fp8_rows(tx, gran=g, fmt=fmt)
    torch.cuda.synchronize()
    q, s = q.cpu().numpy(), s.cpu().numpy()
    rq, rs = oracle.quantize_rows_fmt(x, g, fmt)
    assert s.shape == (rows, cols // g)
    assert np.array_equal(s.view(np.uint32), rs.view(np.uint32)), "factors differ"
    bad = q != rq
    assert not bad.any(), "%d codes differ, first at %s" % (int(bad.sum()), np.argwhere(bad)[0])
