"""E5M2 and mixed-format operands, and g = 256 block scales, on the GPU
(through the C ABI) against the CPU oracle.

The pages name E4M3 and E5M2 as the FP8 input formats (DeepGEMM实战 §2.2)
and 64, 128 and 256 as block granularities (§3.1). Each kernel class is hit
by a shape the tile planner sends to it; the tile is asserted. Bars as for
E4M3: elementwise |gpu - ref| <= 1e-2*|ref| + 1e-2*rms(ref), and bit for bit
for closed forms whose FP32 accumulation is exact, and for the quantiser.
"""

import numpy as np
import pytest

import oracle
import synth
from tests import _common
from tests._gpu import device_inputs, say

pytestmark = pytest.mark.gpu

E4, E5 = 0, 1


def _gemm_fmt(a8, sa, b8, sb, g, fa, fb):
    import torch

    import fp8_block_scaled_scales_amd as dg

    ta, tsa, tb, tsb = device_inputs(a8, sa, b8, sb)
    out = dg.dg_gemm_fp8_nt_fmt(ta, tb, tsa, tsb, gran=g, fmt_a=fa, fmt_b=fb)
    torch.cuda.synchronize()
    bits = out.view(torch.int16).cpu().numpy().view(np.uint16)
    return out.float().cpu().numpy().astype(np.float64), bits


def _assert_parity(got, ref, label):
    ok, rms = _common.within_tolerance(got, ref)
    if not ok.all():
        idx = np.argwhere(~ok)[:5]
        detail = ", ".join("(%d,%d) got %.6g ref %.6g" % (i, j, got[i, j], ref[i, j]) for i, j in idx)
        raise AssertionError("%s: %d of %d outside tolerance: %s" % (label, int((~ok).sum()), ok.size, detail))
    say("%s: max|err|/rms = %.3g" % (label, np.max(np.abs(got - ref)) / rms))


def _operands(M, N, K, g, fa, fb, seed):
    x = synth.normal(seed, (M, K))
    y = synth.normal(seed + 1, (N, K), sigma=0.02)
    a8, sa = oracle.quantize_blocks_fmt(x, g, fa)
    b8, sb = oracle.quantize_blocks_fmt(y, g, fb)
    return a8, sa, b8, sb


# (M, N, K, g, expected (bm, bn)): one shape per kernel class, ragged edges,
# K % 128 == 64 at g = 64.
SHAPES = [
    (64, 4096, 1024, 128, (32, 32)),     # streaming
    (64, 4096, 1536, 256, (32, 32)),
    (64, 520, 2048, 256, (32, 32)),      # streaming, few tiles
    (100, 520, 1088, 64, (32, 32)),
    (257, 1024, 7168, 256, (32, 32)),    # streaming, M > 128 with few tiles
    (257, 3000, 1024, 256, (64, 64)),    # 64x64 over the whole K
    (600, 1000, 2048, 64, (64, 64)),
    (700, 4100, 1024, 256, (128, 128)),  # tiled
    (1000, 3000, 576, 64, (128, 128)),
    (4000, 4000, 768, 256, (256, 256)),  # 256-row tiles
    (3583, 3585, 512, 256, (256, 256)),
    (2000, 4000, 1024, 256, (256, 128)),
    (2000, 4000, 704, 64, (256, 128)),
]


@pytest.mark.parametrize("fa,fb", [(E5, E5), (E4, E5), (E5, E4)])
@pytest.mark.parametrize("M,N,K,g,tile", SHAPES)
def test_formats_parity(M, N, K, g, tile, fa, fb):
    import fp8_block_scaled_scales_amd as dg

    t = dg.dg_query_tile(M, N, K, g)
    assert (t["bm"], t["bn"]) == tile, t
    a8, sa, b8, sb = _operands(M, N, K, g, fa, fb, seed=7000 + M + 10 * fa + 20 * fb)
    say("formats %d,%d M=%d N=%d K=%d g=%d tile %s" % (fa, fb, M, N, K, g, tile))
    got, _ = _gemm_fmt(a8, sa, b8, sb, g, fa, fb)
    rows = _common.sample_indices(M, 150, seed=M)
    cols = _common.sample_indices(N, 150, seed=N)
    rows = np.unique(np.concatenate([rows, np.arange(0, M, tile[0]), np.arange(tile[0] - 1, M, tile[0])]))
    cols = np.unique(np.concatenate([cols, np.arange(0, N, tile[1]), np.arange(tile[1] - 1, N, tile[1])]))
    ref = oracle.gemm_ref_fmt(a8, b8, sa, sb, g, fa, fb, rows, cols)
    _assert_parity(got[np.ix_(rows, cols)], ref, "fmt %d,%d %dx%dx%d g=%d" % (fa, fb, M, N, K, g))


@pytest.mark.parametrize("M,N,K,g,tile", [s for s in SHAPES if s[3] == 256])
def test_g256_e4m3_parity(M, N, K, g, tile):
    import fp8_block_scaled_scales_amd as dg

    assert (dg.dg_query_tile(M, N, K, g)["bm"], dg.dg_query_tile(M, N, K, g)["bn"]) == tile
    a8, sa, b8, sb = _operands(M, N, K, g, E4, E4, seed=7500 + M)
    say("g=256 E4M3 M=%d N=%d K=%d" % (M, N, K))
    got, bits = _gemm_fmt(a8, sa, b8, sb, g, E4, E4)
    from tests._gpu import gemm

    _, bits_plain = gemm(a8, sa, b8, sb, g)
    assert np.array_equal(bits, bits_plain)  # the plain entry point is the E4M3 x E4M3 case
    rows = np.unique(np.concatenate([_common.sample_indices(M, 150, seed=M), [M - 1]]))
    cols = np.unique(np.concatenate([_common.sample_indices(N, 150, seed=N), [N - 1]]))
    ref = oracle.gemm_ref(a8, b8, sa, sb, g, rows, cols)
    _assert_parity(got[np.ix_(rows, cols)], ref, "g=256 %dx%dx%d" % (M, N, K))


def _pow2_scales(nrb, nkb, f):
    s = np.empty((nrb, nkb), np.float32)
    for r in range(nrb):
        for k in range(nkb):
            s[r, k] = 2.0 ** f(r, k)
    return s


@pytest.mark.parametrize("fa,fb", [(E5, E5), (E4, E5)])
@pytest.mark.parametrize("M,N,K,g", [(64, 4096, 1024, 256), (64, 520, 2048, 256), (1000, 3000, 512, 256),
                                     (4000, 4000, 768, 256), (3583, 3585, 512, 256), (2000, 4000, 1024, 256),
                                     (2000, 4000, 1024, 64)])
def test_closed_form_all_ones_bitwise(M, N, K, g, fa, fb):
    one = {E4: 0x38, E5: 0x3C}
    a8 = np.full((M, K), one[fa], np.uint8)
    b8 = np.full((N, K), one[fb], np.uint8)
    sa = _pow2_scales(-(-M // g), K // g, lambda mb, kb: (mb - kb) % 7 - 3)
    sb = _pow2_scales(-(-N // g), K // g, lambda nb, kb: (2 * nb + kb) % 3)
    say("all-ones fmt %d,%d %dx%dx%d g=%d" % (fa, fb, M, N, K, g))
    _, bits = _gemm_fmt(a8, sa, b8, sb, g, fa, fb)
    rows = np.unique(np.concatenate([np.arange(0, M, 37), [M - 1]]))
    cols = np.unique(np.concatenate([np.arange(0, N, 41), [N - 1]]))
    ref = oracle.gemm_ref_fmt(a8, b8, sa, sb, g, fa, fb, rows, cols)
    assert np.array_equal(bits[np.ix_(rows, cols)], _common.f32_to_bf16_bits(ref.astype(np.float32)))


# ------------------------------------------------------------ quantiser

def _gpu_quant(x, g, fmt):
    import torch

    import fp8_block_scaled_scales_amd as dg

    tx = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda:0")
    q, s = dg.dg_quantize_fp8_blocks(tx, gran=g, fmt=fmt)
    torch.cuda.synchronize()
    return q.cpu().numpy(), s.cpu().numpy()


@pytest.mark.parametrize("fmt,g", [(E5, 64), (E5, 128), (E5, 256), (E4, 256)])
@pytest.mark.parametrize("rows,cols", [(2000, 1024), (64, 7168), (257, 512)])
def test_quantiser_bitwise(fmt, g, rows, cols):
    x = synth.student_t3(8100 + rows, (rows, cols))
    x[:, :g] *= 1e-30  # blocks of tiny values: tiny FP32 scales
    x[::3, g:2 * g] *= 1e-9  # elements far below their block's amax: subnormal codes
    x[-1, -g:] = 0.0
    say("quantise fmt %d g=%d %dx%d" % (fmt, g, rows, cols))
    q, s = _gpu_quant(x, g, fmt)
    rq, rs = oracle.quantize_blocks_fmt(x, g, fmt)
    assert np.array_equal(s.view(np.uint32), rs.view(np.uint32)), "scales differ"
    bad = q != rq
    assert not bad.any(), "%d codes differ, first at %s" % (int(bad.sum()), np.argwhere(bad)[0])
