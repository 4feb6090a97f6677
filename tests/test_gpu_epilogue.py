"""The fused epilogue out = bf16(act(C + bias[j])) on the GPU (through the C
ABI) against the CPU oracle's FP64 epilogue on its reference GEMM.

The template article places bias add, ReLU and GELU at the epilogue, before
the write-back (§2.3, §6). Every kernel class is hit by a shape the planner
sends to it. Bars: the elementwise tolerance of the GEMM on act(ref + bias),
bit for bit for the no-op epilogue (it must be the plain call), and bit for
bit for an all-ones closed form with an exact bias and ReLU.
"""

import numpy as np
import pytest

import oracle
import synth
from tests import _common
from tests._gpu import device_inputs, gemm, say

pytestmark = pytest.mark.gpu

NONE, RELU, GELU = 0, 1, 2

SHAPES = [
    (64, 4096, 1024, 128, (32, 32)),     # streaming
    (64, 520, 2048, 128, (32, 32)),      # streaming, few tiles
    (250, 1000, 2048, 64, (32, 32)),     # streaming, M > 128 with few tiles
    (300, 1031, 1024, 128, (64, 64)),    # 64x64 over the whole K
    (1000, 3000, 512, 64, (128, 128)),   # tiled
    (4000, 4000, 768, 128, (256, 256)),  # 256-row tiles
    (3583, 3585, 512, 128, (256, 256)),
    (2000, 4000, 1024, 64, (256, 128)),
]


def _run(a8, sa, b8, sb, g, bias, act):
    import torch

    import fp8_block_scaled_scales_amd as dg

    ta, tsa, tb, tsb = device_inputs(a8, sa, b8, sb)
    tbias = None if bias is None else torch.from_numpy(bias).to("cuda:0")
    out = dg.dg_gemm_fp8_nt_epi(ta, tb, tsa, tsb, gran=g, bias=tbias, act=act)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), out.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("act,with_bias", [(NONE, True), (RELU, True), (GELU, True), (GELU, False)])
@pytest.mark.parametrize("M,N,K,g,tile", SHAPES)
def test_epilogue_parity(M, N, K, g, tile, act, with_bias):
    import fp8_block_scaled_scales_amd as dg

    t = dg.dg_query_tile(M, N, K, g)
    assert (t["bm"], t["bn"]) == tile, t
    a8, sa = oracle.quantize_blocks(synth.normal(6100 + M, (M, K)), g)
    b8, sb = oracle.quantize_blocks(synth.normal(6200 + N, (N, K), sigma=0.02), g)
    bias = synth.normal(6300 + N, (N,), sigma=0.5).astype(np.float32) if with_bias else None
    say("epilogue act=%d bias=%d %dx%dx%d g=%d" % (act, with_bias, M, N, K, g))
    got, _ = _run(a8, sa, b8, sb, g, bias, act)
    rows = np.unique(np.concatenate([_common.sample_indices(M, 120, seed=M), [0, M - 1]]))
    cols = np.unique(np.concatenate([_common.sample_indices(N, 120, seed=N), [0, N - 1],
                                     np.arange(tile[1] - 1, N, tile[1])]))
    ref = oracle.epilogue(oracle.gemm_ref(a8, b8, sa, sb, g, rows, cols), bias, act, cols)
    ok, rms = _common.within_tolerance(got[np.ix_(rows, cols)], ref)
    assert ok.all(), "%d of %d outside tolerance" % (int((~ok).sum()), ok.size)
    if act == RELU:
        assert np.all(got >= 0.0)


@pytest.mark.parametrize("M,N,K,g,tile", SHAPES)
def test_noop_epilogue_is_the_plain_call(M, N, K, g, tile):
    a8, sa = oracle.quantize_blocks(synth.normal(6400 + M, (M, K)), g)
    b8, sb = oracle.quantize_blocks(synth.normal(6500 + N, (N, K), sigma=0.02), g)
    say("no-op epilogue %dx%dx%d g=%d" % (M, N, K, g))
    _, bits = _run(a8, sa, b8, sb, g, None, NONE)
    _, plain = gemm(a8, sa, b8, sb, g)
    assert np.array_equal(bits, plain)


@pytest.mark.parametrize("M,N,K,g,tile", SHAPES)
def test_closed_form_bias_relu_bitwise(M, N, K, g, tile):
    # all-ones operands with power-of-two scales: C = g * sum_kb 2^(p+q), exact
    # in FP32; a bias of integer multiples of g keeps C + bias exact, so ReLU(C + bias)
    # is exact and must round to bf16 exactly as the oracle's value does.
    a8 = np.full((M, K), 0x38, np.uint8)
    b8 = np.full((N, K), 0x38, np.uint8)
    nkb = K // g
    sa = np.array([[2.0 ** ((mb - kb) % 5 - 2) for kb in range(nkb)] for mb in range(-(-M // g))], np.float32)
    sb = np.array([[2.0 ** ((nb + kb) % 3) for kb in range(nkb)] for nb in range(-(-N // g))], np.float32)
    bias = (-(np.arange(N) % 13) * float(2 * g * nkb)).astype(np.float32)  # a share of outputs goes negative
    say("closed form bias+ReLU %dx%dx%d g=%d" % (M, N, K, g))
    _, bits = _run(a8, sa, b8, sb, g, bias, RELU)
    rows = np.unique(np.concatenate([np.arange(0, M, 29), [M - 1]]))
    cols = np.unique(np.concatenate([np.arange(0, N, 31), [N - 1]]))
    ref = oracle.epilogue(oracle.gemm_ref(a8, b8, sa, sb, g, rows, cols), bias, RELU, cols)
    assert (ref == 0).any() and (ref > 0).any()
    assert np.array_equal(bits[np.ix_(rows, cols)], _common.f32_to_bf16_bits(ref.astype(np.float32)))
