"""dg_gemm_fp8_noalloc on the GPU (through the C ABI): the same results as
dg_gemm_fp8_ws, bit for bit, with the workspace taken from the library's
fixed scratch array instead of an argument. Two split-K calls in a row, the
second smaller than the first (the scratch keeps the first call's contents),
then a shape whose plan does not split, then the first shape again."""

import numpy as np
import pytest

import oracle
import synth
from tests import _common
from tests._gpu import device_inputs, say

pytestmark = pytest.mark.gpu


def _case(M, N, K, g, seed):
    a8, sa = oracle.quantize_blocks(synth.normal(seed, (M, K)), g)
    b8, sb = oracle.quantize_blocks(synth.normal(seed + 1, (N, K), sigma=0.02), g)
    return a8, sa, b8, sb


def _bits(out):
    import torch

    torch.cuda.synchronize()
    return out.view(torch.int16).cpu().numpy().view(np.uint16)


def test_noalloc_matches_workspace_call():
    import torch

    import fp8_block_scaled_scales_amd as dg

    shapes = [(64, 512, 24576, 128), (8, 300, 24576, 128), (64, 4096, 1024, 128), (64, 512, 24576, 128)]
    for i, (M, N, K, g) in enumerate(shapes):
        plan = dg.dg_query_tile(M, N, K, g, workspace=True)
        assert (plan["ksplit"] > 1) == (i != 2), plan
        assert plan["workspace_bytes"] <= dg.dg_noalloc_scratch_bytes()
        a8, sa, b8, sb = _case(M, N, K, g, 9100 + i)
        ta, tsa, tb, tsb = device_inputs(a8, sa, b8, sb)
        out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0")
        say("noalloc call %d: %dx%dx%d g=%d ksplit=%d" % (i, M, N, K, g, plan["ksplit"]))
        dg.dg_gemm_fp8_noalloc(ta, tb, tsa, tsb, out, gran=g)
        got = _bits(out)
        want = _bits(dg.dg_gemm_fp8_ws(ta, tb, tsa, tsb, gran=g, workspace=dg.dg_workspace(M, N, K, g)))
        assert np.array_equal(got, want), (M, N, K)
        ref = oracle.gemm_ref(a8, b8, sa, sb, g)
        ok, _ = _common.within_tolerance(_common.bf16_bits_to_f64(got), ref)
        assert ok.all(), (M, N, K)


def test_noalloc_rejects_a_plan_beyond_the_scratch():
    import torch

    import fp8_block_scaled_scales_amd as dg

    M, N, K, g = 128, 1088, 32768, 128  # 34 tiles x 8 splits: 4.25 MiB of partials
    assert dg.dg_query_tile(M, N, K, g, workspace=True)["workspace_bytes"] > dg.dg_noalloc_scratch_bytes()
    a8, sa, b8, sb = _case(M, N, K, g, 9200)
    ta, tsa, tb, tsb = device_inputs(a8, sa, b8, sb)
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(dg.DGError) as e:
        dg.dg_gemm_fp8_noalloc(ta, tb, tsa, tsb, out, gran=g)
    assert e.value.code == dg.DG_ESCRATCH


def test_noalloc_layout_and_row_factors():
    # a transposed layout with per-row A factors through the split path, the
    # scratch holding the previous test's contents: bit for bit the workspace call
    import torch

    import fp8_block_scaled_scales_amd as dg

    M, N, K, g, layout = 96, 528, 24576, 128, 3
    plan = dg.dg_query_tile(M, N, K, g, layout, workspace=True)
    assert plan["ksplit"] > 1 and plan["workspace_bytes"] <= dg.dg_noalloc_scratch_bytes()
    x = synth.normal(9300, (M, K)) * np.exp(np.random.default_rng(9300).uniform(-3, 3, size=(M, 1)))
    a8, sa = oracle.quantize_rows_fmt(x.astype(np.float32), g, 0)
    b8, sb = oracle.quantize_blocks(synth.normal(9301, (N, K), sigma=0.02), g)
    dev = "cuda:0"
    ta = torch.from_numpy(np.ascontiguousarray(a8.T)).to(dev)  # A stored [K, M]
    tb = torch.from_numpy(np.ascontiguousarray(b8.T)).to(dev)  # B stored [K, N]
    tsa, tsb = torch.from_numpy(sa).to(dev), torch.from_numpy(sb).to(dev)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    say("noalloc TN per-row %dx%dx%d ksplit=%d" % (M, N, K, plan["ksplit"]))
    dg.dg_gemm_fp8_noalloc(ta, tb, tsa, tsb, out, gran=g, layout=layout, sa_rows=1)
    got = _bits(out)
    want = _bits(dg.dg_gemm_fp8_ws(ta, tb, tsa, tsb, gran=g, layout=layout, sa_rows=1,
                                   workspace=dg.dg_workspace(M, N, K, g, layout)))
    assert np.array_equal(got, want)
    ok, _ = _common.within_tolerance(_common.bf16_bits_to_f64(got), oracle.gemm_ref_rowa(a8, b8, sa, sb, g))
    assert ok.all()
