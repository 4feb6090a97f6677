"""The default calls inside a captured HIP graph: the quantise-then-multiply
pipeline (DeepGEMM实战 §4.4: activations quantised online, then the GEMM)
captured once and replayed, with eager work and synchronisations between the
replays. Every replay must give the eager pipeline's bits, also after the input
buffer's contents change (the graph reads the buffers, not copies of them)."""

import numpy as np
import pytest

import synth
from tests._gpu import say

pytestmark = pytest.mark.gpu


def _bits(t):
    import torch

    return t.view(torch.int16).cpu().numpy().copy()


@pytest.mark.parametrize("g,fmt", [(128, 0), (64, 1)])
def test_quantise_and_gemm_pipeline_replays(g, fmt):
    import torch

    import fp8_block_scaled_scales_amd as dg

    M, N, K = 300, 1000, 16 * g
    dev = "cuda:0"
    a_in = torch.from_numpy(synth.make_a(3, M=M, K=K)).to(dev).to(torch.bfloat16)
    a_alt = torch.from_numpy(synth.make_a(5, M=M, K=K)).to(dev).to(torch.bfloat16)
    b_in = torch.from_numpy(synth.make_b(3, N=N, K=K)).to(dev).to(torch.bfloat16)

    def eager(a):
        a8, sa = dg.dg_quantize_fp8_rows_typed(a, gran=g, fmt=fmt)
        b8, sb = dg.dg_quantize_fp8_blocks_typed(b_in, gran=g, fmt=fmt)
        out = dg.dg_gemm_fp8_nt_ex(a8, b8, sa, sb, gran=g, sa_rows=1, fmt_a=fmt, fmt_b=fmt)
        torch.cuda.synchronize()
        return _bits(out)

    say("graph pipeline g=%d fmt=%d" % (g, fmt))
    want = eager(a_in)
    want_alt = eager(a_alt)

    a_buf = a_in.clone()
    a8 = torch.empty((M, K), dtype=torch.uint8, device=dev)
    sa = torch.empty((M, K // g), dtype=torch.float32, device=dev)
    b8 = torch.empty((N, K), dtype=torch.uint8, device=dev)
    sb = torch.empty(((N + g - 1) // g, K // g), dtype=torch.float32, device=dev)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(graph, stream=cap):
            dg.dg_quantize_fp8_rows_typed(a_buf, gran=g, fmt=fmt, q=a8, scales=sa, stream=cap)
            dg.dg_quantize_fp8_blocks_typed(b_in, gran=g, fmt=fmt, q=b8, scales=sb, stream=cap)
            dg.dg_gemm_fp8_nt_ex(a8, b8, sa, sb, out=out, gran=g, sa_rows=1, fmt_a=fmt, fmt_b=fmt, stream=cap)
    torch.cuda.synchronize()
    for r in range(6):
        alt = r == 3
        a_buf.copy_(a_alt if alt else a_in)
        for t in (a8, sa, b8, sb, out):
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(_bits(out), want_alt if alt else want), "replay %d" % r
        assert np.array_equal(eager(a_in), want), "eager call after replay %d" % r
