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
