"""The race check build gives the release build's bits.

libdg_sync.so is compiled from the same sources with an extra full memory
wait and workgroup barrier after every pipeline step (a full wait only in the
streaming class, whose LDS rings are per wave): the extra barrier per buffer
switch that the template article's §5.5 recommends for finding ring races.
If the release kernels' own waits and barriers are right, those extras change
only timing, so both libraries must give identical outputs on identical
inputs; a slot read before its copy landed, or refilled while still being
read, would show as a difference. One case per kernel class and path: the
streaming class (NT, both transposed layouts, per-row factors, g = 64), the
split-K class through a workspace, the 128x128 tiles, and the 256-row tiles
256 and 128 wide at g = 64, 128 and 256, with epilogues and E5M2.
"""

from __future__ import annotations

import ctypes

import pytest

from tests._gpu import say

pytestmark = pytest.mark.gpu

# M, N, K, g, layout, per-row A factors, fmt_a, fmt_b, act, bias, workspace, expected (bm, bn, split)
CASES = [
    (64, 4096, 1024, 128, 0, False, 0, 0, 0, False, False, (32, 32, False)),
    (64, 4095, 1024, 128, 1, False, 0, 0, 1, True, False, (32, 32, False)),
    (97, 531, 1088, 64, 2, True, 0, 0, 0, False, False, (32, 32, False)),
    (96, 528, 24576, 128, 0, False, 0, 1, 0, False, True, (64, 64, True)),
    (96, 528, 24576, 128, 3, True, 0, 0, 2, True, True, (64, 64, True)),
    (250, 1008, 2048, 128, 2, False, 0, 0, 0, False, False, (32, 32, False)),
    (608, 1008, 2048, 64, 1, False, 1, 1, 0, False, False, (64, 64, False)),
    (704, 4096, 1024, 128, 0, False, 0, 0, 0, False, False, (128, 128, False)),
    (1008, 3008, 2048, 64, 3, True, 0, 0, 1, True, False, (128, 128, False)),
    (4000, 4000, 768, 128, 0, False, 0, 0, 2, True, False, (256, 256, False)),
    (4001, 3999, 512, 128, 3, False, 0, 0, 0, False, False, (256, 256, False)),
    (4000, 4000, 704, 64, 0, True, 0, 0, 0, False, False, (256, 256, False)),
    (2000, 4000, 1024, 128, 0, True, 0, 0, 1, False, False, (256, 128, False)),
    (2000, 4000, 704, 64, 2, False, 0, 0, 0, False, False, (256, 128, False)),
    (3584, 3584, 512, 256, 0, False, 1, 0, 0, False, False, (256, 256, False)),
]


def _codes(gen, shape, fmt, dev):
    import torch

    c = torch.randint(0, 256, shape, generator=gen, dtype=torch.int32).to(torch.uint8)
    if fmt == 0:
        c = torch.where((c & 0x7F) == 0x7F, c ^ 1, c)  # no E4M3 NaN
    else:
        c = torch.where((c & 0x7C) == 0x7C, c & 0xF3, c)  # no E5M2 inf or NaN
    return c.to(dev)


@pytest.fixture(scope="module")
def sync_lib():
    import fp8_block_scaled_scales_amd as dg

    return dg.load_library(dg.SYNC_LIB_PATH)


@pytest.mark.parametrize("M,N,K,g,layout,rowa,fa,fb,act,with_bias,ws,expect", CASES)
def test_extra_sync_build_same_bits(sync_lib, M, N, K, g, layout, rowa, fa, fb, act, with_bias, ws, expect):
    import torch

    import fp8_block_scaled_scales_amd as dg

    dev = torch.device("cuda:0")
    plan = dg.dg_query_tile(M, N, K, g, layout, workspace=ws)
    assert (plan["bm"], plan["bn"], plan["ksplit"] > 1) == expect, plan
    gen = torch.Generator().manual_seed(900 + M + N + K + layout)
    a = _codes(gen, (K, M) if layout & 2 else (M, K), fa, dev)
    b = _codes(gen, (K, N) if layout & 1 else (N, K), fb, dev)
    nks = K // g
    sa = (torch.rand((M if rowa else -(-M // g), nks), generator=gen) * 2.0 + 0.25).to(dev)
    sb = (torch.rand((-(-N // g), nks), generator=gen) * 2.0 + 0.25).to(dev)
    bias = (torch.randn((N,), generator=gen) * 0.5).to(dev) if with_bias else None
    sa_rows = 1 if rowa else g
    stream = torch.cuda.current_stream(dev).cuda_stream

    def run(lib):
        out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        wsb = dg.dg_workspace(M, N, K, g, layout, device=dev) if ws else None
        rc = lib.dg_gemm_fp8_ws(a.data_ptr(), b.data_ptr(), sa.data_ptr(), sb.data_ptr(), out.data_ptr(), M, N, K, g,
                                layout, sa_rows, fa, fb, None if bias is None else bias.data_ptr(), act,
                                None if wsb is None else wsb.data_ptr(), 0 if wsb is None else wsb.numel(),
                                ctypes.c_void_p(stream))
        assert rc == dg.DG_OK, (rc, lib.dg_strerror(rc))
        torch.cuda.synchronize(dev)
        return out.view(torch.int16).cpu()

    say("extra-sync build M=%d N=%d K=%d g=%d layout=%d rowa=%d tile %s" % (M, N, K, g, layout, rowa, expect))
    want = run(dg.lib)
    got = run(sync_lib)
    assert bool(torch.isfinite(want.view(torch.bfloat16).float()).all())
    diff = int((want != got).sum())
    assert diff == 0, "%d of %d outputs differ between the release and the race check build" % (diff, want.numel())
