"""dg_gemm_fp8_ws on the GPU (through the C ABI) against the CPU oracle: the
cross-workgroup K split for small M (DeepGEMM实战 §3.2: K segments summed
separately, then added; §5.3: small shapes lack parallelism), with the FP32
partial tiles in a workspace the caller owns.

Bars: the elementwise tolerance against the oracle; bit for bit between
repeated calls (the partials are added in split order, whichever split ran
when), for all-ones closed forms, and against the call without a
workspace wherever the workspace plan does not split. The workspace needs no
initialisation and keeps nothing a later call reads: calls on garbage or on
another call's partials give the same bits as calls on a fresh workspace.
Two calls on two streams at once, each with its own workspace, both match
the oracle.

The plan splits only long K ranges (K >= 16384 cut at least 8 ways); the
split kernel is also run on short ones through the tile override, so its
edges (ragged M and N, few steps per split) are covered where the oracle is
quick.
"""

import numpy as np
import pytest

import oracle
import synth
from tests import _common
from tests._gpu import device_inputs, say

pytestmark = pytest.mark.gpu

# Few tiles, long K: the workspace plan splits K over 64x64 tiles.
SPLITK = [
    (1, 2048, 32768, 128), (64, 1000, 24576, 64), (100, 520, 24576, 128), (33, 700, 64 * 400, 64),
    (128, 512, 32768, 128), (7, 64, 65536, 64), (96, 1000, 24576, 128), (64, 512, 24576, 128), (8, 300, 24576, 256),
    (256, 500, 16384, 128), (1000, 100, 16384, 64),  # larger M, few tiles
]
# Short K ranges the plan streams, split through the tile override.
SPLITK_FORCED = [(64, 512, 7168, 128), (8, 300, 2048, 256), (100, 520, 2048, 128), (33, 700, 64 * 37, 64),
                 (96, 2000, 1024, 128), (1, 4096, 7168, 128)]


def _operands(M, N, K, g, seed, fa=0, fb=0):
    x = synth.normal(seed, (M, K))
    y = synth.normal(seed + 1, (N, K), sigma=0.02)
    a8, sa = oracle.quantize_blocks_fmt(x, g, fa)
    b8, sb = oracle.quantize_blocks_fmt(y, g, fb)
    return a8, sa, b8, sb


def _ws_call(t, g, workspace, layout=0, sa_rows=None, fa=0, fb=0, bias=None, act=0, out=None, stream=None):
    import fp8_block_scaled_scales_amd as dg

    ta, tsa, tb, tsb = t
    return dg.dg_gemm_fp8_ws(ta, tb, tsa, tsb, out=out, gran=g, layout=layout, sa_rows=sa_rows, fmt_a=fa, fmt_b=fb,
                             bias=bias, act=act, workspace=workspace, stream=stream)


def _bits(out):
    import torch

    torch.cuda.synchronize()
    return out.view(torch.int16).cpu().numpy().view(np.uint16)


def _vals(out):
    import torch

    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


def _assert_parity(got, ref, label):
    ok, rms = _common.within_tolerance(got, ref)
    if not ok.all():
        idx = np.argwhere(~ok)[:5]
        detail = ", ".join("(%d,%d) got %.6g ref %.6g" % (i, j, got[i, j], ref[i, j]) for i, j in idx)
        raise AssertionError("%s: %d of %d outside tolerance: %s" % (label, int((~ok).sum()), ok.size, detail))
    say("%s: max|err|/rms = %.3g" % (label, np.max(np.abs(got - ref)) / rms))


@pytest.mark.parametrize("M,N,K,g,forced", [s + (False,) for s in SPLITK] + [s + (True,) for s in SPLITK_FORCED])
def test_ws_splitk_parity(M, N, K, g, forced):
    import contextlib

    import torch

    import fp8_block_scaled_scales_amd as dg

    assert dg.dg_query_tile(M, N, K, g)["ksplit"] == 1
    assert (dg.dg_query_tile(M, N, K, g, workspace=True)["ksplit"] > 1) != forced
    a8, sa, b8, sb = _operands(M, N, K, g, 5000 + M + N)
    t = device_inputs(a8, sa, b8, sb)
    ref = oracle.gemm_ref_fmt(a8, b8, sa, sb, g, 0, 0)
    with _common.forced_split(g) if forced else contextlib.nullcontext():
        plan = dg.dg_query_tile(M, N, K, g, workspace=True)
        assert plan["ksplit"] > 1 and plan["workspace_bytes"] > 0, plan
        ws = dg.dg_workspace(M, N, K, g)
        say("ws split-K M=%d N=%d K=%d g=%d ksplit=%d ws=%d forced=%d" % (M, N, K, g, plan["ksplit"], ws.numel(),
                                                                          forced))
        out = _ws_call(t, g, ws)
        _assert_parity(_vals(out), ref, "ws split-K %dx%dx%d g=%d" % (M, N, K, g))
        bits = _bits(out)
        # again on the same workspace, and on a larger one
        assert np.array_equal(_bits(_ws_call(t, g, ws)), bits)
        big = torch.empty(ws.numel() + (1 << 20), dtype=torch.uint8, device="cuda:0")
        assert np.array_equal(_bits(_ws_call(t, g, big)), bits)
    # the call without a workspace (in-workgroup K split) on the same inputs is also within tolerance
    _assert_parity(_vals(dg.dg_gemm_fp8_nt_fmt(t[0], t[2], t[1], t[3], gran=g)), ref,
                   "no workspace %dx%dx%d g=%d" % (M, N, K, g))


def test_ws_all_ones_bitwise():
    M, N, K, g = 64, 384, 24576, 128
    a8 = np.full((M, K), 0x38, np.uint8)
    b8 = np.full((N, K), 0x38, np.uint8)
    sa = np.array([[2.0 ** ((mb - kb) % 7 - 3) for kb in range(K // g)] for mb in range(-(-M // g))], np.float32)
    sb = np.array([[2.0 ** ((2 * nb + kb) % 3) for kb in range(K // g)] for nb in range(-(-N // g))], np.float32)
    import fp8_block_scaled_scales_amd as dg

    assert dg.dg_query_tile(M, N, K, g, workspace=True)["ksplit"] > 1
    say("ws all-ones")
    out = _ws_call(device_inputs(a8, sa, b8, sb), g, dg.dg_workspace(M, N, K, g))
    ref = oracle.gemm_ref(a8, b8, sa, sb, g)
    assert np.array_equal(_bits(out), _common.f32_to_bf16_bits(ref.astype(np.float32)))


def test_ws_garbage_and_stale_contents():
    """No initialisation needed, nothing carried over: every call writes each
    partial it adds before adding it, so a workspace full of 0xFF bytes (NaN
    floats), of random bytes, or of another shape's partials gives the
    fresh-workspace bits."""
    import torch

    import fp8_block_scaled_scales_amd as dg

    M, N, K, g = 64, 512, 24576, 128
    a8, sa, b8, sb = _operands(M, N, K, g, 8100)
    t = device_inputs(a8, sa, b8, sb)
    plan = dg.dg_query_tile(M, N, K, g, workspace=True)
    assert plan["ksplit"] > 1
    ws = torch.zeros(plan["workspace_bytes"], dtype=torch.uint8, device="cuda:0")
    say("ws garbage/stale: fresh")
    want = _bits(_ws_call(t, g, ws))
    other = (8, 300, 24576, 128)
    t_other = device_inputs(*_operands(*other, seed=8101))
    cases = {
        "ones": lambda: ws.fill_(0xFF),
        "random": lambda: ws.copy_(torch.randint(0, 256, ws.shape, dtype=torch.uint8, device="cuda:0",
                                                 generator=torch.Generator(device="cuda:0").manual_seed(3))),
        "another shape's partials": lambda: _ws_call(t_other, other[3], ws[:dg.dg_query_tile(
            *other, workspace=True)["workspace_bytes"]]),
    }
    for name, plant in cases.items():
        plant()
        torch.cuda.synchronize()
        say("ws garbage/stale: %s" % name)
        assert np.array_equal(_bits(_ws_call(t, g, ws)), want), name


def test_ws_interleaved_shapes_one_workspace():
    """Two split shapes with different split counts and tile counts, alternating
    on one workspace (one stream) 20 times: every result bit for bit the same."""
    import fp8_block_scaled_scales_amd as dg

    shapes = [(64, 512, 24576, 128), (128, 1024, 24576, 128)]
    plans = [dg.dg_query_tile(*s, workspace=True) for s in shapes]
    assert plans[0]["ksplit"] != plans[1]["ksplit"] and all(p["ksplit"] > 1 for p in plans), plans
    ws = dg.dg_workspace(*max(shapes, key=lambda s: dg.dg_query_tile(*s, workspace=True)["workspace_bytes"]))
    ops = [_operands(*s, seed=8200 + i) for i, s in enumerate(shapes)]
    ts = [device_inputs(*o) for o in ops]
    say("ws interleaved x20")
    first = [_bits(_ws_call(ts[i], shapes[i][3], ws)) for i in range(2)]
    for _ in range(20):
        for i in range(2):
            assert np.array_equal(_bits(_ws_call(ts[i], shapes[i][3], ws)), first[i]), shapes[i]
    for i, (M, N, K, g) in enumerate(shapes):
        a8, sa, b8, sb = ops[i]
        _assert_parity(_common.bf16_bits_to_f64(first[i]),
                       oracle.gemm_ref(a8, b8, sa, sb, g), "interleaved %dx%dx%d" % (M, N, K))


def test_ws_two_streams_concurrently():
    """Two split-K GEMMs in flight at once on two streams, each with its own
    workspace, enqueued alternately 10 times each with no synchronisation in
    between: every output matches the oracle and its own first result."""
    import torch

    import fp8_block_scaled_scales_amd as dg

    shapes = [(64, 512, 24576, 128), (100, 520, 24576, 128)]
    assert all(dg.dg_query_tile(*s, workspace=True)["ksplit"] > 1 for s in shapes)
    ops = [_operands(*s, seed=8300 + i) for i, s in enumerate(shapes)]
    ts = [device_inputs(*o) for o in ops]
    wss = [dg.dg_workspace(*s) for s in shapes]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [[torch.empty((s[0], s[1]), dtype=torch.bfloat16, device="cuda:0") for _ in range(10)] for s in shapes]
    torch.cuda.synchronize()
    say("ws two streams")
    for r in range(10):
        for i in range(2):
            _ws_call(ts[i], shapes[i][3], wss[i], out=outs[i][r], stream=streams[i])
    torch.cuda.synchronize()
    for i, (M, N, K, g) in enumerate(shapes):
        a8, sa, b8, sb = ops[i]
        ref = oracle.gemm_ref(a8, b8, sa, sb, g)
        b0 = _bits(outs[i][0])
        _assert_parity(_common.bf16_bits_to_f64(b0), ref, "stream %d %dx%dx%d" % (i, M, N, K))
        for r in range(1, 10):
            assert np.array_equal(_bits(outs[i][r]), b0), (i, r)


def test_ws_graph_replays():
    """A split-K call captured into a HIP graph (its counter tag fixed at
    capture) replayed five times, with eager calls on the same workspace and
    synchronisations in between: every replay's output equals the eager one."""
    import torch

    import fp8_block_scaled_scales_amd as dg

    M, N, K, g = 64, 512, 24576, 128
    assert dg.dg_query_tile(M, N, K, g, workspace=True)["ksplit"] > 1
    a8, sa, b8, sb = _operands(M, N, K, g, 8700)
    t = device_inputs(a8, sa, b8, sb)
    ws = dg.dg_workspace(M, N, K, g)
    say("ws graph replays")
    want = _bits(_ws_call(t, g, ws))
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0")
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(graph, stream=cap):
            _ws_call(t, g, ws, out=out, stream=cap)
    torch.cuda.synchronize()
    for r in range(5):
        out.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(_bits(out), want), r
        assert np.array_equal(_bits(_ws_call(t, g, ws)), want), r  # an eager call between replays


@pytest.mark.parametrize("M,N,K,g,layout", [(64, 4096, 7168, 128, 0), (2000, 4000, 1024, 128, 0),
                                            (256, 256, 256, 128, 0), (1008, 3008, 512, 128, 2),
                                            (64, 512, 7168, 128, 3), (8, 4096, 32768, 128, 0)])
def test_ws_without_split_is_the_plain_call(M, N, K, g, layout):
    """Shapes the workspace plan does not split run the call without a
    workspace, bit for bit, and leave the workspace untouched."""
    import torch

    import fp8_block_scaled_scales_amd as dg

    plan = dg.dg_query_tile(M, N, K, g, layout, workspace=True)
    assert plan["ksplit"] == 1 and plan["workspace_bytes"] == 0
    a8, sa, b8, sb = _operands(M, N, K, g, 8400 + M)
    a_st = np.ascontiguousarray(a8.T) if layout & 2 else a8
    b_st = np.ascontiguousarray(b8.T) if layout & 1 else b8
    t = device_inputs(a_st, sa, b_st, sb)
    ws = torch.full((1 << 16,), 0x5A, dtype=torch.uint8, device="cuda:0")
    say("ws without split %dx%dx%d layout %d" % (M, N, K, layout))
    got = _bits(_ws_call(t, g, ws, layout=layout))
    want = _bits(dg.dg_gemm_fp8_layout(t[0], t[2], t[1], t[3], gran=g, layout=layout))
    assert np.array_equal(got, want)
    assert bool((ws == 0x5A).all().item())


# The split path with the call's other options: operand formats, the fused
# epilogue, per-row A factors, transposed layouts, g = 64 with K % 128 == 64.
@pytest.mark.parametrize("case", ["e5m2", "e4m3xe5m2", "bias_gelu", "relu", "rowa_g128", "rowa_g64", "nn", "tt", "tn",
                                  "g64_half_step"])
def test_ws_split_variants(case):
    import torch

    import fp8_block_scaled_scales_amd as dg

    M, N, K, g, layout, fa, fb, act, with_bias, rowa = 96, 528, 24576, 128, 0, 0, 0, 0, False, False
    if case == "e5m2":
        fa = fb = 1
    elif case == "e4m3xe5m2":
        fb = 1
    elif case == "bias_gelu":
        act, with_bias = 2, True
    elif case == "relu":
        act, with_bias = 1, True
    elif case.startswith("rowa"):
        rowa, g = True, int(case[-3:].lstrip("g"))
        K = 24576 if g == 128 else 64 * 385
    elif case in ("nn", "tt", "tn"):
        layout = {"nn": 1, "tt": 2, "tn": 3}[case]
    elif case == "g64_half_step":
        g, K = 64, 64 * 385  # 192.5 steps of 128
    plan = dg.dg_query_tile(M, N, K, g, layout, workspace=True)
    assert plan["ksplit"] > 1, plan
    x = synth.normal(8500, (M, K))
    if rowa:
        x = x * np.exp(np.random.default_rng(8500).uniform(-4, 4, size=(M, 1))).astype(np.float32)
        a8, sa = oracle.quantize_rows_fmt(x.astype(np.float32), g, fa)
    else:
        a8, sa = oracle.quantize_blocks_fmt(x, g, fa)
    b8, sb = oracle.quantize_blocks_fmt(synth.normal(8501, (N, K), sigma=0.02), g, fb)
    bias = synth.normal(8502, (N,), sigma=0.5).astype(np.float32) if with_bias else None
    a_st = np.ascontiguousarray(a8.T) if layout & 2 else a8
    b_st = np.ascontiguousarray(b8.T) if layout & 1 else b8
    t = device_inputs(a_st, sa, b_st, sb)
    tbias = None if bias is None else torch.from_numpy(bias).to("cuda:0")
    say("ws variant %s ksplit=%d" % (case, plan["ksplit"]))
    out = _ws_call(t, g, dg.dg_workspace(M, N, K, g, layout), layout=layout, sa_rows=1 if rowa else None, fa=fa, fb=fb,
                   bias=tbias, act=act)
    if rowa:
        ref = oracle.gemm_ref_rowa(a8, b8, sa, sb, g, fa, fb)
    else:
        ref = oracle.gemm_ref_fmt(a8, b8, sa, sb, g, fa, fb)
    if with_bias or act:
        ref = oracle.epilogue(ref, bias, act)
    _assert_parity(_vals(out), ref, "ws variant %s" % case)
