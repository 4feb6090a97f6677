"""The quantisers on BF16 and FP16 input (dg_quantize_fp8_blocks_typed,
dg_quantize_fp8_rows_typed) against the oracle's 16-bit quantisers.

The inputs are the seeded FP32 matrices rounded to BF16 or FP16 by torch (the
input preparation both sides share); the oracle receives their bit patterns
and decodes them itself. Codes and factors must agree bit for bit.
"""

import numpy as np
import pytest

import oracle
import synth
from tests._gpu import say

pytestmark = pytest.mark.gpu

KINDS = {"bf16": oracle.IN_BF16, "f16": oracle.IN_F16}


def _as16(x32, kind):
    """(torch 16-bit tensor on the GPU, its bit patterns as uint16) of an FP32 matrix."""
    import torch

    dt = torch.bfloat16 if kind == "bf16" else torch.float16
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(dt)
    bits = t.view(torch.int16).numpy().view(np.uint16).copy()
    return t.to("cuda:0"), bits


def _check(x32, g, fmt, kind, rows_kind=False, label=""):
    import torch

    import fp8_block_scaled_scales_amd as dg

    say("quantise16 %s %s %s g=%d fmt=%d %s" % (label, kind, x32.shape, g, fmt, "1xg" if rows_kind else "gxg"))
    t, bits = _as16(x32, kind)
    fn = dg.dg_quantize_fp8_rows_typed if rows_kind else dg.dg_quantize_fp8_blocks_typed
    q, s = fn(t, gran=g, fmt=fmt)
    torch.cuda.synchronize()
    ref = oracle.quantize_rows_16 if rows_kind else oracle.quantize_blocks_16
    rq, rs = ref(bits, KINDS[kind], g, fmt)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), rs.view(np.uint32)), "scales differ"
    bad = q.cpu().numpy() != rq
    assert not bad.any(), "%d codes differ, first at %s" % (int(bad.sum()), np.argwhere(bad)[0])


@pytest.mark.parametrize("kind", ["bf16", "f16"])
@pytest.mark.parametrize("c", [1, 2, 3, 5])
def test_workload_operands_bitwise(kind, c):
    w = synth.WORKLOADS[c]
    M, N = min(w["M"], 1000), min(w["N"], 1000)
    for fmt in (0, 1):
        _check(synth.make_a(c, M=M), w["g"], fmt, kind, label="A of workload %d" % c)
        _check(synth.make_b(c, N=N), w["g"], fmt, kind, label="B of workload %d" % c)


@pytest.mark.parametrize("kind", ["bf16", "f16"])
@pytest.mark.parametrize("rows,cols,g", [(1, 64, 64), (1, 256, 256), (17, 192, 64), (129, 256, 128),
                                         (200, 640, 64), (300, 768, 256), (1023, 384, 128)])
def test_ragged_bitwise(kind, rows, cols, g):
    x = synth.normal(5100 + rows, (rows, cols))
    _check(x, g, 0, kind, label="ragged")
    _check(x, g, 1, kind, rows_kind=True, label="ragged")


@pytest.mark.parametrize("rows_kind", [False, True])
def test_bf16_range_and_subnormals(rows_kind):
    """BF16 keeps FP32's exponent range: blocks of values near 1e38, blocks of
    BF16 subnormals (whose factor is subnormal, so the kernels divide per
    element), signed zeros and an all-zero block."""
    g = 64
    x = synth.normal(5200, (128, 256)).astype(np.float32)
    x[0:64, 0:64] *= np.float32(1e37)
    x[0:64, 64:128] *= np.float32(1e-39)   # BF16 subnormals (below 2^-126)
    x[64:128, 0:64] = 0.0
    x[64:128, 64:128] = -0.0
    x[64:128, 128] = np.float32(-3.0e38)
    x[100, 200] = np.float32(2.0 ** -133)  # smallest BF16 subnormal
    for fmt in (0, 1):
        _check(x, g, fmt, "bf16", rows_kind=rows_kind, label="range")


@pytest.mark.parametrize("rows_kind", [False, True])
def test_f16_range_and_subnormals(rows_kind):
    """FP16 subnormals (below 2^-14) widen to normal FP32 values; the largest
    FP16 value, 65504, and the smallest subnormal, 2^-24."""
    g = 128
    x = synth.normal(5300, (256, 384)).astype(np.float32)
    x[0:128, 0:128] *= np.float32(3e-6)     # mostly FP16 subnormals
    x[0:128, 128:256] = np.float32(65504.0) * np.sign(x[0:128, 128:256])
    x[128:256, 0:128] = -0.0
    x[200, 300] = np.float32(2.0 ** -24)
    x[129, 1] = np.float32(2.0 ** -24)      # the only non-zero of its block
    for fmt in (0, 1):
        _check(x, g, fmt, "f16", rows_kind=rows_kind, label="range")


@pytest.mark.parametrize("kind", ["bf16", "f16"])
@pytest.mark.parametrize("g", [64, 128, 256])
def test_same_as_the_fp32_call_on_the_widened_copy(kind, g):
    """A 16-bit matrix and its exact FP32 copy quantise identically (the
    16-bit path only widens its loads)."""
    import torch

    import fp8_block_scaled_scales_amd as dg

    t, _ = _as16(synth.normal(5400 + g, (3 * g + 5, 4 * g)), kind)
    say("quantise16 vs fp32 %s g=%d" % (kind, g))
    for fmt in (0, 1):
        q16, s16 = dg.dg_quantize_fp8_blocks_typed(t, gran=g, fmt=fmt)
        q32, s32 = dg.dg_quantize_fp8_blocks(t.float(), gran=g, fmt=fmt)
        r16, rs16 = dg.dg_quantize_fp8_rows_typed(t, gran=g, fmt=fmt)
        r32, rs32 = dg.dg_quantize_fp8_rows(t.float(), gran=g, fmt=fmt)
        torch.cuda.synchronize()
        assert torch.equal(q16, q32) and torch.equal(s16, s32)
        assert torch.equal(r16, r32) and torch.equal(rs16, rs32)


@pytest.mark.parametrize("kind", ["bf16", "f16"])
def test_full_size_square_operand(kind):
    """The 8192 x 8192 operand of the large square GEMM, in the launch the
    benchmark times (g = 128, E4M3): every code and factor against the oracle."""
    _check(synth.make_a(4), 128, 0, kind, label="A of the 8192^3 workload")


def test_fp32_through_the_typed_call():
    import torch

    import fp8_block_scaled_scales_amd as dg

    x = synth.normal(5500, (257, 512))
    say("quantise typed fp32")
    q, s = dg.dg_quantize_fp8_blocks_typed(torch.from_numpy(x).to("cuda:0"), gran=128, fmt=1)
    torch.cuda.synchronize()
    rq, rs = oracle.quantize_blocks_fmt(x, 128, 1)
    assert np.array_equal(q.cpu().numpy(), rq) and np.array_equal(s.cpu().numpy().view(np.uint32), rs.view(np.uint32))


@pytest.mark.parametrize("kind", ["bf16", "f16"])
@pytest.mark.parametrize("g", [64, 128])
def test_16bit_operands_quantised_then_multiplied(kind, g):
    """The use the quantiser exists for: 16-bit activations (per-row factors)
    and weights (g x g blocks) quantised on the GPU, then the GEMM; against the
    oracle's 16-bit quantisers and its reference GEMM on the same bits."""
    import torch

    import fp8_block_scaled_scales_amd as dg
    from tests._common import within_tolerance

    M, N, K = 300, 520, 8 * g
    a16, abits = _as16(synth.make_a(3, M=M, K=K), kind)
    b16, bbits = _as16(synth.make_b(3, N=N, K=K), kind)
    say("quantise16 then gemm %s g=%d %dx%dx%d" % (kind, g, M, N, K))
    a8, sa = dg.dg_quantize_fp8_rows_typed(a16, gran=g)
    b8, sb = dg.dg_quantize_fp8_blocks_typed(b16, gran=g)
    out = dg.dg_gemm_fp8_nt_ex(a8, b8, sa, sb, gran=g, sa_rows=1)
    torch.cuda.synchronize()
    ra8, rsa = oracle.quantize_rows_16(abits, KINDS[kind], g)
    rb8, rsb = oracle.quantize_blocks_16(bbits, KINDS[kind], g)
    assert np.array_equal(a8.cpu().numpy(), ra8) and np.array_equal(b8.cpu().numpy(), rb8)
    assert np.array_equal(sa.cpu().numpy().view(np.uint32), rsa.view(np.uint32))
    assert np.array_equal(sb.cpu().numpy().view(np.uint32), rsb.view(np.uint32))
    ref = oracle.gemm_ref_rowa(ra8, rb8, rsa, rsb, g)
    ok, _ = within_tolerance(out.float().cpu().numpy(), ref)
    assert ok.all(), "%d outputs outside the bar" % int((~ok).sum())


# The per-row quantiser takes 8, 4, 2 or 1 loads per lane by the number of
# 1 x g segments (the most that still give 2048 workgroups). These shapes land
# on each choice at g = 128 for FP32 (32 segments per workgroup and load) and
# for 16-bit input (64), and just below a boundary.
@pytest.mark.parametrize("kind,rows,cols", [
    ("f32", 4096, 8192), ("f32", 2048, 8192), ("f32", 1024, 8192), ("f32", 1023, 8192), ("f32", 64, 7168),
    ("bf16", 4096, 8192), ("bf16", 2048, 8192), ("bf16", 2047, 8192), ("bf16", 1024, 8192), ("bf16", 64, 7168),
    ("f16", 1100, 7680)])
def test_rows_each_unroll_bitwise(kind, rows, cols):
    import torch

    import fp8_block_scaled_scales_amd as dg

    g = 128
    x = synth.normal(5600 + rows, (rows, cols))
    if kind == "f32":
        say("quantise rows unroll f32 %dx%d" % (rows, cols))
        q, s = dg.dg_quantize_fp8_rows(torch.from_numpy(x).to("cuda:0"), gran=g)
        torch.cuda.synchronize()
        rq, rs = oracle.quantize_rows_fmt(x, g, 0)
        assert np.array_equal(s.cpu().numpy().view(np.uint32), rs.view(np.uint32)), "scales differ"
        assert np.array_equal(q.cpu().numpy(), rq), "codes differ"
    else:
        _check(x, g, 0, kind, rows_kind=True, label="unroll")


def test_quantisers_on_concurrent_streams():
    """Quantiser calls of every input kind and both block shapes on three
    streams at once, repeated: each result equals the same call made alone
    (the quantisers keep no state between calls)."""
    import torch

    import fp8_block_scaled_scales_amd as dg

    g = 128
    xs = [torch.from_numpy(synth.normal(5700 + i, (1500 + 37 * i, 2048))).to("cuda:0") for i in range(3)]
    xs[1] = xs[1].to(torch.bfloat16)
    xs[2] = xs[2].to(torch.float16)
    calls = [(dg.dg_quantize_fp8_blocks_typed, xs[0], 0), (dg.dg_quantize_fp8_rows_typed, xs[1], 1),
             (dg.dg_quantize_fp8_blocks_typed, xs[2], 0)]
    say("quantisers on three streams")
    alone = []
    for fn, x, fmt in calls:
        q, s = fn(x, gran=g, fmt=fmt)
        torch.cuda.synchronize()
        alone.append((q.clone(), s.clone()))
    streams = [torch.cuda.Stream() for _ in calls]
    for _ in range(4):
        outs = []
        for (fn, x, fmt), st in zip(calls, streams):
            st.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(st):
                outs.append(fn(x, gran=g, fmt=fmt, stream=st))
        torch.cuda.synchronize()
        for (q, s), (q0, s0) in zip(outs, alone):
            assert torch.equal(q, q0) and torch.equal(s.view(torch.int32), s0.view(torch.int32))
