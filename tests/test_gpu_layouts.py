"""The transposed operand layouts on the GPU (through the C ABI) against the
CPU oracle.

DeepGEMM实战 §3.3: A and B may each be stored transposed ([K,M], [K,N]) and are
read that way. Every layout runs on shapes of every class the transposed
layouts use (64x64 over the whole K for M <= 128; the 256-row tiles 256 and 128
wide, with 16x16x128 and 32x32x64 fragments; 128x128), with ragged M and N
(multiples of 16), K % 128 == 64 at g = 64, and g = 256. Bars: the
elementwise tolerance against the oracle's layout reference; bit for bit
across NN, TT and TN (one kernel family, the same K order), for all-ones
closed forms, and for NT through the layout call against the NT call.
"""

import numpy as np
import pytest

import oracle
import synth
from tests import _common
from tests._gpu import say

pytestmark = pytest.mark.gpu

NT, NN, TT, TN = 0, 1, 2, 3
TRANSPOSED = [NN, TT, TN]

# (M, N, K, g, expected tile): ragged M, N (multiples of 16)
SHAPES = [
    (64, 4096, 1024, 128, (32, 32)),    # streaming 32x32 over the whole K
    (96, 528, 1088, 64, (32, 32)),
    (128, 512, 1024, 256, (32, 32)),
    (64, 4096, 7168, 128, (32, 32)),    # the decode shape
    (256, 1008, 2048, 64, (32, 32)),    # streaming, M > 128 with few tiles
    (608, 1008, 2048, 64, (64, 64)),    # 64x64 over the whole K
    (512, 1040, 768, 256, (64, 64)),
    (704, 4096, 1024, 128, (128, 128)),  # tiled
    (1024, 2000, 576, 64, (128, 128)),
    (1008, 3008, 2048, 64, (128, 128)),
    (1008, 3008, 512, 128, (256, 128)),
    (4000, 4000, 768, 128, (256, 256)),  # 256-row tiles: 16x16x128 fragments
    (4000, 4000, 704, 64, (256, 256)),   # 32x32x64 fragments, K % 128 == 64
    (3584, 3584, 512, 256, (256, 256)),
    (2000, 4000, 1024, 128, (256, 128)),
    (2000, 4000, 704, 64, (256, 128)),
]


def _store(a8, b8, layout):
    a_st = np.ascontiguousarray(a8.T) if layout & 2 else a8
    b_st = np.ascontiguousarray(b8.T) if layout & 1 else b8
    return a_st, b_st


def _run(a_st, b_st, sa, sb, g, layout, fa=0, fb=0, bias=None, act=0):
    import torch

    import fp8_block_scaled_scales_amd as dg

    dev = "cuda:0"
    ta = torch.from_numpy(a_st).to(dev)
    tb = torch.from_numpy(b_st).to(dev)
    tsa = torch.from_numpy(np.ascontiguousarray(sa)).to(dev)
    tsb = torch.from_numpy(np.ascontiguousarray(sb)).to(dev)
    tbias = None if bias is None else torch.from_numpy(bias).to(dev)
    out = dg.dg_gemm_fp8_layout(ta, tb, tsa, tsb, gran=g, layout=layout, fmt_a=fa, fmt_b=fb, bias=tbias, act=act)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), out.view(torch.int16).cpu().numpy().view(np.uint16)


def _operands(M, N, K, g, fa, fb, seed):
    a8, sa = oracle.quantize_blocks_fmt(synth.normal(seed, (M, K)), g, fa)
    b8, sb = oracle.quantize_blocks_fmt(synth.normal(seed + 1, (N, K), sigma=0.02), g, fb)
    return a8, sa, b8, sb


def _sample(M, N, tile, seed):
    rows = np.unique(np.concatenate([_common.sample_indices(M, 120, seed=seed), np.arange(0, M, tile[0]),
                                     np.arange(tile[0] - 1, M, tile[0]), [M - 1]]))
    cols = np.unique(np.concatenate([_common.sample_indices(N, 120, seed=seed + 1), np.arange(0, N, tile[1]),
                                     np.arange(tile[1] - 1, N, tile[1]), [N - 1]]))
    return rows, cols


def _assert_parity(got, ref, label):
    ok, rms = _common.within_tolerance(got, ref)
    if not ok.all():
        idx = np.argwhere(~ok)[:5]
        detail = ", ".join("(%d,%d) got %.6g ref %.6g" % (i, j, got[i, j], ref[i, j]) for i, j in idx)
        raise AssertionError("%s: %d of %d outside tolerance: %s" % (label, int((~ok).sum()), ok.size, detail))
    say("%s: max|err|/rms = %.3g" % (label, np.max(np.abs(got - ref)) / rms))


@pytest.mark.parametrize("layout", TRANSPOSED)
@pytest.mark.parametrize("M,N,K,g,tile", SHAPES)
def test_layout_parity(M, N, K, g, tile, layout):
    import fp8_block_scaled_scales_amd as dg

    t = dg.dg_query_tile(M, N, K, g, layout)
    assert (t["bm"], t["bn"]) == tile, t
    a8, sa, b8, sb = _operands(M, N, K, g, 0, 0, seed=11000 + M + K)
    a_st, b_st = _store(a8, b8, layout)
    say("layout %d M=%d N=%d K=%d g=%d" % (layout, M, N, K, g))
    got, _ = _run(a_st, b_st, sa, sb, g, layout)
    rows, cols = _sample(M, N, tile, M + N)
    ref = oracle.gemm_ref_layout(a_st, b_st, sa, sb, g, layout, M, N, K, rows=rows, cols=cols)
    _assert_parity(got[np.ix_(rows, cols)], ref, "layout %d %dx%dx%d g=%d" % (layout, M, N, K, g))


@pytest.mark.parametrize("layout,fa,fb,act,with_bias", [(NN, 1, 0, 0, False), (TN, 0, 1, 2, True),
                                                        (TT, 1, 1, 1, True)])
@pytest.mark.parametrize("M,N,K,g,tile", [SHAPES[1], SHAPES[3], SHAPES[7], SHAPES[9]])
def test_layout_with_formats_and_epilogue(M, N, K, g, tile, layout, fa, fb, act, with_bias):
    a8, sa, b8, sb = _operands(M, N, K, g, fa, fb, seed=12000 + M + 10 * layout)
    bias = synth.normal(12100 + N, (N,), sigma=0.5).astype(np.float32) if with_bias else None
    a_st, b_st = _store(a8, b8, layout)
    say("layout %d fmt %d,%d act=%d bias=%d M=%d N=%d K=%d g=%d" % (layout, fa, fb, act, with_bias, M, N, K, g))
    got, _ = _run(a_st, b_st, sa, sb, g, layout, fa, fb, bias, act)
    rows, cols = _sample(M, N, tile, M + 3 * N)
    ref = oracle.epilogue(oracle.gemm_ref_layout(a_st, b_st, sa, sb, g, layout, M, N, K, fa, fb, rows, cols),
                          bias, act, cols)
    _assert_parity(got[np.ix_(rows, cols)], ref, "layout %d fmt %d,%d act %d" % (layout, fa, fb, act))


@pytest.mark.parametrize("M,N,K,g,tile", SHAPES)
def test_transposed_layouts_agree_bitwise(M, N, K, g, tile):
    a8, sa, b8, sb = _operands(M, N, K, g, 0, 0, seed=13000 + M + K)
    # every layout's fragments hold the NT K order, so all four give the same bits
    bits = {}
    for layout in [NT] + TRANSPOSED:
        a_st, b_st = _store(a8, b8, layout)
        say("layout %d bits M=%d N=%d K=%d g=%d" % (layout, M, N, K, g))
        bits[layout] = _run(a_st, b_st, sa, sb, g, layout)[1]
    for layout in TRANSPOSED:
        assert np.array_equal(bits[layout], bits[NT]), layout


@pytest.mark.parametrize("layout", TRANSPOSED)
@pytest.mark.parametrize("M,N,K,g,tile", [SHAPES[0], SHAPES[1], SHAPES[3], SHAPES[5], SHAPES[6], SHAPES[7],
                                         SHAPES[10]])
def test_layout_closed_form_all_ones_bitwise(M, N, K, g, tile, layout):
    a8 = np.full((M, K), 0x38, np.uint8)
    b8 = np.full((N, K), 0x38, np.uint8)
    nkb = K // g
    sa = (2.0 ** ((np.arange((M + g - 1) // g)[:, None] - np.arange(nkb)[None, :]) % 7 - 3)).astype(np.float32)
    sb = (2.0 ** ((2 * np.arange((N + g - 1) // g)[:, None] + np.arange(nkb)[None, :]) % 3)).astype(np.float32)
    a_st, b_st = _store(a8, b8, layout)
    say("layout %d closed form M=%d N=%d K=%d g=%d" % (layout, M, N, K, g))
    _, bits = _run(a_st, b_st, sa, sb, g, layout)
    rows = np.unique(np.concatenate([np.arange(0, M, 7), [M - 1]]))
    cols = np.unique(np.concatenate([np.arange(0, N, 37), [N - 1]]))
    ref = oracle.gemm_ref_layout(a_st, b_st, sa, sb, g, layout, M, N, K, rows=rows, cols=cols)
    assert np.array_equal(bits[np.ix_(rows, cols)], _common.f32_to_bf16_bits(ref.astype(np.float32)))


def test_layout_permutation_closed_form_bitwise():
    # A[i,k] = 1 where k = p(i): out[i,j] = sa*sb*B[j, p(i)], one element each,
    # which any transposed index or misplaced transposing read gets wrong
    for M, N, K, g in [(1008, 528, 1024, 128), (4000, 4000, 768, 128), (2000, 4000, 704, 64)]:
        _permutation_case(M, N, K, g)


def _permutation_case(M, N, K, g):
    rng = np.random.default_rng(14000)
    p = rng.integers(0, K, size=M)
    a8 = np.zeros((M, K), np.uint8)
    a8[np.arange(M), p] = 0x38
    b8 = rng.integers(0, 0x7F, size=(N, K), dtype=np.uint8)
    sa = np.ones(((M + g - 1) // g, K // g), np.float32)
    sb = np.ones(((N + g - 1) // g, K // g), np.float32)
    for layout in TRANSPOSED:
        a_st, b_st = _store(a8, b8, layout)
        say("layout %d permutation closed form" % layout)
        _, bits = _run(a_st, b_st, sa, sb, g, layout)
        rows = np.unique(np.concatenate([np.arange(0, M, 13), np.arange(255, M, 256), [M - 1]]))
        ref = oracle.gemm_ref_layout(a_st, b_st, sa, sb, g, layout, M, N, K, rows=rows)
        assert np.array_equal(bits[rows], _common.f32_to_bf16_bits(ref.astype(np.float32))), layout


def test_nt_through_the_layout_call_is_the_nt_call_bitwise():
    import torch

    import fp8_block_scaled_scales_amd as dg

    M, N, K, g = 1000, 3000, 512, 128
    a8, sa, b8, sb = _operands(M, N, K, g, 0, 0, seed=15000)
    o1 = _run(a8, b8, sa, sb, g, NT)[1]
    dev = "cuda:0"
    o2 = dg.dg_gemm_fp8_nt(torch.from_numpy(a8).to(dev), torch.from_numpy(b8).to(dev),
                           torch.from_numpy(sa).to(dev), torch.from_numpy(sb).to(dev), gran=g)
    torch.cuda.synchronize()
    assert np.array_equal(o1, o2.view(torch.int16).cpu().numpy().view(np.uint16))


# Ragged stored rows: M (A stored [K,M]) and N (B stored [K,N]) not multiples
# of 16, so the transposed rows are not 16-byte aligned, on the 64x64, 128x128
# and 256-row tiles (256 and 128 wide), K % 128 == 64 at g = 64.
RAGGED_T = [
    (7, 4095, 1024, 128), (97, 531, 1088, 64), (1001, 3003, 512, 128), (999, 2001, 576, 64),
    (4001, 3999, 512, 128), (2003, 3997, 704, 64),
]


@pytest.mark.parametrize("layout", TRANSPOSED)
@pytest.mark.parametrize("M,N,K,g", RAGGED_T)
def test_layout_ragged_parity(M, N, K, g, layout):
    import fp8_block_scaled_scales_amd as dg

    t = dg.dg_query_tile(M, N, K, g, layout)
    tile = (t["bm"], t["bn"])
    a8, sa, b8, sb = _operands(M, N, K, g, 0, 0, seed=16000 + M + N)
    a_st, b_st = _store(a8, b8, layout)
    say("ragged layout %d M=%d N=%d K=%d g=%d tile %s" % (layout, M, N, K, g, tile))
    got, bits = _run(a_st, b_st, sa, sb, g, layout)
    assert np.all(np.isfinite(got))
    rows, cols = _sample(M, N, tile, M + 5 * N)
    ref = oracle.gemm_ref_layout(a_st, b_st, sa, sb, g, layout, M, N, K, rows=rows, cols=cols)
    _assert_parity(got[np.ix_(rows, cols)], ref, "ragged layout %d %dx%dx%d g=%d" % (layout, M, N, K, g))


@pytest.mark.parametrize("M,N,K,g", [RAGGED_T[1], RAGGED_T[2], RAGGED_T[4], RAGGED_T[5]])
def test_layout_ragged_closed_form_and_agreement_bitwise(M, N, K, g):
    # all-ones codes with power-of-two block factors: exact, so every layout
    # matches bf16(ref) bit for bit, ragged edges included
    a8 = np.full((M, K), 0x38, np.uint8)
    b8 = np.full((N, K), 0x38, np.uint8)
    nkb = K // g
    sa = (2.0 ** ((np.arange((M + g - 1) // g)[:, None] - np.arange(nkb)[None, :]) % 7 - 3)).astype(np.float32)
    sb = (2.0 ** ((2 * np.arange((N + g - 1) // g)[:, None] + np.arange(nkb)[None, :]) % 3)).astype(np.float32)
    rows = np.unique(np.concatenate([np.arange(0, M, 7), [M - 1]]))
    cols = np.unique(np.concatenate([np.arange(0, N, 37), [N - 1]]))
    ref = oracle.gemm_ref(a8, b8, sa, sb, g, rows, cols)
    for layout in TRANSPOSED:
        a_st, b_st = _store(a8, b8, layout)
        say("ragged closed form layout %d M=%d N=%d K=%d g=%d" % (layout, M, N, K, g))
        _, bits = _run(a_st, b_st, sa, sb, g, layout)
        assert np.array_equal(bits[np.ix_(rows, cols)], _common.f32_to_bf16_bits(ref.astype(np.float32))), layout


def _run_ws(a_st, b_st, sa, sb, g, layout, sa_rows=None, fa=0, fb=0, bias=None, act=0, workspace=False):
    import torch

    import fp8_block_scaled_scales_amd as dg

    dev = "cuda:0"
    t = [torch.from_numpy(np.ascontiguousarray(x)).to(dev) for x in (a_st, b_st, sa, sb)]
    tbias = None if bias is None else torch.from_numpy(bias).to(dev)
    ws = None
    if workspace:
        K, M = a_st.shape if layout & 2 else a_st.shape[::-1]
        N = b_st.shape[1] if layout & 1 else b_st.shape[0]
        ws = dg.dg_workspace(M, N, K, g, layout, device=dev)
    out = dg.dg_gemm_fp8_ws(t[0], t[1], t[2], t[3], gran=g, layout=layout, sa_rows=sa_rows, fmt_a=fa, fmt_b=fb,
                            bias=tbias, act=act, workspace=ws)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), out.view(torch.int16).cpu().numpy().view(np.uint16)


# Per-row A factors (one per row and K segment) with a transposed layout, on
# the 64x64, 128x128 and 256-row tiles; ragged M and N included.
ROWA_T = [(64, 4096, 1024, 128), (97, 531, 1088, 64), (1008, 3008, 512, 128), (1001, 3003, 576, 64),
          (4000, 4000, 768, 128), (2003, 3997, 704, 64), (512, 1040, 768, 256)]


@pytest.mark.parametrize("layout", TRANSPOSED)
@pytest.mark.parametrize("M,N,K,g", ROWA_T)
def test_layout_rowscales_parity(M, N, K, g, layout):
    import fp8_block_scaled_scales_amd as dg

    t = dg.dg_query_tile(M, N, K, g, layout, workspace=False)
    tile = (t["bm"], t["bn"])
    x = synth.normal(17000 + M, (M, K)) * np.exp(np.random.default_rng(M).uniform(-4, 4, size=(M, 1)))
    a8, sa = oracle.quantize_rows_fmt(x.astype(np.float32), g, 0)
    b8, sb = oracle.quantize_blocks_fmt(synth.normal(17001 + N, (N, K), sigma=0.02), g, 0)
    a_st, b_st = _store(a8, b8, layout)
    say("per-row layout %d M=%d N=%d K=%d g=%d tile %s" % (layout, M, N, K, g, tile))
    got, _ = _run_ws(a_st, b_st, sa, sb, g, layout, sa_rows=1)
    rows, cols = _sample(M, N, tile, M + 7 * N)
    ref = oracle.gemm_ref_rowa(a8, b8, sa, sb, g, rows=rows, cols=cols)
    _assert_parity(got[np.ix_(rows, cols)], ref, "per-row layout %d %dx%dx%d g=%d" % (layout, M, N, K, g))


@pytest.mark.parametrize("M,N,K,g", [(4000, 4000, 768, 128), (2003, 3997, 704, 64), (1008, 3008, 512, 128)])
def test_layout_rowscales_same_bits_as_nt(M, N, K, g):
    # the transposed tiles read the same K order as the NT tiles of the same
    # class, so per-row results agree with the NT per-row call bit for bit
    import torch

    import fp8_block_scaled_scales_amd as dg

    x = synth.normal(18000 + M, (M, K)) * np.exp(np.random.default_rng(M + 1).uniform(-4, 4, size=(M, 1)))
    a8, sa = oracle.quantize_rows_fmt(x.astype(np.float32), g, 0)
    b8, sb = oracle.quantize_blocks_fmt(synth.normal(18001 + N, (N, K), sigma=0.02), g, 0)
    dev = "cuda:0"
    nt = dg.dg_gemm_fp8_nt_ex(torch.from_numpy(a8).to(dev), torch.from_numpy(b8).to(dev), torch.from_numpy(sa).to(dev),
                              torch.from_numpy(sb).to(dev), gran=g, sa_rows=1)
    torch.cuda.synchronize()
    want = nt.view(torch.int16).cpu().numpy().view(np.uint16)
    for layout in TRANSPOSED:
        t = dg.dg_query_tile(M, N, K, g, layout)
        assert t["kernel_id"] == dg.dg_query_tile(M, N, K, g)["kernel_id"], (layout, t)
        a_st, b_st = _store(a8, b8, layout)
        say("per-row layout %d vs NT bits M=%d N=%d K=%d g=%d" % (layout, M, N, K, g))
        assert np.array_equal(_run_ws(a_st, b_st, sa, sb, g, layout, sa_rows=1)[1], want), layout


# The smallest shapes: stored rows of 1-3 bytes (shorter than one 4-byte word,
# so the tensor's last K row comes entirely from the tail patch), one-row and
# one-column outputs, K of a single segment, and a few tile-edge sizes; every
# layout against the oracle and bit for bit against NT, g x g and per-row
# factors. The whole output is compared.
TINY = [(1, 1, 64, 64), (1, 17, 128, 128), (3, 2, 192, 64), (2, 130, 256, 128), (33, 3, 128, 64),
        (5, 7, 256, 256), (130, 129, 128, 128), (259, 6, 192, 64)]


@pytest.mark.parametrize("rowa", [False, True])
@pytest.mark.parametrize("M,N,K,g", TINY)
def test_tiny_shapes_every_layout(M, N, K, g, rowa):
    x = synth.normal(19000 + M + N, (M, K))
    if rowa:
        a8, sa = oracle.quantize_rows_fmt(x, g, 0)
    else:
        a8, sa = oracle.quantize_blocks_fmt(x, g, 0)
    b8, sb = oracle.quantize_blocks_fmt(synth.normal(19001 + N, (N, K), sigma=0.02), g, 0)
    ref = oracle.gemm_ref_rowa(a8, b8, sa, sb, g) if rowa else oracle.gemm_ref_fmt(a8, b8, sa, sb, g, 0, 0)
    bits = {}
    for layout in [NT] + TRANSPOSED:
        a_st, b_st = _store(a8, b8, layout)
        say("tiny layout %d M=%d N=%d K=%d g=%d rowa=%d" % (layout, M, N, K, g, rowa))
        got, bits[layout] = _run_ws(a_st, b_st, sa, sb, g, layout, sa_rows=1 if rowa else None)
        _assert_parity(got, ref, "tiny layout %d %dx%dx%d g=%d" % (layout, M, N, K, g))
    for layout in TRANSPOSED:
        assert np.array_equal(bits[layout], bits[NT]), layout


@pytest.mark.parametrize("rowa", [False, True])
@pytest.mark.parametrize("M,N,K,g", [(1, 1, 2048, 128), (3, 2, 1088, 64), (2, 130, 1024, 128), (33, 3, 2048, 64),
                                     (5, 7, 1536, 256), (97, 5, 1088, 64)])
def test_tiny_shapes_every_layout_split_k(M, N, K, g, rowa):
    # the same through the split-K class with a workspace (the tile override:
    # the plan itself streams K ranges this short): these few tiles split K
    # over workgroups, and only the last split's final step holds the
    # tensor's last bytes
    with _common.forced_split(g):
        _tiny_split_k(M, N, K, g, rowa)


def _tiny_split_k(M, N, K, g, rowa):
    import fp8_block_scaled_scales_amd as dg

    assert all(dg.dg_query_tile(M, N, K, g, layout, workspace=True)["ksplit"] > 1 for layout in range(4))
    x = synth.normal(19500 + M + N, (M, K))
    if rowa:
        a8, sa = oracle.quantize_rows_fmt(x, g, 0)
    else:
        a8, sa = oracle.quantize_blocks_fmt(x, g, 0)
    b8, sb = oracle.quantize_blocks_fmt(synth.normal(19501 + N, (N, K), sigma=0.02), g, 0)
    ref = oracle.gemm_ref_rowa(a8, b8, sa, sb, g) if rowa else oracle.gemm_ref_fmt(a8, b8, sa, sb, g, 0, 0)
    bits = {}
    for layout in [NT] + TRANSPOSED:
        a_st, b_st = _store(a8, b8, layout)
        say("tiny split-K layout %d M=%d N=%d K=%d g=%d rowa=%d" % (layout, M, N, K, g, rowa))
        got, bits[layout] = _run_ws(a_st, b_st, sa, sb, g, layout, sa_rows=1 if rowa else None, workspace=True)
        _assert_parity(got, ref, "tiny split-K layout %d %dx%dx%d g=%d" % (layout, M, N, K, g))
    for layout in TRANSPOSED:
        assert np.array_equal(bits[layout], bits[NT]), layout
