"""Largest accepted sizes on the GPU (through the C ABI) against the CPU oracle.

DG_MAX_DIM = 2^24 - 256 bounds M, N and K. At K = DG_MAX_DIM a 256-row tile
covers 256 * K = 2^32 - 65536 bytes, the edge of what a buffer descriptor
reaches, so these cases check that no tile's byte range or offset wraps:
- K = DG_MAX_DIM on the 256x128 tiles (g = 128 and 64; NT, TN and TT), the
  32x32 streaming class, the 64x64 class over the whole K, and the split-K
  class of dg_gemm_fp8_ws (M = 64, N = 4096);
- M = DG_MAX_DIM and N = DG_MAX_DIM (K = 256) on the 256x256 tiles, NT and a
  transposed A stored [K, M];
- the g x g and 1 x g quantisers with rows or cols = DG_MAX_DIM, sampled
  blocks bitwise against the oracle's quantisers.

The operands are random E4M3 codes drawn on the GPU by torch's seeded
generator (87 GB in all; drawing them on the host would take minutes), with
the top exponent bit cleared so that no code is NaN (|value| < 2). Only the sampled
rows and columns travel back to the host for the oracle. Along K the block
factors vary per segment; at K = DG_MAX_DIM they are the same for every row
block and column block, so sampled rows and columns form a small problem of
their own. The large-M and large-N cases use per-block factors of every row
block, the oracle taking the sampled rows with their blocks' factors.
"""

import numpy as np
import pytest

import oracle
from tests import _common
from tests._gpu import say

pytestmark = pytest.mark.gpu

MAX_DIM = (1 << 24) - 256
K_MAX = MAX_DIM
POOL_ROWS = 5184  # rows of K_MAX bytes: A [2048] + B [3072] of the tile cases, or B [4096] + A [64]


@pytest.fixture(scope="module")
def pool():
    import torch

    import fp8_block_scaled_scales_amd as dg

    assert dg.DG_MAX_DIM == MAX_DIM
    torch.cuda.empty_cache()
    need = POOL_ROWS * K_MAX
    free, _ = torch.cuda.mem_get_info()
    if free < need + (8 << 30):
        pytest.skip("needs %.0f GB of free device memory, %.0f GB free" % (need / 1e9, free / 1e9))
    say("max-size pool: %d bytes" % need)
    gen = torch.Generator(device="cuda:0").manual_seed(2024)
    p = torch.empty(need, dtype=torch.uint8, device="cuda:0")
    p.random_(0, 256, generator=gen)
    p.bitwise_and_(0xBF)  # top exponent bit off: magnitudes below 2, no NaN code
    torch.cuda.synchronize()
    yield p
    del p
    torch.cuda.empty_cache()


def _kfactors(seed, nkb):
    rng = np.random.default_rng(seed)
    return rng.uniform(0.25, 4.0, size=nkb).astype(np.float32)


def _logical_rows(stored, idx, transposed):
    """Rows idx of the logical [rows, K] operand, on the host."""
    import torch

    t = torch.from_numpy(np.asarray(idx, dtype=np.int64)).to(stored.device)
    if transposed:
        return np.ascontiguousarray(stored.index_select(1, t).cpu().numpy().T)
    return stored.index_select(0, t).cpu().numpy()


def _check_long_k(pool, M, N, g, layout, tile, ws=False):
    import torch

    import fp8_block_scaled_scales_amd as dg

    K = K_MAX
    t = dg.dg_query_tile(M, N, K, g, layout, workspace=ws)
    assert (t["bm"], t["bn"]) == tile, t
    assert (t["ksplit"] > 1) == ws, t
    a_st = pool[:M * K].view(K, M) if layout & 2 else pool[:M * K].view(M, K)
    b_st = pool[M * K:(M + N) * K].view(K, N) if layout & 1 else pool[M * K:(M + N) * K].view(N, K)
    fa, fb = _kfactors(40 + g + layout, K // g), _kfactors(41 + g + layout, K // g)
    sa = torch.from_numpy(np.tile(fa, ((M + g - 1) // g, 1))).to("cuda:0")
    sb = torch.from_numpy(np.tile(fb, ((N + g - 1) // g, 1))).to("cuda:0")
    say("max K: M=%d N=%d K=%d g=%d layout=%d tile=%s ksplit=%d" % (M, N, K, g, layout, tile, t["ksplit"]))
    if ws:
        out = dg.dg_gemm_fp8_ws(a_st, b_st, sa, sb, gran=g, layout=layout,
                                workspace=dg.dg_workspace(M, N, K, g, layout))
    else:
        out = dg.dg_gemm_fp8_layout(a_st, b_st, sa, sb, gran=g, layout=layout)
    torch.cuda.synchronize()
    rows = np.unique(np.array([0, 1, tile[0] - 1, min(tile[0], M - 1), M // 2 + 3, M - 2, M - 1]))
    cols = np.unique(np.array([0, 1, tile[1] - 1, min(tile[1], N - 1), N // 2 + 5, N - 2, N - 1]))
    got = out.float().cpu().numpy().astype(np.float64)[np.ix_(rows, cols)]
    del out, sa, sb
    a_sub = _logical_rows(a_st, rows, layout & 2)
    b_sub = _logical_rows(b_st, cols, layout & 1)
    ref = oracle.gemm_ref(a_sub, b_sub, fa[None, :], fb[None, :], g)
    ok, rms = _common.within_tolerance(got, ref)
    assert ok.all(), (got[~ok][:4], ref[~ok][:4], rms)
    say("max K g=%d layout=%d: max|err|/rms = %.3g" % (g, layout, np.max(np.abs(got - ref)) / rms))


@pytest.mark.parametrize("g,layout", [(128, 0), (64, 0), (128, 3), (64, 2)])
def test_max_k_256x128_tiles(pool, g, layout):
    _check_long_k(pool, 2048, 3072, g, layout, (256, 128))


@pytest.mark.parametrize("layout,N,tile,ws", [(0, 4096, (32, 32), False), (3, 4096, (32, 32), False),
                                              (3, 1024, (64, 64), True)])
def test_max_k_small_m(pool, layout, N, tile, ws):
    _check_long_k(pool, 64, N, 128, layout, tile, ws)


@pytest.mark.parametrize("big_m,layout", [(True, 0), (True, 2), (False, 0)])
def test_max_m_or_n(pool, big_m, layout):
    M, N, K, g = (MAX_DIM, 256, 256, 128) if big_m else (256, MAX_DIM, 256, 128)
    # the 256x256 tiles (table entry 4), whose tiles span the most bytes of
    # A and B (the plan takes 128x128 tiles here)
    with _common.forced_tile(4):
        _max_m_or_n(pool, M, N, K, g, big_m, layout)


def _max_m_or_n(pool, M, N, K, g, big_m, layout):
    import torch

    import fp8_block_scaled_scales_amd as dg

    t = dg.dg_query_tile(M, N, K, g, layout)
    assert (t["bm"], t["bn"]) == (256, 256), t
    a_st = pool[:M * K].view(K, M) if layout & 2 else pool[:M * K].view(M, K)
    b_st = pool[M * K:(M + N) * K].view(N, K)
    rng = np.random.default_rng(50 + layout + 2 * big_m)
    sa = rng.uniform(0.25, 4.0, size=((M + g - 1) // g, K // g)).astype(np.float32)
    sb = rng.uniform(0.25, 4.0, size=((N + g - 1) // g, K // g)).astype(np.float32)
    say("max %s: M=%d N=%d K=%d layout=%d" % ("M" if big_m else "N", M, N, K, layout))
    out = dg.dg_gemm_fp8_layout(a_st, b_st, torch.from_numpy(sa).to("cuda:0"), torch.from_numpy(sb).to("cuda:0"),
                                gran=g, layout=layout)
    torch.cuda.synchronize()
    long_n, short_n = (M, N) if big_m else (N, M)
    idx = np.unique(np.concatenate([_common.sample_indices(long_n, 24, seed=60), np.arange(255, long_n, 1 << 20)]))
    if big_m:
        got = out[torch.from_numpy(idx).to("cuda:0")].float().cpu().numpy().astype(np.float64)
        a_sub = _logical_rows(a_st, idx, layout & 2)
        ref = oracle.gemm_ref_rowa(a_sub, b_st.cpu().numpy(), sa[idx // g], sb, g)
    else:
        got = out[:, torch.from_numpy(idx).to("cuda:0")].float().cpu().numpy().astype(np.float64)
        b_sub = _logical_rows(b_st, idx, False)
        # out[:, idx] = (B[idx] . A^T)^T: B's rows take the per-row factors of their blocks
        ref = oracle.gemm_ref_rowa(b_sub, a_st.cpu().numpy(), sb[idx // g], sa, g).T
    del out
    assert got.shape == ref.shape == ((idx.size, short_n) if big_m else (short_n, idx.size))
    ok, rms = _common.within_tolerance(got, ref)
    assert ok.all(), (got[~ok][:4], ref[~ok][:4], rms)
    say("max %s layout=%d: max|err|/rms = %.3g" % ("M" if big_m else "N", layout, np.max(np.abs(got - ref)) / rms))


@pytest.mark.parametrize("kind", ["f32", "bf16"])
@pytest.mark.parametrize("rows_max", [False, True])
@pytest.mark.parametrize("per_row", [False, True])
def test_max_quantizer(rows_max, per_row, kind):
    # block (g x g) and row (1 x g) quantisers at rows or cols = DG_MAX_DIM, on
    # FP32 or (through the typed calls) BF16 input: sampled blocks bitwise
    # against the oracle's quantiser on those blocks
    import torch

    import fp8_block_scaled_scales_amd as dg

    g = 64
    rows, cols = (MAX_DIM, 256) if rows_max else (64, MAX_DIM)
    gen = torch.Generator(device="cuda:0").manual_seed(77 + rows_max + 2 * per_row)
    x = torch.randn((rows, cols), generator=gen, device="cuda:0", dtype=torch.float32)
    if kind == "bf16":
        x = x.to(torch.bfloat16)
        fn = dg.dg_quantize_fp8_rows_typed if per_row else dg.dg_quantize_fp8_blocks_typed
    else:
        fn = dg.dg_quantize_fp8_rows if per_row else dg.dg_quantize_fp8_blocks
    say("max quantiser: rows=%d cols=%d per_row=%d %s" % (rows, cols, per_row, kind))
    q, s = fn(x, gran=g)
    torch.cuda.synchronize()
    nrb, ncb = rows // g, cols // g
    blocks = [(0, 0), (nrb - 1, ncb - 1), (nrb // 2, ncb // 3), (nrb - 1, 0), (0, ncb - 1)]
    for rb, cb in blocks:
        xt = x[rb * g:(rb + 1) * g, cb * g:(cb + 1) * g].contiguous().cpu()
        qb = q[rb * g:(rb + 1) * g, cb * g:(cb + 1) * g].cpu().numpy()
        if kind == "bf16":
            bits = xt.view(torch.int16).numpy().view(np.uint16)
            ref = oracle.quantize_rows_16 if per_row else oracle.quantize_blocks_16
            want_q, want_s = ref(bits, oracle.IN_BF16, g, 0)
        elif per_row:
            want_q, want_s = oracle.quantize_rows_fmt(xt.numpy(), g)
        else:
            want_q, want_s = oracle.quantize_blocks_fmt(xt.numpy(), g, 0)
        if per_row:
            got_s = s[rb * g:(rb + 1) * g, cb].cpu().numpy()[:, None]
        else:
            got_s = s[rb, cb].cpu().numpy().reshape(1, 1)
        assert np.array_equal(qb, want_q), (rb, cb)
        assert np.array_equal(got_s.view(np.uint32), np.asarray(want_s, np.float32).reshape(got_s.shape).view(np.uint32)), (rb, cb)
    del x, q, s
    torch.cuda.empty_cache()
