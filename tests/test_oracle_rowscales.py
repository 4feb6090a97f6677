"""Pins for the oracle's per-row A scales (CPU only): the 1 x g quantiser and
the reference GEMM whose A factors are one per row and g-wide K segment.

The template article (§3.4) names per-tensor and per-channel scale factors
and takes per channel; read for A as one factor per row of A and K segment
(1 x g blocks), B keeping its g x g blocks.

Pinned by: the block quantiser on one-row matrices (a g x g edge block with
one present row is a 1 x g block); torch's float8 casts on the scaled
values; exact rational brute force; the block-scaled reference when each
row's factors repeat its block's; closed forms with power-of-two factors; and
the one-row doubling invariant.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

TORCH_FP8 = {oracle.E4M3: torch.float8_e4m3fn, oracle.E5M2: torch.float8_e5m2}
FMAX = {oracle.E4M3: 448.0, oracle.E5M2: 57344.0}


def _activations(seed, rows, cols, g):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((rows, cols)) * np.exp(rng.uniform(-6, 6, size=(rows, 1)))).astype(np.float32)
    x[0, :g] = 0.0  # an all-zero segment: factor 1
    x[1, g:2 * g] *= 1e-30  # a segment of tiny values
    return x


# ------------------------------------------------------------- quantiser

@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
@pytest.mark.parametrize("rows,cols,g", [(5, 256, 128), (9, 192, 64), (4, 512, 256)])
def test_rows_quantiser_is_the_block_quantiser_row_by_row(fmt, rows, cols, g):
    x = _activations(rows * 7 + cols + fmt, rows, cols, g)
    q, s = oracle.quantize_rows_fmt(x, g, fmt)
    assert q.shape == x.shape and s.shape == (rows, cols // g)
    for r in range(rows):
        qr, sr = oracle.quantize_blocks_fmt(x[r:r + 1], g, fmt)  # one present row per g x g block
        assert np.array_equal(q[r:r + 1], qr)
        assert np.array_equal(s[r:r + 1].view(np.uint32), sr.view(np.uint32))


@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_rows_quantiser_by_definition(fmt):
    rows, cols, g = 33, 384, 128
    x = _activations(77 + fmt, rows, cols, g)
    q, s = oracle.quantize_rows_fmt(x, g, fmt)
    for r in range(rows):
        for cb in range(cols // g):
            seg = x[r, cb * g:(cb + 1) * g]
            amax = np.float32(np.max(np.abs(seg)))
            scale = np.float32(amax / np.float32(FMAX[fmt])) if amax > 0 else np.float32(1.0)
            assert s[r, cb] == scale
            y = (seg / scale).astype(np.float32)
            ref = torch.from_numpy(np.ascontiguousarray(y)).to(TORCH_FP8[fmt]).view(torch.uint8).numpy()
            assert np.array_equal(q[r, cb * g:(cb + 1) * g], ref), (r, cb)


# ------------------------------------------------------------- reference

def _rand_codes(rng, shape, fmt):
    c = rng.integers(0, 256, size=shape, dtype=np.uint8)
    if fmt == oracle.E5M2:
        c[(c & 0x7F) >= 0x7C] = 0x3C  # no infinity or NaN
    else:
        c[(c & 0x7F) == 0x7F] = 0x38  # no NaN
    return c


def _frac(c, fmt):
    if fmt == oracle.E5M2:
        e, m = (c >> 2) & 31, c & 3
        mag = Fraction(m, 4) * Fraction(1, 2 ** 14) if e == 0 else (1 + Fraction(m, 4)) * Fraction(2) ** (e - 15)
    else:
        e, m = (c >> 3) & 15, c & 7
        mag = Fraction(m, 8) * Fraction(1, 64) if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
    return -mag if c & 0x80 else mag


@pytest.mark.parametrize("fa,fb,M,N,K,g", [(0, 0, 5, 4, 256, 128), (0, 0, 3, 3, 128, 64), (1, 0, 4, 3, 256, 64),
                                          (0, 1, 3, 4, 512, 256), (1, 1, 2, 5, 256, 128)])
def test_rowa_brute_force_exact_rationals(fa, fb, M, N, K, g):
    rng = np.random.default_rng(fa * 10 + fb + K + M)
    a8, b8 = _rand_codes(rng, (M, K), fa), _rand_codes(rng, (N, K), fb)
    sa = rng.uniform(0.01, 3.0, size=(M, K // g)).astype(np.float32)
    sb = rng.uniform(0.01, 3.0, size=((N + g - 1) // g, K // g)).astype(np.float32)
    ref = oracle.gemm_ref_rowa(a8, b8, sa, sb, g, fa, fb)
    nkb = K // g
    for i in range(M):
        for j in range(N):
            exact, mag = Fraction(0), Fraction(0)
            for kb in range(nkb):
                terms = [_frac(int(a8[i, k]), fa) * _frac(int(b8[j, k]), fb) for k in range(kb * g, kb * g + g)]
                s = Fraction(float(sa[i, kb])) * Fraction(float(sb[j // g, kb]))
                exact += s * sum(terms)
                mag += s * sum(abs(t) for t in terms)
            tol = float(mag) * (g + 2) * nkb * 2.0 ** -53
            assert abs(Fraction(ref[i, j]) - exact) <= Fraction(tol), (i, j)


@pytest.mark.parametrize("fa,fb,M,N,K,g", [(0, 0, 300, 70, 512, 128), (1, 0, 130, 65, 384, 64),
                                          (0, 1, 520, 40, 512, 256)])
def test_rowa_with_repeated_block_factors_is_the_block_reference(fa, fb, M, N, K, g):
    rng = np.random.default_rng(M + N + K)
    a8, b8 = _rand_codes(rng, (M, K), fa), _rand_codes(rng, (N, K), fb)
    sa_blk = rng.uniform(0.01, 3.0, size=((M + g - 1) // g, K // g)).astype(np.float32)
    sb = rng.uniform(0.01, 3.0, size=((N + g - 1) // g, K // g)).astype(np.float32)
    sa_row = sa_blk[np.arange(M) // g]
    rows = np.array([0, 1, g - 1, g, M - 1])
    assert np.array_equal(oracle.gemm_ref_rowa(a8, b8, sa_row, sb, g, fa, fb, rows=rows),
                          oracle.gemm_ref_fmt(a8, b8, sa_blk, sb, g, fa, fb, rows=rows))


@pytest.mark.parametrize("M,N,K,g", [(300, 260, 1024, 128), (70, 130, 384, 64), (40, 300, 1024, 256)])
def test_rowa_closed_form_all_ones(M, N, K, g):
    a8 = np.full((M, K), 0x38, np.uint8)  # 1.0
    b8 = np.full((N, K), 0x38, np.uint8)
    nkb = K // g
    sa = np.array([[2.0 ** ((i * 5 + kb) % 9 - 4) for kb in range(nkb)] for i in range(M)], np.float32)
    sb = np.array([[2.0 ** ((nb + 2 * kb) % 3) for kb in range(nkb)] for nb in range((N + g - 1) // g)], np.float32)
    ref = oracle.gemm_ref_rowa(a8, b8, sa, sb, g)
    for i in range(0, M, 3):
        for j in range(0, N, 13):
            want = g * sum(2.0 ** ((i * 5 + kb) % 9 - 4 + ((j // g) + 2 * kb) % 3) for kb in range(nkb))
            assert ref[i, j] == want, (i, j)


def test_rowa_doubling_one_row_factor_moves_that_row_only():
    rng = np.random.default_rng(61)
    M, N, K, g = 40, 33, 512, 128
    a8, b8 = _rand_codes(rng, (M, K), 0), _rand_codes(rng, (N, K), 0)
    sa = rng.uniform(0.5, 2.0, size=(M, K // g)).astype(np.float32)
    sb = rng.uniform(0.5, 2.0, size=((N + g - 1) // g, K // g)).astype(np.float32)
    ref = oracle.gemm_ref_rowa(a8, b8, sa, sb, g)
    sa2 = sa.copy()
    sa2[17, 3] *= 2.0
    ref2 = oracle.gemm_ref_rowa(a8, b8, sa2, sb, g)
    other = np.arange(M) != 17
    assert np.array_equal(ref[other], ref2[other])
    for j in range(N):
        P = oracle.segment_partials(a8[17], b8[j], g)[3]
        assert ref2[17, j] - ref[17, j] == pytest.approx(float(sa[17, 3]) * float(sb[j // g, 3]) * P,
                                                          rel=1e-12, abs=1e-300)


def test_rowa_rejects_block_shaped_scales():
    a8 = np.zeros((200, 256), np.uint8)
    b8 = np.zeros((64, 256), np.uint8)
    with pytest.raises(ValueError):
        oracle.gemm_ref_rowa(a8, b8, np.ones((2, 2), np.float32), np.ones((1, 2), np.float32), 128)
