"""Pins for the oracle's reference GEMM over the four operand layouts (CPU only).

DeepGEMM实战 §3.3: A and B may each be stored transposed; the product does not
change. Layout codes: bit 1 = A stored [K, M], bit 0 = B stored [K, N] (NT 0,
NN 1, TT 2, TN 3). The scales keep their logical shapes.

Pinned by: numpy's transpose of the stored operands back to the NT layout and
the NT reference (bitwise: the same sums in the same order); exact rational
brute force through each layout; permutation-matrix closed forms that read
one stored element per output, which a transposed index gets wrong.
"""

from fractions import Fraction

import numpy as np
import pytest

import oracle

LAYOUTS = [oracle.NT, oracle.NN, oracle.TT, oracle.TN]


def _codes(rng, shape, fmt=0):
    c = rng.integers(0, 256, size=shape, dtype=np.uint8)
    if fmt:
        c[(c & 0x7F) >= 0x7C] = 0x3C
    else:
        c[(c & 0x7F) == 0x7F] = 0x38
    return c


def _store(a8, b8, layout):
    """Logical A [M,K], B [N,K] -> the stored arrays of the layout."""
    sa_ = np.ascontiguousarray(a8.T) if layout & 2 else a8
    sb_ = np.ascontiguousarray(b8.T) if layout & 1 else b8
    return sa_, sb_


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("M,N,K,g,fa,fb", [(70, 90, 512, 128, 0, 0), (33, 130, 384, 64, 1, 0), (40, 20, 512, 256, 0, 1)])
def test_layout_equals_nt_reference_on_transposed_copies(layout, M, N, K, g, fa, fb):
    rng = np.random.default_rng(layout * 100 + M + K)
    a8, b8 = _codes(rng, (M, K), fa), _codes(rng, (N, K), fb)
    sa = rng.uniform(0.01, 3.0, size=((M + g - 1) // g, K // g)).astype(np.float32)
    sb = rng.uniform(0.01, 3.0, size=((N + g - 1) // g, K // g)).astype(np.float32)
    a_st, b_st = _store(a8, b8, layout)
    rows = np.array([0, 1, M // 2, M - 1])
    assert np.array_equal(oracle.gemm_ref_layout(a_st, b_st, sa, sb, g, layout, M, N, K, fa, fb, rows=rows),
                          oracle.gemm_ref_fmt(a8, b8, sa, sb, g, fa, fb, rows=rows))


def _frac(c):
    e, m = (c >> 3) & 15, c & 7
    mag = Fraction(m, 8) * Fraction(1, 64) if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
    return -mag if c & 0x80 else mag


@pytest.mark.parametrize("layout", LAYOUTS)
def test_layout_brute_force_exact_rationals(layout):
    rng = np.random.default_rng(500 + layout)
    M, N, K, g = 5, 3, 128, 64
    a8, b8 = _codes(rng, (M, K)), _codes(rng, (N, K))
    sa = rng.uniform(0.1, 2.0, size=(1, K // g)).astype(np.float32)
    sb = rng.uniform(0.1, 2.0, size=(1, K // g)).astype(np.float32)
    a_st, b_st = _store(a8, b8, layout)
    ref = oracle.gemm_ref_layout(a_st, b_st, sa, sb, g, layout, M, N, K)
    for i in range(M):
        for j in range(N):
            exact, mag = Fraction(0), Fraction(0)
            for kb in range(K // g):
                # read each element from the stored array by the layout's own definition
                terms = [_frac(int(a_st[k, i] if layout & 2 else a_st[i, k])) *
                         _frac(int(b_st[k, j] if layout & 1 else b_st[j, k])) for k in range(kb * g, kb * g + g)]
                s = Fraction(float(sa[0, kb])) * Fraction(float(sb[0, kb]))
                exact += s * sum(terms)
                mag += s * sum(abs(t) for t in terms)
            assert abs(Fraction(ref[i, j]) - exact) <= Fraction(float(mag) * (g + 2) * 2 * 2.0 ** -53), (i, j)


@pytest.mark.parametrize("layout", LAYOUTS)
def test_layout_permutation_closed_form(layout):
    # A[i,k] = 1 exactly where k = p(i), B arbitrary: C[i,j] = sa*sb * B[j, p(i)]
    rng = np.random.default_rng(700 + layout)
    M, N, K, g = 96, 80, 128, 64
    p = rng.permutation(K)[:M]
    a8 = np.zeros((M, K), np.uint8)
    a8[np.arange(M), p] = 0x38
    b8 = _codes(rng, (N, K))
    sa = np.array([[2.0 ** (mb - kb) for kb in range(K // g)] for mb in range((M + g - 1) // g)], np.float32)
    sb = np.array([[2.0 ** (kb - nb) for kb in range(K // g)] for nb in range((N + g - 1) // g)], np.float32)
    a_st, b_st = _store(a8, b8, layout)
    ref = oracle.gemm_ref_layout(a_st, b_st, sa, sb, g, layout, M, N, K)
    bval = oracle.e4m3_decode(b8)
    for i in range(M):
        kb = p[i] // g
        want = float(sa[i // g, kb]) * np.array([float(sb[j // g, kb]) for j in range(N)]) * bval[:, p[i]]
        assert np.array_equal(ref[i], want), i


def test_layout_rejects_wrong_storage_shape():
    a = np.zeros((64, 256), np.uint8)
    b = np.zeros((32, 256), np.uint8)
    s1 = np.ones((1, 2), np.float32)
    with pytest.raises(ValueError):
        oracle.gemm_ref_layout(a, b, s1, s1, 128, oracle.TN, 64, 32, 256)  # TN wants A [K,M], B [K,N]
