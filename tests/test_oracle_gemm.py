"""Pins for the oracle's reference GEMM (CPU only).

ref[i,j] = sum_kb sa[i/g,kb]*sb[j/g,kb] * P[i,j,kb], P the exact FP64 segment
sums (DeepGEMM实战 §2.2 scales restored in accumulation, §3.2 segments summed
separately then added, §3.3/§4.2 NT layout A[M,K], B[N,K]).

Pinned by: a hand-worked example; exact rational brute force; integer
(int64) recomputation of every segment partial; numpy's float64 matmul when
all scales are 1; closed forms (all-ones, identity) with power-of-two block
scales; the scale-doubling invariants; and mutation power, i.e. each of the
ways the pages say results go wrong (§5.2) makes the parity check fail.
"""

from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from tests import _common, _golden


def _rand_codes(rng, shape):
    c = rng.integers(0, 256, size=shape, dtype=np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x38  # no NaN codes
    return c


def _int_decode(codes):
    """Independent integer decode: value * 2^9 as int64 (exact for E4M3FN)."""
    c = codes.astype(np.int64)
    s = np.where(c & 0x80, -1, 1)
    e = (c >> 3) & 0xF
    m = c & 7
    mag = np.where(e == 0, m, (8 + m) << np.maximum(e - 1, 0))
    return s * mag


def test_worked_example():
    w = _golden.worked_gemm()
    ref = oracle.gemm_ref(w["a8"], w["b8"], w["sa"], w["sb"], w["g"])
    assert np.array_equal(ref, w["ref"])
    bf = _common.bf16_bits_to_f64(_common.f32_to_bf16_bits(ref.astype(np.float32)))
    assert np.array_equal(bf, w["bf16"])


@pytest.mark.parametrize("M,N,K,g", [(1, 1, 64, 64), (3, 5, 128, 64), (20, 17, 256, 128), (13, 20, 128, 128),
                                     (70, 3, 128, 64)])
def test_brute_force_exact_rationals(M, N, K, g):
    rng = np.random.default_rng(M * 100 + N)
    a8, b8 = _rand_codes(rng, (M, K)), _rand_codes(rng, (N, K))
    sa = rng.uniform(0.01, 3.0, size=((M + g - 1) // g, K // g)).astype(np.float32)
    sb = rng.uniform(0.01, 3.0, size=((N + g - 1) // g, K // g)).astype(np.float32)
    ref = oracle.gemm_ref(a8, b8, sa, sb, g)
    dec = {c: Fraction(float(v)) for c, v in enumerate(oracle.e4m3_decode(np.arange(256, dtype=np.uint8)))
           if (c & 0x7F) != 0x7F}
    # decode again by hand from the bit fields so this check does not lean on the oracle codec
    for c in dec:
        e, m = (c >> 3) & 15, c & 7
        mag = Fraction(m, 8) * Fraction(1, 64) if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
        assert dec[c] == (-mag if c & 0x80 else mag)
    nkb = K // g
    for i in range(M):
        for j in range(N):
            exact = Fraction(0)
            mag = Fraction(0)
            for kb in range(nkb):
                p = sum(dec[int(a8[i, k])] * dec[int(b8[j, k])] for k in range(kb * g, kb * g + g))
                term = Fraction(float(sa[i // g, kb])) * Fraction(float(sb[j // g, kb])) * p
                exact += term
                mag += abs(term)
            # the oracle rounds once per segment (scale multiply) and once per add:
            # at most 2*nkb units of 2^-53 relative to the sum of |terms|
            tol = float(mag) * 2 * nkb * 2.0 ** -53
            assert abs(Fraction(ref[i, j]) - exact) <= Fraction(tol), (i, j)


def test_segment_partials_exact_int64():
    rng = np.random.default_rng(3)
    K, g = 16384, 64  # the longest K of the workloads, all codes random (incl. +-448)
    a = _rand_codes(rng, (4, K))
    b = _rand_codes(rng, (4, K))
    ia, ib = _int_decode(a), _int_decode(b)
    for i in range(4):
        P = oracle.segment_partials(a[i], b[i], g)
        Pint = (ia[i] * ib[i]).reshape(-1, g).sum(axis=1)  # exact integers, units of 2^-18
        assert np.array_equal(P, Pint.astype(np.float64) * 2.0 ** -18)
        # the full-K unscaled dot is exact too
        assert np.sum(Pint) == int(np.sum(Pint))


def test_scales_one_equals_float64_matmul():
    rng = np.random.default_rng(5)
    M, N, K, g = 77, 130, 512, 128
    a8, b8 = _rand_codes(rng, (M, K)), _rand_codes(rng, (N, K))
    sa = np.ones(((M + g - 1) // g, K // g), np.float32)
    sb = np.ones(((N + g - 1) // g, K // g), np.float32)
    ref = oracle.gemm_ref(a8, b8, sa, sb, g)
    A = _int_decode(a8).astype(np.float64) * 2.0 ** -9
    B = _int_decode(b8).astype(np.float64) * 2.0 ** -9
    assert np.array_equal(ref, A @ B.T)  # every partial sum is exact, so bitwise


def _pow2_scales(nrb, nkb, f):
    s = np.empty((nrb, nkb), np.float32)
    for r in range(nrb):
        for k in range(nkb):
            s[r, k] = 2.0 ** f(r, k)
    return s


@pytest.mark.parametrize("M,N,K,g", [(256, 384, 512, 128), (200, 130, 320, 64)])
def test_closed_form_all_ones(M, N, K, g):
    a8 = np.full((M, K), 0x38, np.uint8)
    b8 = np.full((N, K), 0x38, np.uint8)
    sa = _pow2_scales((M + g - 1) // g, K // g, lambda mb, kb: mb - kb)
    sb = _pow2_scales((N + g - 1) // g, K // g, lambda nb, kb: (2 * nb + kb) % 3)
    ref = oracle.gemm_ref(a8, b8, sa, sb, g)
    for i in range(M):
        for j in range(N):
            want = g * sum(2.0 ** ((i // g - kb) + (2 * (j // g) + kb) % 3) for kb in range(K // g))
            assert ref[i, j] == want


def test_closed_form_identity():
    M = K = 256
    N, g = 192, 64
    rng = np.random.default_rng(9)
    a8 = np.zeros((M, K), np.uint8)
    a8[np.arange(M), np.arange(K)] = 0x38
    b8 = _rand_codes(rng, (N, K))
    sa = _pow2_scales(M // g, K // g, lambda mb, kb: (mb * 3 + kb) % 5 - 2)
    sb = _pow2_scales(N // g, K // g, lambda nb, kb: (nb + 2 * kb) % 4 - 1)
    ref = oracle.gemm_ref(a8, b8, sa, sb, g)
    Bv = _int_decode(b8).astype(np.float64) * 2.0 ** -9
    for i in range(M):
        for j in range(N):
            assert ref[i, j] == sa[i // g, i // g] * sb[j // g, i // g] * Bv[j, i]


def test_invariant_double_one_block_scale():
    rng = np.random.default_rng(13)
    M, N, K, g = 300, 200, 512, 128
    a8, b8 = _rand_codes(rng, (M, K)), _rand_codes(rng, (N, K))
    sa = rng.uniform(0.1, 2, size=((M + g - 1) // g, K // g)).astype(np.float32)
    sb = rng.uniform(0.1, 2, size=((N + g - 1) // g, K // g)).astype(np.float32)
    ref = oracle.gemm_ref(a8, b8, sa, sb, g)
    mb, kb = 1, 2
    sa2 = sa.copy()
    sa2[mb, kb] *= 2
    ref2 = oracle.gemm_ref(a8, b8, sa2, sb, g)
    rows = np.arange(M) // g == mb
    assert np.array_equal(ref2[~rows], ref[~rows])  # other row blocks bitwise unchanged
    for i in np.flatnonzero(rows)[:40]:
        for j in range(0, N, 7):
            P = oracle.segment_partials(a8[i], b8[j], g)
            delta = float(sa[mb, kb]) * float(sb[j // g, kb]) * P[kb]
            scale = np.sum(np.abs(P) * sa2[mb] * sb[j // g]) + abs(delta)
            assert abs((ref2[i, j] - ref[i, j]) - delta) <= 8 * 2.0 ** -52 * scale


def test_invariant_all_sa_times_two_doubles_output():
    rng = np.random.default_rng(17)
    M, N, K, g = 130, 70, 256, 64
    a8, b8 = _rand_codes(rng, (M, K)), _rand_codes(rng, (N, K))
    sa = rng.uniform(0.1, 2, size=((M + g - 1) // g, K // g)).astype(np.float32)
    sb = rng.uniform(0.1, 2, size=((N + g - 1) // g, K // g)).astype(np.float32)
    ref = oracle.gemm_ref(a8, b8, sa, sb, g)
    assert np.array_equal(oracle.gemm_ref(a8, b8, sa * np.float32(2), sb, g), 2 * ref)


# ---- mutation power: the parity check must reject each wrong variant -------------

_CACHE = {}


def _workload(c):
    """Quantised inputs of workload c and sampled output coordinates."""
    if c not in _CACHE:
        w = synth.WORKLOADS[c]
        g = w["g"]
        a8, sa = oracle.quantize_blocks(synth.make_a(c), g)
        b8, sb = oracle.quantize_blocks(synth.make_b(c), g)
        rows = _common.sample_indices(w["M"], 48, seed=c)
        cols = _common.sample_indices(w["N"], 48, seed=c + 50)
        ref = oracle.gemm_ref(a8, b8, sa, sb, g, rows, cols)
        _CACHE[c] = (w, a8, b8, sa, sb, rows, cols, ref)
    return _CACHE[c]


def _mutations(w, a8, b8, sa, sb):
    g, N, K = w["g"], w["N"], w["K"]
    yield "divide", (a8, b8, (1 / sa).astype(np.float32), (1 / sb).astype(np.float32))
    yield "B_transposed", (a8, np.ascontiguousarray(b8.reshape(K, N).T), sa, sb)
    yield "per_tensor_scale", (a8, b8, np.full_like(sa, sa.max()), np.full_like(sb, sb.max()))
    yield "scale_kb_off_by_one", (a8, b8, np.roll(sa, 1, axis=1), np.roll(sb, 1, axis=1))
    yield "no_promotion", (a8, b8, np.repeat(sa[:, :1], sa.shape[1], axis=1),
                           np.repeat(sb[:, :1], sb.shape[1], axis=1))


@pytest.mark.slow
@pytest.mark.parametrize("c", [2, 3, 4, 5])
def test_mutations_fail_parity(c):
    w, a8, b8, sa, sb, rows, cols, ref = _workload(c)
    for name, (ma, mb, msa, msb) in _mutations(w, a8, b8, sa, sb):
        got = oracle.gemm_ref(ma, mb, msa, msb, w["g"], rows, cols)
        ok, _ = _common.within_tolerance(got, ref)
        assert not ok.all(), "mutation %s passed the parity check on workload %d" % (name, c)
