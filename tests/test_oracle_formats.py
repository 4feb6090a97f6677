"""Pins for the oracle's E5M2 codec, its format-generic quantiser and
reference GEMM, and block granularity g = 256 (CPU only).

The pages name E4M3 and E5M2 as the two FP8 input formats (DeepGEMM实战
§2.2) and 64, 128 and 256 as block granularities (§3.1). E5M2 is the OCP
format torch.float8_e5m2 implements.

Pinned by: torch's CPU float8_e5m2 cast on all 256 codes (decode) and inside
the finite range (encode); a brute-force nearest-value search with ties to the
even code; hand-derived code points; exact rational brute force for mixed
formats and g = 256; numpy's float64 matmul where every sum is exact; closed
forms with power-of-two scales; and the scale-doubling invariant at g = 256.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

ALL = np.arange(256, dtype=np.uint8)


# ---------------------------------------------------------------- E5M2 codec

def test_e5m2_decode_matches_torch_all_codes():
    mine = oracle.e5m2_decode(ALL)
    ref = torch.from_numpy(ALL.copy()).view(torch.float8_e5m2).to(torch.float32).double().numpy()
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    fin = ~np.isnan(mine)
    assert np.array_equal(mine[fin], ref[fin])
    assert np.signbit(mine[0x80]) and not np.signbit(mine[0x00])
    assert mine[0x7C] == np.inf and mine[0xFC] == -np.inf
    assert set(np.flatnonzero(np.isnan(mine)).tolist()) == {0x7D, 0x7E, 0x7F, 0xFD, 0xFE, 0xFF}


@pytest.mark.parametrize("code,val", [(0x01, 2.0 ** -16), (0x03, 3 * 2.0 ** -16), (0x04, 2.0 ** -14),
                                      (0x3C, 1.0), (0x3D, 1.25), (0x3F, 1.75), (0x40, 2.0),
                                      (0x7B, 57344.0), (0x7A, 49152.0), (0xBC, -1.0), (0x00, 0.0)])
def test_e5m2_decode_hand_points(code, val):
    # (1 + m/4) * 2^(e-15) for e > 0, m/4 * 2^-14 for e == 0, worked by hand
    assert oracle.e5m2_decode(np.array([code], np.uint8))[0] == val


def _e5m2_finite_positive():
    codes = np.arange(0, 0x7C)  # 0x00 .. 0x7B
    return codes, oracle.e5m2_decode(codes.astype(np.uint8))


def _brute_e5m2(y):
    codes, vals = _e5m2_finite_positive()
    a = np.abs(y.astype(np.float64))
    d = np.abs(a[:, None] - vals[None, :])
    cand = d == d.min(axis=1, keepdims=True)
    even = (codes % 2 == 0)[None, :]
    pick = np.where((cand & even).any(axis=1), np.argmax(cand & even, axis=1), np.argmax(cand, axis=1))
    out = codes[pick].astype(np.uint8)
    out[a >= 57344.0] = 0x7B
    out |= np.where(np.signbit(y), 0x80, 0).astype(np.uint8)
    return out


def _e5m2_probe_points():
    _, vals = _e5m2_finite_positive()
    mids = (vals[1:] + vals[:-1]) / 2.0
    p32 = np.concatenate([vals, mids]).astype(np.float32)
    near = np.concatenate([p32, np.nextafter(p32, np.float32(np.inf)), np.nextafter(p32, np.float32(0))])
    extra = np.array([57344.0, 59392.0, 61439.0, 61440.0, 1e6, 3.4e38, 1e-30, 2.0 ** -17, 3 * 2.0 ** -18],
                     dtype=np.float32)
    pos = np.concatenate([near, extra])
    return np.concatenate([pos, -pos]).astype(np.float32)


def test_e5m2_encode_brute_force():
    rng = np.random.default_rng(21)
    mag = np.exp(rng.uniform(np.log(2.0 ** -18), np.log(70000.0), size=100_000))
    y = np.concatenate([_e5m2_probe_points(), (mag * rng.choice([-1.0, 1.0], size=mag.size)).astype(np.float32)])
    assert np.array_equal(oracle.e5m2_encode(y), _brute_e5m2(y))


def test_e5m2_encode_matches_torch_in_range():
    rng = np.random.default_rng(23)
    mag = np.exp(rng.uniform(np.log(2.0 ** -18), np.log(57344.0), size=1_000_000))
    y = np.concatenate([(mag * rng.choice([-1.0, 1.0], size=mag.size)).astype(np.float32), _e5m2_probe_points()])
    y = y[np.abs(y) <= 57344.0]
    ref = torch.from_numpy(y).to(torch.float8_e5m2).view(torch.uint8).numpy()
    assert np.array_equal(oracle.e5m2_encode(y), ref)


def test_e5m2_round_trip_all_finite_codes():
    codes = np.array([c for c in range(256) if (c & 0x7F) < 0x7C], dtype=np.uint8)
    vals = oracle.e5m2_decode(codes).astype(np.float32)
    assert np.array_equal(oracle.e5m2_encode(vals), codes)


# ---------------------------------------------------------- quantiser

@pytest.mark.parametrize("rows,cols,g", [(300, 256, 128), (65, 192, 64), (513, 512, 256), (1, 256, 256)])
def test_quantize_e4m3_is_the_plain_quantiser(rows, cols, g):
    rng = np.random.default_rng(rows + cols)
    x = (rng.standard_normal((rows, cols)) * np.exp(rng.uniform(-6, 6, size=(rows, 1)))).astype(np.float32)
    q0, s0 = oracle.quantize_blocks(x, g)
    q1, s1 = oracle.quantize_blocks_fmt(x, g, oracle.E4M3)
    assert np.array_equal(q0, q1) and np.array_equal(s0, s1)


@pytest.mark.parametrize("rows,cols,g", [(300, 256, 128), (65, 192, 64), (513, 512, 256)])
def test_quantize_e5m2_by_definition(rows, cols, g):
    rng = np.random.default_rng(rows * 3 + cols)
    x = (rng.standard_normal((rows, cols)) * np.exp(rng.uniform(-8, 8, size=(rows, 1)))).astype(np.float32)
    x[0, :g] = 0.0
    q, s = oracle.quantize_blocks_fmt(x, g, oracle.E5M2)
    assert s.shape == ((rows + g - 1) // g, cols // g)
    for rb in range(s.shape[0]):
        for cb in range(s.shape[1]):
            rs, cs = slice(rb * g, min(rb * g + g, rows)), slice(cb * g, cb * g + g)
            blk = x[rs, cs]
            amax = np.float32(np.max(np.abs(blk)))
            scale = np.float32(amax / np.float32(57344.0)) if amax > 0 else np.float32(1.0)
            assert s[rb, cb] == scale
            y = (blk / scale).astype(np.float32)  # <= 57344 up to one rounding, which torch also rounds down
            ref = torch.from_numpy(np.ascontiguousarray(y)).to(torch.float8_e5m2).view(torch.uint8).numpy()
            assert np.array_equal(q[rs, cs], ref)


# ---------------------------------------------------------- reference GEMM

def _rand_e4m3(rng, shape):
    c = rng.integers(0, 256, size=shape, dtype=np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x38
    return c


def _rand_e5m2(rng, shape):
    c = rng.integers(0, 256, size=shape, dtype=np.uint8)
    c[(c & 0x7F) >= 0x7C] = 0x3C  # no infinity or NaN codes
    return c


def _frac_e4m3(c):
    e, m = (c >> 3) & 15, c & 7
    mag = Fraction(m, 8) * Fraction(1, 64) if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
    return -mag if c & 0x80 else mag


def _frac_e5m2(c):
    e, m = (c >> 2) & 31, c & 3
    mag = Fraction(m, 4) * Fraction(1, 2 ** 14) if e == 0 else (1 + Fraction(m, 4)) * Fraction(2) ** (e - 15)
    return -mag if c & 0x80 else mag


def test_ref_fmt_e4m3_is_the_plain_reference():
    rng = np.random.default_rng(31)
    M, N, K, g = 37, 50, 512, 128
    a8, b8 = _rand_e4m3(rng, (M, K)), _rand_e4m3(rng, (N, K))
    sa = rng.uniform(0.01, 3.0, size=((M + g - 1) // g, K // g)).astype(np.float32)
    sb = rng.uniform(0.01, 3.0, size=((N + g - 1) // g, K // g)).astype(np.float32)
    assert np.array_equal(oracle.gemm_ref(a8, b8, sa, sb, g), oracle.gemm_ref_fmt(a8, b8, sa, sb, g, 0, 0))


@pytest.mark.parametrize("fa,fb,M,N,K,g", [(1, 1, 3, 4, 128, 64), (0, 1, 5, 3, 128, 64), (1, 0, 4, 4, 512, 256),
                                          (0, 0, 3, 5, 512, 256), (1, 1, 2, 3, 256, 256)])
def test_ref_fmt_brute_force_exact_rationals(fa, fb, M, N, K, g):
    rng = np.random.default_rng(fa * 10 + fb + K)
    a8 = _rand_e5m2(rng, (M, K)) if fa else _rand_e4m3(rng, (M, K))
    b8 = _rand_e5m2(rng, (N, K)) if fb else _rand_e4m3(rng, (N, K))
    sa = rng.uniform(0.01, 3.0, size=((M + g - 1) // g, K // g)).astype(np.float32)
    sb = rng.uniform(0.01, 3.0, size=((N + g - 1) // g, K // g)).astype(np.float32)
    ref = oracle.gemm_ref_fmt(a8, b8, sa, sb, g, fa, fb)
    da = _frac_e5m2 if fa else _frac_e4m3
    db = _frac_e5m2 if fb else _frac_e4m3
    nkb = K // g
    for i in range(M):
        for j in range(N):
            exact, mag = Fraction(0), Fraction(0)
            for kb in range(nkb):
                terms = [da(int(a8[i, k])) * db(int(b8[j, k])) for k in range(kb * g, kb * g + g)]
                s = Fraction(float(sa[i // g, kb])) * Fraction(float(sb[j // g, kb]))
                exact += s * sum(terms)
                mag += s * sum(abs(t) for t in terms)
            # FP64 segment sums (g adds) plus one multiply and one add per segment
            tol = float(mag) * (g + 2) * nkb * 2.0 ** -53
            assert abs(Fraction(ref[i, j]) - exact) <= Fraction(tol), (i, j)


def test_ref_fmt_scales_one_equals_float64_matmul():
    # E5M2 codes with exponent fields 10..20 (multiples of 2^-7 below 2^6) times
    # E4M3 codes (multiples of 2^-9 below 2^9): every product is a multiple of
    # 2^-16 below 2^15, so every sum of 512 of them is exact in FP64.
    rng = np.random.default_rng(41)
    M, N, K, g = 60, 70, 512, 256
    e = rng.integers(10, 21, size=(M, K))
    a8 = ((rng.integers(0, 2, size=(M, K)) << 7) | (e << 2) | rng.integers(0, 4, size=(M, K))).astype(np.uint8)
    b8 = _rand_e4m3(rng, (N, K))
    sa = np.ones(((M + g - 1) // g, K // g), np.float32)
    sb = np.ones(((N + g - 1) // g, K // g), np.float32)
    ref = oracle.gemm_ref_fmt(a8, b8, sa, sb, g, 1, 0)
    A = np.array([[float(_frac_e5m2(int(c))) for c in row] for row in a8])
    B = np.array([[float(_frac_e4m3(int(c))) for c in row] for row in b8])
    assert np.array_equal(ref, A @ B.T)


def _pow2_scales(nrb, nkb, f):
    s = np.empty((nrb, nkb), np.float32)
    for r in range(nrb):
        for k in range(nkb):
            s[r, k] = 2.0 ** f(r, k)
    return s


@pytest.mark.parametrize("fa,fb,M,N,K,g", [(1, 1, 300, 520, 1024, 256), (0, 1, 200, 130, 384, 128)])
def test_ref_fmt_closed_form_all_ones(fa, fb, M, N, K, g):
    one = {0: 0x38, 1: 0x3C}  # 1.0 in E4M3 and in E5M2
    a8 = np.full((M, K), one[fa], np.uint8)
    b8 = np.full((N, K), one[fb], np.uint8)
    sa = _pow2_scales((M + g - 1) // g, K // g, lambda mb, kb: mb - kb)
    sb = _pow2_scales((N + g - 1) // g, K // g, lambda nb, kb: (2 * nb + kb) % 3)
    ref = oracle.gemm_ref_fmt(a8, b8, sa, sb, g, fa, fb)
    for i in range(0, M, 7):
        for j in range(0, N, 11):
            want = g * sum(2.0 ** ((i // g - kb) + (2 * (j // g) + kb) % 3) for kb in range(K // g))
            assert ref[i, j] == want


def test_ref_g256_invariant_double_one_block_scale():
    rng = np.random.default_rng(43)
    M, N, K, g = 520, 40, 768, 256
    a8, b8 = _rand_e4m3(rng, (M, K)), _rand_e4m3(rng, (N, K))
    sa = _pow2_scales((M + g - 1) // g, K // g, lambda mb, kb: (mb + kb) % 3 - 1)
    sb = _pow2_scales((N + g - 1) // g, K // g, lambda nb, kb: kb % 2)
    ref = oracle.gemm_ref_fmt(a8, b8, sa, sb, g, 0, 0)
    sa2 = sa.copy()
    sa2[1, 2] *= 2.0  # rows 256..511, K block 2
    ref2 = oracle.gemm_ref_fmt(a8, b8, sa2, sb, g, 0, 0)
    rows = np.arange(M)
    other = (rows // g) != 1
    assert np.array_equal(ref[other], ref2[other])
    for i in (256, 300, 511):
        for j in (0, 17, 39):
            P = oracle.segment_partials(a8[i], b8[j], g)[2]
            assert ref2[i, j] - ref[i, j] == pytest.approx(float(sa[1, 2]) * float(sb[j // g, 2]) * P, rel=1e-12)
