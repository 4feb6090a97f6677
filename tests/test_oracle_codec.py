"""Pins for the oracle's E4M3FN codec (CPU only).

Decode is pinned to torch's CPU float8_e4m3fn -> float32 cast on all 256 codes
and to hand-listed code points; encode to a brute-force nearest-value search
(ties to the even code) and to torch's cast inside the finite range.
"""

import numpy as np
import pytest
import torch

import oracle
from tests import _golden

ALL = np.arange(256, dtype=np.uint8)


def test_decode_matches_torch_all_codes():
    mine = oracle.e4m3_decode(ALL)
    ref = torch.from_numpy(ALL.copy()).view(torch.float8_e4m3fn).to(torch.float32).double().numpy()
    both_nan = np.isnan(mine) & np.isnan(ref)
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    assert np.all(both_nan | (mine == ref))
    # signed zero survives
    assert np.signbit(mine[0x80]) and not np.signbit(mine[0x00])
    assert set(np.flatnonzero(np.isnan(mine)).tolist()) == {0x7F, 0xFF}


def test_decode_hand_points():
    for code, val in _golden.e4m3_points():
        got = oracle.e4m3_decode(np.array([code], np.uint8))[0]
        if np.isnan(val):
            assert np.isnan(got), hex(code)
        else:
            assert got == val and np.signbit(got) == np.signbit(val), (hex(code), got, val)


def _finite_positive_table():
    vals = oracle.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))  # 0x00..0x7E
    return np.arange(0, 0x7F), vals


def _brute_encode(y: np.ndarray) -> np.ndarray:
    """Nearest finite E4M3 value by exhaustive search; ties go to the even code."""
    codes, vals = _finite_positive_table()
    a = np.abs(y.astype(np.float64))
    d = np.abs(a[:, None] - vals[None, :])
    dmin = d.min(axis=1, keepdims=True)
    cand = d == dmin
    # among ties prefer the even code
    even = (codes % 2 == 0)[None, :]
    pick = np.where((cand & even).any(axis=1), np.argmax(cand & even, axis=1), np.argmax(cand, axis=1))
    out = codes[pick].astype(np.uint8)
    out[a >= 448.0] = 0x7E  # saturation
    out |= np.where(np.signbit(y), 0x80, 0).astype(np.uint8)
    return out


def _probe_points():
    codes, vals = _finite_positive_table()
    mids = (vals[1:] + vals[:-1]) / 2.0
    pts = np.concatenate([vals, mids])
    # neighbours of every value and midpoint in float32
    p32 = pts.astype(np.float32)
    near = np.concatenate([p32, np.nextafter(p32, np.float32(np.inf)), np.nextafter(p32, np.float32(0))])
    extra = np.array([448.0, 448.5, 460.0, 463.99, 464.0, 464.01, 479.9, 480.0, 1e6, 3.4e38,
                      1e-30, 2.0 ** -10, 2.0 ** -11], dtype=np.float32)
    pos = np.concatenate([near, extra])
    return np.concatenate([pos, -pos]).astype(np.float32)


def test_encode_brute_force_boundaries():
    y = _probe_points()
    assert np.array_equal(oracle.e4m3_encode(y), _brute_encode(y))


def test_encode_brute_force_random():
    rng = np.random.default_rng(7)
    # log-uniform magnitudes over the whole E4M3 range and beyond, both signs
    mag = np.exp(rng.uniform(np.log(2.0 ** -12), np.log(600.0), size=200_000))
    y = (mag * rng.choice([-1.0, 1.0], size=mag.size)).astype(np.float32)
    assert np.array_equal(oracle.e4m3_encode(y), _brute_encode(y))


def test_encode_matches_torch_in_range():
    rng = np.random.default_rng(11)
    mag = np.exp(rng.uniform(np.log(2.0 ** -12), np.log(448.0), size=1_000_000))
    y = (mag * rng.choice([-1.0, 1.0], size=mag.size)).astype(np.float32)
    y = np.concatenate([y, _probe_points()])
    y = y[np.abs(y) <= 448.0]
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.e4m3_encode(y), ref)


def test_encode_round_trip_all_finite_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = oracle.e4m3_decode(codes).astype(np.float32)
    assert np.array_equal(oracle.e4m3_encode(vals), codes)


@pytest.mark.parametrize("y,code", [(448.0, 0x7E), (1000.0, 0x7E), (-1e30, 0xFE), (463.9, 0x7E),
                                    (0.0, 0x00), (-0.0, 0x80), (-1e-9, 0x80), (2.0 ** -10, 0x00),
                                    (3 * 2.0 ** -11, 0x01), (3 * 2.0 ** -10, 0x02), (5 * 2.0 ** -10, 0x02), (7 * 2.0 ** -10, 0x04), (1.0625, 0x38), (1.1875, 0x3A)])
def test_encode_special_cases(y, code):
    assert oracle.e4m3_encode(np.array([y], np.float32))[0] == code
