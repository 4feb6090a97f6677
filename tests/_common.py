"""Helpers shared by the tests: the parity tolerance, BF16 rounding, sampling."""

from __future__ import annotations

import numpy as np


def within_tolerance(got, ref, rms=None):
    """Parity bar: |got - ref| <= 1e-2*|ref| + 1e-2*rms(ref), elementwise.

    rms is taken over ``ref`` (the whole output, or the sampled outputs when only
    a sample is computed). Returns (ok_mask, rms).
    """
    ref = np.asarray(ref, dtype=np.float64)
    got = np.asarray(got, dtype=np.float64)
    if rms is None:
        rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    ok = np.abs(got - ref) <= 1e-2 * np.abs(ref) + 1e-2 * rms
    return ok, rms


def f32_to_bf16_bits(x) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f64(bits) -> np.ndarray:
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def sample_indices(n: int, count: int, seed: int) -> np.ndarray:
    """Sorted distinct indices in [0, n): the first and last 8, plus random ones."""
    rng = np.random.default_rng(seed)
    edge = list(range(min(8, n))) + list(range(max(0, n - 8), n))
    rest = rng.choice(n, size=min(n, count), replace=False).tolist()
    return np.array(sorted(set(edge + rest)), dtype=np.int64)
