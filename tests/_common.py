"""Helpers shared by the tests: the parity tolerance, BF16 rounding, sampling."""

from __future__ import annotations

import contextlib
import os

import numpy as np

# Table ids of the split-K class (64x64 tiles) for K segments of 128 and 64.
SPLIT_TILE = {128: 2, 256: 2, 64: 3}


@contextlib.contextmanager
def forced_tile(kernel_id: int):
    """Inside, every call of a matching granularity runs table entry
    kernel_id (DG_FORCE_TILE, which the library reads at each call)."""
    old = os.environ.get("DG_FORCE_TILE")
    os.environ["DG_FORCE_TILE"] = str(kernel_id)
    try:
        yield
    finally:
        if old is None:
            del os.environ["DG_FORCE_TILE"]
        else:
            os.environ["DG_FORCE_TILE"] = old


def forced_split(g: int):
    """Inside, every call runs the split-K class, splitting K over workgroups
    when a workspace is given, whatever the shape. The plan itself splits
    only long K ranges (16384 and up); this reaches the split path on shapes
    the oracle finishes in moments."""
    return forced_tile(SPLIT_TILE[g])


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


def fp32_promotion_emulation(a_dec, b_dec, sa, sb, g: int, rows, cols) -> np.ndarray:
    """What an ideal FP32 implementation of the method gives on outputs rows x
    cols: each g-segment partial exact (a float64 product of decoded operands;
    every such sum is exact in float64) then rounded to FP32, the factor
    product sa*sb rounded to FP32, and acc = fma(P, s, acc) in FP32 over the
    segments in order. The single rounding of the FMA is emulated in float64
    (P*s is exact there; the add then rounds once in float64 and once to FP32).

    Diagnostic only: it bounds how close to the FP64 reference an FP32
    accumulator can be expected to stay, which is what the GPU's share of
    outputs within one BF16 ulp is compared with."""
    rows = np.asarray(rows)
    cols = np.asarray(cols)
    A = np.asarray(a_dec, np.float64)[rows]
    B = np.asarray(b_dec, np.float64)[cols]
    K = A.shape[1]
    acc = np.zeros((rows.size, cols.size), np.float32)
    for kb in range(K // g):
        seg = slice(kb * g, (kb + 1) * g)
        P = (A[:, seg] @ B[:, seg].T).astype(np.float32)
        s = (np.asarray(sa, np.float32)[rows // g, kb][:, None] * np.asarray(sb, np.float32)[cols // g, kb][None, :])
        acc = (P.astype(np.float64) * s.astype(np.float64) + acc.astype(np.float64)).astype(np.float32)
    return acc.astype(np.float64)


def within_one_ulp(got, ref) -> float:
    """Share of outputs within one BF16 ulp of bf16(ref) (ulp = |bf16(ref)| * 2^-8)."""
    bf_ref = bf16_bits_to_f64(f32_to_bf16_bits(np.asarray(ref, np.float64).astype(np.float32)))
    ulp = np.abs(bf_ref) * 2.0 ** -8 + 1e-30
    return float(np.mean(np.abs(np.asarray(got, np.float64) - bf_ref) <= ulp))
