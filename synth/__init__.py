"""Seeded synthetic inputs shared by the tests, the oracle and the benchmark.

This module holds random numbers only: it draws FP32 matrices from a seed and
knows the workload shapes and value distributions. It holds none of the GEMM's
arithmetic (no FP8 codec, no block scales, no quantisation) and imports neither
the oracle nor the HIP library.

Generator: SplitMix64 used as a counter-based generator. For a stream key s
and element index i (0-based) the 64-bit word is mix(s + (i+1)*GAMMA), where
GAMMA = 0x9E3779B97F4A7C15 and mix is SplitMix64's finaliser
(xor-shift 30, *0xBF58476D1CE4E5B9, xor-shift 27, *0x94D049BB133111EB,
xor-shift 31). The stream key is mix(seed*GAMMA + stream), so distinct
(seed, stream) pairs give unrelated sequences. Uniforms are
u = ((word >> 11) + 0.5) * 2^-53, never 0 or 1. Normals come from Box-Muller
in float64 on consecutive uniform pairs (2p, 2p+1) -> (r cos t, r sin t).
Every value is cast to float32 last.

Workloads (the five shapes the GEMM is measured and checked on; seeds
2c+1000 for A and 2c+1001 for B of workload c):

  1  M=N=K=256,            g=128  A ~ N(0,1),  B ~ N(0,0.02)
  2  M=64, N=4096, K=7168, g=128  A ~ N(0,1) with 1% of its K columns x20,
                                  B ~ N(0,0.02)                (small-M decode)
  3  M=4096,N=7168,K=2048, g=128  A ~ N(0,1) * r_i, r_i = 10^U(-1,1) per row,
                                  B ~ N(0,0.02)                (prefill FFN)
  4  M=N=K=8192,           g=128  A, B ~ N(0,1)                (large square)
  5  M=2000,N=4000,K=16384,g=64   A ~ Student-t(3), B ~ N(0,0.02) (long K, ragged)

N(0,0.02) is read as standard deviation 0.02. The outlier columns of
workload 2 are round(0.01*K) = 72 distinct columns chosen uniformly without
replacement; every row of those columns is multiplied by 20. Student-t(3) is
Z / sqrt(chi2_3 / 3) with chi2_3 the sum of three squared standard normals.
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

GAMMA = 0x9E3779B97F4A7C15
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_MASK = (1 << 64) - 1
_CHUNK = 1 << 20

# Stream numbers within one seed.
S_MAIN, S_CHI1, S_CHI2, S_CHI3, S_ROWSCALE, S_OUTLIER = range(6)


def _mix_scalar(z: int) -> int:
    z &= _MASK
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK
    return z ^ (z >> 31)


def _mix(z: np.ndarray) -> np.ndarray:
    """SplitMix64 finaliser, in place on a uint64 array."""
    t = np.empty_like(z)
    with np.errstate(over="ignore"):
        np.right_shift(z, np.uint64(30), out=t)
        z ^= t
        z *= _M1
        np.right_shift(z, np.uint64(27), out=t)
        z ^= t
        z *= _M2
        np.right_shift(z, np.uint64(31), out=t)
        z ^= t
    return z


def stream_key(seed: int, stream: int) -> int:
    return _mix_scalar((seed * GAMMA + stream) & _MASK)


def words(seed: int, stream: int, start: int, n: int) -> np.ndarray:
    """64-bit words i = start .. start+n-1 of stream (seed, stream)."""
    z = np.arange(start + 1, start + n + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z *= np.uint64(GAMMA)
        z += np.uint64(stream_key(seed, stream))
    return _mix(z)


def uniform(seed: int, stream: int, n: int, start: int = 0) -> np.ndarray:
    """n float64 uniforms in (0,1)."""
    w = words(seed, stream, start, n)
    w >>= np.uint64(11)
    u = w.astype(np.float64)
    u += 0.5
    u *= 2.0 ** -53
    return u


def _normal_chunk(seed: int, stream: int, p0: int, p1: int, n: int, out: np.ndarray) -> None:
    u = uniform(seed, stream, 2 * (p1 - p0), start=2 * p0)
    r = np.sqrt(-2.0 * np.log(u[0::2]))
    t = 2.0 * np.pi * u[1::2]
    z = np.empty(2 * (p1 - p0), dtype=np.float64)
    z[0::2] = r * np.cos(t)
    z[1::2] = r * np.sin(t)
    lo, hi = 2 * p0, min(n, 2 * p1)
    out[lo:hi] = z[: hi - lo]


def std_normal(seed: int, stream: int, n: int) -> np.ndarray:
    """n float64 standard normals (Box-Muller on uniform pairs).

    Chunks are independent (counter-based), so they are filled by a small
    thread pool; the values do not depend on the chunking or thread count.
    """
    out = np.empty(n, dtype=np.float64)
    npairs = (n + 1) // 2
    spans = [(p0, min(npairs, p0 + _CHUNK)) for p0 in range(0, npairs, _CHUNK)]
    if len(spans) <= 1:
        for p0, p1 in spans:
            _normal_chunk(seed, stream, p0, p1, n, out)
        return out
    workers = max(1, min(len(spans), os.cpu_count() or 1, 16))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        list(ex.map(lambda sp: _normal_chunk(seed, stream, sp[0], sp[1], n, out), spans))
    return out


def normal(seed: int, shape, sigma: float = 1.0) -> np.ndarray:
    n = int(np.prod(shape))
    z = std_normal(seed, S_MAIN, n)
    if sigma != 1.0:
        z *= sigma
    return z.astype(np.float32).reshape(shape)


def student_t3(seed: int, shape) -> np.ndarray:
    n = int(np.prod(shape))
    z = std_normal(seed, S_MAIN, n)
    chi = np.zeros(n, dtype=np.float64)
    for s in (S_CHI1, S_CHI2, S_CHI3):
        c = std_normal(seed, s, n)
        chi += c * c
    return (z / np.sqrt(chi / 3.0)).astype(np.float32).reshape(shape)


def outlier_columns(seed: int, K: int, frac: float = 0.01) -> np.ndarray:
    """round(frac*K) distinct column indices, uniform without replacement (sorted)."""
    count = int(round(frac * K))
    order = np.argsort(uniform(seed, S_OUTLIER, K), kind="stable")
    return np.sort(order[:count])


def row_scales_loguniform(seed: int, rows: int, lo: float = 0.1, hi: float = 10.0) -> np.ndarray:
    u = uniform(seed, S_ROWSCALE, rows)
    return np.power(10.0, np.log10(lo) + u * (np.log10(hi) - np.log10(lo)))


# name -> (M, N, K, g)
WORKLOADS = {
    1: dict(name="square256", M=256, N=256, K=256, g=128),
    2: dict(name="decode_m64_n4096_k7168", M=64, N=4096, K=7168, g=128),
    3: dict(name="prefill_m4096_n7168_k2048", M=4096, N=7168, K=2048, g=128),
    4: dict(name="square8192", M=8192, N=8192, K=8192, g=128),
    5: dict(name="longk_m2000_n4000_k16384_g64", M=2000, N=4000, K=16384, g=64),
}


def seeds(c: int):
    return 2 * c + 1000, 2 * c + 1001


def make_a(c: int, M: int | None = None, K: int | None = None) -> np.ndarray:
    """A [M,K] float32 of workload c (shape overridable for reduced-size cases)."""
    w = WORKLOADS[c]
    M = w["M"] if M is None else M
    K = w["K"] if K is None else K
    sA, _ = seeds(c)
    if c in (1, 4):
        return normal(sA, (M, K))
    if c == 2:
        a = normal(sA, (M, K))
        a[:, outlier_columns(sA, K)] *= np.float32(20.0)
        return a
    if c == 3:
        a = std_normal(sA, S_MAIN, M * K).reshape(M, K)
        a *= row_scales_loguniform(sA, M)[:, None]
        return a.astype(np.float32)
    if c == 5:
        return student_t3(sA, (M, K))
    raise KeyError(c)


def make_b(c: int, N: int | None = None, K: int | None = None) -> np.ndarray:
    """B [N,K] float32 of workload c."""
    w = WORKLOADS[c]
    N = w["N"] if N is None else N
    K = w["K"] if K is None else K
    _, sB = seeds(c)
    if c == 4:
        return normal(sB, (N, K))
    return normal(sB, (N, K), sigma=0.02)
