"""Pins for the oracle's block quantiser (CPU only).

The quantiser is the step just before the GEMM: one FP32 scale per g x g block
(DeepGEMM实战 §2.2), quantise by dividing (§5.2), same granularity as the GEMM
(§4.4). Pinned by a hand-worked block, by reconstructing every code by brute
force from the definition (FP32 amax, FP32 divide, nearest even E4M3), and by
the dequantisation error bound that round-to-nearest guarantees.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from tests import _golden


def test_worked_block():
    w = _golden.worked_quant()
    q, s = oracle.quantize_blocks(w["x"], w["g"])
    assert s.shape == (1, 1) and s[0, 0] == np.float32(w["scale"])
    assert np.array_equal(q, w["codes"])


def _blocks(rows, cols, g):
    for rb in range(0, rows, g):
        for cb in range(0, cols, g):
            yield rb // g, cb // g, slice(rb, min(rb + g, rows)), slice(cb, cb + g)


@pytest.mark.parametrize("rows,cols,g", [(300, 256, 128), (65, 192, 64), (1, 128, 128), (130, 64, 64)])
def test_scales_and_codes_by_definition(rows, cols, g):
    rng = np.random.default_rng(rows * 7 + cols)
    x = (rng.standard_normal((rows, cols)) * np.exp(rng.uniform(-8, 8, size=(rows, 1)))).astype(np.float32)
    x[0, 0] = 0.0
    q, s = oracle.quantize_blocks(x, g)
    assert s.shape == ((rows + g - 1) // g, cols // g)
    for rb, cb, rs, cs in _blocks(rows, cols, g):
        blk = x[rs, cs]
        amax = np.float32(np.max(np.abs(blk)))
        scale = np.float32(amax / np.float32(448.0)) if amax > 0 else np.float32(1.0)
        assert s[rb, cb] == scale
        # torch's float8 cast is an independent RNE encoder; x/scale stays <= 448
        # up to one FP32 rounding, which torch also rounds to 448.
        y = (blk / scale).astype(np.float32)
        ref = torch.from_numpy(np.ascontiguousarray(y)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(q[rs, cs], ref)


def test_all_zero_block_scale_one():
    x = np.zeros((128, 256), np.float32)
    x[:, 128:] = 1.0
    q, s = oracle.quantize_blocks(x, 128)
    assert s[0, 0] == 1.0 and np.all(q[:, :128] == 0)
    assert s[0, 1] == np.float32(1.0 / 448.0) and np.all(q[:, 128:] == 0x7E)


def test_edge_block_uses_present_rows_only():
    # 130 rows, g=64: the third row block holds rows 128..129 only.
    x = np.full((130, 64), 1.0, np.float32)
    x[128:, :] = 0.5
    q, s = oracle.quantize_blocks(x, 64)
    assert s[2, 0] == np.float32(0.5 / 448.0)
    assert np.all(q[128:] == 0x7E)


def test_dequantisation_error_bound():
    """|dec(q)*s - x| <= half a step of E4M3 at |x/s| (relative 2^-4, absolute 2^-10 below 2^-6)."""
    x = synth.make_a(5, M=192, K=256)  # heavy-tailed Student-t rows
    g = 64
    q, s = oracle.quantize_blocks(x, g)
    deq = oracle.e4m3_decode(q)
    srep = np.repeat(np.repeat(s.astype(np.float64), g, axis=0)[: x.shape[0]], g, axis=1)
    y = np.abs(x.astype(np.float64) / srep)
    step = np.where(y < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(y, 2.0 ** -6))) - 3))
    err = np.abs(deq - x.astype(np.float64) / srep)
    assert np.all(err <= step / 2 * (1 + 1e-6) + 1e-12)
    # every block's largest element lands on +-448
    for rb, cb, rs, cs in _blocks(*x.shape, g):
        assert np.max(np.abs(deq[rs, cs])) == 448.0


@pytest.mark.parametrize("fmt,mag", [(0, 1e-44), (1, 1e-42), (1, 3e-41)])
def test_underflowing_scale_is_one(fmt, mag):
    # amax / fmax rounds to zero in FP32 for these blocks (fmax 448 or 57344):
    # the factor is then 1.0, as for an all-zero block, and every value (far
    # below the smallest FP8 subnormal) encodes as a zero of its own sign
    fmax = np.float32(448.0 if fmt == 0 else 57344.0)
    x = (np.random.default_rng(7).uniform(-1.0, 1.0, (64, 64)) * mag).astype(np.float32)
    x[0, 0] = np.float32(-mag)
    assert np.float32(np.abs(x).max()) / fmax == np.float32(0.0)
    for q, s in (oracle.quantize_blocks_fmt(x, 64, fmt), oracle.quantize_rows_fmt(x, 64, fmt)):
        assert np.all(s == np.float32(1.0))
        assert np.array_equal(q, np.where(np.signbit(x), 0x80, 0x00).astype(np.uint8))


def test_scale_just_above_underflow():
    # the smallest amax whose quotient does not underflow keeps amax / 448
    x = np.zeros((64, 64), np.float32)
    x[3, 5] = np.float32(448.0) * np.float32(2.0 ** -149)  # amax / 448 = 2^-149, the smallest subnormal
    q, s = oracle.quantize_blocks(x, 64)
    assert s[0, 0] == np.float32(2.0 ** -149)
    assert q[3, 5] == 0x7E  # 448
