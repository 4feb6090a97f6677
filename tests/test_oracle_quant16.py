"""Pins of the oracle's 16-bit quantiser input (BF16 and FP16, DeepGEMM实战 §4.4).

The decoders are checked on every one of the 65536 patterns against torch's
bfloat16 and numpy's float16 conversions (library routines, not the oracle's
bit-field code) and on hand-listed values. The quantisers are checked on blocks
with a closed-form result: FP8 values that a 16-bit format carries exactly,
with the block's amax at fmax * 2^k, quantise to scale 2^k and to their own
codes, so a wrong decode (bias, field width, byte order, sign) or a dropped
decode step changes codes or scales.
"""

import numpy as np
import pytest
import torch

import oracle

ALL = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)


def test_bf16_decode_all_patterns_match_torch():
    got = oracle.bf16_decode(ALL)
    ref = torch.from_numpy(ALL.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))  # signed zeros too


def test_f16_decode_all_patterns_match_numpy():
    got = oracle.f16_decode(ALL)
    ref = ALL.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


@pytest.mark.parametrize("bits,value", [
    (0x3F80, 1.0), (0xC000, -2.0), (0x0001, 2.0 ** -133), (0x0080, 2.0 ** -126),
    (0x7F7F, (2 - 2.0 ** -7) * 2.0 ** 127), (0x4040, 3.0), (0x3E00, 0.125), (0x7F80, np.inf),
])
def test_bf16_decode_values(bits, value):
    assert oracle.bf16_decode(np.array([bits], dtype=np.uint16))[0] == np.float32(value)


@pytest.mark.parametrize("bits,value", [
    (0x3C00, 1.0), (0xC000, -2.0), (0x0001, 2.0 ** -24), (0x0400, 2.0 ** -14),
    (0x7BFF, 65504.0), (0x4200, 3.0), (0x3000, 0.125), (0xFC00, -np.inf),
])
def test_f16_decode_values(bits, value):
    assert oracle.f16_decode(np.array([bits], dtype=np.uint16))[0] == np.float32(value)


def test_negative_zero_keeps_its_sign():
    z = np.array([0x8000], dtype=np.uint16)
    assert np.signbit(oracle.bf16_decode(z)[0]) and np.signbit(oracle.f16_decode(z)[0])


def _finite_codes(fmt):
    codes = np.arange(256, dtype=np.uint8)
    dec = oracle.e4m3_decode(codes) if fmt == 0 else oracle.e5m2_decode(codes)
    return codes[np.isfinite(dec)], dec[np.isfinite(dec)]


def _bits_of(values, kind):
    """16-bit patterns of values that the format holds exactly (checked)."""
    v = np.asarray(values, dtype=np.float32)
    if kind == oracle.IN_BF16:
        u = v.view(np.uint32)
        assert not np.any(u & 0xFFFF), "value not exact in BF16"
        return (u >> 16).astype(np.uint16)
    h = v.astype(np.float16)
    assert np.array_equal(h.astype(np.float32), v), "value not exact in FP16"
    return h.view(np.uint16)


def _closed_form_block(fmt, g, rows, seed):
    """rows x g FP8 codes covering every finite code, with the format's largest value present."""
    codes, _ = _finite_codes(fmt)
    rng = np.random.default_rng(seed)
    q = rng.choice(codes, size=(rows, g))
    q[rows // 2, g // 3] = 0x7E if fmt == 0 else 0x7B  # +fmax
    q.reshape(-1)[: codes.size] = codes
    return q


# (kind, fmt, power k of two): the scaled FP8 values stay exact in the 16-bit format
CASES = [(oracle.IN_BF16, 0, 0), (oracle.IN_BF16, 0, -20), (oracle.IN_BF16, 0, 40), (oracle.IN_BF16, 1, 0),
         (oracle.IN_BF16, 1, -30), (oracle.IN_F16, 0, 0), (oracle.IN_F16, 0, -10), (oracle.IN_F16, 0, 5),
         (oracle.IN_F16, 1, 0)]


@pytest.mark.parametrize("kind,fmt,k", CASES)
@pytest.mark.parametrize("g", [64, 128])
def test_blocks_closed_form(kind, fmt, k, g):
    q0 = _closed_form_block(fmt, g, g, seed=g + 7 * abs(k) + 3 * fmt + kind)
    vals = (oracle.e4m3_decode(q0) if fmt == 0 else oracle.e5m2_decode(q0)) * 2.0 ** k
    q, s = oracle.quantize_blocks_16(_bits_of(vals, kind), kind, g, fmt)
    assert s.shape == (1, 1) and s[0, 0] == np.float32(2.0 ** k)
    assert np.array_equal(q, q0)


@pytest.mark.parametrize("kind,fmt,k", CASES)
def test_rows_closed_form(kind, fmt, k):
    g, rows = 64, 5
    q0 = _closed_form_block(fmt, g * 2, rows, seed=11 + abs(k))
    q0[:, g // 2] = 0x7E if fmt == 0 else 0x7B      # every 1 x g segment holds +fmax
    q0[:, g + g // 2] = 0xFE if fmt == 0 else 0xFB  # or -fmax
    vals = (oracle.e4m3_decode(q0) if fmt == 0 else oracle.e5m2_decode(q0)) * 2.0 ** k
    q, s = oracle.quantize_rows_16(_bits_of(vals, kind), kind, g, fmt)
    assert s.shape == (rows, 2) and np.all(s == np.float32(2.0 ** k))
    assert np.array_equal(q, q0)


def test_e5m2_codes_are_the_high_byte_of_fp16():
    # E5M2 is FP16 with the low 8 fraction bits dropped: code c is the FP16
    # pattern c << 8. A block holding +-57344 has scale 1 and returns each code.
    codes, _ = _finite_codes(1)
    q0 = np.resize(codes, (64, 64)).astype(np.uint8)
    q0[0, 0] = 0x7B
    bits = q0.astype(np.uint16) << 8
    q, s = oracle.quantize_blocks_16(bits, oracle.IN_F16, 64, fmt=1)
    assert s[0, 0] == 1.0 and np.array_equal(q, q0)


def test_partial_edge_block_and_ragged_rows():
    # rows past the end leave the edge block partial: its amax is over the
    # rows present, so a large value beyond the last row cannot exist and the
    # block's scale follows the rows that do.
    g = 64
    v = np.zeros((g + 3, g), dtype=np.float32)
    v[:g] = 1.0
    v[g:] = 2.0 ** -5
    v[0, 0] = 448.0
    q, s = oracle.quantize_blocks_16(_bits_of(v, oracle.IN_BF16), oracle.IN_BF16, g, 0)
    assert s[0, 0] == 1.0 and s[1, 0] == np.float32(2.0 ** -5 / 448)
    assert np.all(q[g:] == 0x7E)  # each edge-block value is its block's amax -> +448


def test_matches_the_fp32_quantiser_on_the_decoded_values():
    # the 16-bit path is the FP32 rule on exact values: seeded normals rounded
    # to BF16 by torch give the same result through either entry
    x = torch.from_numpy(np.random.default_rng(5).standard_normal((200, 256)).astype(np.float32))
    xb = x.to(torch.bfloat16)
    bits = xb.view(torch.int16).numpy().view(np.uint16)
    for fmt in (0, 1):
        q16, s16 = oracle.quantize_blocks_16(bits, oracle.IN_BF16, 128, fmt)
        q32, s32 = oracle.quantize_blocks_fmt(xb.float().numpy(), 128, fmt)
        assert np.array_equal(q16, q32) and np.array_equal(s16, s32)
