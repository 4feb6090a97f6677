"""bench.py's host logic on the CPU: the algorithmic FLOP and byte counts the
roofline fractions divide by, the bound each workload is measured against,
and the refusal of more than one GPU. The expected counts are worked out by
hand from the shapes: FLOP = 2MNK; bytes = FP8 A and B once (MK + NK), the
FP32 factors (4 per g x g block of each operand, or per 1 x g segment of A),
and the BF16 output (2MN)."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synth  # noqa: E402

# workload: (FLOP, algorithmic bytes, bound)
EXPECTED = {
    1: (2 * 256 ** 3, 256 * 256 * 2 + 4 * (2 + 2) * 2 + 2 * 256 * 256, "hbm"),
    2: (2 * 64 * 4096 * 7168, 64 * 7168 + 4096 * 7168 + 4 * (1 + 32) * 56 + 2 * 64 * 4096, "hbm"),
    3: (2 * 4096 * 7168 * 2048, 4096 * 2048 + 7168 * 2048 + 4 * (32 + 56) * 16 + 2 * 4096 * 7168, "mfma"),
    4: (2 * 8192 ** 3, 2 * 8192 * 8192 + 4 * (64 + 64) * 64 + 2 * 8192 * 8192, "mfma"),
    5: (2 * 2000 * 4000 * 16384, 2000 * 16384 + 4000 * 16384 + 4 * (32 + 63) * 256 + 2 * 2000 * 4000, "mfma"),
}


@pytest.mark.parametrize("c", sorted(EXPECTED))
def test_algorithmic_counts_and_bound(c):
    w = synth.WORKLOADS[c]
    flops, nbytes = bench.algorithmic(w)
    assert (flops, nbytes) == EXPECTED[c][:2]
    assert bench.bound_of(w) == EXPECTED[c][2]


def test_decode_bytes_value():
    # the decode shape's figure quoted next to its roofline: 30,350,560 bytes
    assert bench.algorithmic(synth.WORKLOADS[2])[1] == 30350560


def test_per_row_factor_bytes():
    # 1 x g factors of A: one per row and K segment
    w = synth.WORKLOADS[4]
    _, blocks = bench.algorithmic(w)
    _, rows = bench.algorithmic(w, sa_rows=1)
    assert rows - blocks == 4 * (8192 - 64) * 64


def test_g256_factor_bytes():
    w = synth.WORKLOADS[4]
    _, b128 = bench.algorithmic(w)
    _, b256 = bench.algorithmic(w, g=256)
    assert b128 - b256 == 4 * (64 + 64) * 64 - 4 * (32 + 32) * 32


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
