"""The seeded input generators: published SplitMix64 vector, determinism, shapes."""

import numpy as np

import synth


def test_splitmix64_published_vector():
    # SplitMix64 from state 1234567: the widely published first five outputs.
    want = [6457827717110365317, 3203168211198807973, 9817491932198370423,
            4593380528125082431, 16408922859458223821]
    got = [synth._mix_scalar(1234567 + i * synth.GAMMA) for i in range(1, 6)]
    assert got == want
    key = 1234567
    arr = synth._mix(np.arange(1, 6, dtype=np.uint64) * np.uint64(synth.GAMMA) + np.uint64(key))
    assert arr.tolist() == want


def test_counter_based_and_chunk_independent():
    a = synth.std_normal(5, 0, 3_000_001)
    b = synth.std_normal(5, 0, 1001)
    assert np.array_equal(a[:1001], b)
    u1 = synth.uniform(9, 2, 100, start=50)
    u2 = synth.uniform(9, 2, 150)[50:]
    assert np.array_equal(u1, u2)
    assert np.all((u2 > 0) & (u2 < 1))


def test_distributions():
    z = synth.normal(1, (1000, 1000), sigma=0.02).astype(np.float64)
    assert abs(z.mean()) < 1e-4 and abs(z.std() - 0.02) < 1e-4
    t = synth.student_t3(2, (400, 1000)).astype(np.float64)
    # t3: median |t| = 0.7649, variance 3
    assert abs(np.median(np.abs(t)) - 0.7649) < 0.01
    cols = synth.outlier_columns(1004, 7168)
    assert cols.size == 72 and np.unique(cols).size == 72
    r = synth.row_scales_loguniform(1006, 4096)
    assert r.min() >= 0.1 and r.max() <= 10.0 and abs(np.mean(np.log10(r))) < 0.05


def test_workload_2_outliers_applied():
    a = synth.make_a(2)
    cols = synth.outlier_columns(synth.seeds(2)[0], 7168)
    base = synth.normal(synth.seeds(2)[0], (64, 7168))
    assert np.array_equal(a[:, cols], base[:, cols] * np.float32(20))
    mask = np.ones(7168, bool)
    mask[cols] = False
    assert np.array_equal(a[:, mask], base[:, mask])
