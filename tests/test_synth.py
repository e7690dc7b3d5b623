"""Properties of the seeded input generator (CPU only)."""
import numpy as np

import synth
from synth.workloads import get


def test_workload_totals():
    expect = {"tiny": 10_272, "gpt2_small": 124_439_808, "llama3_8b": 8_030_261_248,
              "llama2_70b": 68_976_648_192, "dna_20b": 19_987_850_990}
    counts = {"tiny": 3, "gpt2_small": 148, "llama3_8b": 291, "llama2_70b": 723,
              "dna_20b": 2178}
    for name, total in expect.items():
        w = get(name)
        assert w.total == total and len(w.shapes) == counts[name]
    sizes = synth.small_sizes(2000)
    assert min(sizes) >= 64 and max(sizes) <= 6144


def test_normal_moments_and_support():
    k = synth.key(0, synth.STREAM_GRAD, 1)
    z = synth.host_values(k, 0, 1 << 20, 1.0).astype(np.float64)
    assert abs(z.mean()) < 5e-3 and abs(z.var() - 1) < 5e-3
    assert np.abs(z).max() <= 2 * np.sqrt(3) + 1e-6
    # bounded support: fp16 grads at the largest loss scale used stay finite
    assert 1e-3 * 2 * np.sqrt(3) * 65536 < 65504


def test_counter_based_and_reproducible():
    k = synth.key(0, synth.STREAM_GRAD, 3)
    a = synth.host_values(k, 1000, 5000, 1e-3)
    b = synth.host_values(k, 1000, 5000, 1e-3)
    assert np.array_equal(a, b)
    idx = np.array([1000, 1001, 4321, 5999], np.int64)
    assert np.array_equal(synth.host_gather(k, idx, 1e-3), a[idx - 1000])
    other = synth.host_values(synth.key(0, synth.STREAM_GRAD, 4), 1000, 5000, 1e-3)
    assert not np.array_equal(a, other)


def test_outlier_rate():
    k = synth.key(0, synth.STREAM_GRAD, 1)
    base = synth.host_values(k, 0, 1 << 20, 1e-3)
    out = synth.host_values(k, 0, 1 << 20, 1e-3, 1.0, synth.outlier_thresh(0.01), 100.0)
    hit = base != out
    assert abs(hit.mean() - 0.01) < 1e-3
    assert np.allclose(out[hit], base[hit] * 100, rtol=1e-6)


def test_injection_rate():
    hits = [synth.inject(0, it, 1 << 30, 0.1) for it in range(1, 4001)]
    rate = np.mean([h is not None for h in hits])
    assert abs(rate - 0.1) < 0.02
    assert all(0 <= h < (1 << 30) for h in hits if h is not None)
