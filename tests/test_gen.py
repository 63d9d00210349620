"""Seeded generator: determinism, the published SplitMix64 sequence, moments, bf16 rounding."""
import numpy as np

import gen


def test_splitmix64_published_sequence():
    # First outputs of SplitMix64 started from state 0 (Steele, Lea & Flood, OOPSLA 2014;
    # the same values are printed with the public reference implementation).
    got = [int(x) for x in gen.raw_u64(np.uint64(0), 3)]
    assert got == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_deterministic_and_distinct_streams():
    a = gen.tensor(3, 0, "q", (2, 3, 5, 8))
    b = gen.tensor(3, 0, "q", (2, 3, 5, 8))
    assert np.array_equal(a, b)
    assert not np.array_equal(a, gen.tensor(3, 0, "k", (2, 3, 5, 8)))
    assert not np.array_equal(a, gen.tensor(3, 1, "q", (2, 3, 5, 8)))
    assert not np.array_equal(a, gen.tensor(4, 0, "q", (2, 3, 5, 8)))
    # chunked generation gives the same numbers as one shot
    key = gen.stream_key(9, 2, 1)
    assert np.array_equal(gen.normals(key, 1000, chunk=64), gen.normals(key, 1000))


def test_moments():
    z = gen.normals(gen.stream_key(1, 0, 0), 400_000)
    assert abs(z.mean()) < 0.01
    assert abs(z.std() - 1.0) < 0.01
    assert abs(np.mean(z ** 4) - 3.0) < 0.05  # Gaussian kurtosis
    x = gen.tensor(2, 0, "do", (400_000,), sigma=0.1)
    assert abs(x.std() - 0.1) < 0.001


def test_bf16_round_to_nearest_even():
    vals = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20, -1.0 - 2 ** -8,
                     3.0e38], dtype=np.float32)
    want = np.array([1.0, 1.0, 1.0 + 2 ** -6, 1.0 + 2 ** -7, -1.0, 2.9993e38], dtype=np.float32)
    got = gen.round_bf16(vals)
    assert np.array_equal(got[:5], want[:5])
    assert np.all(gen.bf16_bits(got) >= 0)
    x = gen.tensor(1, 0, "q", (10000,), dtype="bf16")
    assert np.all(x.view(np.uint32) & 0xFFFF == 0)
    # rounding error is at most half a bf16 ulp
    x32 = gen.tensor(1, 0, "q", (10000,), dtype="f32")
    rel = np.abs(x - x32) / np.abs(x32)
    assert rel.max() <= 2.0 ** -8 + 1e-12


def test_outlier_keys_exact_count():
    w = gen.Workload("t", 2, 2, 2, 300, 8, "bf16", outlier_frac=0.01, outlier_scale=8.0, seed=5)
    q, k, v, do = gen.layer_inputs(w)
    plain = gen.tensor(5, 0, "k", k.shape, dtype="bf16")
    for b in range(2):
        for g in range(2):
            ratio = k[b, g] / plain[b, g]
            scaled = np.where(np.all(ratio == 8.0, axis=1))[0]
            same = np.where(np.all(ratio == 1.0, axis=1))[0]
            assert len(scaled) == 3 and len(same) == 297
            assert np.array_equal(scaled, gen.pick_positions(5, 0, b, g, 300, 3))


def test_workload_shapes():
    w = gen.WORKLOADS[3]
    assert (w.B, w.Hq, w.Hkv, w.T, w.D, w.G) == (16, 12, 4, 512, 64, 3)
    assert w.causal_pairs == 25_214_976
    assert gen.WORKLOADS[5].causal_pairs == 134_283_264
    assert gen.WORKLOADS[1].causal_pairs == 33_024
