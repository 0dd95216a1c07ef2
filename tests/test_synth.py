"""CPU tier: the seeded input generator (no method arithmetic here)."""
import math

import numpy as np

import synth


def test_deterministic_and_stream_separated():
    a = synth.normal_f32(1000, 1.0, 0, synth.tag(synth.TAG_WBASE))
    b = synth.normal_f32(1000, 1.0, 0, synth.tag(synth.TAG_WBASE))
    c = synth.normal_f32(1000, 1.0, 0, synth.tag(synth.TAG_X))
    d = synth.normal_f32(1000, 1.0, 1, synth.tag(synth.TAG_WBASE))
    assert np.array_equal(a, b)
    assert not np.array_equal(a, c) and not np.array_equal(a, d)
    # element i is a function of i alone: a prefix of a longer draw is the short draw
    assert np.array_equal(synth.normal_f32(4000, 1.0, 0, synth.tag(synth.TAG_WBASE))[:1000], a)


def test_splitmix64_published_outputs():
    """The finaliser chain is SplitMix64: stream key derived from (seed, tag),
    element i = mix(key + (i+1) gamma).  Check against a direct Python
    rendering of the published algorithm (Steele, Lea, Flood 2014)."""
    M = (1 << 64) - 1
    G = 0x9E3779B97F4A7C15

    def mix(z):
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & M
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & M
        return z ^ (z >> 31)

    # SplitMix64 seeded with 0: first output is mix(gamma) = 0xE220A8397B1DCDAF
    assert mix(G) == 0xE220A8397B1DCDAF
    key = mix(mix((7 + G) & M) ^ ((3 * 0xD1B54A32D192ED03 + 0x632BE59BD9B4E019) & M))
    got = synth.u64(5, 7, 3)
    assert [int(v) for v in got] == [mix((key + (i + 1) * G) & M) for i in range(5)]


def test_distributions():
    n = 200000
    z = synth.normal_f32(n, 0.02, 3, 11).astype(np.float64)
    assert abs(z.mean()) < 5 * 0.02 / math.sqrt(n) and abs(z.std() / 0.02 - 1) < 0.01
    lp = synth.laplace_f32(n, 1e-3, 3, 12).astype(np.float64)
    assert abs(np.abs(lp).mean() / 1e-3 - 1) < 0.01          # E|X| = b
    assert abs(lp.std() / (math.sqrt(2) * 1e-3) - 1) < 0.02   # sd = b sqrt 2
    assert abs((lp >= 0).mean() - 0.5) < 0.01
    u = synth.uniform(n, 3, 13)
    assert u.min() > 0 and u.max() < 1 and abs(u.mean() - 0.5) < 0.005


def test_zipf_split_and_ids():
    counts = synth.zipf_counts(4096, 14, 1.1)
    assert counts == [1397, 652, 417, 304, 238, 195, 164, 142, 125, 111, 100, 91, 83, 77]
    ids = synth.variant_ids(counts, seed=0)
    assert np.array_equal(np.bincount(ids, minlength=14), counts)
    assert not np.array_equal(ids, np.sort(ids))
    scales = synth.variant_scales(14)
    assert scales.min() >= 3e-4 and scales.max() <= 3e-3


def test_layer_recipe():
    w_base, w_ft = synth.layer(64, 256)
    wb = synth.bf16_bits_to_f32(w_base)
    assert w_base.dtype == np.uint16 and w_ft.dtype == np.float32
    d = w_ft - wb
    assert abs(np.abs(d).mean() / 1e-3 - 1) < 0.05
