"""The input generator: determinism, index keying and value distributions."""
import numpy as np

import synth


def test_keyed_by_global_index():
    sp = synth.spec(5, synth.STREAM_MASTER, 0, 0.02)
    whole = synth.cpu_f32(10_000, 0, sp)
    part = synth.cpu_f32(3_000, 4_000, sp)
    assert np.array_equal(whole[4_000:7_000], part)
    at = synth.cpu_at_f32(np.array([0, 9_999, 4_321]), sp)
    assert np.array_equal(at, whole[[0, 9_999, 4_321]])


def test_streams_and_steps_differ():
    a = synth.cpu_f32(1000, 0, synth.spec(5, synth.STREAM_CONTRIB + 0, 1, 1e-3))
    b = synth.cpu_f32(1000, 0, synth.spec(5, synth.STREAM_CONTRIB + 1, 1, 1e-3))
    c = synth.cpu_f32(1000, 0, synth.spec(5, synth.STREAM_CONTRIB + 0, 2, 1e-3))
    assert not np.array_equal(a, b) and not np.array_equal(a, c)


def test_normal_moments():
    x = synth.cpu_f32(1_000_000, 0, synth.spec(1, synth.STREAM_MASTER, 0, 0.02)).astype(np.float64)
    assert abs(x.mean()) < 0.02 * 0.005
    assert abs(x.std() / 0.02 - 1) < 0.005
    k = ((x / 0.02) ** 4).mean()
    assert abs(k - 3) < 0.15  # Irwin-Hall(12) kurtosis is 2.9
    assert np.abs(x).max() <= 6 * 0.02


def test_padding_is_zero():
    x = synth.cpu_bf16(100, 0, synth.spec(1, synth.STREAM_CONTRIB, 1, 1e-3, valid_hi=97))
    assert np.all(x[97:] == 0) and np.count_nonzero(x[:97]) >= 90


def test_shared_zero_mask():
    n = 400_000
    a = synth.cpu_bf16(n, 0, synth.spec(1, synth.STREAM_CONTRIB + 0, 1, 1e-3, zero_prob=0.01))
    b = synth.cpu_bf16(n, 0, synth.spec(1, synth.STREAM_CONTRIB + 7, 3, 1e-3, zero_prob=0.01))
    za, zb = a == 0, b == 0
    assert abs(za.mean() - 0.01) < 0.001
    # the masked positions are the same for every contribution and step
    assert (za & ~zb).sum() <= 10 and (zb & ~za).sum() <= 10


def test_heavy_tail_rate():
    n = 1_000_000
    x = synth.cpu_f32(n, 0, synth.spec(2, synth.STREAM_CONTRIB, 1, 1e-3, tail_sigma=0.1,
                                       tail_prob=0.001))
    big = np.abs(x) > 7e-3  # beyond the bulk's +-6 sigma support
    assert 0.0008 < big.mean() < 0.0011
