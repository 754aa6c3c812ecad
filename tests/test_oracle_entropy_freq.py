"""Pins for oracle.entropy and oracle.freq (closed forms, hand-worked cases)."""

import math

import numpy as np
import pytest

from oracle import entropy, freq


@pytest.mark.parametrize("m", [1, 2, 3, 16, 256])
def test_uniform_entropy_is_log2_m(m):
    sym = np.repeat(np.arange(m), 7)
    assert entropy.empirical_entropy(sym, 256) == pytest.approx(math.log2(m), abs=1e-12)


def test_uniform_ternary_is_1585_bits():
    # the ternary page: three equiprobable values carry log2(3) ~= 1.585 bits
    sym = np.array([0, 1, 2] * 1000)
    h = entropy.empirical_entropy(sym, 3)
    assert h == pytest.approx(1.584962500721156, abs=1e-12)
    assert round(h, 3) == 1.585


def test_single_symbol_is_zero_bits():
    assert entropy.empirical_entropy(np.full(100, 5), 16) == 0.0


@pytest.mark.parametrize("a,b", [(1, 3), (1, 9), (3, 5), (1, 1)])
def test_two_symbols_binary_entropy(a, b):
    sym = np.array([0] * a + [1] * b)
    p = a / (a + b)
    h = -p * math.log2(p) - (1 - p) * math.log2(1 - p)
    assert entropy.empirical_entropy(sym, 2) == pytest.approx(h, abs=1e-12)


def test_discrete_gaussian_entropy_close_form():
    # rint(N(0, 8)) has entropy close to 0.5*log2(2*pi*e*sigma^2) = 5.047 for sigma >> 1
    rng = np.random.default_rng(1)
    sym = (np.clip(np.rint(rng.normal(0, 8, 2_000_000)), -127, 127).astype(np.int64) + 128)
    h = entropy.empirical_entropy(sym, 256)
    assert h == pytest.approx(0.5 * math.log2(2 * math.pi * math.e * 64), abs=0.01)


def test_histogram_rejects_out_of_alphabet():
    with pytest.raises(ValueError):
        entropy.histogram(np.array([0, 16]), 16)


# ------------------------------------------------------------------ freq
def test_freq_hand_worked_ties():
    # counts [1,1,1], M=4: floors 1,1,1 (sum 3); d=1 goes to the smallest symbol
    # among equal remainders (4 mod 3 = 1 for all)
    assert list(freq.quantize_freqs([1, 1, 1], 2)) == [2, 1, 1]


def test_freq_hand_worked_floor_to_one():
    # counts [1, 100], M=16: f0 = max(1, floor(16/101)) = 1, f1 = floor(1600/101) = 15
    assert list(freq.quantize_freqs([1, 100], 4)) == [1, 15]


def test_freq_hand_worked_reduce_largest():
    # five singletons bumped to 1 plus floor(8000/1005) = 7 -> sum 12, d = -4
    assert list(freq.quantize_freqs([1, 1, 1, 1, 1, 1000], 3)) == [1, 1, 1, 1, 1, 3]


def test_freq_hand_worked_remainders():
    # counts [5, 3, 2], M=16: exact 8, 4.8, 3.2 -> floors 8,4,3 (sum 15);
    # remainders (80%10=0, 48%10=8, 32%10=2): +1 to symbol 1
    assert list(freq.quantize_freqs([5, 3, 2], 4)) == [8, 5, 3]


def test_freq_exact_when_divisible():
    counts = np.array([2048, 1024, 512, 512]) * 3
    assert list(freq.quantize_freqs(counts, 12)) == [2048, 1024, 512, 512]


def test_freq_single_symbol_gets_everything():
    f = freq.quantize_freqs([0, 0, 77, 0], 12)
    assert list(f) == [0, 0, 4096, 0]


@pytest.mark.parametrize("seed", range(20))
def test_freq_invariants_random(seed):
    rng = np.random.default_rng(seed)
    alpha = int(rng.integers(2, 257))
    counts = rng.integers(0, 1000, alpha) * (rng.random(alpha) < 0.7)
    counts[rng.integers(alpha)] += 1
    f = freq.quantize_freqs(counts, 12)
    assert f.sum() == 4096
    assert ((f > 0) == (counts > 0)).all()
    assert list(f) == list(freq.quantize_freqs(counts, 12))  # deterministic
    c = freq.cumulative(f)
    s2 = freq.slot_to_symbol(f)
    assert s2.size == 4096
    for s in np.nonzero(f)[0]:
        assert (s2[c[s]:c[s] + f[s]] == s).all()


def test_freq_errors():
    with pytest.raises(ValueError):
        freq.quantize_freqs([0, 0], 12)
    with pytest.raises(ValueError):
        freq.quantize_freqs(np.ones(20), 4)  # 20 symbols > M = 16


def test_freq_quantisation_cost_is_small():
    # cross-entropy with the quantised table stays within 0.01 bit of H for
    # peaked and flat 8-bit histograms
    rng = np.random.default_rng(3)
    for sigma in (1.0, 8.0, 40.0):
        sym = np.clip(np.rint(rng.normal(128, sigma, 500_000)), 0, 255).astype(np.int64)
        counts = entropy.histogram(sym, 256)
        f = freq.quantize_freqs(counts, 12)
        p = counts / counts.sum()
        cross = -(p[p > 0] * np.log2(f[p > 0] / 4096)).sum()
        assert cross - entropy.entropy_from_counts(counts) < 0.01
