"""Pins for oracle.rans: hand-worked golden streams, brute-force round trips,
scalar-vs-vectorised equality, size bounds and integrity errors."""

import itertools
import json
import math
import os

import numpy as np
import pytest

from oracle import entropy, freq, rans


def _golden(golden_dir):
    with open(os.path.join(golden_dir, "rans_tiny.json")) as fh:
        return json.load(fh)["cases"]


def test_golden_hand_worked_streams(golden_dir):
    for case in _golden(golden_dir):
        st, w, k = rans.encode_scalar(case["symbols_j_order"], case["freqs"],
                                      case["lanes"], case["prob_bits"], case["kmax"])
        assert st == case["states"], case["name"]
        assert list(w) == case["words"], case["name"]
        assert k == case["k"], case["name"]
        S = len(case["symbols_j_order"]) // case["lanes"]
        out = rans.decode_scalar(st, w, case["freqs"], case["lanes"], S, k, case["prob_bits"])
        assert out == case["symbols_j_order"]
        # the vectorised coder produces the same bytes
        st2, w2, k2 = rans.encode_tiles(np.array([case["symbols_j_order"]]), case["freqs"],
                                        case["lanes"], case["prob_bits"], case["kmax"])
        assert list(st2[0]) == case["states"] and list(w2[0]) == case["words"] and k2[0] == k


TABLES = {
    2: [[1, 4095], [2048, 2048], [4095, 1]],
    3: [[1, 1, 4094], [1, 4094, 1], [1365, 1365, 1366], [100, 3000, 996]],
}


@pytest.mark.parametrize("alpha", [2, 3])
@pytest.mark.parametrize("lanes", [1, 2, 3])
@pytest.mark.parametrize("kmax", [0, 16])
def test_brute_force_round_trip(alpha, lanes, kmax):
    """Every sequence up to length 6 (multiple of R) over small alphabets."""
    for table in TABLES[alpha]:
        for length in range(lanes, 7, lanes):
            for seq in itertools.product(range(alpha), repeat=length):
                st, w, k = rans.encode_scalar(seq, table, lanes, 12, kmax)
                assert all(rans.L <= v < 2 ** 32 for v in st)
                assert all(0 <= v < 2 ** 16 for v in w)
                out = rans.decode_scalar(st, w, table, lanes, length // lanes, k, 12)
                assert tuple(out) == seq


@pytest.mark.parametrize("seed", range(12))
def test_vectorised_equals_scalar(seed):
    rng = np.random.default_rng(seed)
    alpha = int(rng.integers(2, 40))
    lanes = int(rng.choice([1, 2, 4, 16, 32, 64, 128]))
    steps = int(rng.integers(1, 40))
    tiles = int(rng.integers(1, 5))
    counts = rng.integers(1, 500, alpha) ** 2
    f = freq.quantize_freqs(counts, 12)
    p = f / f.sum()
    sym = rng.choice(alpha, size=(tiles, steps * lanes), p=p)
    kmax = int(rng.choice([0, 3, 16]))
    st, ws, ks = rans.encode_tiles(sym, f, lanes, 12, kmax)
    for t in range(tiles):
        s1, w1, k1 = rans.encode_scalar(sym[t], f, lanes, 12, kmax)
        assert list(st[t]) == s1 and list(ws[t]) == list(w1) and ks[t] == k1
        assert rans.decode_scalar(s1, w1, f, lanes, steps, k1, 12) == list(sym[t])
    out = rans.decode_tiles(st, ws, f, lanes, steps, ks, 12)
    assert np.array_equal(out, sym)


def test_size_near_entropy_and_above_gibbs_bound():
    """Stream bits >= N*H_emp - (state bits); <= N*H + 0.1 bit/sym at long lanes."""
    rng = np.random.default_rng(7)
    sym = np.clip(np.rint(rng.normal(8, 1.2, (64, 16384))), 0, 15).astype(np.int64)
    counts = entropy.histogram(sym, 16)
    h = entropy.entropy_from_counts(counts)
    f = freq.quantize_freqs(counts, 12)
    st, ws, ks = rans.encode_tiles(sym, f, 64, 12)
    bits = st.size * 32 + sum(len(w) for w in ws) * 16
    n = sym.size
    assert bits >= n * h - 32 * st.size   # a static code cannot beat H by more than its states
    assert bits / n <= h + 0.1


def test_integrity_errors():
    rng = np.random.default_rng(9)
    f = freq.quantize_freqs([5, 1, 30, 3], 12)
    sym = rng.choice(4, size=(1, 64 * 32), p=np.array([5, 1, 30, 3]) / 39)
    st, ws, ks = rans.encode_tiles(sym, f, 64, 12)
    # truncated stream
    with pytest.raises(rans.IntegrityError):
        rans.decode_tiles(st, [ws[0][:-1]], f, 64, 32, ks)
    # a corrupted state
    bad = st.copy()
    bad[0, 5] ^= 0x1234
    with pytest.raises(rans.IntegrityError):
        rans.decode_tiles(bad, ws, f, 64, 32, ks)
    # wrong payload count
    with pytest.raises(rans.IntegrityError):
        rans.decode_tiles(st, ws, f, 64, 32, ks + 1)


def test_zero_frequency_symbol_rejected():
    with pytest.raises(ValueError):
        rans.encode_scalar([0, 1], [4096, 0], 1)
    with pytest.raises(ValueError):
        rans.encode_tiles(np.array([[0, 1]]), [4096, 0], 1)


def test_constant_layer_costs_only_states():
    f = [0, 4096, 0]
    sym = np.ones((2, 64 * 16), dtype=np.int64)
    st, ws, ks = rans.encode_tiles(sym, f, 64, 12)
    assert all(len(w) == 0 for w in ws)
    assert (st == rans.L).all() and (ks == 16).all()
    assert np.array_equal(rans.decode_tiles(st, ws, f, 64, 16, ks), sym)


def test_payload_reduces_flush_cost():
    rng = np.random.default_rng(11)
    sym = np.clip(np.rint(rng.normal(8, 1.2, (32, 8192))), 0, 15).astype(np.int64)
    f = freq.quantize_freqs(entropy.histogram(sym, 16), 12)
    sizes = {}
    for kmax in (0, 16):
        st, ws, ks = rans.encode_tiles(sym, f, 64, 12, kmax)
        sizes[kmax] = st.size * 32 + sum(len(w) for w in ws) * 16
    per_lane_saving = (sizes[0] - sizes[16]) / (32 * 64)
    assert per_lane_saving > 4.0
    assert math.isfinite(per_lane_saving)
