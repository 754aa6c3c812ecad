"""Alternative codings of bf16 weights (a size study on the oracle, CPU only).

[P1 §4.1] codes bf16 with 16-bit symbols and notes a table-precision cost;
[P2] (DFloat11) codes the 8-bit exponent and stores sign and mantissa.  The
library decodes the byte split (format 4) and the exponent split (format 6);
full 16-bit symbols need a decode table of 2^n slots with n well above the
12 bits a 160 KB LDS holds beside the staged streams, so they are sized here
only, with the oracle's own coder run at n = 13..16.
"""

import numpy as np

import workloads
from oracle import blob, entropy, freq, order, rans


def _sixteen_bit_bits_per_weight(w, prob_bits, tile_n=128, tile_k=64, lanes=64):
    """Blob bits/weight with each bf16 pattern one symbol (alphabet 65536):
    header, a u16 table of 65536 entries, index, payload counts, streams."""
    w = np.asarray(w, dtype=np.uint16)
    n, k = w.shape
    counts = np.bincount(w.ravel(), minlength=65536)
    f = freq.quantize_freqs(counts, prob_bits)
    ts = order.gather_tiles(w.astype(np.int64), tile_n, tile_k, lanes)
    states, words, ks = rans.encode_tiles(ts, f, lanes, prob_bits)
    tiles = ts.shape[0]
    nwords = sum(len(x) + (len(x) & 1) for x in words)
    total = 128 + 2 * 65536 + 4 * (tiles + 1) + tiles + 4 * lanes * tiles + 2 * nwords
    return 8.0 * total / (n * k), (f, ts, states, words, ks)


def test_sixteen_bit_symbols_round_trip_at_n16():
    d = workloads.random_small(blob.FMT_BF16, 128, 128, seed=21)
    w = np.asarray(d["codes"])
    _, (f, ts, states, words, ks) = _sixteen_bit_bits_per_weight(w, 16)
    out = rans.decode_tiles(states, words, f, 64, 128 * 64 // 64, ks, 16)
    assert np.array_equal(np.asarray(out), ts)


def test_bf16_codings_order_on_a_layer_slice():
    """On 1024 rows of the 14336x4096 bf16 layer: 16-bit symbols at n = 16 <
    exponent split < byte split; at n = 13 (the largest table a decode LUT of
    64 KB holds) the 16-bit code loses its edge to the table precision."""
    d = workloads.make("bf16_mlp")
    w = np.asarray(d["codes"])[:1024]
    n, k = w.shape
    byte = blob.bits_per_weight(blob.compress_layer(blob.FMT_BF16, w, 128, 64, 64), n, k)
    expo = blob.bits_per_weight(blob.compress_layer(blob.FMT_BF16_EXP, w, 128, 64, 64), n, k)
    # the 65536-entry table is 1 bit/weight per 131072 weights: compare streams
    table_share = 8.0 * (2 * 65536 - 2 * 256) / (n * k)
    b16, _ = _sixteen_bit_bits_per_weight(w, 16)
    b13, _ = _sixteen_bit_bits_per_weight(w, 13)
    h16 = entropy.empirical_entropy(w, 65536)
    assert h16 < b16 - table_share < expo < byte
    assert b13 - table_share > byte
    assert 0.08 < byte - expo < 0.2
