"""Pins for oracle.order: bijections and hand-checked positions."""

import numpy as np
import pytest

from oracle import order

GEOMS = [(16, 8, 16), (16, 32, 64), (128, 32, 32), (128, 64, 64), (256, 64, 64),
         (32, 16, 32), (48, 24, 16), (32, 64, 128), (128, 64, 128), (256, 64, 128),
         (96, 128, 128)]


@pytest.mark.parametrize("tn,tk,R", GEOMS)
def test_positions_are_bijections(tn, tk, R):
    for fn in (order.tile_positions, order.raw_positions):
        r, c = fn(tn, tk, R)
        assert r.min() == 0 and r.max() == tn - 1 and c.min() == 0 and c.max() == tk - 1
        lin = r * tk + c
        assert np.array_equal(np.sort(lin), np.arange(tn * tk))


def test_hand_checked_positions_r64():
    r, c = order.tile_positions(32, 64, 64)
    # j = step*64 + lane; lane p -> row p%16, column group p//16 (8 columns each)
    assert (r[0], c[0]) == (0, 0)
    assert (r[1], c[1]) == (1, 0)
    assert (r[16], c[16]) == (0, 8)
    assert (r[63], c[63]) == (15, 24 + 0)
    assert (r[64], c[64]) == (0, 1)          # step 1 = element 1 of lane 0
    assert (r[7 * 64 + 63], c[7 * 64 + 63]) == (15, 31)
    assert (r[8 * 64], c[8 * 64]) == (16, 0)  # fragment 1 = second row band
    assert (r[16 * 64], c[16 * 64]) == (0, 32)  # fragment 2 = next column block


def test_hand_checked_positions_r32():
    r, c = order.tile_positions(128, 32, 32)
    assert (r[31], c[31]) == (15, 8)   # lane 31: row 15, column group 1
    assert (r[32], c[32]) == (0, 1)    # step 1
    assert (r[8 * 32], c[8 * 32]) == (16, 0)
    assert (r[8 * 8 * 32], c[8 * 8 * 32]) == (0, 16)  # after 8 row bands: column block 1


def test_hand_checked_positions_two_states_per_lane():
    """R = 128 on a 64x64 tile: states 0..63 walk the top 32 rows as an R = 64
    tile would, states 64..127 the bottom 32 rows."""
    r, c = order.tile_positions(64, 64, 128)
    assert (r[0], c[0]) == (0, 0)
    assert (r[17], c[17]) == (1, 8)            # state 17: row 1, column group 1
    assert (r[64], c[64]) == (32, 0)           # state 64 = lane 0 of the bottom half
    assert (r[127], c[127]) == (47, 24)        # state 127 = lane 63 of the bottom half
    assert (r[128], c[128]) == (0, 1)          # step 1
    assert (r[8 * 128], c[8 * 128]) == (16, 0)       # fragment 1: the half's second band
    assert (r[16 * 128], c[16 * 128]) == (0, 32)     # fragment 2: next column block
    assert (r[16 * 128 + 64], c[16 * 128 + 64]) == (32, 32)
    # raw bytes: block g = 0 holds state p's 8 values at q = p*8 + e
    rr, cr = order.raw_positions(64, 64, 128)
    assert (rr[8 * 64 + 3], cr[8 * 64 + 3]) == (32, 3)
    assert (rr[1024], cr[1024]) == (16, 0)


@pytest.mark.parametrize("tn,tk", [(64, 64), (128, 64), (256, 64), (64, 128)])
def test_two_states_share_the_column_of_two_row_bands(tn, tk):
    """At every step, a wave lane's two states (p and 64 + p) decode the same
    column in rows Tn/2 apart, and over 8 steps lane p's values form the
    matrix-core operand of its row (p % 16) and 8 columns (8 * (p // 16) + e)."""
    r, c = order.tile_positions(tn, tk, 128)
    S = tn * tk // 128
    for s in range(S):
        for p in range(64):
            ja, jb = s * 128 + p, s * 128 + 64 + p
            assert c[ja] == c[jb] and r[jb] == r[ja] + tn // 2
            assert r[ja] % 16 == p % 16 and (c[ja] % 32) == 8 * (p // 16) + s % 8


@pytest.mark.parametrize("tn,tk,R", GEOMS)
def test_raw_order_is_lane_major_symbol_order(tn, tk, R):
    """raw index q = g*8R + p*8 + e holds the element of symbol j = (8g+e)*R + p."""
    rs, cs = order.tile_positions(tn, tk, R)
    rr, cr = order.raw_positions(tn, tk, R)
    T = tn * tk
    q = np.arange(T)
    g, p, e = q // (8 * R), (q % (8 * R)) // 8, q % 8
    j = (8 * g + e) * R + p
    assert np.array_equal(rr, rs[j]) and np.array_equal(cr, cs[j])


def test_gather_scatter_inverse():
    rng = np.random.default_rng(0)
    w = rng.integers(0, 256, (256, 192)).astype(np.uint8)
    for R, tn, tk in [(64, 128, 64), (32, 128, 32), (16, 16, 8), (128, 128, 64), (128, 64, 64)]:
        for raw in (False, True):
            t = order.gather_tiles(w, tn, tk, R, raw=raw)
            assert t.shape == ((256 // tn) * (192 // tk), tn * tk)
            assert np.array_equal(order.scatter_tiles(t, 256, 192, tn, tk, R, raw=raw), w)
    # tile id t = bn*(K/Tk) + bk, and the first symbol of a tile is its corner
    t = order.gather_tiles(w, 128, 64, 64)
    assert t[1, 0] == w[0, 64] and t[3, 0] == w[128, 0]


def test_geometry_errors():
    for args in [(100, 64, 128, 64, 64), (128, 64, 128, 64, 48), (128, 64, 120, 64, 64),
                 (128, 48, 128, 48, 64), (96, 64, 48, 64, 128), (128, 16, 128, 16, 128)]:
        with pytest.raises(ValueError):
            order.check_geometry(*args)


@pytest.mark.parametrize("tn,tk,R", [(32, 16, 16), (128, 32, 64), (128, 16, 32), (256, 32, 64),
                                     (128, 32, 128), (64, 64, 128)])
def test_pair_positions_cover_each_lanes_eight_weights(tn, tk, R):
    """Pair layout (epl = 4 on the [rows, tk] pair matrix, i.e. tiles of 2*tk
    weights): lane p's 4 symbols of fragment g are exactly the weights that
    lane p decodes at fragment g in the one-weight layout, two per symbol in
    column order (symbol e covers weight columns 2e and 2e + 1)."""
    rows, cols = order.tile_positions(tn, tk, R, epl=4)
    rows1, cols1 = order.tile_positions(tn, 2 * tk, R)
    S = tn * tk // R
    for s in range(S):
        g, e = divmod(s, 4)
        for p in range(R):
            j = s * R + p
            j_lo = (8 * g + 2 * e) * R + p
            j_hi = (8 * g + 2 * e + 1) * R + p
            assert (rows[j], 2 * cols[j]) == (rows1[j_lo], cols1[j_lo])
            assert (rows[j], 2 * cols[j] + 1) == (rows1[j_hi], cols1[j_hi])
    # and it is a bijection on the pair tile
    assert len(set(zip(rows.tolist(), cols.tolist()))) == tn * tk
