"""Tile partition and tile-local symbol order (oracle).

[P1 §3.1]: offline, each layer is cut into tiles in the downstream GEMM's
tiling geometry (e.g. 128x32, 256x64); every tile is an independently decodable
sub-stream, and each tile's stream is split into R sub-streams, one rANS state
per lane.  The pages do not fix which lane codes which element nor in which
order; the reading used here follows the matrix-core operand layout so that a
lane's decoded values are directly its operand for a 16-row x 32-deep product:

Layer W is [N, K] row-major (out x in).  Tile (bn, bk) covers rows
bn*Tn .. bn*Tn+Tn-1 and columns bk*Tk .. bk*Tk+Tk-1; tile id t = bn*(K/Tk)+bk.

Inside a tile (Tn % 16 == 0, R % 16 == 0, FW = R/2 divides Tk):
  fragments of 16 rows x FW columns; Fn = Tn/16, Fk = Tk/FW, G = Fn*Fk;
  fragment index g = fk*Fn + fn  (all row bands of column block 0 first);
  lane p in [0, R): row a = p % 16 of the band, column group cg = p // 16;
  element e in [0, 8): column cg*8 + e of the fragment;
  (row, col) in tile = (fn*16 + a, fk*FW + cg*8 + e);
  decode step s = g*8 + e (S = T/R steps), symbol index j = s*R + p.
So at every step each of the R lanes decodes one symbol, and after 8 steps a
lane holds 8 consecutive-column values of one row.

Raw (uncoded) bytes of a tile, where a format stores them, are kept in the
lane-major order q = g*8*R + p*8 + e, i.e. a lane's 8 values are contiguous.

Formats whose symbol packs two weights (int4 pairs) apply the same map to
the matrix of symbols with epl = 4 symbols per lane per fragment: a fragment
is then 16 rows x (R/16)*4 symbols, i.e. the same 16 x R/2 weights, and a
lane's 4 symbols are its 8 consecutive-column weights.

Two states per lane (R = 128, a reading for a 64-wide wavefront: the pages
put one state on each of the warp's lanes and leave R free): the tile's top
Tn/2 rows and bottom Tn/2 rows are two halves, each ordered as an R = 64 tile
of shape (Tn/2) x Tk; state p < 64 codes the top half's lane p, state 64 + p
the bottom half's lane p, and both share the tile's one word stream through
the interleaving j = s*128 + p.  A wave lane p then holds states p and
64 + p, whose values at a step are the same column of two row bands, so the
two matrix-core products of a fragment share their X operand.  Raw bytes:
q = g*1024 + p*8 + e with p in [0, 128), the half's R = 64 raw order.
"""

import numpy as np


def check_geometry(n: int, k: int, tile_n: int, tile_k: int, lanes: int,
                   epl: int = 8) -> None:
    if min(n, k, tile_n, tile_k, lanes) <= 0:
        raise ValueError("sizes must be positive")
    if n % tile_n or k % tile_k:
        raise ValueError("N and K must be multiples of the tile shape")
    if lanes == 128:  # two R = 64 halves of Tn/2 rows
        if tile_n % 32:
            raise ValueError("two states per lane need tile_n a multiple of 32")
        lanes = 64
    if lanes % 16 or tile_n % 16:
        raise ValueError("lanes and tile_n must be multiples of 16")
    if tile_k % ((lanes // 16) * epl):
        raise ValueError("tile_k must be a multiple of the fragment width")


def _halves(pos_of_half, tile_n: int, count: int, per_block: int):
    """Positions for R = 128 from the R = 64 positions of a (Tn/2)-row half:
    index i splits into (block b, state p in [0,128), rest) with per_block
    entries per state; p // 64 picks the half, p % 64 the half's lane."""
    i = np.arange(count, dtype=np.int64)
    b, rem = i // (128 * per_block), i % (128 * per_block)
    p, r = rem // per_block, rem % per_block
    h = p // 64
    i_half = (b * 64 + p % 64) * per_block + r
    rows, cols = pos_of_half
    return rows[i_half] + h * (tile_n // 2), cols[i_half]


def tile_positions(tile_n: int, tile_k: int, lanes: int, epl: int = 8):
    """(rows[j], cols[j]) inside the tile for symbol index j = s*R + p."""
    if lanes == 128:
        half = tile_positions(tile_n // 2, tile_k, 64, epl)
        return _halves(half, tile_n, tile_n * tile_k, 1)
    R = lanes
    fw = (R // 16) * epl
    fn_count = tile_n // 16
    fk_count = tile_k // fw
    T = tile_n * tile_k
    j = np.arange(T, dtype=np.int64)
    s, p = j // R, j % R
    g, e = s // epl, s % epl
    fk, fn = g // fn_count, g % fn_count
    a, cg = p % 16, p // 16
    rows = fn * 16 + a
    cols = fk * fw + cg * epl + e
    assert fk.max() < fk_count
    return rows, cols


def raw_positions(tile_n: int, tile_k: int, lanes: int):
    """(rows[q], cols[q]) inside the tile for raw-byte index q = g*8R + p*8 + e."""
    if lanes == 128:
        half = raw_positions(tile_n // 2, tile_k, 64)
        return _halves(half, tile_n, tile_n * tile_k, 8)
    R = lanes
    fw = R // 2
    fn_count = tile_n // 16
    T = tile_n * tile_k
    q = np.arange(T, dtype=np.int64)
    g, rem = q // (8 * R), q % (8 * R)
    p, e = rem // 8, rem % 8
    fk, fn = g // fn_count, g % fn_count
    rows = fn * 16 + p % 16
    cols = fk * fw + (p // 16) * 8 + e
    return rows, cols


def tile_origin(t: int, k: int, tile_n: int, tile_k: int):
    kt = k // tile_k
    return (t // kt) * tile_n, (t % kt) * tile_k


def _positions(tile_n, tile_k, lanes, raw, epl):
    if raw:
        return raw_positions(tile_n, tile_k, lanes)
    return tile_positions(tile_n, tile_k, lanes, epl)


def gather_tiles(w, tile_n: int, tile_k: int, lanes: int, raw: bool = False, epl: int = 8):
    """[tiles, T] array: tile t's elements in symbol order (or raw order)."""
    w = np.asarray(w)
    n, k = w.shape
    check_geometry(n, k, tile_n, tile_k, lanes, 8 if raw else epl)
    rows, cols = _positions(tile_n, tile_k, lanes, raw, epl)
    nt, kt = n // tile_n, k // tile_k
    # view W as [nt, Tn, kt, Tk] -> [nt, kt, Tn, Tk]
    blocks = w.reshape(nt, tile_n, kt, tile_k).transpose(0, 2, 1, 3)
    blocks = blocks.reshape(nt * kt, tile_n, tile_k)
    return blocks[:, rows, cols]


def scatter_tiles(tiles, n: int, k: int, tile_n: int, tile_k: int, lanes: int,
                  raw: bool = False, epl: int = 8):
    """Inverse of gather_tiles: rebuild [N, K] from per-tile ordered values."""
    tiles = np.asarray(tiles)
    check_geometry(n, k, tile_n, tile_k, lanes, 8 if raw else epl)
    rows, cols = _positions(tile_n, tile_k, lanes, raw, epl)
    nt, kt = n // tile_n, k // tile_k
    blocks = np.zeros((nt * kt, tile_n, tile_k), dtype=tiles.dtype)
    blocks[:, rows, cols] = tiles
    return blocks.reshape(nt, kt, tile_n, tile_k).transpose(0, 2, 1, 3).reshape(n, k)
