"""Interleaved R-lane rANS coder (oracle).

[P1 §2.2, §3.1]: rANS (asymmetric numeral systems) is the coder of choice:
near-entropy efficiency with byte-granular streaming decode; every tile's stream
is split into R independent sub-streams, one rANS state per warp lane, so the
serial state machine is spread over the lanes.  [P4] reference list: Duda's
ANS papers; the range variant (rANS) is written here from its definition.

Parameters (the pages fix none of them; readings):
  state x is an integer in [L, 2**32) with L = 2**16, renormalisation moves
  16-bit words, M = 2**n (n = prob_bits = 12 in the format), frequencies f_s,
  cumulative c_s (see ``oracle.freq``).

Encode one symbol s on a lane with state x:
  if x >= f_s * 2**(32-n): emit the word (x mod 2**16); x = floor(x / 2**16)
  x = floor(x / f_s) * M + (x mod f_s) + c_s
Decode one symbol from state x:
  r = x mod M;  s = the symbol with c_s <= r < c_s + f_s
  x = f_s * floor(x / M) + r - c_s
  if x < L: x = x * 2**16 + next_word

Interleaving of R lanes over S steps (symbol j = step*R + lane): the encoder
walks step = S-1 .. 0 and, inside a step, lane = R-1 .. 0, appending emitted
words to a list E.  The decoder walks step = 0 .. S-1 and lane = 0 .. R-1 and
lanes that renormalise take the next word of reverse(E), which is therefore
the stream.  The stored per-lane states are the encoder's final states.

Initial-state payload (a reading chosen to cut the per-lane flush cost): a
textbook encoder starts at x = L, so the 16 bits of the initial state carry
nothing.  Here the encoder first codes the first k encoded symbols of every
lane (the last k decoded: steps S-1 .. S-k) into y, starting from y = 0 and
with no renormalisation, then starts the normal coder at x = L + y.  k is the
largest value <= min(kmax, S) for which every lane of the tile keeps
y < 2**32 - L; it is stored per tile.  The decoder runs steps 0 .. S-k-1
normally, sets y = x - L, and decodes steps S-k .. S-1 from y without reading
words.  Integrity: every lane ends with y == 0 and the stream is consumed
exactly.  kmax = 0 gives the textbook coder.

Two implementations are given: ``encode_scalar`` / ``decode_scalar`` follow the
description literally with Python integers (tiny inputs), and
``encode_tiles`` / ``decode_tiles`` run the same steps with NumPy across many
tiles and lanes at once (lanes are independent; only the word order couples
them).  Tests pin the second against the first.
"""

import numpy as np

from .freq import cumulative, slot_to_symbol

STATE_BITS = 32
WORD_BITS = 16
L = 1 << 16          # lower bound of the normalised state interval
Y_LIMIT = (1 << 32) - L  # payload must keep L + y inside 32 bits
KMAX = 16            # payload steps per tile in the format


class IntegrityError(ValueError):
    """A tile stream did not decode back to the initial states / its length."""


def _enc_step(x, fs, cs, M):
    return (x // fs) * M + (x % fs) + cs


# ----------------------------------------------------------------- scalar form
def encode_scalar(symbols, freqs, lanes: int, prob_bits: int = 12, kmax: int = KMAX):
    """Literal encoder for one tile: returns (final_states[R], words, k)."""
    sym = [int(s) for s in np.asarray(symbols).ravel()]
    R = lanes
    if len(sym) % R:
        raise ValueError("symbol count must be a multiple of the lane count")
    S = len(sym) // R
    f = [int(v) for v in freqs]
    c = [int(v) for v in cumulative(freqs)]
    M = 1 << prob_bits
    if any(f[s] <= 0 for s in sym):
        raise ValueError("symbol with zero frequency")
    # payload phase: steps S-1, S-2, ... into y (no renormalisation)
    y = [0] * R
    k = 0
    while k < min(kmax, S):
        step = S - 1 - k
        cand = [_enc_step(y[r], f[sym[step * R + r]], c[sym[step * R + r]], M)
                for r in range(R)]
        if any(v >= Y_LIMIT for v in cand):
            break
        y = cand
        k += 1
    x = [L + v for v in y]
    E = []
    for step in range(S - 1 - k, -1, -1):
        for r in range(R - 1, -1, -1):
            s = sym[step * R + r]
            fs = f[s]
            if x[r] >= fs << (STATE_BITS - prob_bits):
                E.append(x[r] & 0xFFFF)
                x[r] >>= WORD_BITS
            x[r] = _enc_step(x[r], fs, c[s], M)
    return x, E[::-1], k


def decode_scalar(states, words, freqs, lanes: int, steps: int, k: int,
                  prob_bits: int = 12):
    """Literal decoder: returns the symbols in j order; checks integrity."""
    R = lanes
    f = [int(v) for v in freqs]
    c = [int(v) for v in cumulative(freqs)]
    sym_of = slot_to_symbol(freqs)
    M = 1 << prob_bits
    x = [int(v) for v in states]
    out = [0] * (steps * R)
    ptr = 0
    for step in range(steps):
        if step == steps - k:
            if any(v < L for v in x):
                raise IntegrityError("state below L at payload switch")
            x = [v - L for v in x]
        for r in range(R):
            slot = x[r] % M
            s = int(sym_of[slot])
            out[step * R + r] = s
            x[r] = f[s] * (x[r] // M) + slot - c[s]
            if step < steps - k and x[r] < L:
                if ptr >= len(words):
                    raise IntegrityError("stream exhausted")
                x[r] = (x[r] << WORD_BITS) | int(words[ptr])
                ptr += 1
    final = 0 if k > 0 else L
    if any(v != final for v in x) or ptr != len(words):
        raise IntegrityError("final state / stream length mismatch")
    return out


# ------------------------------------------------------------ vectorised form
def encode_tiles(symbols, freqs, lanes: int, prob_bits: int = 12, kmax: int = KMAX):
    """Encode many tiles at once.

    symbols: [tiles, T] symbol indices in j order (T = S*R).
    Returns (states [tiles, R] uint32, words: list of uint16 arrays in stream
    (decoder) order, ks [tiles] payload step counts).
    """
    sym = np.asarray(symbols, dtype=np.int64)
    if sym.ndim == 1:
        sym = sym[None, :]
    tiles, T = sym.shape
    R = lanes
    if T % R:
        raise ValueError("symbol count must be a multiple of the lane count")
    S = T // R
    f = np.asarray(freqs, dtype=np.int64)
    c = cumulative(f)
    M = 1 << prob_bits
    if (f[sym] <= 0).any():
        raise ValueError("symbol with zero frequency")
    s3 = sym.reshape(tiles, S, R)

    y = np.zeros((tiles, R), dtype=np.int64)
    ks = np.zeros(tiles, dtype=np.int64)
    alive = np.ones(tiles, dtype=bool)
    for k in range(min(kmax, S)):
        ss = s3[:, S - 1 - k, :]
        cand = _enc_step(y, f[ss], c[ss], M)
        ok = alive & (cand < Y_LIMIT).all(axis=1)
        y = np.where(ok[:, None], cand, y)
        ks += ok
        alive = ok
    x = L + y

    emit = np.zeros((tiles, S, R), dtype=bool)
    word = np.zeros((tiles, S, R), dtype=np.uint16)
    for step in range(S - 1, -1, -1):
        active = (step < S - ks)[:, None]  # this step is a normal-coder step
        ss = s3[:, step, :]
        fs = f[ss]
        e = active & (x >= (fs << (STATE_BITS - prob_bits)))
        emit[:, step, :] = e
        word[:, step, :] = (x & 0xFFFF).astype(np.uint16)
        xr = np.where(e, x >> WORD_BITS, x)
        x = np.where(active, _enc_step(xr, fs, c[ss], M), x)
    # E is appended in (step desc, lane desc) order, so reverse(E) lists the
    # emitted words in (step asc, lane asc) order: boolean selection in C order.
    words = [word[t][emit[t]] for t in range(tiles)]
    return x.astype(np.uint32), words, ks


def decode_tiles(states, words, freqs, lanes: int, steps: int, ks, prob_bits: int = 12,
                 check: bool = True, return_consumed: bool = False):
    """Decode many tiles at once.

    states: [tiles, R]; words: list of per-tile uint16 arrays (stream order);
    ks: per-tile payload step counts.  Returns symbols [tiles, S*R] in j order
    (and, with return_consumed, the words each tile consumed).  Raises
    IntegrityError if a stream under-runs, if a lane does not end at its
    initial value, or (check=True) if a stream is not consumed exactly.
    """
    x = np.asarray(states, dtype=np.int64).copy()
    if x.ndim == 1:
        x = x[None, :]
    tiles, R = x.shape
    if R != lanes:
        raise ValueError("state count does not match lanes")
    ks = np.broadcast_to(np.asarray(ks, dtype=np.int64), (tiles,))
    f = np.asarray(freqs, dtype=np.int64)
    c = cumulative(f)
    sym_of = slot_to_symbol(f)
    M = 1 << prob_bits
    if sym_of.size != M:
        raise ValueError("frequencies do not sum to 2**prob_bits")
    nwords = np.array([len(w) for w in words], dtype=np.int64)
    width = int(nwords.max()) if tiles else 0
    warr = np.zeros((tiles, width + 1), dtype=np.int64)
    for t, w in enumerate(words):
        warr[t, : len(w)] = w
    ptr = np.zeros(tiles, dtype=np.int64)
    out = np.zeros((tiles, steps, R), dtype=np.int64)
    rows = np.arange(tiles)[:, None]
    for step in range(steps):
        switch = (step == steps - ks)[:, None]
        if (switch & (x < L)).any():
            raise IntegrityError("state below L at payload switch")
        x = np.where(switch, x - L, x)
        normal = (step < steps - ks)[:, None]
        slot = x & (M - 1)
        s = sym_of[slot]
        out[:, step, :] = s
        x = f[s] * (x >> prob_bits) + slot - c[s]
        need = normal & (x < L)
        rank = np.cumsum(need, axis=1) - need
        idx = ptr[:, None] + rank
        if (need & (idx >= nwords[:, None])).any():
            raise IntegrityError("stream exhausted")
        w = warr[rows, np.minimum(idx, width)]
        x = np.where(need, (x << WORD_BITS) | w, x)
        ptr += need.sum(axis=1)
    final = np.where(ks > 0, 0, L)[:, None]
    if (x != final).any():
        raise IntegrityError("final state mismatch")
    if check and (ptr != nwords).any():
        raise IntegrityError("stream length mismatch")
    out = out.reshape(tiles, steps * R)
    return (out, ptr) if return_consumed else out
