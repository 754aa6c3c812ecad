"""Integer frequency quantisation for the shared per-layer codebook (oracle).

[P1 §3.1]: all tiles of a layer share one compact ANS codebook.
[P1 §4.1]: the frequency table is normalised with finite precision, which
costs a little over the entropy.  The pages give no rule; the reading used
here (integer only, so that independent implementations agree bit for bit):

  M = 2**prob_bits, N = sum of counts, m = number of symbols with c_s > 0.
  1. m > M is an error; N == 0 is an error.
  2. f_s = 0 if c_s == 0, else max(1, floor(c_s * M / N)).
  3. d = M - sum(f).
  4. while d > 0: give +1 to the present symbols in order of remainder
     (c_s * M mod N) descending, ties by the smaller symbol, one pass.
  5. while d < 0: take 1 from the symbol with the largest f_s (ties by the
     smaller symbol) among those with f_s > 1.
  6. cumulative c_s = sum_{t < s} f_t in natural symbol order.
A layer with a single distinct symbol gets f = M (it then costs zero bits).
"""

import numpy as np


def quantize_freqs(counts, prob_bits: int = 12) -> np.ndarray:
    counts = [int(c) for c in np.asarray(counts).ravel()]
    M = 1 << prob_bits
    N = sum(counts)
    if N <= 0:
        raise ValueError("empty histogram")
    present = [s for s, c in enumerate(counts) if c > 0]
    if len(present) > M:
        raise ValueError("more distinct symbols than 2**prob_bits")
    f = [0] * len(counts)
    for s in present:
        f[s] = max(1, (counts[s] * M) // N)
    d = M - sum(f)
    if d > 0:
        # remainder descending, then smaller symbol first
        ranked = sorted(present, key=lambda s: (-((counts[s] * M) % N), s))
        for s in ranked:
            if d == 0:
                break
            f[s] += 1
            d -= 1
        if d != 0:  # cannot happen: sum of floors loses < 1 per present symbol
            raise AssertionError("quantisation did not converge")
    while d < 0:
        best = None
        for s in present:
            if f[s] > 1 and (best is None or f[s] > f[best]):
                best = s
        if best is None:
            raise AssertionError("cannot reduce frequencies")
        f[best] -= 1
        d += 1
    return np.asarray(f, dtype=np.int64)


def cumulative(freqs) -> np.ndarray:
    """c_s = sum of f_t for t < s, natural order; length alphabet + 1."""
    f = np.asarray(freqs, dtype=np.int64)
    c = np.zeros(f.size + 1, dtype=np.int64)
    c[1:] = np.cumsum(f)
    return c


def slot_to_symbol(freqs) -> np.ndarray:
    """For every slot r in [0, M): the symbol s with c_s <= r < c_s + f_s."""
    f = np.asarray(freqs, dtype=np.int64)
    return np.repeat(np.arange(f.size, dtype=np.int64), f)
