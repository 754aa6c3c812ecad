"""Empirical Shannon entropy of a layer's symbol histogram (oracle).

[P1 §2.1]: each layer's weights are treated as a sequence of discrete symbols,
an empirical histogram is taken and its Shannon entropy computed.
[P2 "实验方法"]: Shannon entropy of a discrete random variable X over the
value set chi with probability mass p; the formula itself did not survive
extraction, the plain reading is H(X) = -sum_x p(x) log2 p(x).
"""

import numpy as np


def histogram(symbols, alphabet: int) -> np.ndarray:
    """Counts c_s of every symbol s in [0, alphabet) (int64)."""
    s = np.asarray(symbols).ravel().astype(np.int64)
    if s.size and (s.min() < 0 or s.max() >= alphabet):
        raise ValueError("symbol outside alphabet")
    return np.bincount(s, minlength=alphabet).astype(np.int64)


def entropy_from_counts(counts) -> float:
    """H = -sum p log2 p with p = c/N over symbols with c > 0, in fp64 bits."""
    c = np.asarray(counts, dtype=np.float64)
    n = c.sum()
    if n <= 0:
        return 0.0
    p = c[c > 0] / n
    return float(-(p * np.log2(p)).sum())


def empirical_entropy(symbols, alphabet: int) -> float:
    """Entropy in bits per symbol of the empirical histogram of ``symbols``."""
    return entropy_from_counts(histogram(symbols, alphabet))
