"""Number formats the GEMM consumes (oracle, fp64).

[P1 §2.1] lists the formats whose symbols are coded (bf16, fp8, int8, int4,
awq4 among them); [P1 §2.1 end] and [P1 §5] note the coding is orthogonal to
quantisation: the coded symbols are the quantised codes themselves, and the
GEMM consumes the values those codes stand for.  The pages give no arithmetic
for this step; the readings used (plain, standard definitions):

  bf16     : the top 16 bits of an IEEE fp32; fp32 -> bf16 rounds to nearest,
             ties to even (RNE).
  e4m3     : OCP FP8 E4M3 ("fn": bias 7, no infinities, 0x7F/0xFF are NaN,
             max finite 448); fp32 -> e4m3 rounds to nearest even and
             saturates finite values to +-448.
  int8     : the code's own integer value (exact in bf16).
  int4     : code q in [0, 15] with zero point 8 and one bf16 scale per group
             of 128 along K: value = bf16_RNE(fp32(q - 8) * fp32(scale)).
  fp8 path : activations are quantised per tensor before the fp8 product:
             amax = max|x|, inv = fl32(448 / amax), sx = fl32(amax / 448),
             xq = e4m3(fl32(x * inv)); Y = sx * sw * (Xq . Wq^T).
"""

import numpy as np

E4M3_MAX = 448.0


# ---------------------------------------------------------------------- bf16
def bf16_bits_to_f64(bits) -> np.ndarray:
    b = (np.asarray(bits, dtype=np.uint32) << 16).astype(np.uint32)
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def f32_to_bf16_bits(x) -> np.ndarray:
    """Round fp32 values (given as float32) to bf16 bit patterns, RNE."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    is_nan = np.isnan(np.asarray(x, dtype=np.float32))
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) & 0xFFFF
    r = np.where(is_nan, (u >> 16) | 0x40, r)  # quiet NaN keeps its sign
    return r.astype(np.uint16)


# ---------------------------------------------------------------------- e4m3
def e4m3_to_f64(codes) -> np.ndarray:
    b = np.asarray(codes, dtype=np.int64) & 0xFF
    sign = np.where(b & 0x80, -1.0, 1.0)
    exp = (b >> 3) & 0xF
    man = b & 0x7
    val = np.where(exp == 0, man * 2.0 ** -9,
                   (1.0 + man / 8.0) * np.exp2(exp.astype(np.float64) - 7.0))
    val = np.where((exp == 15) & (man == 7), np.nan, val)
    return sign * val


def _e4m3_positive_table():
    codes = np.arange(0, 0x7F, dtype=np.int64)  # 0x00 .. 0x7E: all finite >= 0
    return codes, e4m3_to_f64(codes)


def f64_to_e4m3(x) -> np.ndarray:
    """Nearest e4m3 code, ties to the even code, finite values saturate."""
    x = np.asarray(x, dtype=np.float64)
    codes, vals = _e4m3_positive_table()  # ascending values
    a = np.abs(x)
    a_c = np.minimum(a, E4M3_MAX)
    hi = np.searchsorted(vals, a_c, side="left")  # first value >= a
    hi = np.minimum(hi, vals.size - 1)
    lo = np.maximum(hi - 1, 0)
    d_hi = vals[hi] - a_c
    d_lo = a_c - vals[lo]
    pick_lo = (d_lo < d_hi) | ((d_lo == d_hi) & ((codes[lo] & 1) == 0))
    mag = np.where(pick_lo, codes[lo], codes[hi])
    mag = np.where(vals[hi] == a_c, codes[hi], mag)
    out = np.where(np.signbit(x), mag | 0x80, mag)
    out = np.where(np.isnan(x), 0x7F, out)
    return out.astype(np.uint8)


# ----------------------------------------------------------- decoded values
def int4_dequant_bf16_bits(q, scales_bf16_bits, group: int = 128) -> np.ndarray:
    """bf16 bits of bf16_RNE(fp32(q - 8) * fp32(scale[n, k // group]))."""
    q = np.asarray(q, dtype=np.int64)
    n, k = q.shape
    s = bf16_bits_to_f64(scales_bf16_bits).reshape(n, k // group)
    s_full = np.repeat(s, group, axis=1)
    prod = (q - 8).astype(np.float64) * s_full  # exact: <= 4 x 8 significant bits
    return f32_to_bf16_bits(prod.astype(np.float32))


def fp8_quantize_activations(x_bf16_bits):
    """Per-tensor e4m3 quantisation of bf16 activations.

    Returns (xq codes uint8, sx float32 value as Python float).
    """
    x = bf16_bits_to_f64(x_bf16_bits)
    amax = float(np.abs(x).max()) if x.size else 0.0
    if amax == 0.0 or not np.isfinite(amax):
        return np.zeros(x.shape, dtype=np.uint8), 1.0
    inv = float(np.float32(E4M3_MAX / amax))
    sx = float(np.float32(amax / E4M3_MAX))
    scaled = (x * inv).astype(np.float32).astype(np.float64)
    return f64_to_e4m3(scaled), sx
