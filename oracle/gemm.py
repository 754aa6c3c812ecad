"""fp64 reference GEMM Y = X W^T over the decoded weights (oracle).

[P1 §3.1]: the decoded tile feeds the GEMM that consumes it; the method is
lossless ([P1 §1]: decompressed weights are bit-identical to the originals),
so the product it computes has a plain definition: the ordinary matrix
product with the original weights.  W is [N, K] (out x in), X is [M, K],
Y = X . W^T is [M, N], evaluated here in fp64 from exactly representable
inputs (bf16 activations, decoded weight values).
"""

import numpy as np

from . import numerics

FMT_INT8, FMT_INT4, FMT_FP8, FMT_BF16, FMT_INT4_PAIR, FMT_BF16_EXP = 1, 2, 3, 4, 5, 6
FMT_BF16_PAIR = 7
FMT_BF16_WORD = 8


def gemm_fp64(x, w) -> np.ndarray:
    """Y[m, n] = sum_k x[m, k] * w[n, k] in float64 (library matmul)."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    return x @ w.T


def gemm_loop(x, w) -> np.ndarray:
    """The same product as explicit sums (small shapes; pins gemm_fp64)."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    m, k = x.shape
    n = w.shape[0]
    y = np.zeros((m, n))
    for i in range(m):
        for j in range(n):
            acc = 0.0
            for t in range(k):
                acc += x[i, t] * w[j, t]
            y[i, j] = acc
    return y


def weight_values(fmt: int, codes, scales_bf16_bits=None) -> np.ndarray:
    """fp64 values of the weights the GEMM consumes, per format.

    int8: the signed code; int4 (single or pair symbols: the same codes and
    values, only the coding differs): bf16_RNE((q-8)*scale); fp8: the e4m3 value
    (the per-tensor weight scale is applied to the product, not here);
    bf16 (any of the four codings): the bf16 value of the 16-bit pattern.
    """
    if fmt == FMT_INT8:
        return np.asarray(codes).astype(np.int8).astype(np.float64)
    if fmt in (FMT_INT4, FMT_INT4_PAIR):
        bits = numerics.int4_dequant_bf16_bits(codes, scales_bf16_bits)
        return numerics.bf16_bits_to_f64(bits)
    if fmt == FMT_FP8:
        return numerics.e4m3_to_f64(codes)
    if fmt in (FMT_BF16, FMT_BF16_EXP, FMT_BF16_PAIR, FMT_BF16_WORD):
        return numerics.bf16_bits_to_f64(codes)
    raise ValueError("unknown format")


def reference_output(fmt: int, codes, x_bf16_bits, scales_bf16_bits=None,
                     w_scale: float = 1.0) -> np.ndarray:
    """Y64 for the fused product: fp64 of what the device must compute."""
    w = weight_values(fmt, codes, scales_bf16_bits)
    if fmt == FMT_FP8:
        xq, sx = numerics.fp8_quantize_activations(x_bf16_bits)
        return (float(sx) * float(w_scale)) * gemm_fp64(numerics.e4m3_to_f64(xq), w)
    return gemm_fp64(numerics.bf16_bits_to_f64(x_bf16_bits), w)


def rel_frobenius(y, ref) -> float:
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    num = np.linalg.norm(y - ref)
    return float(num / den) if den > 0 else float(num)
