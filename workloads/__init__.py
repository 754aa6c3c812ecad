"""Seeded synthetic inputs shared by the tests, the bench and the oracle's callers.

This module only draws random inputs with the shapes and value distributions
of the workloads; it holds none of the coding or GEMM arithmetic, and both the
HIP library's callers and the CPU oracle's callers read its outputs.  The
method's pages measure real checkpoints (Qwen, Llama, Mistral, Mixtral); none
are available, so these draws stand in for them.

Recipe (numpy.random.default_rng(seed); W first, then scales, then X):
  int8_1024     W 1024x1024 int8 = rint(N(0, 8)) clipped to [-127, 127];
                X bf16 [16, 1024] N(0, 1).  Tiles 128x32, 32 lanes.
  int4_4096     W 4096x4096 codes rint(N(8, 1.2)) clipped to [0, 15]; scales
                bf16 [4096, 32] N(0.01, 0.002) redrawn while <= 0 (one per 128
                columns); X bf16 [16, 4096] N(0, 1).  Tiles 128x64, 32 lanes.
  fp8_8192      W 8192x8192 bf16 N(0, 0.02), per-tensor scale
                sw = fl32(amax|W| / 448), codes = e4m3(fl32(W / sw)) (torch's
                cast); X bf16 [64, 8192] N(0, 1).  Tiles 256x64, 64 lanes.
  bf16_mlp      W 14336x4096 bf16 N(0, 0.02) (Llama-3-8B MLP projection shape);
                X bf16 [256, 4096] N(0, 1).  Tiles 256x64, 64 lanes.
  int4_ffn405   W 53248x16384 int4 rint(N(8, 1.0)) clipped, scales as int4_4096;
                X bf16 [256, 16384].  Tiles 256x64, 64 lanes.
  int4_4096_pair, int4_ffn405_pair: the two int4 layers above (same seeds,
                same draws) in the pair-symbol format.
  bf16_mlp_exp  the bf16_mlp layer (same seed, same draws) in the exponent split.
  bf16_mlp_pair, bf16_ffn405_pair: the two bf16 layers (same seeds, same draws)
                in the byte split with the high bytes coded in pairs.
  bf16_mlp_word, bf16_ffn405_word: the same layers coded as whole 16-bit
                words, frequency precision 16 bits.
  *_r128        the named layer (same seed, same draws) coded with two rANS
                states per lane (R = 128: tile halves of tile_n/2 rows).
  bf16_mlp_t128, int4_ffn405_t128, bf16_mlp_r32, int4_ffn405_r32,
  int4_4096_r64 the named layer (same draws) in another tile geometry
                (128x64 tiles; 32 or 64 lanes).
Where the configuration leaves the tile geometry or the lane count free, the
default is one whose compressed size stays within 0.1 bit per weight of the
empirical entropy (256x64 tiles, or 32 lanes at 128x64).
  bf16_ffn405   W 53248x16384 bf16 N(0, 0.01); X bf16 [256, 16384].
                Tiles 256x64, 64 lanes.
rint is numpy's (ties to even); clipping follows rounding.  Casts to bf16 and
e4m3 are torch's CPU casts (round to nearest even).
"""

from dataclasses import dataclass, field

import numpy as np

FMT_INT8, FMT_INT4, FMT_FP8, FMT_BF16, FMT_INT4_PAIR, FMT_BF16_EXP = 1, 2, 3, 4, 5, 6
FMT_BF16_PAIR = 7
FMT_BF16_WORD = 8
_BF16_FORMATS = (FMT_BF16, FMT_BF16_EXP, FMT_BF16_PAIR, FMT_BF16_WORD)
_CHUNK = 1 << 24


@dataclass(frozen=True)
class Workload:
    name: str
    fmt: int
    n: int
    k: int
    tile_n: int
    tile_k: int
    lanes: int
    seed: int
    m_values: tuple
    w_sigma: float = 0.0
    w_mean: float = 0.0
    prob_bits: int = 12
    note: str = field(default="", compare=False)

    @property
    def m_max(self) -> int:
        return max(self.m_values)


WORKLOADS = {
    "int8_1024": Workload("int8_1024", FMT_INT8, 1024, 1024, 128, 32, 32, 101, (16,),
                          w_sigma=8.0, note="int8 codes, H ~ 5 bits"),
    "int4_4096": Workload("int4_4096", FMT_INT4, 4096, 4096, 128, 64, 32, 202, (1, 16),
                          w_sigma=1.2, w_mean=8.0, note="AWQ-style int4 + group-128 scales"),
    "fp8_8192": Workload("fp8_8192", FMT_FP8, 8192, 8192, 256, 64, 64, 303, (1, 16, 64),
                         w_sigma=0.02, note="e4m3 with per-tensor scale"),
    "bf16_mlp": Workload("bf16_mlp", FMT_BF16, 14336, 4096, 256, 64, 64, 404, (1, 8, 64, 256),
                         w_sigma=0.02, note="bf16 N(0,0.02) byte split, Llama-3-8B MLP shape"),
    "int4_ffn405": Workload("int4_ffn405", FMT_INT4, 53248, 16384, 256, 64, 64, 505,
                            (1, 8, 64, 256), w_sigma=1.0, w_mean=8.0,
                            note="405B-scale FFN, int4"),
    "bf16_ffn405": Workload("bf16_ffn405", FMT_BF16, 53248, 16384, 256, 64, 64, 506,
                            (1, 8, 64, 256), w_sigma=0.01, note="405B-scale FFN, bf16"),
    # the same int4 layers (same seeds, codes and scales) coded two weights per symbol
    "int4_4096_pair": Workload("int4_4096_pair", FMT_INT4_PAIR, 4096, 4096, 128, 64, 32, 202,
                               (1, 16), w_sigma=1.2, w_mean=8.0,
                               note="int4_4096 coded as int4 pairs"),
    "int4_ffn405_pair": Workload("int4_ffn405_pair", FMT_INT4_PAIR, 53248, 16384, 256, 64, 64,
                                 505, (1, 8, 64, 256), w_sigma=1.0, w_mean=8.0,
                                 note="int4_ffn405 coded as int4 pairs"),
    # the bf16 MLP layer (same draws) with its exponent coded, sign + mantissa raw
    "bf16_mlp_exp": Workload("bf16_mlp_exp", FMT_BF16_EXP, 14336, 4096, 256, 64, 64, 404,
                             (1, 8, 64, 256), w_sigma=0.02,
                             note="bf16 N(0,0.02) exponent split, Llama-3-8B MLP shape"),
}
# the bf16 layers (same draws) with the high bytes of adjacent weights coded in pairs
for _base in ("bf16_mlp", "bf16_ffn405"):
    _w = WORKLOADS[_base]
    WORKLOADS[_base + "_pair"] = Workload(
        _base + "_pair", FMT_BF16_PAIR, _w.n, _w.k, _w.tile_n, _w.tile_k, _w.lanes, _w.seed,
        _w.m_values, w_sigma=_w.w_sigma, prob_bits=_w.prob_bits,
        note=_w.note + ", high bytes coded in pairs")
# the same layers in other tile geometries (the configurations leave tile shape
# or lane count free for these): 256x64 tiles, or 32 lanes per tile
for _base, _tn, _tk, _r, _suffix in (("bf16_mlp", 128, 64, 64, "_t128"),
                                     ("bf16_mlp", 128, 64, 32, "_r32"),
                                     ("int4_ffn405", 128, 64, 64, "_t128"),
                                     ("int4_ffn405", 128, 64, 32, "_r32"),
                                     ("int4_4096", 128, 64, 64, "_r64")):
    _w = WORKLOADS[_base]
    WORKLOADS[_base + _suffix] = Workload(
        _base + _suffix, _w.fmt, _w.n, _w.k, _tn, _tk, _r, _w.seed, _w.m_values,
        w_sigma=_w.w_sigma, w_mean=_w.w_mean, prob_bits=_w.prob_bits,
        note=_w.note + ", the other tile geometry")
# the bf16 layers (same draws) coded as whole 16-bit words at 16-bit precision
for _base in ("bf16_mlp", "bf16_ffn405"):
    _w = WORKLOADS[_base]
    WORKLOADS[_base + "_word"] = Workload(
        _base + "_word", FMT_BF16_WORD, _w.n, _w.k, _w.tile_n, _w.tile_k, _w.lanes, _w.seed,
        _w.m_values, w_sigma=_w.w_sigma, prob_bits=16,
        note=_w.note.replace("byte split", "whole 16-bit words"))
# two states per lane: the same layers with R = 128
for _base in ("int4_4096", "fp8_8192", "bf16_mlp", "int4_ffn405", "bf16_ffn405"):
    _w = WORKLOADS[_base]
    WORKLOADS[_base + "_r128"] = Workload(
        _base + "_r128", _w.fmt, _w.n, _w.k, _w.tile_n, _w.tile_k, 128, _w.seed, _w.m_values,
        w_sigma=_w.w_sigma, w_mean=_w.w_mean, prob_bits=_w.prob_bits,
        note=_w.note + ", two states per lane (R = 128)")


def _normal(rng, count: int, mean: float, sigma: float) -> np.ndarray:
    out = np.empty(count, dtype=np.float64)
    for s in range(0, count, _CHUNK):
        e = min(count, s + _CHUNK)
        out[s:e] = rng.normal(mean, sigma, e - s)
    return out


def _to_bf16_bits(values_f64) -> np.ndarray:
    import torch
    t = torch.from_numpy(np.ascontiguousarray(values_f64, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def _normal_bf16_bits(rng, count: int, mean: float, sigma: float) -> np.ndarray:
    """Same draws and casts as _to_bf16_bits(_normal(...)), chunk by chunk."""
    out = np.empty(count, dtype=np.uint16)
    for s in range(0, count, _CHUNK):
        e = min(count, s + _CHUNK)
        out[s:e] = _to_bf16_bits(rng.normal(mean, sigma, e - s))
    return out


def _int_codes(rng, n, k, mean, sigma, lo, hi) -> np.ndarray:
    out = np.empty(n * k, dtype=np.int16)
    for s in range(0, n * k, _CHUNK):
        e = min(n * k, s + _CHUNK)
        out[s:e] = np.clip(np.rint(rng.normal(mean, sigma, e - s)), lo, hi)
    return out.reshape(n, k)


def _scales(rng, rows: int, groups: int) -> np.ndarray:
    s = rng.normal(0.01, 0.002, rows * groups)
    bad = s <= 0
    while bad.any():
        s[bad] = rng.normal(0.01, 0.002, int(bad.sum()))
        bad = s <= 0
    return _to_bf16_bits(s).reshape(rows, groups)


def make_weights(wl: Workload, rng=None):
    """Return dict with 'codes' (the stored weights) and, where the format has
    them, 'scales' (bf16 bits [N, K/128]) and 'w_scale' (fp32 per-tensor)."""
    if rng is None:
        rng = np.random.default_rng(wl.seed)
    n, k = wl.n, wl.k
    out = {"w_scale": 1.0, "scales": None}
    if wl.fmt == FMT_INT8:
        out["codes"] = _int_codes(rng, n, k, 0.0, wl.w_sigma, -127, 127).astype(np.int8)
    elif wl.fmt in (FMT_INT4, FMT_INT4_PAIR):
        out["codes"] = _int_codes(rng, n, k, wl.w_mean, wl.w_sigma, 0, 15).astype(np.uint8)
        out["scales"] = _scales(rng, n, k // 128)
    elif wl.fmt == FMT_FP8:
        import torch
        wb = _normal_bf16_bits(rng, n * k, 0.0, wl.w_sigma).reshape(n, k)
        wt = torch.from_numpy(wb.view(np.int16)).view(torch.bfloat16).float()
        amax = wt.abs().max()
        sw = (amax / 448.0).to(torch.float32)
        q = (wt / sw).to(torch.float8_e4m3fn)
        out["codes"] = q.view(torch.uint8).numpy().copy()
        out["w_scale"] = float(sw)
    elif wl.fmt in _BF16_FORMATS:
        out["codes"] = _normal_bf16_bits(rng, n * k, 0.0, wl.w_sigma).reshape(n, k)
    else:
        raise ValueError("unknown format")
    return out


def make_activations(wl: Workload, m: int, rng) -> np.ndarray:
    """bf16 bits [m, K] drawn N(0, 1)."""
    return _to_bf16_bits(rng.normal(0.0, 1.0, m * wl.k)).reshape(m, wl.k)


def make(wl_name: str, m: int = None):
    """Weights then activations ([m_max, K], first m rows returned if m given)."""
    wl = WORKLOADS[wl_name]
    rng = np.random.default_rng(wl.seed)
    d = make_weights(wl, rng)
    x = make_activations(wl, wl.m_max, rng)
    d["x"] = x if m is None else x[:m].copy()
    d["workload"] = wl
    return d


def random_small(fmt: int, n: int, k: int, seed: int, sigma: float = None,
                 mean: float = None, m: int = 4):
    """Small seeded layer of any shape for parity cases (same distributions)."""
    rng = np.random.default_rng(seed)
    d = {"w_scale": 1.0, "scales": None}
    if fmt == FMT_INT8:
        d["codes"] = _int_codes(rng, n, k, 0.0, 8.0 if sigma is None else sigma,
                                -127, 127).astype(np.int8)
    elif fmt in (FMT_INT4, FMT_INT4_PAIR):
        d["codes"] = _int_codes(rng, n, k, 8.0 if mean is None else mean,
                                1.2 if sigma is None else sigma, 0, 15).astype(np.uint8)
        d["scales"] = _scales(rng, n, k // 128) if k % 128 == 0 else None
    elif fmt == FMT_FP8:
        import torch
        wb = _to_bf16_bits(_normal(rng, n * k, 0.0, 0.02 if sigma is None else sigma))
        wt = torch.from_numpy(wb.view(np.int16)).view(torch.bfloat16).float()
        sw = (wt.abs().max() / 448.0).to(torch.float32)
        d["codes"] = (wt / sw).to(torch.float8_e4m3fn).view(torch.uint8).numpy().reshape(n, k).copy()
        d["w_scale"] = float(sw)
    elif fmt in _BF16_FORMATS:
        d["codes"] = _to_bf16_bits(_normal(rng, n * k, 0.0,
                                           0.02 if sigma is None else sigma)).reshape(n, k)
    d["x"] = _to_bf16_bits(rng.normal(0.0, 1.0, m * k)).reshape(m, k)
    return d
