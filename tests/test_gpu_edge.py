"""GPU parity on the degenerate tables the method has.

- a constant layer: one symbol with f = 2^12, so every decode step is a
  zero-bit step and a tile's streams are its R states alone;
- one rare symbol among a constant field (f = 1 for it);
- full 8-bit alphabets (every int8 byte; every finite e4m3 code);
- constant bf16 layers in the four bf16 codings (one high byte, one
  exponent, one high-byte pair, one whole word: f = 2^16) and a two-valued
  one (four high-byte pairs); one rare whole word (f = 1).

Each layer decodes bit-exactly (every tile status 0) and the fused GEMM is
within 1e-5 relative Frobenius of the fp64 oracle at M = 1 and 16; for the
constant bf16 layer at 1.0 the oracle's result is also checked against the
closed form Y[m, n] = sum_k X[m, k]."""

import zlib

import numpy as np
import pytest

import decode_gemm_tile_amd as dgt
from oracle import blob as oblob
from oracle import numerics
from tests.gpu_util import (codes_as_u8_or_u16, decoded_to_numpy, reference, rel_err, to_dev,
                            x_dev)

pytestmark = pytest.mark.gpu
TOL = 1e-5
N, K = 256, 512


def _bf16(a):
    return numerics.f32_to_bf16_bits(np.asarray(a, np.float32))


def _x(rng, m):
    return _bf16(rng.normal(0.0, 1.0, (m, K)))


def _layer(name, rng):
    d = {"w_scale": 1.0, "scales": None}
    if name == "int4_constant":
        fmt, codes = dgt.DGT_FMT_INT4, np.full((N, K), 3, np.uint8)
    elif name == "int4_rare_symbol":
        fmt, codes = dgt.DGT_FMT_INT4, np.full((N, K), 8, np.uint8)
        codes[17, 301] = 15
    elif name == "int4_pair_constant":
        fmt, codes = dgt.DGT_FMT_INT4_PAIR, np.full((N, K), 11, np.uint8)
    elif name == "int8_all_bytes":
        fmt = dgt.DGT_FMT_INT8
        codes = rng.integers(0, 256, (N, K)).astype(np.uint8).view(np.int8)
        codes.flat[:256] = np.arange(256, dtype=np.uint8).view(np.int8)
    elif name == "fp8_all_finite_codes":
        fmt = dgt.DGT_FMT_FP8_E4M3
        finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
        codes = rng.choice(finite, (N, K))
        codes.flat[:finite.size] = finite
        d["w_scale"] = 0.01
    elif name.startswith("bf16_constant"):
        fmt = {"split": dgt.DGT_FMT_BF16_SPLIT, "exp": dgt.DGT_FMT_BF16_EXP,
               "pair": dgt.DGT_FMT_BF16_PAIR, "word": dgt.DGT_FMT_BF16_WORD}[name.split("_")[-1]]
        codes = np.full((N, K), 0x3F80, np.uint16)  # 1.0
    elif name == "bf16_rare_word":
        # one word among 2^17 (f = 1) and copies of another (f = 2^16 - 1)
        fmt, codes = dgt.DGT_FMT_BF16_WORD, np.full((N, K), 0x3C24, np.uint16)
        codes[77, 401] = 0xC2F0
    elif name == "bf16_many_rare_words":
        # 6000 words once each (f = 1, runs of starts inside every 4-slot
        # bucket) around one common word
        fmt, codes = dgt.DGT_FMT_BF16_WORD, np.full((N, K), 0x3F80, np.uint16)
        words = np.array([w for w in range(0x3000, 0x3000 + 6001) if w != 0x3F80], np.uint16)
        codes.flat[rng.permutation(N * K)[:words.size]] = words
    elif name == "bf16_two_values_pair":
        fmt = dgt.DGT_FMT_BF16_PAIR
        codes = np.where(rng.random((N, K)) < 0.3, 0xBC24, 0x3C24).astype(np.uint16)
    else:
        raise KeyError(name)
    if fmt in (dgt.DGT_FMT_INT4, dgt.DGT_FMT_INT4_PAIR):
        d["scales"] = _bf16(rng.uniform(0.005, 0.015, (N, K // 128)))
    d["codes"] = codes
    d["x"] = _x(rng, 16)
    return fmt, d


NAMES = ["int4_constant", "int4_rare_symbol", "int4_pair_constant", "int8_all_bytes",
         "fp8_all_finite_codes", "bf16_constant_split", "bf16_constant_exp",
         "bf16_constant_pair", "bf16_two_values_pair"]


WORD_NAMES = ["bf16_constant_word", "bf16_rare_word", "bf16_many_rare_words"]


@pytest.mark.parametrize("name,R", [(n, r) for n in NAMES for r in (32, 64, 128)] +
                         [(n, 64) for n in WORD_NAMES])  # whole words: 64 lanes
def test_degenerate_layer_decodes_and_multiplies(name, R):
    import torch
    rng = np.random.default_rng(zlib.crc32(("%s/%d" % (name, R)).encode()))
    fmt, d = _layer(name, rng)
    blob = dgt.dgt_compress_layer(fmt, d["codes"], 128, 64, R)
    assert np.array_equal(codes_as_u8_or_u16(fmt, oblob.decompress_layer(blob)),
                          codes_as_u8_or_u16(fmt, d["codes"]))
    layer = dgt.DeviceLayer(blob)
    status = torch.full((layer.info.tiles,), -1, dtype=torch.int32, device="cuda")
    out = dgt.dgt_decode_tiles(layer, status=status)
    torch.cuda.synchronize()
    assert np.array_equal(decoded_to_numpy(fmt, out), codes_as_u8_or_u16(fmt, d["codes"]))
    assert (status.cpu().numpy() == 0).all()
    scales = to_dev(d["scales"]) if d["scales"] is not None else None
    for m in (1, 16):
        xb = d["x"][:m]
        status.fill_(-1)
        y = dgt.dgt_fused_decode_gemm(layer, x_dev(xb), scales=scales, w_scale=d["w_scale"],
                                      status=status)
        torch.cuda.synchronize()
        ref = reference(fmt, d, xb)
        if name in ("bf16_constant_split", "bf16_constant_word"):
            closed = numerics.bf16_bits_to_f64(xb).sum(axis=1, keepdims=True) * np.ones((1, N))
            assert np.allclose(ref, closed, rtol=0, atol=1e-9)
        assert rel_err(y.cpu().numpy(), ref) <= TOL, (name, R, m)
        assert (status.cpu().numpy() == 0).all()
