"""The Python binding rejects malformed arguments before anything reaches the
C ABI (which receives raw device pointers and cannot see shapes, dtypes,
layouts or devices), and never falls back to the CPU.  Host-only: the layer's
"device" copy is a CPU tensor here, so every call must raise."""

import numpy as np
import pytest
import torch

import decode_gemm_tile_amd as dgt
import workloads


class _HostLayer:
    """Stand-in for DeviceLayer whose blob sits in host memory."""

    def __init__(self, blob):
        self.info = dgt.dgt_layer_info(blob)
        self.blob = torch.frombuffer(bytearray(blob), dtype=torch.uint8)
        self.nbytes = len(blob)


def _layer(fmt, n=256, k=512, tn=128, tk=64, lanes=64):
    d = workloads.random_small(fmt, n, k, seed=5)
    return _HostLayer(dgt.dgt_compress_layer(fmt, d["codes"], tn, tk, lanes)), d


def _x(m, k, dtype=torch.bfloat16):
    return torch.zeros((m, k), dtype=dtype)


def _raises(match, fn, *a, **kw):
    with pytest.raises(ValueError, match=match):
        fn(*a, **kw)


def test_fused_rejects_bad_x():
    layer, _ = _layer(dgt.DGT_FMT_BF16_SPLIT)
    _raises("x has dtype", dgt.dgt_fused_decode_gemm, layer, _x(4, 512, torch.float32))
    _raises("x has shape", dgt.dgt_fused_decode_gemm, layer, _x(4, 256))
    _raises("x has shape", dgt.dgt_fused_decode_gemm, layer, torch.zeros(512, dtype=torch.bfloat16))
    _raises("x must be contiguous", dgt.dgt_fused_decode_gemm, layer, _x(512, 8).t())
    _raises("x is required", dgt.dgt_fused_decode_gemm, layer, None)


def test_fused_rejects_bad_y_status_ws():
    layer, _ = _layer(dgt.DGT_FMT_BF16_SPLIT)
    x = _x(4, 512)
    _raises("y has shape", dgt.dgt_fused_decode_gemm, layer, x,
            y=torch.zeros((4, 255), dtype=torch.float32))
    _raises("y has dtype", dgt.dgt_fused_decode_gemm, layer, x,
            y=torch.zeros((4, 256), dtype=torch.float16))
    _raises("status holds", dgt.dgt_fused_decode_gemm, layer, x,
            y=torch.zeros((4, 256)), status=torch.zeros(layer.info.tiles - 1, dtype=torch.int32))
    _raises("status has dtype", dgt.dgt_fused_decode_gemm, layer, x,
            y=torch.zeros((4, 256)), status=torch.zeros(layer.info.tiles, dtype=torch.int64))
    _raises("ws has dtype", dgt.dgt_fused_decode_gemm, layer, x, y=torch.zeros((4, 256)),
            ws=torch.zeros(4096, dtype=torch.float32))


def test_fused_rejects_bad_scales():
    layer, d = _layer(dgt.DGT_FMT_INT4)
    x = _x(2, 512)
    _raises("scales is required", dgt.dgt_fused_decode_gemm, layer, x)
    _raises("scales has shape", dgt.dgt_fused_decode_gemm, layer, x,
            scales=torch.zeros((256, 3), dtype=torch.int16))
    _raises("scales has dtype", dgt.dgt_fused_decode_gemm, layer, x,
            scales=torch.zeros((256, 4), dtype=torch.float32))
    layer8, _ = _layer(dgt.DGT_FMT_INT8)
    _raises("only taken by the int4", dgt.dgt_fused_decode_gemm, layer8, x,
            scales=torch.zeros((256, 4), dtype=torch.int16))


def test_no_cpu_fallback():
    """Well-formed host tensors are refused too: the library computes on the GPU only."""
    layer, _ = _layer(dgt.DGT_FMT_BF16_SPLIT)
    _raises("arguments must be in GPU memory", dgt.dgt_fused_decode_gemm, layer, _x(4, 512),
            y=torch.zeros((4, 256)))
    _raises("arguments must be in GPU memory", dgt.dgt_decode_tiles, layer,
            out=torch.zeros((256, 512), dtype=torch.int16))


def test_decode_rejects_bad_ids_and_out():
    layer, _ = _layer(dgt.DGT_FMT_INT8)
    tiles = layer.info.tiles
    out = torch.zeros((256, 512), dtype=torch.uint8)
    _raises("tile ids must lie", dgt.dgt_decode_tiles, layer, tile_ids=[0, tiles], out=out)
    _raises("tile ids must lie", dgt.dgt_decode_tiles, layer, tile_ids=[-1], out=out)
    _raises("tile ids must lie", dgt.dgt_decode_tiles, layer,
            tile_ids=np.array([3, 2 ** 32 - 1], np.int64), out=out)
    _raises("1-D integer", dgt.dgt_decode_tiles, layer, tile_ids=[0.5], out=out)
    _raises("out has shape", dgt.dgt_decode_tiles, layer,
            out=torch.zeros((256, 511), dtype=torch.uint8))
    _raises("out has dtype", dgt.dgt_decode_tiles, layer,
            out=torch.zeros((256, 512), dtype=torch.int16))
    layer16, _ = _layer(dgt.DGT_FMT_BF16_SPLIT)
    _raises("out has dtype", dgt.dgt_decode_tiles, layer16,
            out=torch.zeros((256, 512), dtype=torch.uint8))


def test_dense_rejects_bad_arguments():
    w = torch.zeros((256, 512), dtype=torch.uint8)
    _raises("x has shape", dgt.dgt_dense_gemm, dgt.DGT_FMT_INT8, w, _x(2, 256))
    _raises("w has dtype", dgt.dgt_dense_gemm, dgt.DGT_FMT_BF16_SPLIT, w, _x(2, 512))
    _raises("scales is required", dgt.dgt_dense_gemm, dgt.DGT_FMT_INT4, w, _x(2, 512))
    _raises("arguments must be in GPU memory", dgt.dgt_dense_gemm, dgt.DGT_FMT_INT8, w, _x(2, 512))
