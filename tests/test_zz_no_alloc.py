"""The allocation-free fused entry point (workspace in the library's static
device scratch) against the workspace entry point: identical outputs (both run
the same kernels in a fixed reduction order), on two calls in a row with the
second smaller, through the C ABI; oversize calls are refused."""

import numpy as np
import pytest

import decode_gemm_tile_amd as dgt
import workloads
from tests.gpu_util import to_dev, x_dev

pytestmark = pytest.mark.gpu

# (fmt, N, K, tile_n, tile_k, lanes, seed)
LAYERS = [
    (dgt.DGT_FMT_BF16_SPLIT, 512, 4096, 128, 64, 64, 91),
    (dgt.DGT_FMT_FP8_E4M3, 512, 1024, 256, 64, 64, 92),
    (dgt.DGT_FMT_INT4, 256, 2048, 128, 64, 64, 93),
    (dgt.DGT_FMT_INT8, 256, 512, 128, 32, 32, 94),
]


def _run_pair(fmt, n, k, tn, tk, lanes, seed, m):
    import torch
    d = workloads.random_small(fmt, n, k, seed=seed, m=m)
    layer = dgt.DeviceLayer(dgt.dgt_compress_layer(fmt, d["codes"], tn, tk, lanes))
    x = x_dev(d["x"])
    scales = to_dev(d["scales"]) if d["scales"] is not None else None
    ref = dgt.dgt_fused_decode_gemm(layer, x, scales=scales, w_scale=d["w_scale"])
    y = torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda")
    st = torch.full((layer.info.tiles,), -1, dtype=torch.int32, device="cuda")
    dgt.dgt_fused_decode_gemm_noalloc(layer, x, y, scales=scales, w_scale=d["w_scale"], status=st)
    torch.cuda.synchronize()
    assert torch.equal(y, ref), (fmt, m)
    assert int((st != 0).sum().item()) == 0


@pytest.mark.parametrize("layer", LAYERS)
def test_noalloc_matches_workspace_entry_point_twice(layer):
    # a first call, then a smaller one on the same scratch
    _run_pair(*layer, m=16)
    fmt, n, k, tn, tk, lanes, seed = layer
    _run_pair(fmt, n // 2, k // 2, tn, tk, lanes, seed + 100, m=3)


def test_noalloc_refuses_oversize_workspace():
    """fp8 8192 x 8192 at M = 256 needs 77 MiB of workspace: refused, nothing run."""
    import torch
    fmt, n, k = dgt.DGT_FMT_FP8_E4M3, 8192, 8192
    d = workloads.random_small(fmt, 1024, 1024, seed=95, m=1)
    codes = np.tile(d["codes"], (n // 1024, k // 1024))
    layer = dgt.DeviceLayer(dgt.dgt_compress_layer(fmt, codes, 256, 64, 64))
    m = 256
    assert dgt.dgt_gemm_workspace(layer, m) > dgt.dgt_noalloc_scratch_bytes()
    x = torch.zeros((m, k), dtype=torch.bfloat16, device="cuda")
    y = torch.zeros((m, n), dtype=torch.float32, device="cuda")
    with pytest.raises(dgt.DgtError) as e:
        dgt.dgt_fused_decode_gemm_noalloc(layer, x, y, w_scale=d["w_scale"])
    assert e.value.code == -4
    torch.cuda.synchronize()
    assert (y == 0).all()
