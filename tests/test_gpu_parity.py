"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Decoded weights must be bit-exact (the method is lossless: the decoded layer is
the input itself, and the oracle's decoder gives the same symbols); GEMM
outputs (fp32 accumulation) must be within 1e-5 relative Frobenius error of the
fp64 oracle.  Sizes span several tiles, several workgroups per strip and
ragged wave/workgroup tails."""

import numpy as np
import pytest

import decode_gemm_tile_amd as dgt
import workloads
from oracle import blob as oblob
from oracle import gemm as ogemm
from tests.gpu_util import (codes_as_u8_or_u16, decoded_to_numpy, reference, rel_err, to_dev,
                            x_dev)

pytestmark = pytest.mark.gpu
TOL = 1e-5

F8, F4, FE, FB, FP, FX = (dgt.DGT_FMT_INT8, dgt.DGT_FMT_INT4, dgt.DGT_FMT_FP8_E4M3,
                          dgt.DGT_FMT_BF16_SPLIT, dgt.DGT_FMT_INT4_PAIR, dgt.DGT_FMT_BF16_EXP)
FH = dgt.DGT_FMT_BF16_PAIR
FW = dgt.DGT_FMT_BF16_WORD

# (fmt, N, K, tile_n, tile_k, lanes, seed)
CASES = [
    (F8, 256, 512, 128, 32, 32, 1),       # 32 lanes: two tiles per wave
    (F8, 384, 256, 128, 64, 64, 2),
    (F4, 256, 1024, 128, 64, 64, 3),
    (F4, 128, 384, 128, 64, 32, 4),       # ragged: 6 k-tiles
    (FE, 512, 448, 256, 64, 64, 5),       # 7 k-tiles: odd count
    (FE, 256, 256, 128, 32, 32, 6),
    (FB, 384, 640, 128, 64, 64, 7),
    (FB, 512, 192, 256, 64, 64, 8),
    (FB, 256, 4096, 128, 64, 64, 9),      # 64 k-tiles: several workgroups per strip
    (FP, 256, 1024, 128, 64, 64, 10),     # int4 pairs: 4 symbols per lane per fragment
    (FP, 128, 768, 128, 64, 32, 11),      # int4 pairs, two tiles per wave
    (FP, 512, 2048, 256, 64, 64, 12),     # int4 pairs, tile_n 256
    (FX, 384, 1024, 128, 64, 64, 13),     # bf16 exponent split
    (FX, 256, 256, 128, 32, 32, 14),      # bf16 exponent split, two tiles per wave
    # two states per lane (R = 128)
    (F8, 256, 512, 128, 32, 128, 15),
    (F4, 256, 1024, 128, 64, 128, 16),
    (FE, 512, 448, 256, 64, 128, 17),     # 7 k-tiles, tile_n 256
    (FB, 384, 640, 128, 64, 128, 18),
    (FB, 256, 4096, 128, 64, 128, 19),    # several workgroups per strip
    (FP, 256, 1024, 128, 64, 128, 20),
    (FX, 384, 1024, 128, 64, 128, 22),
    # bf16 byte split with high-byte pairs (16-bit symbols)
    (FH, 384, 1024, 128, 64, 64, 23),
    (FH, 512, 448, 256, 64, 64, 24),      # tile_n 256, 7 k-tiles
    (FH, 256, 256, 128, 32, 32, 25),      # two tiles per wave
    (FH, 256, 4096, 128, 64, 64, 26),     # several workgroups per strip
    (FH, 384, 1024, 128, 64, 128, 27),    # two states per lane
    # bf16 whole words (16-bit symbols at 16-bit precision, 64 lanes)
    (FW, 384, 1024, 128, 64, 64, 28),
    (FW, 512, 448, 256, 64, 64, 29),      # tile_n 256, 7 k-tiles
    (FW, 256, 4096, 128, 64, 64, 30),     # several workgroups per strip
]


def _layer(fmt, n, k, tn, tk, R, seed, m=16):
    d = workloads.random_small(fmt, n, k, seed=seed, m=m)
    blob = dgt.dgt_compress_layer(fmt, d["codes"], tn, tk, R)
    return d, blob


@pytest.mark.parametrize("fmt,n,k,tn,tk,R,seed", CASES)
def test_decode_tiles_bit_exact(fmt, n, k, tn, tk, R, seed):
    import torch
    d, blob = _layer(fmt, n, k, tn, tk, R, seed)
    layer = dgt.DeviceLayer(blob)
    status = torch.full((layer.info.tiles,), -1, dtype=torch.int32, device="cuda")
    out = dgt.dgt_decode_tiles(layer, status=status)
    torch.cuda.synchronize()
    got = decoded_to_numpy(fmt, out)
    assert np.array_equal(got, codes_as_u8_or_u16(fmt, d["codes"]))
    assert (status.cpu().numpy() == 0).all()
    # the oracle's decoder agrees symbol for symbol
    assert np.array_equal(oblob.decompress_layer(blob), d["codes"])


@pytest.mark.parametrize("fmt,n,k,tn,tk,R,seed", CASES[:4] + CASES[6:7])
def test_decode_tile_subset(fmt, n, k, tn, tk, R, seed):
    import torch
    d, blob = _layer(fmt, n, k, tn, tk, R, seed)
    layer = dgt.DeviceLayer(blob)
    tiles = layer.info.tiles
    ids = [tiles - 1, 0, tiles // 2] if tiles > 2 else [0]
    out = dgt.dgt_decode_tiles(layer, tile_ids=ids)
    torch.cuda.synchronize()
    got = decoded_to_numpy(fmt, out)
    want = codes_as_u8_or_u16(fmt, d["codes"])
    kt = k // tk
    mask = np.zeros((n, k), bool)
    for t in ids:
        r0, c0 = (t // kt) * tn, (t % kt) * tk
        mask[r0:r0 + tn, c0:c0 + tk] = True
    assert np.array_equal(got[mask], want[mask])
    assert (got[~mask] == 0).all()


@pytest.mark.parametrize("fmt,n,k,tn,tk,R,seed", CASES)
@pytest.mark.parametrize("m", [1, 2, 5, 8, 16, 33, 64, 100])
def test_fused_gemm_matches_fp64_oracle(fmt, n, k, tn, tk, R, seed, m):
    import torch
    if fmt in (F4, FP) and k % 128:
        pytest.skip("int4 needs K % 128 == 0 for its scale groups")
    d, blob = _layer(fmt, n, k, tn, tk, R, seed, m=m)
    layer = dgt.DeviceLayer(blob)
    scales = to_dev(d["scales"]) if d["scales"] is not None else None
    status = torch.full((layer.info.tiles,), -1, dtype=torch.int32, device="cuda")
    y = dgt.dgt_fused_decode_gemm(layer, x_dev(d["x"]), scales=scales, w_scale=d["w_scale"],
                                  status=status)
    torch.cuda.synchronize()
    ref = reference(fmt, d, d["x"])
    assert rel_err(y.cpu().numpy(), ref) <= TOL
    assert (status.cpu().numpy() == 0).all()


# Large M: every tile decoded once and its fragments shared through LDS by the
# waves that own the row blocks (tile_n 128: 16 waves x 16 rows; tile_n 256:
# 8 waves x 32 rows).  Shapes cover strips finished by one workgroup (direct
# store) and by several (workspace hand-off), ragged M and idle row blocks.
XM_CASES = [
    (FB, 256, 1024, 128, 64, 64, 41),     # one batch per strip
    (FB, 384, 4096, 128, 64, 64, 42),     # four workgroups per strip
    (F8, 256, 2048, 128, 64, 64, 43),
    (F4, 256, 2048, 128, 64, 64, 44),
    (FE, 512, 1024, 256, 64, 64, 45),     # tile_n 256: two batches per strip
    (FB, 512, 512, 256, 64, 64, 46),
    (F4, 256, 1024, 256, 64, 64, 47),
    (FP, 384, 2048, 128, 64, 64, 49),     # int4 pairs
    (FP, 512, 1024, 256, 64, 64, 50),
    (FX, 256, 2048, 128, 64, 64, 51),     # bf16 exponent split
    (FH, 384, 1024, 128, 64, 64, 57),     # bf16 high-byte pairs (16-bit symbols)
    (FH, 512, 1024, 256, 64, 64, 58),
    (FB, 256, 8192, 256, 64, 64, 59),     # tile_n 256, eight batches per strip
    (FW, 384, 2048, 128, 64, 64, 60),     # bf16 whole words
    (FW, 512, 1024, 256, 64, 64, 61),
    (FB, 384, 4096, 128, 64, 128, 55),    # two states per lane: two operands per fragment
    (FE, 512, 1024, 256, 64, 128, 56),
    (F4, 256, 2048, 128, 64, 128, 57),
    (FP, 512, 1024, 256, 64, 128, 58),
    (FX, 256, 2048, 128, 64, 128, 59),
    (FH, 384, 2048, 128, 64, 64, 62),     # bf16 high-byte pairs
    (FH, 512, 1024, 256, 64, 64, 63),
    (FH, 256, 2048, 128, 64, 128, 64),
]


@pytest.mark.parametrize("fmt,n,k,tn,tk,R,seed", XM_CASES)
@pytest.mark.parametrize("m", [17, 64, 65, 100, 128, 256])
def test_fused_gemm_large_m_matches_fp64_oracle(fmt, n, k, tn, tk, R, seed, m):
    import torch
    d, blob = _layer(fmt, n, k, tn, tk, R, seed, m=m)
    layer = dgt.DeviceLayer(blob)
    scales = to_dev(d["scales"]) if d["scales"] is not None else None
    status = torch.full((layer.info.tiles,), -1, dtype=torch.int32, device="cuda")
    ws = dgt.alloc_workspace(dgt.dgt_gemm_workspace(layer, m))
    y = dgt.dgt_fused_decode_gemm(layer, x_dev(d["x"]), scales=scales, w_scale=d["w_scale"],
                                  status=status, ws=ws)
    torch.cuda.synchronize()
    ref = reference(fmt, d, d["x"])
    assert rel_err(y.cpu().numpy(), ref) <= TOL
    assert (status.cpu().numpy() == 0).all()
    strips = n // tn
    assert int(ws[:4 * strips].sum().item()) == 0   # strip counters returned to zero


@pytest.mark.parametrize("fmt,n,k,tn,tk,R,seed", [c for c in XM_CASES if c[5] == 64])
@pytest.mark.parametrize("staging", ["ring", "whole"])
def test_large_m_single_buffer_matches_oracle(fmt, n, k, tn, tk, R, seed, staging, monkeypatch):
    """The large-M kernel with one fragment buffer (a barrier after every
    group's products instead of ping-pong buffers) gives the oracle's results
    and the same values as the two-buffer kernel."""
    import torch
    monkeypatch.setenv("DGT_STAGING", staging)
    monkeypatch.setenv("DGT_XM_SUBSETS", "0")  # the 8-wave form, which has the one-buffer rung
    d, blob = _layer(fmt, n, k, tn, tk, R, seed, m=100)
    layer = dgt.DeviceLayer(blob)
    scales = to_dev(d["scales"]) if d["scales"] is not None else None
    ws = dgt.alloc_workspace(dgt.dgt_gemm_workspace(layer, 100))
    y2 = dgt.dgt_fused_decode_gemm(layer, x_dev(d["x"]), scales=scales, w_scale=d["w_scale"],
                                   ws=ws).clone()
    monkeypatch.setenv("DGT_XM_SINGLE_BUFFER", "1")
    status = torch.full((layer.info.tiles,), -1, dtype=torch.int32, device="cuda")
    y1 = dgt.dgt_fused_decode_gemm(layer, x_dev(d["x"]), scales=scales, w_scale=d["w_scale"],
                                   status=status, ws=ws)
    torch.cuda.synchronize()
    assert rel_err(y1.cpu().numpy(), reference(fmt, d, d["x"])) <= TOL
    assert torch.equal(y1, y2)
    assert (status.cpu().numpy() == 0).all()


# The 16-wave subset form of the large-M kernel (256-row tiles, 64 lanes,
# M <= 128): each wave multiplies a quarter (M <= 64) or half (M <= 128) of a
# batch's 16 tiles and the subsets' sums are added through LDS.
@pytest.mark.parametrize("staging", ["ring", "whole"])
@pytest.mark.parametrize("k", [1024, 4096])
@pytest.mark.parametrize("m", [17, 64, 65, 128])
def test_large_m_subsets_exact_integer_case(m, k, staging, monkeypatch):
    """int8 W at 256x64 tiles and integer X in [-4, 4]: every fp32 partial sum
    is an integer below 2^24, so the subset kernel and the 8-wave kernel must
    both give the fp64 product exactly (one strip per workgroup at K = 1024,
    four workgroups per strip at K = 4096)."""
    import torch
    monkeypatch.setenv("DGT_STAGING", staging)
    rng = np.random.default_rng(900 + m + k)
    d = workloads.random_small(F8, 512, k, seed=910 + m)
    xi = rng.integers(-4, 5, (m, k)).astype(np.float32)
    xb = (xi.view(np.uint32) >> 16).astype(np.uint16)
    blob = dgt.dgt_compress_layer(F8, d["codes"], 256, 64, 64)
    layer = dgt.DeviceLayer(blob)
    status = torch.full((layer.info.tiles,), -1, dtype=torch.int32, device="cuda")
    ws = dgt.alloc_workspace(dgt.dgt_gemm_workspace(layer, m))
    y = dgt.dgt_fused_decode_gemm(layer, x_dev(xb), status=status, ws=ws).clone()
    monkeypatch.setenv("DGT_XM_SUBSETS", "0")   # (its workspace holds 256-row slots)
    ws8 = dgt.alloc_workspace(dgt.dgt_gemm_workspace(layer, m))
    y8 = dgt.dgt_fused_decode_gemm(layer, x_dev(xb), ws=ws8)
    torch.cuda.synchronize()
    ref = ogemm.gemm_fp64(xi.astype(np.float64), d["codes"].astype(np.float64))
    assert np.array_equal(y.cpu().numpy().astype(np.float64), ref)
    assert np.array_equal(y8.cpu().numpy().astype(np.float64), ref)
    assert (status.cpu().numpy() == 0).all()
    assert int(ws[:4 * 2].sum().item()) == 0   # strip counters returned to zero


@pytest.mark.parametrize("fmt,n,k,tn,tk,R,seed", [c for c in XM_CASES
                                                   if c[3] == 256 and c[5] == 64])
@pytest.mark.parametrize("m", [33, 100])
def test_large_m_subsets_match_eight_wave_kernel(fmt, n, k, tn, tk, R, seed, m, monkeypatch):
    """Subset form and 8-wave form: both within the bound of the fp64 oracle,
    each deterministic run to run (they add in different orders)."""
    import torch
    d, blob = _layer(fmt, n, k, tn, tk, R, seed, m=m)
    layer = dgt.DeviceLayer(blob)
    scales = to_dev(d["scales"]) if d["scales"] is not None else None
    run = lambda: dgt.dgt_fused_decode_gemm(
        layer, x_dev(d["x"]), scales=scales, w_scale=d["w_scale"],
        ws=dgt.alloc_workspace(dgt.dgt_gemm_workspace(layer, m))).clone()
    ys, ys2 = run(), run()
    monkeypatch.setenv("DGT_XM_SUBSETS", "0")
    y8 = run()
    torch.cuda.synchronize()
    ref = reference(fmt, d, d["x"])
    assert rel_err(ys.cpu().numpy(), ref) <= TOL
    assert rel_err(y8.cpu().numpy(), ref) <= TOL
    assert torch.equal(ys, ys2)


@pytest.mark.parametrize("fmt,n,k,tn,tk,R,seed", [
    (FB, 384, 4096, 128, 64, 64, 52),
    (FE, 512, 1024, 256, 64, 64, 53),     # one fp8 activation scale across passes
    (FP, 256, 2048, 128, 64, 64, 54),
    (FB, 384, 4096, 128, 64, 128, 60),
])
@pytest.mark.parametrize("m", [257, 300, 513])
def test_fused_gemm_beyond_one_pass(fmt, n, k, tn, tk, R, seed, m):
    import torch
    d, blob = _layer(fmt, n, k, tn, tk, R, seed, m=m)
    layer = dgt.DeviceLayer(blob)
    scales = to_dev(d["scales"]) if d["scales"] is not None else None
    y = dgt.dgt_fused_decode_gemm(layer, x_dev(d["x"]), scales=scales, w_scale=d["w_scale"])
    torch.cuda.synchronize()
    assert rel_err(y.cpu().numpy(), reference(fmt, d, d["x"])) <= TOL


STAGING_CASES = [
    (FB, 384, 4096, 128, 64, 64, 71),
    (FB, 256, 2048, 128, 64, 128, 72),
    (FE, 512, 1024, 256, 64, 64, 73),
    (FE, 512, 1024, 256, 64, 128, 74),
    (FP, 256, 2048, 128, 64, 128, 75),
    (F8, 256, 2048, 128, 64, 128, 76),
    (FH, 384, 4096, 128, 64, 64, 77),
    (FW, 384, 4096, 128, 64, 64, 78),
]


@pytest.mark.parametrize("fmt,n,k,tn,tk,R,seed", STAGING_CASES)
@pytest.mark.parametrize("staging", ["ring", "whole"])
def test_forced_staging_matches_oracle(fmt, n, k, tn, tk, R, seed, staging, monkeypatch):
    """Both ways of bringing tile streams on chip (whole, or a two-chunk ring)
    give the oracle's results, for the decode and for the fused GEMM at small
    (register path) and large (LDS-shared fragments) M."""
    import torch
    monkeypatch.setenv("DGT_STAGING", staging)
    d, blob = _layer(fmt, n, k, tn, tk, R, seed, m=100)
    layer = dgt.DeviceLayer(blob)
    status = torch.full((layer.info.tiles,), -1, dtype=torch.int32, device="cuda")
    out = dgt.dgt_decode_tiles(layer, status=status)
    torch.cuda.synchronize()
    assert np.array_equal(decoded_to_numpy(fmt, out), codes_as_u8_or_u16(fmt, d["codes"]))
    assert (status.cpu().numpy() == 0).all()
    scales = to_dev(d["scales"]) if d["scales"] is not None else None
    for m in (1, 16, 100):
        xb = d["x"][:m]
        status.fill_(-1)
        y = dgt.dgt_fused_decode_gemm(layer, x_dev(xb), scales=scales, w_scale=d["w_scale"],
                                      status=status)
        torch.cuda.synchronize()
        assert rel_err(y.cpu().numpy(), reference(fmt, d, xb)) <= TOL, m
        assert (status.cpu().numpy() == 0).all()


ROUNDS_CASES = [
    (FB, 256, 4096, 128, 64, 64, 81),     # two strips of 64 chains
    (FH, 256, 4096, 128, 64, 64, 82),
    (F8, 256, 1024, 128, 32, 32, 83),     # chains of two tiles
    (FE, 512, 1024, 256, 64, 128, 84),    # tile_n 256, two states per lane
    (FP, 384, 2048, 128, 64, 64, 85),     # int4 pairs with scales
    (FW, 256, 4096, 128, 64, 64, 86),     # bf16 whole words
]


@pytest.mark.parametrize("fmt,n,k,tn,tk,R,seed", ROUNDS_CASES)
@pytest.mark.parametrize("rounds", [2, 3, 7])
@pytest.mark.parametrize("staging", ["ring", "whole"])
def test_rounds_per_workgroup_match_oracle(fmt, n, k, tn, tk, R, seed, rounds, staging,
                                           monkeypatch):
    """Workgroups that run several rounds of chains (one LUT build, partial
    sums reduced when a round starts another strip) give the oracle's
    results; forced here on small layers, where ranges straddle strips."""
    import torch
    monkeypatch.setenv("DGT_ROUNDS", str(rounds))
    monkeypatch.setenv("DGT_STAGING", staging)
    d, blob = _layer(fmt, n, k, tn, tk, R, seed, m=16)
    layer = dgt.DeviceLayer(blob)
    status = torch.full((layer.info.tiles,), -1, dtype=torch.int32, device="cuda")
    scales = to_dev(d["scales"]) if d["scales"] is not None else None
    ws = dgt.alloc_workspace(dgt.dgt_gemm_workspace(layer, 16))
    for m in (1, 5, 16):
        xb = d["x"][:m]
        status.fill_(-1)
        y = dgt.dgt_fused_decode_gemm(layer, x_dev(xb), scales=scales, w_scale=d["w_scale"],
                                      status=status, ws=ws)
        torch.cuda.synchronize()
        assert rel_err(y.cpu().numpy(), reference(fmt, d, xb)) <= TOL, m
        assert (status.cpu().numpy() == 0).all()


@pytest.mark.parametrize("fmt,n,k,tn,seed", [(FB, 2048, 4096, 256, 94), (F4, 1024, 4096, 128, 95),
                                              (FE, 1024, 2048, 256, 96), (FW, 1024, 2048, 256, 97)])
@pytest.mark.parametrize("rounds", ["0", "3"])
def test_packed_rows_match_row_blocks(fmt, n, k, tn, seed, rounds, monkeypatch):
    """2..8 rows with the tile's bands packed four (M <= 4) or two (M <= 8) per
    accumulator give the 16-row block kernels' output bit for bit (the same
    products in the same order) and the oracle's within the bound, in one
    round and forced into three rounds per workgroup."""
    import torch
    monkeypatch.setenv("DGT_STAGING", "ring")
    monkeypatch.setenv("DGT_ROUNDS", rounds)
    d, blob = _layer(fmt, n, k, tn, 64, 64, seed, m=8)
    layer = dgt.DeviceLayer(blob)
    scales = to_dev(d["scales"]) if d["scales"] is not None else None
    for m in (2, 3, 4, 5, 8):
        out = {}
        for packed in ("1", "0"):
            monkeypatch.setenv("DGT_PACKED", packed)
            status = torch.full((layer.info.tiles,), -1, dtype=torch.int32, device="cuda")
            y = dgt.dgt_fused_decode_gemm(layer, x_dev(d["x"][:m]), scales=scales,
                                          w_scale=d["w_scale"], status=status)
            torch.cuda.synchronize()
            assert (status.cpu().numpy() == 0).all()
            out[packed] = y.cpu()
        assert torch.equal(out["1"], out["0"]), m
        assert rel_err(out["1"].numpy(), reference(fmt, d, d["x"][:m])) <= TOL, m


@pytest.mark.parametrize("fmt,seed", [(F4, 86), (FB, 87)])
def test_rounds_two_chains_per_wave_match_oracle(fmt, seed, monkeypatch):
    """A layer large enough for 32 chains per workgroup (16 waves, two chains
    each) through the ring, forced into 3 rounds so that workgroup ranges of
    96 chains straddle the 256-chain strips: every output column against the
    fp64 oracle."""
    import torch
    monkeypatch.setenv("DGT_STAGING", "ring")
    monkeypatch.setenv("DGT_ROUNDS", "3")
    d, blob = _layer(fmt, 4096, 16384, 128, 64, 64, seed, m=16)
    layer = dgt.DeviceLayer(blob)
    status = torch.full((layer.info.tiles,), -1, dtype=torch.int32, device="cuda")
    scales = to_dev(d["scales"]) if d["scales"] is not None else None
    for m in (1, 16):
        xb = d["x"][:m]
        status.fill_(-1)
        y = dgt.dgt_fused_decode_gemm(layer, x_dev(xb), scales=scales, w_scale=d["w_scale"],
                                      status=status)
        torch.cuda.synchronize()
        assert rel_err(y.cpu().numpy(), reference(fmt, d, xb)) <= TOL, m
        assert (status.cpu().numpy() == 0).all()


def test_fused_gemm_large_m_repeatable():
    import torch
    d, blob = _layer(FB, 384, 4096, 128, 64, 64, 48, m=256)
    layer = dgt.DeviceLayer(blob)
    x = x_dev(d["x"])
    ws = dgt.alloc_workspace(dgt.dgt_gemm_workspace(layer, 256))
    y1 = dgt.dgt_fused_decode_gemm(layer, x, ws=ws).clone()
    y2 = dgt.dgt_fused_decode_gemm(layer, x, ws=ws).clone()
    y3 = dgt.dgt_fused_decode_gemm(layer, x[:200].contiguous(), ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)               # fixed accumulation and reduction order
    assert torch.equal(y3, y1[:200])         # row results do not depend on M in this path


def test_fused_gemm_repeatable_and_workspace_reusable():
    import torch
    d, blob = _layer(FB, 256, 4096, 128, 64, 64, 21, m=16)
    layer = dgt.DeviceLayer(blob)
    x = x_dev(d["x"])
    ws = dgt.alloc_workspace(dgt.dgt_gemm_workspace(layer, 16))
    y1 = dgt.dgt_fused_decode_gemm(layer, x, ws=ws).clone()
    y2 = dgt.dgt_fused_decode_gemm(layer, x, ws=ws).clone()
    y3 = dgt.dgt_fused_decode_gemm(layer, x[:3].contiguous(), ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)               # deterministic reduction order
    assert torch.equal(y3, y1[:3])           # row results do not depend on M
    assert int(ws[:256].sum().item()) == 0   # strip counters returned to zero


def test_exact_integer_case():
    """int8 weights and integer activations in [-4, 4]: every fp32 partial sum is
    an integer below 2^24, so the device result must equal the oracle exactly."""
    import torch
    rng = np.random.default_rng(3)
    d = workloads.random_small(F8, 512, 1024, seed=31)
    xi = rng.integers(-4, 5, (16, 1024)).astype(np.float32)
    xb = (xi.view(np.uint32) >> 16).astype(np.uint16)
    blob = dgt.dgt_compress_layer(F8, d["codes"], 128, 32, 32)
    y = dgt.dgt_fused_decode_gemm(dgt.DeviceLayer(blob), x_dev(xb))
    torch.cuda.synchronize()
    ref = ogemm.gemm_fp64(xi.astype(np.float64), d["codes"].astype(np.float64))
    assert np.array_equal(y.cpu().numpy().astype(np.float64), ref)


@pytest.mark.parametrize("fmt,tn", [(F8, 128), (F4, 128), (FE, 256), (FB, 128), (FB, 256),
                                    (FP, 128), (FX, 128), (FH, 128)])
@pytest.mark.parametrize("m", [1, 16, 33, 64, 200])
def test_dense_baseline_matches_oracle(fmt, tn, m):
    """The uncompressed baseline (GEMV at M = 1, strip kernel below 32 rows,
    LDS-tiled GEMM from 32 rows, ragged row blocks) against the oracle."""
    import torch
    n, k = 512, 1024
    d = workloads.random_small(fmt, n, k, seed=40 + fmt, m=m)
    w = to_dev(codes_as_u8_or_u16(fmt, d["codes"]))
    scales = to_dev(d["scales"]) if d["scales"] is not None else None
    y = dgt.dgt_dense_gemm(fmt, w, x_dev(d["x"]), tile_n=tn, scales=scales,
                           w_scale=d["w_scale"])
    torch.cuda.synchronize()
    assert rel_err(y.cpu().numpy(), reference(fmt, d, d["x"])) <= TOL


@pytest.mark.parametrize("fmt", [FB, F4, FE, F8])
@pytest.mark.parametrize("n,k,m", [(2048, 4096, 1), (2048, 4096, 256), (32768, 256, 129),
                                   (32768, 256, 256)])
def test_dense_baseline_several_blocks_match_oracle(fmt, n, k, m):
    """Several blocks per XCD and a K of 64 stages (tiled GEMM with 64-row W
    blocks), 512 blocks and more (128-row W blocks, ragged last row block),
    and a GEMV over 2048 rows: every output against the fp64 oracle."""
    import torch
    d = workloads.random_small(fmt, n, k, seed=60 + fmt, m=m)
    w = to_dev(codes_as_u8_or_u16(fmt, d["codes"]))
    scales = to_dev(d["scales"]) if d["scales"] is not None else None
    y = dgt.dgt_dense_gemm(fmt, w, x_dev(d["x"]), tile_n=128, scales=scales,
                           w_scale=d["w_scale"])
    torch.cuda.synchronize()
    assert rel_err(y.cpu().numpy(), reference(fmt, d, d["x"])) <= TOL


@pytest.mark.parametrize("R,staging", [(64, "whole"), (64, "ring"), (128, "whole"),
                                       (128, "ring")])
def test_corrupt_stream_sets_status_and_stays_in_bounds(R, staging, monkeypatch):
    """Bytes flipped inside tile word streams (the index untouched): the
    kernel's clamps keep every access in bounds and the tile status reports it."""
    import torch
    monkeypatch.setenv("DGT_STAGING", staging)
    d, blob = _layer(F8, 256, 512, 128, 64, R, 51)
    info = dgt.dgt_layer_info(blob)
    h = oblob.parse(blob)
    b = bytearray(blob)
    bad_tiles = [1, 5]
    for t in bad_tiles:
        start = info.streams_off + 4 * int(h["index"][t]) + 4 * info.lanes
        for j in range(6):
            b[start + 2 * j] ^= 0xA5
    layer = dgt.DeviceLayer(bytes(b))
    status = torch.full((info.tiles,), -1, dtype=torch.int32, device="cuda")
    # the output sits inside a larger buffer whose guard rows must stay untouched
    buf = torch.full((info.n + 32, info.k), 0x5A, dtype=torch.uint8, device="cuda")
    dgt.dgt_decode_tiles(layer, out=buf[16:16 + info.n], status=status)
    torch.cuda.synchronize()
    st = status.cpu().numpy()
    assert all(st[t] != 0 for t in bad_tiles)
    assert all(st[t] == 0 for t in range(info.tiles) if t not in bad_tiles)
    host = buf.cpu().numpy()
    assert (host[:16] == 0x5A).all() and (host[16 + info.n:] == 0x5A).all()
    # tiles whose streams are intact still decode exactly
    got = host[16:16 + info.n]
    want = codes_as_u8_or_u16(F8, d["codes"])
    kt = info.k // info.tile_k
    for t in range(info.tiles):
        if t in bad_tiles:
            continue
        r0, c0 = (t // kt) * info.tile_n, (t % kt) * info.tile_k
        assert np.array_equal(got[r0:r0 + info.tile_n, c0:c0 + info.tile_k],
                              want[r0:r0 + info.tile_n, c0:c0 + info.tile_k]), t


@pytest.mark.parametrize("R", [32, 64, 128])
def test_decode_tiles_skips_ids_past_the_layer(R):
    """Tile ids >= the tile count reach the C ABI (the binding would refuse
    them): the kernel decodes the valid ids and writes nothing for the others,
    neither output nor status."""
    import ctypes
    import torch
    d, blob = _layer(F8, 256, 512, 128, 64 if R != 32 else 32, R, 52)
    layer = dgt.DeviceLayer(blob)
    info = layer.info
    valid = [info.tiles - 1, 2, 0]
    raw_ids = valid[:1] + [info.tiles, 0xFFFFFFFF] + valid[1:] + [info.tiles + 7]
    ids = torch.tensor(np.array(raw_ids, np.uint32).view(np.int32), device="cuda")
    buf = torch.full((info.n + 32, info.k), 0x5A, dtype=torch.uint8, device="cuda")
    status = torch.full((info.tiles + 8,), -1, dtype=torch.int32, device="cuda")
    rc = dgt.lib().dgt_decode_tiles(ctypes.c_void_p(layer.blob.data_ptr()), ctypes.byref(info),
                                    ctypes.c_void_p(ids.data_ptr()), len(raw_ids),
                                    ctypes.c_void_p(buf[16:].data_ptr()),
                                    ctypes.c_void_p(status.data_ptr()),
                                    ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0
    torch.cuda.synchronize()
    host = buf.cpu().numpy()
    st = status.cpu().numpy()
    assert (host[:16] == 0x5A).all() and (host[16 + info.n:] == 0x5A).all()
    got = host[16:16 + info.n]
    want = codes_as_u8_or_u16(F8, d["codes"])
    kt = info.k // info.tile_k
    mask = np.zeros(got.shape, bool)
    for t in valid:
        r0, c0 = (t // kt) * info.tile_n, (t % kt) * info.tile_k
        mask[r0:r0 + info.tile_n, c0:c0 + info.tile_k] = True
    assert np.array_equal(got[mask], want[mask])
    assert (got[~mask] == 0x5A).all()
    assert all(st[t] == 0 for t in valid)
    assert all(st[t] == -1 for t in range(info.tiles + 8) if t not in valid)


def test_argument_errors():
    d, blob = _layer(F8, 256, 512, 128, 64, 64, 61)
    layer = dgt.DeviceLayer(blob)
    x = x_dev(d["x"])
    with pytest.raises(dgt.DgtError) as e:
        dgt.dgt_fused_decode_gemm(layer, x, ws=dgt.alloc_workspace(256)[:0])
    assert e.value.code in (-1, -4)
    import torch
    big = torch.zeros(((1 << 16) + 1, 512), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(dgt.DgtError) as e:
        dgt.dgt_fused_decode_gemm(layer, big)
    assert e.value.code == -1


def _fp8_layer_from_codes(codes, tn, tk, R):
    blob = dgt.dgt_compress_layer(FE, codes, tn, tk, R)
    return dgt.DeviceLayer(blob)


def _bf16_bits(values):
    import torch
    return torch.tensor(np.asarray(values, np.float32)).to(torch.bfloat16).view(
        torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("tn,tk,R", [(256, 64, 64), (128, 32, 32), (128, 64, 128)])
@pytest.mark.parametrize("m", [3, 40, 200])
def test_fp8_activation_quant_bit_exact(tn, tk, R, m):
    """The device's per-tensor e4m3 quantisation of X, read through a layer
    whose weights are the identity (e4m3 1.0 on the diagonal): Y[m, j] is
    fl32(xq[m, j] * sx) exactly.  X's maximum is 0.5234375, and it holds values
    whose product with inv rounds across an e4m3 boundary only in fp32, so the
    device must round x * inv to fp32 before the e4m3 rounding, as the oracle
    does.  M = 3 and 40 quantise in one workgroup, M = 200 in two launches."""
    import torch
    from oracle import numerics
    n = k = 512
    codes = np.zeros((n, k), np.uint8)
    codes[np.arange(n), np.arange(k)] = 0x38
    layer = _fp8_layer_from_codes(codes, tn, tk, R)
    rng = np.random.default_rng(70 + m)
    v = rng.uniform(-0.5, 0.5, (m, k)) * np.exp2(rng.integers(-14, 1, (m, k)))
    v[0, :4] = [0.5234375, 2.396106719970703e-05, -4.792213439941406e-05, 2.0742416381835938e-05]
    xb = _bf16_bits(v)
    y = dgt.dgt_fused_decode_gemm(layer, x_dev(xb), w_scale=1.0)
    torch.cuda.synchronize()
    xq, sx = numerics.fp8_quantize_activations(xb)
    want = (numerics.e4m3_to_f64(xq) * sx).astype(np.float32)
    assert np.array_equal(y.cpu().numpy(), want)


@pytest.mark.parametrize("tn,tk,R", [(256, 64, 64), (128, 32, 32)])
@pytest.mark.parametrize("m", [1, 16, 64])
def test_fp8_exact_integer_gemm(tn, tk, R, m):
    """amax|X| = 448 makes inv = sx = 1; X holds integers in [-16, 16] and e4m3
    midpoints (1.0625 -> 1, 1.1875 -> 1.25 under ties-to-even), W small integers:
    every partial sum is a multiple of 1/4 below 2^17, so Y is exact."""
    import torch
    from oracle import numerics
    n, k = 512, 512
    rng = np.random.default_rng(80 + m)
    wv = rng.integers(-8, 9, (n, k)).astype(np.float64)
    codes = numerics.f64_to_e4m3(wv)
    xv = rng.integers(-16, 17, (m, k)).astype(np.float64)
    xv[0, 0] = 448.0
    xv[:, 1] = 1.0625
    xv[:, 2] = -1.1875
    xb = _bf16_bits(xv)
    layer = _fp8_layer_from_codes(codes, tn, tk, R)
    y = dgt.dgt_fused_decode_gemm(layer, x_dev(xb), w_scale=1.0)
    torch.cuda.synchronize()
    xq = np.round(xv)  # the e4m3 values of X: integers, with the two midpoints below
    xq[:, 1] = 1.0
    xq[:, 2] = -1.25
    want = ogemm.gemm_fp64(xq, wv)
    assert np.array_equal(y.cpu().numpy().astype(np.float64), want)
    assert np.array_equal(ogemm.reference_output(FE, codes, xb, w_scale=1.0), want)
