"""GPU parity at the workloads' full sizes, in the launch configuration the
bench uses (the library's own planner):

- the whole layer decodes bit-exactly to the generated weights (the plain
  definition of the decoded result for a lossless coder), every tile status 0;
- the C++ encoder's streams for sampled tiles equal the oracle's encoding of
  those tiles (the oracle builds its own table from the full histogram);
- sampled output columns of the fused GEMM match the fp64 oracle within 1e-5
  relative Frobenius error at every M the workload lists.
"""

import numpy as np
import pytest

import decode_gemm_tile_amd as dgt
import workloads
from oracle import blob as oblob
from oracle import entropy as oent
from oracle import freq as ofreq
from oracle import gemm as ogemm
from oracle import order as oorder
from oracle import rans as orans
from tests.gpu_util import BF16_FORMATS, codes_as_u8_or_u16, to_dev, x_dev

pytestmark = pytest.mark.gpu
TOL = 1e-5
NAMES = ["int8_1024", "int4_4096", "fp8_8192", "bf16_mlp", "int4_ffn405", "bf16_ffn405",
         "int4_4096_pair", "int4_ffn405_pair", "bf16_mlp_exp", "int4_4096_r128",
         "fp8_8192_r128", "bf16_mlp_r128", "bf16_mlp_pair", "bf16_ffn405_pair"]
_CACHE = {}


def _setup(name):
    if name in _CACHE:
        return _CACHE[name]
    _CACHE.clear()  # keep one full-size layer in memory at a time
    d = workloads.make(name)
    wl = d["workload"]
    blob = dgt.dgt_compress_layer(wl.fmt, d["codes"], wl.tile_n, wl.tile_k, wl.lanes)
    layer = dgt.DeviceLayer(blob)
    _CACHE[name] = (d, wl, blob, layer)
    return _CACHE[name]


@pytest.mark.parametrize("name", NAMES)
def test_fullsize_decode_bit_exact(name):
    import torch
    d, wl, blob, layer = _setup(name)
    status = torch.full((layer.info.tiles,), -1, dtype=torch.int32, device="cuda")
    out = dgt.dgt_decode_tiles(layer, status=status)
    ref = to_dev(codes_as_u8_or_u16(wl.fmt, d["codes"]))
    if wl.fmt in BF16_FORMATS:
        ref = ref.view(torch.int16)
    torch.cuda.synchronize()
    assert torch.equal(out.view(ref.dtype), ref)
    assert int((status != 0).sum().item()) == 0
    print("%s: %.4f bits/weight, %d tiles" % (name, layer.info.bits_per_weight, layer.info.tiles))


@pytest.mark.parametrize("name", NAMES)
def test_fullsize_encoder_matches_oracle_on_sampled_tiles(name):
    d, wl, blob, layer = _setup(name)
    sym, _ = oblob.symbolise(wl.fmt, d["codes"])
    f = ofreq.quantize_freqs(oent.histogram(sym, oblob.alphabet_of(wl.fmt)), wl.prob_bits)
    h = oblob.parse(blob)
    assert np.array_equal(h["freq"], f)
    rng = np.random.default_rng(7)
    tiles = sorted(set([0, h["tiles"] - 1] + list(rng.integers(0, h["tiles"], 14))))
    kt = wl.k // wl.tile_k
    _, tks, epl = oblob.symbol_geometry(wl.fmt, wl.n, wl.k, wl.tile_n, wl.tile_k)
    for t in tiles:
        r0, c0 = (t // kt) * wl.tile_n, (t % kt) * tks
        block = sym[r0:r0 + wl.tile_n, c0:c0 + tks]
        ts = oorder.gather_tiles(block, wl.tile_n, tks, wl.lanes, epl=epl)
        st, ws, ks = orans.encode_tiles(ts, f, wl.lanes, wl.prob_bits)
        gst, gws = oblob.tile_stream(blob, h, t)
        assert np.array_equal(gst, st[0]), t
        n = len(ws[0])
        assert np.array_equal(gws[:n], ws[0]) and len(gws) in (n, n + 1), t
        assert h["ks"][t] == ks[0], t


@pytest.mark.parametrize("name", NAMES)
def test_fullsize_fused_gemm_sampled_columns(name):
    import torch
    d, wl, blob, layer = _setup(name)
    rng = np.random.default_rng(11)
    cols = np.sort(rng.choice(wl.n, size=96, replace=False))
    scales = to_dev(d["scales"]) if d["scales"] is not None else None
    codes_s = np.asarray(d["codes"])[cols]
    scales_s = d["scales"][cols] if d["scales"] is not None else None
    for m in wl.m_values:
        xb = d["x"][:m]
        status = torch.full((layer.info.tiles,), -1, dtype=torch.int32, device="cuda")
        y = dgt.dgt_fused_decode_gemm(layer, x_dev(xb), scales=scales, w_scale=d["w_scale"],
                                      status=status)
        torch.cuda.synchronize()
        ys = y.cpu().numpy()[:, cols]
        ref = ogemm.reference_output(wl.fmt, codes_s, xb, scales_s, d["w_scale"])
        err = ogemm.rel_frobenius(ys, ref)
        assert err <= TOL, (name, m, err)
        assert int((status != 0).sum().item()) == 0
        assert np.isfinite(y.cpu().numpy()).all()
