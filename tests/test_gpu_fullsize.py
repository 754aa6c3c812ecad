"""GPU parity at the workloads' full sizes, in the launch configuration the
bench uses (the library's own planner):

- the whole layer decodes bit-exactly to the generated weights (the plain
  definition of the decoded result for a lossless coder), every tile status 0;
- the C++ encoder's streams for sampled tiles equal the oracle's encoding of
  those tiles (the oracle builds its own table from the full histogram);
- the fused GEMM matches the fp64 oracle within 1e-5 relative Frobenius error
  at every M the workload lists: over the whole output at M <= 8, and at
  M <= 64 on layers up to 8192 x 8192; elsewhere over one column of every
  strip (tile_n columns of Y) plus 96 random columns.  Y starts as NaN, so an
  output the kernel never writes fails the check everywhere.
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
# codings of the same weights are adjacent, so they share one oracle output
NAMES = ["int8_1024", "int4_4096", "int4_4096_pair", "int4_4096_r128", "fp8_8192",
         "fp8_8192_r128", "bf16_mlp", "bf16_mlp_exp", "bf16_mlp_r128", "bf16_mlp_pair",
         "bf16_mlp_word",
         "int4_ffn405", "int4_ffn405_pair", "bf16_ffn405", "bf16_ffn405_pair"]
_CACHE = {}


def _setup(name):
    if name in _CACHE:
        return _CACHE[name]
    _CACHE.clear()  # keep one full-size layer in memory at a time
    d = workloads.make(name)
    wl = d["workload"]
    blob = dgt.dgt_compress_layer(wl.fmt, d["codes"], wl.tile_n, wl.tile_k, wl.lanes, wl.prob_bits)
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


FULL_WEIGHTS = 8192 * 8192  # whole-output comparison up to this layer size at M <= 64
_REF = {}  # oracle outputs of the first rows, shared by codings of the same weights


def _family(wl):
    """Key of the weight values a workload multiplies (codings of one layer share it)."""
    fam = {dgt.DGT_FMT_INT4_PAIR: dgt.DGT_FMT_INT4, dgt.DGT_FMT_BF16_EXP: dgt.DGT_FMT_BF16_SPLIT,
           dgt.DGT_FMT_BF16_PAIR: dgt.DGT_FMT_BF16_SPLIT,
           dgt.DGT_FMT_BF16_WORD: dgt.DGT_FMT_BF16_SPLIT}.get(wl.fmt, wl.fmt)
    return (fam, wl.n, wl.k, wl.seed)


def _reference_cols(wl, d, xb, cols=None, chunk=2048):
    """fp64 oracle output Y[:, cols] (all columns if None), computed over
    chunks of W's rows so the fp64 weights of a chunk are all that is held."""
    codes = np.asarray(d["codes"])
    idx = np.arange(wl.n) if cols is None else np.asarray(cols)
    out = np.empty((xb.shape[0], len(idx)))
    for s in range(0, len(idx), chunk):
        sel = idx[s:s + chunk]
        c = codes[s:s + chunk] if cols is None else codes[sel]
        sc = None
        if d["scales"] is not None:
            sc = d["scales"][s:s + chunk] if cols is None else d["scales"][sel]
        out[:, s:s + len(sel)] = ogemm.reference_output(wl.fmt, c, xb, sc, d["w_scale"])
    return out


def _full_reference(wl, d, m):
    if wl.fmt == dgt.DGT_FMT_FP8_E4M3:  # the activation scale depends on the rows
        return _reference_cols(wl, d, d["x"][:m])
    key = _family(wl)
    if key not in _REF or _REF[key].shape[0] < m:
        _REF.clear()
        rows = max(mm for mm in wl.m_values if _whole_output(wl, mm))
        _REF[key] = _reference_cols(wl, d, d["x"][:rows])
    return _REF[key][:m]


def _whole_output(wl, m):
    return m <= 8 or (wl.n * wl.k <= FULL_WEIGHTS and m <= 64)


@pytest.mark.parametrize("name", NAMES)
def test_fullsize_fused_gemm(name):
    import torch
    d, wl, blob, layer = _setup(name)
    rng = np.random.default_rng(11)
    strips = wl.n // wl.tile_n
    per_strip = np.arange(strips) * wl.tile_n + rng.integers(0, wl.tile_n, strips)
    cols = np.unique(np.concatenate([per_strip, rng.choice(wl.n, size=96, replace=False)]))
    scales = to_dev(d["scales"]) if d["scales"] is not None else None
    for m in wl.m_values:
        xb = d["x"][:m]
        status = torch.full((layer.info.tiles,), -1, dtype=torch.int32, device="cuda")
        y = torch.full((m, wl.n), float("nan"), dtype=torch.float32, device="cuda")
        dgt.dgt_fused_decode_gemm(layer, x_dev(xb), scales=scales, w_scale=d["w_scale"], y=y,
                                  status=status)
        torch.cuda.synchronize()
        yh = y.cpu().numpy()
        assert np.isfinite(yh).all(), (name, m, int((~np.isfinite(yh)).sum()))
        assert int((status != 0).sum().item()) == 0
        if _whole_output(wl, m):
            err = ogemm.rel_frobenius(yh, _full_reference(wl, d, m))
        else:
            err = ogemm.rel_frobenius(yh[:, cols], _reference_cols(wl, d, xb, cols))
        print("%s M=%d: rel err %.2e (%s)" % (name, m, err,
                                             "all columns" if _whole_output(wl, m)
                                             else "%d columns" % len(cols)))
        assert err <= TOL, (name, m, err)
