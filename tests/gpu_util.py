"""Helpers shared by the GPU tests (inputs, device transfer, oracle values)."""

import numpy as np

import decode_gemm_tile_amd as dgt
from oracle import gemm as ogemm


BF16_FORMATS = dgt.BF16_FORMATS


def to_dev(arr, dtype=None):
    import torch
    a = np.ascontiguousarray(arr)
    if a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16))
    else:
        t = torch.from_numpy(a)
    if dtype is not None:
        t = t.view(dtype)
    return t.to("cuda")


def x_dev(x_bits):
    import torch
    return to_dev(x_bits).view(torch.bfloat16)


def codes_as_u8_or_u16(fmt, codes):
    c = np.asarray(codes)
    if fmt == dgt.DGT_FMT_INT8:
        return c.astype(np.int8).view(np.uint8)
    if fmt in BF16_FORMATS:
        return c.astype(np.uint16)
    return c.astype(np.uint8)


def decoded_to_numpy(fmt, out):
    a = out.cpu().numpy()
    if fmt in BF16_FORMATS:
        return a.view(np.uint16)
    return a


def reference(fmt, d, x_bits):
    return ogemm.reference_output(fmt, d["codes"], x_bits, d.get("scales"), d.get("w_scale", 1.0))


def rel_err(y, ref):
    return ogemm.rel_frobenius(y, ref)
