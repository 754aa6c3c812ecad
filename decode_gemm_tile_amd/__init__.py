"""Python binding of libdgt (ctypes): argument marshalling only.

Every step of the decode and the GEMM runs in the HIP library; PyTorch only
provides device memory and the current HIP stream.  Function names follow the
C ABI in include/dgt.h one to one.  There is no CPU fallback: when libdgt.so
is missing or no GPU is present the device entry points raise.
"""

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdgt.so")

DGT_FMT_INT8, DGT_FMT_INT4, DGT_FMT_FP8_E4M3, DGT_FMT_BF16_SPLIT = 1, 2, 3, 4
DGT_FMT_INT4_PAIR = 5
DGT_FMT_BF16_EXP = 6
DGT_FMT_BF16_PAIR = 7
DGT_FMT_BF16_WORD = 8
BF16_FORMATS = (DGT_FMT_BF16_SPLIT, DGT_FMT_BF16_EXP, DGT_FMT_BF16_PAIR, DGT_FMT_BF16_WORD)
STATUS = {0: "DGT_OK", -1: "DGT_E_ARG", -2: "DGT_E_SHAPE", -3: "DGT_E_ALPHABET",
          -4: "DGT_E_BUFSIZE", -5: "DGT_E_FORMAT", -6: "DGT_E_CORRUPT", -7: "DGT_E_HIP",
          -8: "DGT_E_UNSUPPORTED"}
EXPORTS = ["dgt_version", "dgt_status_string", "dgt_compress_bound", "dgt_compress_layer",
           "dgt_layer_info", "dgt_decode_tiles", "dgt_gemm_workspace",
           "dgt_fused_decode_gemm", "dgt_dense_workspace", "dgt_dense_gemm",
           "dgt_noalloc_scratch_bytes", "dgt_fused_decode_gemm_noalloc"]


class DgtError(RuntimeError):
    def __init__(self, code: int, where: str):
        super().__init__("%s failed: %s (%d)" % (where, STATUS.get(code, "?"), code))
        self.code = code


class dgt_params(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint32) for n in
                ("fmt", "n", "k", "tile_n", "tile_k", "lanes", "prob_bits", "flags")]


class dgt_info(ctypes.Structure):
    _fields_ = ([(n, ctypes.c_uint32) for n in
                 ("fmt", "n", "k", "tile_n", "tile_k", "lanes", "prob_bits", "alphabet",
                  "tiles", "max_tile_words4", "kmax", "flags")] +
                [(n, ctypes.c_uint64) for n in
                 ("table_off", "index_off", "ktab_off", "streams_off", "raw_off",
                  "total_bytes", "stream_bytes")] +
                [("bits_per_weight", ctypes.c_double)])

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}


_lib = None


def lib():
    """Load the in-tree libdgt.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libdgt.so not built: run python -m decode_gemm_tile_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        vp, u32, sz = ctypes.c_void_p, ctypes.c_uint32, ctypes.c_size_t
        L.dgt_version.restype = ctypes.c_int
        L.dgt_status_string.restype = ctypes.c_char_p
        L.dgt_status_string.argtypes = [ctypes.c_int]
        L.dgt_compress_bound.restype = sz
        L.dgt_compress_bound.argtypes = [ctypes.POINTER(dgt_params)]
        L.dgt_compress_layer.restype = ctypes.c_int
        L.dgt_compress_layer.argtypes = [ctypes.POINTER(dgt_params), vp, vp, sz,
                                         ctypes.POINTER(sz)]
        L.dgt_layer_info.restype = ctypes.c_int
        L.dgt_layer_info.argtypes = [vp, sz, ctypes.POINTER(dgt_info)]
        L.dgt_decode_tiles.restype = ctypes.c_int
        L.dgt_decode_tiles.argtypes = [vp, ctypes.POINTER(dgt_info), vp, u32, vp, vp, vp]
        L.dgt_gemm_workspace.restype = sz
        L.dgt_gemm_workspace.argtypes = [ctypes.POINTER(dgt_info), u32]
        L.dgt_fused_decode_gemm.restype = ctypes.c_int
        L.dgt_fused_decode_gemm.argtypes = [vp, ctypes.POINTER(dgt_info), vp, u32, vp,
                                            ctypes.c_float, vp, vp, sz, vp, vp]
        L.dgt_noalloc_scratch_bytes.restype = sz
        L.dgt_noalloc_scratch_bytes.argtypes = []
        L.dgt_fused_decode_gemm_noalloc.restype = ctypes.c_int
        L.dgt_fused_decode_gemm_noalloc.argtypes = [vp, ctypes.POINTER(dgt_info), vp, u32, vp,
                                                    ctypes.c_float, vp, vp, vp]
        L.dgt_dense_workspace.restype = sz
        L.dgt_dense_workspace.argtypes = [u32, u32, u32, u32, u32]
        L.dgt_dense_gemm.restype = ctypes.c_int
        L.dgt_dense_gemm.argtypes = [u32, u32, u32, u32, vp, vp, u32, vp, ctypes.c_float, vp,
                                     vp, sz, vp]
        _lib = L
    return _lib


def _check(code: int, where: str):
    if code != 0:
        raise DgtError(code, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


# Argument checks made before anything is launched: the C ABI receives raw
# device pointers and cannot tell a tensor's shape, dtype, layout or device.
_TWO_BYTE = ("torch.bfloat16", "torch.int16", "torch.uint16", "torch.float16")


def _need(cond, msg):
    if not cond:
        raise ValueError(msg)


def _check_tensor(t, name, shape, dtypes, device):
    """t must be a contiguous tensor of one of `dtypes` (by name), with
    `shape` (None entries are free), on `device`."""
    _need(t is not None, "%s is required" % name)
    _need(hasattr(t, "data_ptr") and hasattr(t, "is_contiguous"), "%s must be a tensor" % name)
    _need(str(t.dtype) in dtypes, "%s has dtype %s, expected one of %s"
          % (name, t.dtype, ", ".join(dtypes)))
    _need(t.dim() == len(shape) and all(s is None or s == d for s, d in zip(shape, t.shape)),
          "%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    _need(t.is_contiguous(), "%s must be contiguous" % name)
    _need(t.device == device, "%s is on %s, expected %s" % (name, t.device, device))


def _check_gpu(device):
    """Checked after every argument's shape and dtype: all of them live on
    `device`, which must be a GPU."""
    _need(device.type == "cuda", "arguments must be in GPU memory (the library has no CPU path)")


def _check_status(status, tiles, device):
    if status is not None:
        _check_tensor(status, "status", (None,), ("torch.int32",), device)
        _need(status.numel() >= tiles, "status holds %d entries, the layer has %d tiles"
              % (status.numel(), tiles))


def _check_scales(fmt, scales, n, k, device):
    if fmt in (DGT_FMT_INT4, DGT_FMT_INT4_PAIR):
        _need(k % 128 == 0, "int4 layers need K divisible by 128 (one scale per 128 columns)")
        _check_tensor(scales, "scales", (n, k // 128), _TWO_BYTE, device)
    else:
        _need(scales is None, "scales are only taken by the int4 formats")


# ----------------------------------------------------------------- host side
def dgt_version() -> int:
    return lib().dgt_version()


def dgt_status_string(code: int) -> str:
    return lib().dgt_status_string(code).decode()


def dgt_compress_bound(fmt, n, k, tile_n, tile_k, lanes, prob_bits=12) -> int:
    p = dgt_params(fmt, n, k, tile_n, tile_k, lanes, prob_bits, 0)
    return lib().dgt_compress_bound(ctypes.byref(p))


def dgt_compress_layer(fmt, w, tile_n, tile_k, lanes, prob_bits=None) -> bytes:
    """Offline encoder.  w: [N, K] numpy array (int8 / uint8 codes, or uint16
    bf16 bit patterns for the bf16 formats).  prob_bits defaults to 12 (16 for
    whole bf16 words)."""
    if prob_bits is None:
        prob_bits = 16 if fmt == DGT_FMT_BF16_WORD else 12
    w = np.ascontiguousarray(w)
    n, k = w.shape
    p = dgt_params(fmt, n, k, tile_n, tile_k, lanes, prob_bits, 0)
    cap = lib().dgt_compress_bound(ctypes.byref(p))
    if cap == 0:
        _check(-2, "dgt_compress_bound")
    out = np.empty(cap, dtype=np.uint8)
    size = ctypes.c_size_t(0)
    _check(lib().dgt_compress_layer(ctypes.byref(p), w.ctypes.data_as(ctypes.c_void_p),
                                    out.ctypes.data_as(ctypes.c_void_p), cap,
                                    ctypes.byref(size)), "dgt_compress_layer")
    return out[: size.value].tobytes()


def dgt_layer_info(blob: bytes) -> dgt_info:
    info = dgt_info()
    buf = np.frombuffer(blob, dtype=np.uint8)
    _check(lib().dgt_layer_info(buf.ctypes.data_as(ctypes.c_void_p), len(blob),
                                ctypes.byref(info)), "dgt_layer_info")
    return info


# --------------------------------------------------------------- device side
class DeviceLayer:
    """A blob resident in HBM plus its parsed header."""

    def __init__(self, blob: bytes, device="cuda"):
        import torch
        self.info = dgt_layer_info(blob)
        host = torch.frombuffer(bytearray(blob), dtype=torch.uint8)
        self.blob = host.to(device)
        if self.blob.data_ptr() % 16:
            raise RuntimeError("device blob is not 16-byte aligned")
        self.nbytes = len(blob)


def dgt_decode_tiles(layer: DeviceLayer, tile_ids=None, out=None, status=None, stream=None):
    """Decode tiles into W layout [N, K] (uint8 codes, or int16 bf16 bits)."""
    import torch
    inf = layer.info
    dev = layer.blob.device
    wide = inf.fmt in BF16_FORMATS
    if out is None:
        out = torch.zeros((inf.n, inf.k), dtype=torch.int16 if wide else torch.uint8, device=dev)
    _check_tensor(out, "out", (inf.n, inf.k), _TWO_BYTE if wide else ("torch.uint8", "torch.int8"),
                  dev)
    _check_status(status, inf.tiles, dev)
    ids = None
    n_ids = 0
    if tile_ids is not None:
        if isinstance(tile_ids, torch.Tensor):
            ids = tile_ids
        else:
            a = np.asarray(tile_ids)
            _need(a.dtype.kind in "iub" or a.size == 0, "tile_ids must be a 1-D integer list")
            ids = torch.from_numpy(a.astype(np.int64).reshape(a.shape))
        _need(ids.dim() == 1 and not ids.is_floating_point(), "tile_ids must be a 1-D integer list")
        if ids.numel():
            lo, hi = int(ids.min()), int(ids.max())
            _need(0 <= lo and hi < inf.tiles, "tile ids must lie in [0, %d); got %d..%d"
                  % (inf.tiles, lo, hi))
        _check_gpu(dev)
        ids = ids.to(dtype=torch.int32, device=dev).contiguous()
        n_ids = ids.numel()
        if n_ids == 0:
            return out
    _check_gpu(dev)
    _check(lib().dgt_decode_tiles(_ptr(layer.blob), ctypes.byref(inf), _ptr(ids), n_ids,
                                  _ptr(out), _ptr(status), _stream(stream)),
           "dgt_decode_tiles")
    return out


def dgt_gemm_workspace(layer: DeviceLayer, m: int) -> int:
    return lib().dgt_gemm_workspace(ctypes.byref(layer.info), m)


def alloc_workspace(nbytes: int, device="cuda"):
    import torch
    return torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def dgt_fused_decode_gemm(layer: DeviceLayer, x, scales=None, w_scale=1.0, y=None, ws=None,
                          status=None, stream=None):
    """Y[m, n] = sum_k X[m, k] W[n, k] with W decoded on chip; x: bf16 [M, K]."""
    import torch
    inf = layer.info
    dev = layer.blob.device
    _check_tensor(x, "x", (None, inf.k), ("torch.bfloat16",), dev)
    m = x.shape[0]
    _need(1 <= m, "x needs at least one row")
    if y is None:
        y = torch.empty((m, inf.n), dtype=torch.float32, device=dev)
    _check_tensor(y, "y", (m, inf.n), ("torch.float32",), dev)
    _check_scales(inf.fmt, scales, inf.n, inf.k, dev)
    _check_status(status, inf.tiles, dev)
    if ws is not None:
        _check_tensor(ws, "ws", (None,), ("torch.uint8",), dev)
    _check_gpu(dev)
    if ws is None:
        ws = alloc_workspace(dgt_gemm_workspace(layer, m), dev)
    _check(lib().dgt_fused_decode_gemm(_ptr(layer.blob), ctypes.byref(inf), _ptr(x), m,
                                       _ptr(scales), float(w_scale), _ptr(y), _ptr(ws),
                                       ws.numel(), _ptr(status), _stream(stream)),
           "dgt_fused_decode_gemm")
    return y


def dgt_noalloc_scratch_bytes() -> int:
    return lib().dgt_noalloc_scratch_bytes()


def dgt_fused_decode_gemm_noalloc(layer: DeviceLayer, x, y, scales=None, w_scale=1.0,
                                  status=None, stream=None):
    """dgt_fused_decode_gemm on the library's static scratch: no workspace and,
    given y, no allocation at all."""
    inf = layer.info
    dev = layer.blob.device
    _check_tensor(x, "x", (None, inf.k), ("torch.bfloat16",), dev)
    m = x.shape[0]
    _need(1 <= m, "x needs at least one row")
    _check_tensor(y, "y", (m, inf.n), ("torch.float32",), dev)
    _check_scales(inf.fmt, scales, inf.n, inf.k, dev)
    _check_status(status, inf.tiles, dev)
    _check_gpu(dev)
    _check(lib().dgt_fused_decode_gemm_noalloc(_ptr(layer.blob), ctypes.byref(inf), _ptr(x), m,
                                               _ptr(scales), float(w_scale), _ptr(y),
                                               _ptr(status), _stream(stream)),
           "dgt_fused_decode_gemm_noalloc")
    return y


def dgt_dense_workspace(fmt, n, k, tile_n, m) -> int:
    return lib().dgt_dense_workspace(fmt, n, k, tile_n, m)


def dgt_dense_gemm(fmt, w, x, tile_n=128, scales=None, w_scale=1.0, y=None, ws=None,
                   stream=None):
    """Uncompressed baseline; w: device [N, K] (uint8 codes or bf16 bits)."""
    import torch
    wide = fmt in BF16_FORMATS
    _need(hasattr(w, "shape") and w.dim() == 2, "w must be a 2-D tensor [N, K]")
    n, k = w.shape
    dev = w.device
    _check_tensor(w, "w", (n, k), _TWO_BYTE if wide else ("torch.uint8", "torch.int8"), dev)
    _check_tensor(x, "x", (None, k), ("torch.bfloat16",), dev)
    m = x.shape[0]
    if y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=dev)
    _check_tensor(y, "y", (m, n), ("torch.float32",), dev)
    _check_scales(fmt, scales, n, k, dev)
    if ws is not None:
        _check_tensor(ws, "ws", (None,), ("torch.uint8",), dev)
    _check_gpu(dev)
    if ws is None:
        ws = alloc_workspace(dgt_dense_workspace(fmt, n, k, tile_n, m), dev)
    _check(lib().dgt_dense_gemm(fmt, n, k, tile_n, _ptr(w), _ptr(x), m, _ptr(scales),
                                float(w_scale), _ptr(y), _ptr(ws), ws.numel(),
                                _stream(stream)), "dgt_dense_gemm")
    return y
