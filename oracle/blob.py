"""Compressed-layer byte format: writer and reader (oracle).

[P1 §3.1]: offline, a layer is cut into GEMM-aligned tiles, all tiles share
one compact codebook, each tile is coded independently (R lane sub-streams)
and a light index records each tile's start offset, so any tile can be
decoded on its own.  The byte layout below is this project's reading (the
pages give none); all integers are little-endian.

header (128 bytes)
   0 magic  b"DGT1"              4 u16 version = 1     6 u16 header bytes = 128
   8 u32 fmt (1 int8, 2 int4, 3 fp8 e4m3, 4 bf16 byte split, 5 int4 pairs,
              6 bf16 exponent split, 7 bf16 byte split with high-byte pairs,
              8 bf16 whole words)
  12 u32 flags = 0              16 u32 N     20 u32 K
  24 u32 tile_n  28 u32 tile_k  32 u32 lanes R  36 u32 prob_bits n
  40 u32 alphabet (16 for int4, 256 for the other dense tables; formats 7
         and 8: the number P of table entries)     44 u32 tiles
  48 u64 table_off   56 u64 index_off   64 u64 ktab_off   72 u64 streams_off
  80 u64 raw_off (0 when the format stores no raw bytes)   88 u64 total bytes
  96 u32 max tile stream length in 4-byte units
 100 u32 kmax (payload-step cap, 16)    104..127 zero
table   u16 f[alphabet]; formats 7 and 8 (alphabet 65536, at most 2**n
        symbols present): u32 entry[P] for the symbols with f > 0, in
        increasing symbol order, entry = symbol | f << 16 (format 7) or
        symbol | (f - 1) << 16 (format 8, whose n = 16 allows f = 2**16)
                                                          (16-byte aligned)
index   u32 off[tiles + 1], 4-byte units from streams_off, off[0] = 0 (aligned)
ktab    u8 k[tiles]: payload steps of each tile (see ``oracle.rans``) (aligned)
streams tile t at streams_off + 4*off[t]: R u32 states (lane order) then the
        u16 words in decoder order, then one zero u16 if the count is odd
raw     (bf16 splits only, 16-byte aligned) T raw bytes per tile, tiles in id
        order, each tile in the lane-major raw order of ``oracle.order``
total = end of raw (bf16 split) or end of streams.

Symbols: int8 code & 0xFF; int4 code; e4m3 byte; bf16 bits >> 8 (sign and
top seven exponent bits) with the low byte (exponent LSB + mantissa) raw;
bf16 exponent split: the 8 exponent bits (bits >> 7) & 0xFF coded, the sign
and the 7 mantissa bits raw as one byte (sign << 7 | mantissa), the split
DFloat11 uses ([P2]); int4 pairs: q[n, 2c] | q[n, 2c+1] << 4 (two weights adjacent along K per
symbol, alphabet 256; tile_n and tile_k stay in weights, a tile holds
tile_n*tile_k/2 symbols laid out by ``oracle.order`` with epl = 4); bf16
high-byte pairs (format 7): the bf16 byte split with the high bytes of two
weights adjacent along K coded as one 16-bit symbol hi[n, 2c] | hi[n, 2c+1] << 8
(the same pair geometry as int4 pairs), the low bytes raw as in format 4;
bf16 whole words (format 8): the 16-bit pattern itself is the symbol, nothing
is stored raw, and the table has 2**16 slots (n = 16), the precision the
pages' 16-bit coding needs ([P1 §4.1] puts the table-precision cost of
16-bit symbols at 0.1-0.2 bit).
"""

import struct

import numpy as np

from . import entropy, freq, order, rans

MAGIC = b"DGT1"
VERSION = 1
HEADER_BYTES = 128
FMT_INT8, FMT_INT4, FMT_FP8, FMT_BF16, FMT_INT4_PAIR, FMT_BF16_EXP = 1, 2, 3, 4, 5, 6
FMT_BF16_PAIR = 7
FMT_BF16_WORD = 8
_PAIR_FORMATS = (FMT_INT4_PAIR, FMT_BF16_PAIR)
_HDR = struct.Struct("<4sHHIIIIIIIIII QQQQQQ II 24x")
assert _HDR.size == HEADER_BYTES


def _align(v: int, a: int) -> int:
    return (v + a - 1) // a * a


def alphabet_of(fmt: int) -> int:
    if fmt == FMT_INT4:
        return 16
    if fmt in (FMT_INT8, FMT_FP8, FMT_BF16, FMT_INT4_PAIR, FMT_BF16_EXP):
        return 256
    if fmt in (FMT_BF16_PAIR, FMT_BF16_WORD):
        return 65536
    raise ValueError("unknown format")


def sparse_table(fmt: int) -> bool:
    """Formats whose table lists only the present symbols (symbol, f)."""
    return fmt in (FMT_BF16_PAIR, FMT_BF16_WORD)


def sparse_f_bias(fmt: int) -> int:
    """A sparse entry stores f - bias in its top 16 bits (format 8: f may be 2**16)."""
    return 1 if fmt == FMT_BF16_WORD else 0


def weights_per_symbol(fmt: int) -> int:
    return 2 if fmt in _PAIR_FORMATS else 1


def symbol_geometry(fmt: int, n: int, k: int, tile_n: int, tile_k: int):
    """(symbol-matrix columns, tile columns in symbols, symbols per lane per
    fragment) of a format: pairs halve K and the fragment's symbol count."""
    if fmt in _PAIR_FORMATS:
        if k % 2 or tile_k % 2:
            raise ValueError("pair symbols need even K and tile_k")
        return k // 2, tile_k // 2, 4
    return k, tile_k, 8


def symbolise(fmt: int, w):
    """Return (symbols [N,K] (uint16 [N,K/2] for bf16 pairs, uint8 [N,K/2]
    for int4 pairs, else uint8), raw low bytes uint8 [N,K] or None)."""
    w = np.asarray(w)
    if fmt == FMT_INT8:
        return w.astype(np.int8).view(np.uint8), None
    if fmt == FMT_INT4:
        if w.min() < 0 or w.max() > 15:
            raise ValueError("int4 codes must be in [0, 15]")
        return w.astype(np.uint8), None
    if fmt == FMT_FP8:
        return w.astype(np.uint8), None
    if fmt == FMT_BF16:
        b = w.astype(np.uint16)
        return (b >> 8).astype(np.uint8), (b & 0xFF).astype(np.uint8)
    if fmt == FMT_BF16_EXP:
        b = w.astype(np.uint16)
        sym = ((b >> 7) & 0xFF).astype(np.uint8)
        raw = (((b >> 8) & 0x80) | (b & 0x7F)).astype(np.uint8)
        return sym, raw
    if fmt == FMT_INT4_PAIR:
        if w.min() < 0 or w.max() > 15:
            raise ValueError("int4 codes must be in [0, 15]")
        if w.shape[1] % 2:
            raise ValueError("int4 pairs need an even K")
        q = w.astype(np.uint8)
        return (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8), None
    if fmt == FMT_BF16_PAIR:
        b = w.astype(np.uint16)
        if b.shape[1] % 2:
            raise ValueError("bf16 pairs need an even K")
        hi = (b >> 8).astype(np.uint16)
        return (hi[:, 0::2] | (hi[:, 1::2] << 8)).astype(np.uint16), (b & 0xFF).astype(np.uint8)
    if fmt == FMT_BF16_WORD:
        return w.astype(np.uint16), None
    raise ValueError("unknown format")


def compress_layer(fmt: int, w, tile_n: int, tile_k: int, lanes: int,
                   prob_bits: int = 12) -> bytes:
    w = np.asarray(w)
    n, k = w.shape
    order.check_geometry(n, k, tile_n, tile_k, lanes)
    ks_, tks, epl = symbol_geometry(fmt, n, k, tile_n, tile_k)
    order.check_geometry(n, ks_, tile_n, tks, lanes, epl)
    sym, raw = symbolise(fmt, w)
    alpha = alphabet_of(fmt)
    counts = entropy.histogram(sym, alpha)
    f = freq.quantize_freqs(counts, prob_bits)
    tsym = order.gather_tiles(sym, tile_n, tks, lanes, epl=epl)
    states, words, ks = rans.encode_tiles(tsym, f, lanes, prob_bits, rans.KMAX)
    tiles = tsym.shape[0]
    T = tile_n * tile_k

    chunks, off = [], [0]
    for t in range(tiles):
        wd = words[t]
        if wd.size % 2:
            wd = np.concatenate([wd, np.zeros(1, np.uint16)])
        c = states[t].astype("<u4").tobytes() + wd.astype("<u2").tobytes()
        chunks.append(c)
        off.append(off[-1] + len(c) // 4)
    table_off = HEADER_BYTES
    if sparse_table(fmt):
        present = np.nonzero(f)[0]
        fv = f[present].astype(np.uint32) - sparse_f_bias(fmt)
        table = (present.astype(np.uint32) | (fv << 16)).astype("<u4")
        table_bytes, alpha_field = table.tobytes(), int(present.size)
    else:
        table_bytes, alpha_field = f.astype("<u2").tobytes(), alpha
    index_off = _align(table_off + len(table_bytes), 16)
    ktab_off = _align(index_off + 4 * (tiles + 1), 16)
    streams_off = _align(ktab_off + tiles, 16)
    streams_end = streams_off + 4 * off[-1]
    if raw is not None:
        raw_off = _align(streams_end, 16)
        total = raw_off + tiles * T
    else:
        raw_off, total = 0, streams_end
    max_len = max(off[t + 1] - off[t] for t in range(tiles))
    hdr = _HDR.pack(MAGIC, VERSION, HEADER_BYTES, fmt, 0, n, k, tile_n, tile_k,
                    lanes, prob_bits, alpha_field, tiles, table_off, index_off,
                    ktab_off, streams_off, raw_off, total, max_len, rans.KMAX)
    buf = bytearray(total)
    buf[0:HEADER_BYTES] = hdr
    buf[table_off:table_off + len(table_bytes)] = table_bytes
    buf[index_off:index_off + 4 * (tiles + 1)] = np.asarray(off, "<u4").tobytes()
    buf[ktab_off:ktab_off + tiles] = ks.astype(np.uint8).tobytes()
    buf[streams_off:streams_end] = b"".join(chunks)
    if raw is not None:
        rtiles = order.gather_tiles(raw, tile_n, tile_k, lanes, raw=True)
        buf[raw_off:total] = rtiles.astype(np.uint8).tobytes()
    return bytes(buf)


def parse(blob) -> dict:
    """Header fields plus table, index; validates what a reader must trust."""
    b = bytes(blob) if not isinstance(blob, (bytes, bytearray)) else blob
    if len(b) < HEADER_BYTES:
        raise ValueError("blob shorter than header")
    v = _HDR.unpack_from(b, 0)
    keys = ["magic", "version", "header_bytes", "fmt", "flags", "n", "k",
            "tile_n", "tile_k", "lanes", "prob_bits", "alphabet", "tiles",
            "table_off", "index_off", "ktab_off", "streams_off", "raw_off", "total",
            "max_tile_words4", "kmax"]
    h = dict(zip(keys, v))
    if h["magic"] != MAGIC or h["version"] != VERSION or h["header_bytes"] != HEADER_BYTES:
        raise ValueError("bad magic / version")
    if h["total"] != len(b):
        raise ValueError("size mismatch")
    order.check_geometry(h["n"], h["k"], h["tile_n"], h["tile_k"], h["lanes"])
    if sparse_table(h["fmt"]):
        if not 1 <= h["alphabet"] <= (1 << h["prob_bits"]):
            raise ValueError("bad table size")
    elif h["alphabet"] != alphabet_of(h["fmt"]):
        raise ValueError("bad alphabet")
    ksym, tks, epl = symbol_geometry(h["fmt"], h["n"], h["k"], h["tile_n"], h["tile_k"])
    order.check_geometry(h["n"], ksym, h["tile_n"], tks, h["lanes"], epl)
    h["steps"] = h["tile_n"] * tks // h["lanes"]
    nt = (h["n"] // h["tile_n"]) * (h["k"] // h["tile_k"])
    if h["tiles"] != nt:
        raise ValueError("bad tile count")
    a, t = h["alphabet"], h["tiles"]
    if sparse_table(h["fmt"]):
        ent = np.frombuffer(b, "<u4", a, h["table_off"]).astype(np.int64)
        syms, fs = ent & 0xFFFF, (ent >> 16) + sparse_f_bias(h["fmt"])
        if (fs == 0).any() or (np.diff(syms) <= 0).any():
            raise ValueError("bad sparse table")
        h["freq"] = np.zeros(alphabet_of(h["fmt"]), np.int64)
        h["freq"][syms] = fs
    else:
        h["freq"] = np.frombuffer(b, "<u2", a, h["table_off"]).astype(np.int64)
    if h["freq"].sum() != (1 << h["prob_bits"]):
        raise ValueError("frequencies do not sum to 2**prob_bits")
    h["index"] = np.frombuffer(b, "<u4", t + 1, h["index_off"]).astype(np.int64)
    if h["index"][0] != 0 or (np.diff(h["index"]) < h["lanes"]).any():
        raise ValueError("index not monotone")
    end = h["streams_off"] + 4 * int(h["index"][-1])
    if end > len(b) or (h["raw_off"] and h["raw_off"] < end):
        raise ValueError("streams overrun")
    if int(np.diff(h["index"]).max()) != h["max_tile_words4"]:
        raise ValueError("bad max tile length")
    h["ks"] = np.frombuffer(b, np.uint8, t, h["ktab_off"]).astype(np.int64)
    S = h["steps"]
    if h["kmax"] > 255 or (h["ks"] > min(h["kmax"], S)).any():
        raise ValueError("bad payload step count")
    return h


def tile_stream(blob, h: dict, t: int):
    """(states [R] uint32, words uint16 incl. possible pad) of tile t."""
    start = h["streams_off"] + 4 * int(h["index"][t])
    end = h["streams_off"] + 4 * int(h["index"][t + 1])
    R = h["lanes"]
    states = np.frombuffer(blob, "<u4", R, start).astype(np.uint32)
    words = np.frombuffer(blob, "<u2", (end - start - 4 * R) // 2, start + 4 * R)
    return states, words


def decode_symbols(blob, tiles=None) -> np.ndarray:
    """Decoded symbols [len(tiles), T] in j order (all tiles by default)."""
    h = parse(blob)
    ids = range(h["tiles"]) if tiles is None else list(tiles)
    R = h["lanes"]
    S = h["steps"]
    st, ws = [], []
    for t in ids:
        s, w = tile_stream(blob, h, t)
        st.append(s)
        ws.append(w)
    # a stream holds R states and 2*(len4 - R) word slots; the coder uses
    # all of them, or all but a final zero pad word
    ks = h["ks"][np.asarray(list(ids), dtype=np.int64)]
    syms, used = rans.decode_tiles(np.asarray(st), ws, h["freq"], R, S, ks,
                                   h["prob_bits"], check=False, return_consumed=True)
    for i, w in enumerate(ws):
        if not (used[i] == len(w) or (used[i] == len(w) - 1 and w[-1] == 0)):
            raise rans.IntegrityError("stream length mismatch")
    return syms


def decompress_layer(blob) -> np.ndarray:
    """Rebuild the original codes: int8 -> int8, int4/fp8/int4 pairs -> uint8, bf16 -> uint16."""
    h = parse(blob)
    syms = decode_symbols(blob)
    n, k, tn, tk, R = h["n"], h["k"], h["tile_n"], h["tile_k"], h["lanes"]
    fmt = h["fmt"]
    if fmt == FMT_BF16_PAIR:
        pairs = order.scatter_tiles(syms.astype(np.uint16), n, k // 2, tn, tk // 2, R, epl=4)
        hi = np.empty((n, k), np.uint16)
        hi[:, 0::2] = pairs & 0xFF
        hi[:, 1::2] = pairs >> 8
        T = tn * tk
        raw = np.frombuffer(blob, np.uint8, h["tiles"] * T, h["raw_off"]).reshape(h["tiles"], T)
        lo = order.scatter_tiles(raw, n, k, tn, tk, R, raw=True).astype(np.uint16)
        return (hi << 8) | lo
    if fmt == FMT_BF16_WORD:
        return order.scatter_tiles(syms.astype(np.uint16), n, k, tn, tk, R)
    if fmt == FMT_INT4_PAIR:
        pairs = order.scatter_tiles(syms.astype(np.uint8), n, k // 2, tn, tk // 2, R, epl=4)
        out = np.empty((n, k), np.uint8)
        out[:, 0::2] = pairs & 15
        out[:, 1::2] = pairs >> 4
        return out
    sym = order.scatter_tiles(syms.astype(np.uint8), n, k, tn, tk, R)
    if fmt == FMT_INT8:
        return sym.view(np.int8)
    if fmt in (FMT_INT4, FMT_FP8):
        return sym
    T = tn * tk
    raw = np.frombuffer(blob, np.uint8, h["tiles"] * T, h["raw_off"]).reshape(h["tiles"], T)
    lo = order.scatter_tiles(raw, n, k, tn, tk, R, raw=True).astype(np.uint16)
    if fmt == FMT_BF16_EXP:
        return ((lo & 0x80) << 8) | (sym.astype(np.uint16) << 7) | (lo & 0x7F)
    return (sym.astype(np.uint16) << 8) | lo


def bits_per_weight(blob, n: int, k: int) -> float:
    return 8.0 * len(blob) / (n * k)
