/*
 * dgt.h -- C ABI of libdgt: tile-granular lossless rANS coding of LLM weight
 * matrices, decoded on the fly inside the GEMM that consumes them (AMD
 * MI355X / gfx950).
 *
 * Source of the method: the page "arXiv'26 | 无损压缩逼近 Shannon 极限：你的
 * LLM 权重里一半以上的 bit 是白存的" (write-up of "Approaching Shannon Bound
 * with Lossless LLM Weight Compression"), cited below as [P §n]:
 *   §2.2  decode must keep up with memory bandwidth, any tile must decode on
 *         its own, decoded weights go to on-chip memory and never to global
 *         memory;
 *   §3.1  offline, each layer is cut into tiles in the GEMM's tiling geometry,
 *         all tiles share one compact ANS codebook, a light index records each
 *         tile's start offset, every tile stream is split into R lane
 *         sub-streams with one rANS state per lane; at run time tile k+1 is
 *         decoded while tile k is multiplied, in a static tile-swizzle order,
 *         packaged as a kernel a framework can call directly;
 *   §4.1  finite-precision frequency normalisation.
 *
 * Conventions for every entry point:
 *   - Plain C types only.  Pointers prefixed d_ are device (HIP) pointers,
 *     others are host pointers.  `stream` is a hipStream_t passed as void*
 *     (NULL = the default stream).  Device entry points are asynchronous on
 *     that stream and return as soon as the work is enqueued.
 *   - The caller owns every buffer; the library allocates no device memory.
 *   - Return value: DGT_OK (0) or a negative dgt_status.  No exceptions cross
 *     the ABI.  On error nothing has been enqueued.
 *   - Device blobs must be 16-byte aligned.  All multi-byte fields are
 *     little-endian.  Calls are thread-safe.
 *   - Environment: DGT_STAGING=whole|ring overrides the per-layer choice of
 *     how device kernels bring tile streams on chip (whole streams, or a
 *     two-chunk ring for one tile per wave); DGT_ROUNDS=n forces n rounds of
 *     chains per workgroup where the multi-round fused kernel applies (ring
 *     staging, M <= 16 per launch, 64 or 128 lanes) instead of the per-layer
 *     choice (1 = one round); DGT_XM_SINGLE_BUFFER=1 makes the large-M fused
 *     kernel (17 <= M <= 256 per pass, 64 lanes) keep one fragment buffer
 *     instead of two (a comparison point; an error where no such kernel
 *     exists).  Results are identical.  DGT_XM_SUBSETS=0 keeps the 8-wave
 *     large-M kernel where the 16-wave subset form would run (256-row tiles,
 *     64 lanes, 17 <= M <= 128, int4 pairs to 64); results agree within
 *     rounding (another order of additions).  Read at every call;
 *     dgt_gemm_workspace covers every choice.
 *
 * Compressed layer ("blob") format, version 1 (all offsets in bytes):
 *   header (128 B): magic "DGT1", u16 version, u16 header size, u32 fmt,
 *     u32 flags, u32 N, K, tile_n, tile_k, lanes R, prob_bits, alphabet,
 *     tiles; u64 table, index, ktab, streams, raw offsets, u64 total size;
 *     u32 max tile length (4-byte units), u32 kmax (16); zero padding.
 *   table  u16 f[alphabet], sum f = 2^prob_bits (shared by all tiles);
 *          BF16_PAIR and BF16_WORD (alphabet 65536): u32 symbol | f << 16
 *          (BF16_WORD: symbol | (f - 1) << 16) for each symbol with f > 0, in
 *          increasing symbol order, and the header's alphabet field holds the
 *          number of entries.
 *   index  u32 off[tiles+1]: tile t's stream starts at streams + 4*off[t].
 *   ktab   u8 k[tiles]: initial-state payload steps of each tile.
 *   streams per tile: R u32 lane states, u16 words in decode order, zero pad.
 *   raw    (BF16_SPLIT, BF16_EXP, BF16_PAIR) T raw bytes per tile, lane-major.
 * Tile t = bn*(K/tile_k) + bk covers W rows bn*tile_n.. and columns
 * bk*tile_k..  Inside a tile, symbol j = s*R + p (step s, lane p) with
 * s = 8g + e, fragment g = fk*(tile_n/16) + fn: lane p decodes row
 * 16fn + p%16, column fk*R/2 + 8*(p/16) + e.  rANS: state in [2^16, 2^32),
 * INT4_PAIR (and BF16_PAIR, whose symbol is the two weights' high bytes)
 * codes symbol c of a row for the weight pair (2c, 2c+1) and lays
 * out a tile's tile_n*tile_k/2 symbols the same way with 4 symbols per lane
 * per fragment (s = 4g + e, pair column fk*R/4 + 4*(p/16) + e), so a lane's
 * 4 symbols are again its 8 consecutive weights of one row.
 * R = 128 (two states per wave lane; tile_n a multiple of 32): states p < 64
 * order the top tile_n/2 rows and states 64 + p the bottom tile_n/2 rows,
 * each half exactly as an R = 64 tile of tile_n/2 rows; both share the one
 * word stream (interleaving j = s*128 + p); raw byte q = g*1024 + p*8 + e.
 * 16-bit renormalisation words; decode x' = f*(x>>n) + (x mod 2^n) - c_s,
 * then if x' < 2^16 read one word.  The last k[t] steps of a tile decode from
 * y = x - 2^16 without reading words; a valid tile ends with y == 0 on every
 * lane and its stream consumed exactly.
 */
#ifndef DGT_H_
#define DGT_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Weight formats ([P §2.1]: the formats whose codes are entropy coded). */
enum dgt_format {
  DGT_FMT_INT8 = 1,       /* int8 codes; GEMM value = the integer (exact bf16) */
  DGT_FMT_INT4 = 2,       /* codes 0..15, zero point 8, bf16 scale per 128 columns */
  DGT_FMT_FP8_E4M3 = 3,   /* OCP e4m3 bytes, per-tensor fp32 weight scale */
  DGT_FMT_BF16_SPLIT = 4, /* bf16: high byte coded, low byte stored raw */
  DGT_FMT_INT4_PAIR = 5,  /* INT4 weights and scales, coded two per symbol:
                             q[n,2c] | q[n,2c+1] << 4 (alphabet 256) */
  DGT_FMT_BF16_EXP = 6,   /* bf16: exponent (bits 14..7) coded, sign and mantissa
                             stored raw as one byte (sign << 7 | mantissa) */
  DGT_FMT_BF16_PAIR = 7,  /* bf16 byte split with the high bytes of two weights
                             adjacent along K coded as one 16-bit symbol
                             hi[n,2c] | hi[n,2c+1] << 8; low bytes raw */
  DGT_FMT_BF16_WORD = 8   /* bf16 whole words: the 16-bit pattern is the symbol,
                             frequency precision prob_bits = 16 ([P §4.1]:
                             16-bit symbols need a precise table), nothing raw */
};

enum dgt_status {
  DGT_OK = 0,
  DGT_E_ARG = -1,         /* null pointer or out-of-range scalar argument */
  DGT_E_SHAPE = -2,       /* N, K not multiples of the tile; bad tile/lane geometry */
  DGT_E_ALPHABET = -3,    /* code outside the format's alphabet */
  DGT_E_BUFSIZE = -4,     /* output / workspace buffer too small */
  DGT_E_FORMAT = -5,      /* blob header not recognised (magic, version, fmt) */
  DGT_E_CORRUPT = -6,     /* blob inconsistent (sizes, index, table, ktab) */
  DGT_E_HIP = -7,         /* a HIP runtime call or kernel launch failed */
  DGT_E_UNSUPPORTED = -8  /* valid request this library does not implement */
};

/* Layer geometry for compression.  prob_bits: frequency precision n (12;
 * BF16_WORD: 16, which the device kernels require for it). */
typedef struct dgt_params {
  uint32_t fmt, n, k, tile_n, tile_k, lanes, prob_bits, flags;
} dgt_params;

/* Parsed, validated view of a blob (filled by dgt_layer_info). */
typedef struct dgt_info {
  uint32_t fmt, n, k, tile_n, tile_k, lanes, prob_bits, alphabet;
  uint32_t tiles, max_tile_words4, kmax, flags;
  uint64_t table_off, index_off, ktab_off, streams_off, raw_off, total_bytes;
  uint64_t stream_bytes;     /* bytes of the streams section */
  double bits_per_weight;    /* 8 * total_bytes / (N*K) */
} dgt_info;

/* Library ABI version (1). */
int dgt_version(void);

/* Human-readable text for a dgt_status code (static storage). */
const char* dgt_status_string(int status);

/* Upper bound of the blob size dgt_compress_layer can produce for `p`
 * (every symbol costing a full word); 0 if `p` is invalid. */
size_t dgt_compress_bound(const dgt_params* p);

/* Offline encoder ([P §3.1] offline stage), host only.
 *   w: N*K weights row-major: one byte per weight for INT8 (two's
 *      complement), INT4 and INT4_PAIR (values 0..15; INT4_PAIR needs even
 *      K and tile_k) and FP8_E4M3; one uint16 bf16 bit pattern per weight
 *      for BF16_SPLIT, BF16_EXP, BF16_PAIR and BF16_WORD.
 *   out/cap: caller buffer of `cap` bytes; *out_size receives the blob size.
 * Errors: E_ARG, E_SHAPE, E_ALPHABET (INT4 code > 15), E_BUFSIZE.
 * Deterministic: the same input always gives the same bytes. */
int dgt_compress_layer(const dgt_params* p, const void* w, void* out, size_t cap,
                       size_t* out_size);

/* Parse and validate a host copy of a blob (header, table sums to 2^n,
 * index monotone and inside the blob, ktab <= min(kmax, steps)).
 * Errors: E_ARG, E_FORMAT, E_CORRUPT. */
int dgt_layer_info(const void* blob, size_t size, dgt_info* out);

/* Decode tiles to global memory (the layer-granular "decompress first" path,
 * kept for tests and the decompress-then-GEMM comparison; [P §2.2] names it
 * as what the fused path avoids).
 *   d_blob: device copy of the blob described by `info`.
 *   d_tile_ids: n_ids tile ids to decode, or NULL for all tiles (n_ids ignored).
 *          An id >= the layer's tile count is skipped on the device: nothing
 *          is written for it (neither d_out nor d_status), and the reads made
 *          in its place stay inside the blob (tile 0's stream).
 *   d_out: the full W layout, row-major [N, K]: uint8 (INT8 bytes, INT4
 *          and INT4_PAIR codes, FP8 bytes) or uint16 bf16 bits (BF16_SPLIT,
 *          BF16_EXP);
 *          only the elements of the decoded tiles are written.
 *   d_status: NULL or int32[tiles]; entry t is set to 0 when tile t decoded
 *          with a consistent stream, else to a positive error mask
 *          (1 = final state, 2 = stream length, 4 = stream overrun).
 * Errors (synchronous): E_ARG, E_UNSUPPORTED (lanes not 32/64/128; R = 32
 * streams too long for on-chip staging), E_HIP. */
int dgt_decode_tiles(const void* d_blob, const dgt_info* info, const uint32_t* d_tile_ids,
                     uint32_t n_ids, void* d_out, int32_t* d_status, void* stream);

/* Workspace bytes dgt_fused_decode_gemm needs for `m` activation rows.  The
 * workspace must be zero-filled before its first use; every call leaves it
 * ready for the next one (its counters return to zero). */
size_t dgt_gemm_workspace(const dgt_info* info, uint32_t m);

/* Fused decode + GEMM ([P §3.1] run-time stage): Y[m, n] = sum_k X[m, k] W[n, k]
 * with W decoded tile by tile on chip, never written to global memory.
 *   d_x: bf16 bits [m, K] row-major; m in 1..65536.  Up to 256 rows run in
 *        one pass in which every tile is decoded once; more rows run in
 *        passes of 256 (the layer is decoded once per pass).
 *   d_scales: INT4 and INT4_PAIR, bf16 bits [N, K/128]; else NULL.
 *   w_scale: FP8 only, per-tensor weight scale (X is quantised to e4m3 per
 *            tensor on the device first); ignored otherwise.
 *   d_y: fp32 [m, N] row-major, overwritten.
 *   d_ws, ws_bytes: workspace of at least dgt_gemm_workspace(info, m) bytes.
 *   d_status: NULL or int32[tiles], as for dgt_decode_tiles.
 * Values: INT8 -> bf16(code); INT4, INT4_PAIR -> bf16_RNE((q-8)*scale); BF16_SPLIT,
 * BF16_EXP -> the bf16 bits;
 * FP8 -> e4m3 products scaled by sx*w_scale; fp32 accumulation.
 * Errors: E_ARG, E_BUFSIZE (workspace), E_UNSUPPORTED, E_HIP. */
int dgt_fused_decode_gemm(const void* d_blob, const dgt_info* info, const uint16_t* d_x,
                          uint32_t m, const uint16_t* d_scales, float w_scale, float* d_y,
                          void* d_ws, size_t ws_bytes, int32_t* d_status, void* stream);

/* Allocation-free variant of dgt_fused_decode_gemm, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, values and errors, but
 * no workspace argument: the workspace is a static device array of
 * dgt_noalloc_scratch_bytes() bytes (64 MiB) that every device the library
 * runs on holds from the library's load until the process ends.  A call whose
 * workspace (dgt_gemm_workspace) would exceed it returns DGT_E_BUFSIZE and
 * enqueues nothing; M <= 16 fits every layer up to 53248 x 16384 (55 MiB at
 * most), and so does M <= 64 for 256 x 64 tiles at 64 lanes (39 MiB at most)
 * and M <= 256 up to 14336 x 4096 (42 MiB).  Each call
 * first zeroes the array's counters with a small kernel on `stream`.  All
 * calls on one device share the array: calls that overlap in time on one
 * device (other streams, other threads) race and give wrong results.  Calls
 * no hipMalloc, hipFree or allocating library routine. */
size_t dgt_noalloc_scratch_bytes(void);
int dgt_fused_decode_gemm_noalloc(const void* d_blob, const dgt_info* info, const uint16_t* d_x,
                                  uint32_t m, const uint16_t* d_scales, float w_scale,
                                  float* d_y, int32_t* d_status, void* stream);

/* Uncompressed baseline: Y = X W^T with W read from global memory, d_w is
 * [N, K] in the same element layout dgt_decode_tiles writes (INT4_PAIR is
 * read as INT4, BF16_EXP, BF16_PAIR and BF16_WORD as BF16_SPLIT), same weight
 * values and epilogue as the fused call.  M = 1 runs a streaming GEMV (K <=
 * 32768), M >= 32 an LDS-tiled MFMA GEMM reading each W block once per 128
 * rows, the rows between in the fused call's strip decomposition.  Workspace
 * from dgt_dense_workspace (zero-filled before first use); M <= 256. */
size_t dgt_dense_workspace(uint32_t fmt, uint32_t n, uint32_t k, uint32_t tile_n,
                           uint32_t m);
int dgt_dense_gemm(uint32_t fmt, uint32_t n, uint32_t k, uint32_t tile_n, const void* d_w,
                   const uint16_t* d_x, uint32_t m, const uint16_t* d_scales, float w_scale,
                   float* d_y, void* d_ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DGT_H_ */
