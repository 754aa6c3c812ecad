// Internal constants and helpers of the compressed-layer format (library side).
//
// The format follows the execution model of the page "arXiv'26 | 无损压缩逼近
// Shannon 极限" §3.1 (tiles in the GEMM's geometry, one shared frequency
// table per layer, a per-tile offset index, R rANS lane states per tile); the
// byte layout itself is documented in include/dgt.h.
#pragma once

#include <cstddef>
#include <cstdint>

namespace dgt {

constexpr uint32_t kMagic = 0x31544744u;  // "DGT1" little-endian
constexpr uint32_t kVersion = 1;
constexpr uint32_t kHeaderBytes = 128;
constexpr uint32_t kStateL = 1u << 16;     // normalised states live in [L, 2^32)
constexpr uint32_t kKmax = 16;             // payload-step cap per tile
constexpr uint32_t kGroup = 128;           // INT4 scale group along K

// Byte offsets of header fields.
struct HeaderLayout {
  static constexpr size_t magic = 0, version = 4, header_bytes = 6, fmt = 8, flags = 12,
                          n = 16, k = 20, tile_n = 24, tile_k = 28, lanes = 32,
                          prob_bits = 36, alphabet = 40, tiles = 44, table_off = 48,
                          index_off = 56, ktab_off = 64, streams_off = 72, raw_off = 80,
                          total = 88, max_tile_words4 = 96, kmax = 100;
};

inline uint32_t alphabet_of(uint32_t fmt) {
  return fmt == 2 ? 16u : (fmt == 7 || fmt == 8) ? 65536u : 256u;
}
// formats whose table lists the present symbols only: u32 symbol | (f - bias) << 16
inline bool sparse_table(uint32_t fmt) { return fmt == 7 || fmt == 8; }
// BF16_WORD (frequency precision 16 bits) stores f - 1, so that f = 2^16 fits
inline uint32_t sparse_f_bias(uint32_t fmt) { return fmt == 8 ? 1u : 0u; }
// weights coded per symbol (INT4_PAIR and BF16_PAIR pack two along K)
inline uint32_t weights_per_symbol(uint32_t fmt) { return (fmt == 5 || fmt == 7) ? 2u : 1u; }
// symbols per lane per 16-row fragment (8 weights either way)
inline uint32_t symbols_per_lane(uint32_t fmt) { return 8u / weights_per_symbol(fmt); }
// formats that store one raw byte per weight beside the coded symbol
inline bool has_raw(uint32_t fmt) { return fmt == 4 || fmt == 6 || fmt == 7; }

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Tile-local position of symbol j = s*R + p (s = epl*g + e; g = fk*Fn + fn),
// epl symbols per lane per fragment; col counts symbols (weights, or pairs).
// R = 128 (two states per wave lane): states p < 64 order the top tile_n/2
// rows and states 64 + p the bottom ones, each half as an R = 64 tile.
inline void symbol_position(uint32_t j, uint32_t tile_n, uint32_t lanes, uint32_t epl,
                            uint32_t* row, uint32_t* col) {
  if (lanes == 128) {
    const uint32_t s = j / 128, p = j % 128;
    symbol_position(s * 64 + (p & 63), tile_n / 2, 64, epl, row, col);
    *row += (p >> 6) * (tile_n / 2);
    return;
  }
  const uint32_t s = j / lanes, p = j % lanes;
  const uint32_t g = s / epl, e = s % epl;
  const uint32_t fn_count = tile_n / 16;
  const uint32_t fk = g / fn_count, fn = g % fn_count;
  *row = fn * 16 + (p & 15);
  *col = fk * (lanes / 16) * epl + (p >> 4) * epl + e;
}

// Tile-local position of raw byte q = g*8R + p*8 + e (lane-major).
inline void raw_position(uint32_t q, uint32_t tile_n, uint32_t lanes, uint32_t* row,
                         uint32_t* col) {
  if (lanes == 128) {
    const uint32_t g = q / 1024, p = (q % 1024) >> 3;
    raw_position(g * 512 + (p & 63) * 8 + (q & 7), tile_n / 2, 64, row, col);
    *row += (p >> 6) * (tile_n / 2);
    return;
  }
  const uint32_t g = q / (8 * lanes), rem = q % (8 * lanes);
  const uint32_t p = rem >> 3, e = rem & 7;
  const uint32_t fn_count = tile_n / 16;
  const uint32_t fk = g / fn_count, fn = g % fn_count;
  *row = fn * 16 + (p & 15);
  *col = fk * (lanes / 2) + (p >> 4) * 8 + e;
}

}  // namespace dgt
