// Host side of libdgt: the offline encoder and blob validation.
//
// Follows the offline stage of the page "arXiv'26 | 无损压缩逼近 Shannon 极限"
// §3.1: a layer is cut into tiles in the GEMM's tiling geometry, one compact
// frequency table is shared by all tiles (§4.1: finite-precision
// normalisation), every tile is rANS coded on its own as R interleaved lane
// sub-streams, and a light index records where each tile's stream starts.
// rANS is the range variant of Duda's asymmetric numeral systems (named in the
// reference list of the podcast page "Approaching Shannon Bound: Lossless LLM
// Weight Compression").  Tiles are coded in parallel on the host cores.
#include <algorithm>
#include <atomic>
#include <cstring>
#include <thread>
#include <vector>

#include "../../include/dgt.h"
#include "dgt_format.h"

namespace {

using dgt::HeaderLayout;

template <typename T>
void put(uint8_t* base, size_t off, T v) {
  std::memcpy(base + off, &v, sizeof(T));
}
template <typename T>
T get(const uint8_t* base, size_t off) {
  T v;
  std::memcpy(&v, base + off, sizeof(T));
  return v;
}

bool geometry_ok(uint32_t fmt, uint32_t n, uint32_t k, uint32_t tn, uint32_t tk,
                 uint32_t lanes) {
  if (!n || !k || !tn || !tk || !lanes) return false;
  if (n % tn || k % tk) return false;
  if (lanes == 128) {  // two R = 64 halves of tn/2 rows
    if (tn % 32) return false;
    tn /= 2;
    lanes = 64;
  }
  if (lanes % 16 || tn % 16) return false;
  if (tk % (lanes / 2)) return false;  // whole fragments of R/2 weights
  const uint32_t wps = dgt::weights_per_symbol(fmt);
  if (tk % wps) return false;
  if ((uint64_t)tn * (tk / wps) % lanes) return false;
  return true;
}

// frequency precision a format allows: 8..15 bits, or exactly 16 for whole
// bf16 words (a u16 dense entry cannot hold f = 2^16)
bool prob_bits_ok(uint32_t fmt, uint32_t prob_bits) {
  if (fmt == DGT_FMT_BF16_WORD) return prob_bits >= 12 && prob_bits <= 16;
  return prob_bits >= 8 && prob_bits <= 15;
}

bool params_ok(const dgt_params* p) {
  if (!p) return false;
  if (p->fmt < DGT_FMT_INT8 || p->fmt > DGT_FMT_BF16_WORD) return false;
  return prob_bits_ok(p->fmt, p->prob_bits);
}

// Integer frequency quantisation to M = 2^prob_bits (largest remainder, ties
// to the smaller symbol; then take from the largest frequency while the sum
// exceeds M).  Identical integer rule everywhere, so encoders agree bitwise.
bool quantize(const std::vector<uint64_t>& counts, uint32_t prob_bits,
              std::vector<uint32_t>* out) {
  const uint64_t M = 1ull << prob_bits;
  uint64_t N = 0;
  std::vector<uint32_t> present;
  for (size_t s = 0; s < counts.size(); ++s) {
    N += counts[s];
    if (counts[s]) present.push_back((uint32_t)s);
  }
  if (N == 0 || present.size() > M) return false;
  std::vector<int64_t> f(counts.size(), 0);
  int64_t sum = 0;
  for (uint32_t s : present) {
    const uint64_t q = (unsigned __int128)counts[s] * M / N;
    f[s] = q ? (int64_t)q : 1;
    sum += f[s];
  }
  int64_t d = (int64_t)M - sum;
  if (d > 0) {
    std::vector<uint32_t> ranked = present;
    std::sort(ranked.begin(), ranked.end(), [&](uint32_t a, uint32_t b) {
      const uint64_t ra = (uint64_t)((unsigned __int128)counts[a] * M % N);
      const uint64_t rb = (uint64_t)((unsigned __int128)counts[b] * M % N);
      if (ra != rb) return ra > rb;
      return a < b;
    });
    for (uint32_t s : ranked) {
      if (d == 0) break;
      ++f[s];
      --d;
    }
    if (d) return false;
  }
  while (d < 0) {
    int best = -1;
    for (uint32_t s : present)
      if (f[s] > 1 && (best < 0 || f[s] > f[best])) best = (int)s;
    if (best < 0) return false;
    --f[best];
    ++d;
  }
  out->assign(counts.size(), 0);
  for (size_t s = 0; s < counts.size(); ++s) (*out)[s] = (uint32_t)f[s];
  return true;
}

struct TileOut {
  std::vector<uint32_t> states;
  std::vector<uint16_t> words;  // stream (decoder) order
  uint32_t k = 0;
};

// Encode one tile: symbols in j order (j = step*R + lane).
void encode_tile(const uint16_t* sym, uint32_t lanes, uint32_t steps, const uint32_t* f,
                 const uint32_t* c, uint32_t prob_bits, TileOut* out) {
  const uint64_t M = 1ull << prob_bits;
  const uint64_t y_limit = (1ull << 32) - dgt::kStateL;
  std::vector<uint64_t> y(lanes, 0), cand(lanes);
  uint32_t k = 0;
  const uint32_t kcap = std::min<uint32_t>(dgt::kKmax, steps);
  while (k < kcap) {
    const uint32_t step = steps - 1 - k;
    bool ok = true;
    for (uint32_t r = 0; r < lanes; ++r) {
      const uint32_t s = sym[(size_t)step * lanes + r];
      const uint64_t v = (y[r] / f[s]) * M + (y[r] % f[s]) + c[s];
      cand[r] = v;
      ok &= v < y_limit;
    }
    if (!ok) break;
    y.swap(cand);
    ++k;
  }
  std::vector<uint64_t> x(lanes);
  for (uint32_t r = 0; r < lanes; ++r) x[r] = dgt::kStateL + y[r];
  std::vector<uint16_t> E;
  E.reserve((size_t)steps * lanes / 4);
  for (int64_t step = (int64_t)steps - 1 - k; step >= 0; --step) {
    for (int64_t r = (int64_t)lanes - 1; r >= 0; --r) {
      const uint32_t s = sym[(size_t)step * lanes + r];
      const uint64_t fs = f[s];
      uint64_t xr = x[r];
      if (xr >= (fs << (32 - prob_bits))) {
        E.push_back((uint16_t)(xr & 0xFFFF));
        xr >>= 16;
      }
      x[r] = (xr / fs) * M + (xr % fs) + c[s];
    }
  }
  out->states.resize(lanes);
  for (uint32_t r = 0; r < lanes; ++r) out->states[r] = (uint32_t)x[r];
  out->words.assign(E.rbegin(), E.rend());
  out->k = k;
}

unsigned worker_count() {
  unsigned hw = std::thread::hardware_concurrency();
  if (hw == 0) hw = 4;
  return std::min(hw, 32u);
}

}  // namespace

extern "C" {

int dgt_version(void) { return 1; }

const char* dgt_status_string(int status) {
  switch (status) {
    case DGT_OK: return "ok";
    case DGT_E_ARG: return "invalid argument";
    case DGT_E_SHAPE: return "invalid shape or tile geometry";
    case DGT_E_ALPHABET: return "code outside the format alphabet";
    case DGT_E_BUFSIZE: return "buffer too small";
    case DGT_E_FORMAT: return "unrecognised blob format";
    case DGT_E_CORRUPT: return "corrupt blob";
    case DGT_E_HIP: return "HIP runtime error";
    case DGT_E_UNSUPPORTED: return "not supported by this library";
    default: return "unknown status";
  }
}

size_t dgt_compress_bound(const dgt_params* p) {
  if (!params_ok(p) || !geometry_ok(p->fmt, p->n, p->k, p->tile_n, p->tile_k, p->lanes))
    return 0;
  const uint64_t tiles = (uint64_t)(p->n / p->tile_n) * (p->k / p->tile_k);
  const uint64_t T = (uint64_t)p->tile_n * p->tile_k;
  const uint32_t alpha = dgt::alphabet_of(p->fmt);
  const uint64_t table = dgt::sparse_table(p->fmt) ? 4ull << p->prob_bits : 2ull * alpha;
  uint64_t b = dgt::kHeaderBytes + dgt::align_up(table, 16) +
               dgt::align_up(4 * (tiles + 1), 16) + dgt::align_up(tiles, 16);
  b += tiles * (4ull * p->lanes + 2 * T + 4) + 16;
  if (dgt::has_raw(p->fmt)) b += tiles * T + 16;
  return (size_t)b;
}

int dgt_compress_layer(const dgt_params* p, const void* w, void* out, size_t cap,
                       size_t* out_size) {
  if (!params_ok(p) || !w || !out || !out_size) return DGT_E_ARG;
  const uint32_t n = p->n, k = p->k, tn = p->tile_n, tk = p->tile_k, R = p->lanes;
  if (!geometry_ok(p->fmt, n, k, tn, tk, R)) return DGT_E_SHAPE;
  const uint32_t fmt = p->fmt, alpha = dgt::alphabet_of(fmt), pb = p->prob_bits;
  const uint64_t NK = (uint64_t)n * k;
  // the symbol matrix is [n, ks] with tiles of tn x tks symbols
  const uint32_t wps = dgt::weights_per_symbol(fmt), epl = dgt::symbols_per_lane(fmt);
  const uint32_t ks = k / wps, tks = tk / wps;
  const uint64_t NS = (uint64_t)n * ks;

  // symbolise: coded symbol (+ raw low byte for the bf16 splits)
  std::vector<uint16_t> sym(NS);
  std::vector<uint8_t> raw;
  if (fmt == DGT_FMT_BF16_PAIR) {
    raw.resize(NK);
    const uint16_t* b = static_cast<const uint16_t*>(w);
    for (uint64_t i = 0; i < NS; ++i)
      sym[i] = (uint16_t)((b[2 * i] >> 8) | (b[2 * i + 1] & 0xFF00u));
    for (uint64_t i = 0; i < NK; ++i) raw[i] = (uint8_t)(b[i] & 0xFF);
  } else if (fmt == DGT_FMT_INT4_PAIR) {
    const uint8_t* q = static_cast<const uint8_t*>(w);
    for (uint64_t i = 0; i < NS; ++i) {
      const uint8_t a = q[2 * i], b = q[2 * i + 1];
      if (a > 15 || b > 15) return DGT_E_ALPHABET;
      sym[i] = (uint8_t)(a | (b << 4));
    }
  } else if (fmt == DGT_FMT_BF16_WORD) {
    const uint16_t* b = static_cast<const uint16_t*>(w);
    for (uint64_t i = 0; i < NS; ++i) sym[i] = b[i];
  } else if (fmt == DGT_FMT_BF16_SPLIT) {
    raw.resize(NK);
    const uint16_t* b = static_cast<const uint16_t*>(w);
    for (uint64_t i = 0; i < NK; ++i) {
      sym[i] = (uint8_t)(b[i] >> 8);
      raw[i] = (uint8_t)(b[i] & 0xFF);
    }
  } else if (fmt == DGT_FMT_BF16_EXP) {
    raw.resize(NK);
    const uint16_t* b = static_cast<const uint16_t*>(w);
    for (uint64_t i = 0; i < NK; ++i) {
      sym[i] = (uint8_t)((b[i] >> 7) & 0xFF);
      raw[i] = (uint8_t)(((b[i] >> 8) & 0x80) | (b[i] & 0x7F));
    }
  } else {
    const uint8_t* q = static_cast<const uint8_t*>(w);
    for (uint64_t i = 0; i < NK; ++i) sym[i] = q[i];
    if (fmt == DGT_FMT_INT4)
      for (uint64_t i = 0; i < NK; ++i)
        if (sym[i] > 15) return DGT_E_ALPHABET;
  }

  // shared per-layer table
  std::vector<uint64_t> counts(alpha, 0);
  for (uint64_t i = 0; i < NS; ++i) counts[sym[i]]++;
  std::vector<uint32_t> f;
  if (!quantize(counts, pb, &f)) return DGT_E_ALPHABET;
  std::vector<uint32_t> c(alpha + 1, 0);
  for (uint32_t s = 0; s < alpha; ++s) c[s + 1] = c[s] + f[s];

  const uint32_t kt = k / tk;
  const uint64_t tiles = (uint64_t)(n / tn) * kt;
  const uint32_t T = tn * tk, TS = tn * tks, S = TS / R;
  if (tiles > 0xFFFFFFFFull) return DGT_E_SHAPE;

  // tile-local positions, shared by every tile (pos in the symbol matrix,
  // rpos in the weight matrix)
  std::vector<uint32_t> pos(TS), rpos(raw.empty() ? 0 : T);
  for (uint32_t j = 0; j < TS; ++j) {
    uint32_t r, col;
    dgt::symbol_position(j, tn, R, epl, &r, &col);
    pos[j] = r * ks + col;
  }
  for (uint32_t j = 0; j < (uint32_t)rpos.size(); ++j) {
    uint32_t r, col;
    dgt::raw_position(j, tn, R, &r, &col);
    rpos[j] = r * k + col;
  }

  std::vector<TileOut> enc(tiles);
  std::atomic<uint64_t> next{0};
  auto work = [&]() {
    std::vector<uint16_t> ts(TS);
    for (;;) {
      const uint64_t t = next.fetch_add(1);
      if (t >= tiles) break;
      const uint64_t base = (uint64_t)(t / kt) * tn * ks + (uint64_t)(t % kt) * tks;
      for (uint32_t j = 0; j < TS; ++j) ts[j] = sym[base + pos[j]];
      encode_tile(ts.data(), R, S, f.data(), c.data(), pb, &enc[t]);
    }
  };
  const unsigned nw = (unsigned)std::min<uint64_t>(worker_count(), tiles);
  std::vector<std::thread> pool;
  for (unsigned i = 1; i < nw; ++i) pool.emplace_back(work);
  work();
  for (auto& th : pool) th.join();

  // layout
  std::vector<uint32_t> off(tiles + 1, 0);
  uint32_t max_len = 0;
  for (uint64_t t = 0; t < tiles; ++t) {
    const uint64_t len4 = R + (enc[t].words.size() + 1) / 2;
    if ((uint64_t)off[t] + len4 > 0xFFFFFFFFull) return DGT_E_SHAPE;
    off[t + 1] = off[t] + (uint32_t)len4;
    max_len = std::max<uint32_t>(max_len, (uint32_t)len4);
  }
  // the table: dense u16 f[alphabet], or (sparse formats) u32 symbol | f << 16
  // for the present symbols in symbol order; the header's alphabet field then
  // holds the entry count
  uint32_t table_entries = alpha;
  size_t table_bytes = 2 * (size_t)alpha;
  if (dgt::sparse_table(fmt)) {
    table_entries = 0;
    for (uint32_t s = 0; s < alpha; ++s) table_entries += f[s] ? 1 : 0;
    table_bytes = 4 * (size_t)table_entries;
  }
  const size_t table_off = dgt::kHeaderBytes;
  const size_t index_off = dgt::align_up(table_off + table_bytes, 16);
  const size_t ktab_off = dgt::align_up(index_off + 4 * (tiles + 1), 16);
  const size_t streams_off = dgt::align_up(ktab_off + tiles, 16);
  const size_t streams_end = streams_off + 4 * (size_t)off[tiles];
  size_t raw_off = 0, total = streams_end;
  if (dgt::has_raw(fmt)) {
    raw_off = dgt::align_up(streams_end, 16);
    total = raw_off + tiles * (size_t)T;
  }
  *out_size = total;
  if (cap < total) return DGT_E_BUFSIZE;

  uint8_t* o = static_cast<uint8_t*>(out);
  std::memset(o, 0, std::min(total, (size_t)streams_off));
  put<uint32_t>(o, HeaderLayout::magic, dgt::kMagic);
  put<uint16_t>(o, HeaderLayout::version, (uint16_t)dgt::kVersion);
  put<uint16_t>(o, HeaderLayout::header_bytes, (uint16_t)dgt::kHeaderBytes);
  put<uint32_t>(o, HeaderLayout::fmt, fmt);
  put<uint32_t>(o, HeaderLayout::flags, 0);
  put<uint32_t>(o, HeaderLayout::n, n);
  put<uint32_t>(o, HeaderLayout::k, k);
  put<uint32_t>(o, HeaderLayout::tile_n, tn);
  put<uint32_t>(o, HeaderLayout::tile_k, tk);
  put<uint32_t>(o, HeaderLayout::lanes, R);
  put<uint32_t>(o, HeaderLayout::prob_bits, pb);
  put<uint32_t>(o, HeaderLayout::alphabet, table_entries);
  put<uint32_t>(o, HeaderLayout::tiles, (uint32_t)tiles);
  put<uint64_t>(o, HeaderLayout::table_off, table_off);
  put<uint64_t>(o, HeaderLayout::index_off, index_off);
  put<uint64_t>(o, HeaderLayout::ktab_off, ktab_off);
  put<uint64_t>(o, HeaderLayout::streams_off, streams_off);
  put<uint64_t>(o, HeaderLayout::raw_off, raw_off);
  put<uint64_t>(o, HeaderLayout::total, total);
  put<uint32_t>(o, HeaderLayout::max_tile_words4, max_len);
  put<uint32_t>(o, HeaderLayout::kmax, dgt::kKmax);
  if (dgt::sparse_table(fmt)) {
    size_t e = 0;
    for (uint32_t s = 0; s < alpha; ++s)
      if (f[s]) put<uint32_t>(o, table_off + 4 * e++, s | ((f[s] - dgt::sparse_f_bias(fmt)) << 16));
  } else {
    for (uint32_t s = 0; s < alpha; ++s) put<uint16_t>(o, table_off + 2 * s, (uint16_t)f[s]);
  }
  for (uint64_t t = 0; t <= tiles; ++t) put<uint32_t>(o, index_off + 4 * t, off[t]);
  for (uint64_t t = 0; t < tiles; ++t) o[ktab_off + t] = (uint8_t)enc[t].k;
  for (uint64_t t = 0; t < tiles; ++t) {
    uint8_t* dst = o + streams_off + 4 * (size_t)off[t];
    std::memcpy(dst, enc[t].states.data(), 4 * (size_t)R);
    const size_t nw_ = enc[t].words.size();
    if (nw_) std::memcpy(dst + 4 * R, enc[t].words.data(), 2 * nw_);  // (a constant layer has none)
    if (nw_ & 1) put<uint16_t>(dst, 4 * (size_t)R + 2 * nw_, 0);
  }
  if (raw_off) {
    if (raw_off > streams_end) std::memset(o + streams_end, 0, raw_off - streams_end);
    for (uint64_t t = 0; t < tiles; ++t) {
      const uint64_t base = (uint64_t)(t / kt) * tn * k + (uint64_t)(t % kt) * tk;
      uint8_t* dst = o + raw_off + t * (size_t)T;
      for (uint32_t q = 0; q < T; ++q) dst[q] = raw[base + rpos[q]];
    }
  }
  return DGT_OK;
}

int dgt_layer_info(const void* blob, size_t size, dgt_info* out) {
  if (!blob || !out) return DGT_E_ARG;
  const uint8_t* b = static_cast<const uint8_t*>(blob);
  if (size < dgt::kHeaderBytes) return DGT_E_FORMAT;
  if (get<uint32_t>(b, HeaderLayout::magic) != dgt::kMagic ||
      get<uint16_t>(b, HeaderLayout::version) != dgt::kVersion ||
      get<uint16_t>(b, HeaderLayout::header_bytes) != dgt::kHeaderBytes)
    return DGT_E_FORMAT;
  dgt_info in{};
  in.fmt = get<uint32_t>(b, HeaderLayout::fmt);
  in.flags = get<uint32_t>(b, HeaderLayout::flags);
  in.n = get<uint32_t>(b, HeaderLayout::n);
  in.k = get<uint32_t>(b, HeaderLayout::k);
  in.tile_n = get<uint32_t>(b, HeaderLayout::tile_n);
  in.tile_k = get<uint32_t>(b, HeaderLayout::tile_k);
  in.lanes = get<uint32_t>(b, HeaderLayout::lanes);
  in.prob_bits = get<uint32_t>(b, HeaderLayout::prob_bits);
  in.alphabet = get<uint32_t>(b, HeaderLayout::alphabet);
  in.tiles = get<uint32_t>(b, HeaderLayout::tiles);
  in.table_off = get<uint64_t>(b, HeaderLayout::table_off);
  in.index_off = get<uint64_t>(b, HeaderLayout::index_off);
  in.ktab_off = get<uint64_t>(b, HeaderLayout::ktab_off);
  in.streams_off = get<uint64_t>(b, HeaderLayout::streams_off);
  in.raw_off = get<uint64_t>(b, HeaderLayout::raw_off);
  in.total_bytes = get<uint64_t>(b, HeaderLayout::total);
  in.max_tile_words4 = get<uint32_t>(b, HeaderLayout::max_tile_words4);
  in.kmax = get<uint32_t>(b, HeaderLayout::kmax);
  if (in.fmt < DGT_FMT_INT8 || in.fmt > DGT_FMT_BF16_WORD) return DGT_E_FORMAT;
  if (in.flags != 0) return DGT_E_FORMAT;
  if (in.total_bytes != size) return DGT_E_CORRUPT;
  if (!geometry_ok(in.fmt, in.n, in.k, in.tile_n, in.tile_k, in.lanes)) return DGT_E_CORRUPT;
  if (!prob_bits_ok(in.fmt, in.prob_bits)) return DGT_E_CORRUPT;
  const bool sparse = dgt::sparse_table(in.fmt);
  if (sparse ? (in.alphabet == 0 || in.alphabet > (1u << in.prob_bits))
             : in.alphabet != dgt::alphabet_of(in.fmt))
    return DGT_E_CORRUPT;
  const uint64_t table_bytes = (sparse ? 4ull : 2ull) * in.alphabet;
  const uint64_t tiles = (uint64_t)(in.n / in.tile_n) * (in.k / in.tile_k);
  if (tiles != in.tiles) return DGT_E_CORRUPT;
  const uint64_t T = (uint64_t)in.tile_n * in.tile_k;
  const uint64_t S = T / dgt::weights_per_symbol(in.fmt) / in.lanes;
  if (in.kmax > 255) return DGT_E_CORRUPT;
  // section bounds and alignment
  if (in.table_off < dgt::kHeaderBytes || in.table_off % 16 ||
      in.table_off + table_bytes > in.index_off || in.index_off % 16 ||
      in.index_off + 4 * (tiles + 1) > in.ktab_off || in.ktab_off % 16 ||
      in.ktab_off + tiles > in.streams_off || in.streams_off % 16 || in.streams_off > size)
    return DGT_E_CORRUPT;
  uint64_t fsum = 0;
  if (sparse) {
    int64_t prev_sym = -1;
    for (uint32_t e = 0; e < in.alphabet; ++e) {
      const uint32_t v = get<uint32_t>(b, in.table_off + 4 * e);
      const uint32_t fv = (v >> 16) + dgt::sparse_f_bias(in.fmt);
      if ((int64_t)(v & 0xFFFF) <= prev_sym || fv == 0) return DGT_E_CORRUPT;
      prev_sym = v & 0xFFFF;
      fsum += fv;
    }
  } else {
    for (uint32_t s = 0; s < in.alphabet; ++s) fsum += get<uint16_t>(b, in.table_off + 2 * s);
  }
  if (fsum != (1ull << in.prob_bits)) return DGT_E_CORRUPT;
  uint32_t prev = get<uint32_t>(b, in.index_off), maxlen = 0;
  if (prev != 0) return DGT_E_CORRUPT;
  for (uint64_t t = 1; t <= tiles; ++t) {
    const uint32_t v = get<uint32_t>(b, in.index_off + 4 * t);
    if (v < prev + in.lanes) return DGT_E_CORRUPT;
    maxlen = std::max<uint32_t>(maxlen, v - prev);
    prev = v;
  }
  if (maxlen != in.max_tile_words4) return DGT_E_CORRUPT;
  in.stream_bytes = 4ull * prev;
  const uint64_t streams_end = in.streams_off + in.stream_bytes;
  if (streams_end > size) return DGT_E_CORRUPT;
  const uint64_t kcap = std::min<uint64_t>(in.kmax, S);
  for (uint64_t t = 0; t < tiles; ++t)
    if (b[in.ktab_off + t] > kcap) return DGT_E_CORRUPT;
  if (dgt::has_raw(in.fmt)) {
    if (in.raw_off < streams_end || in.raw_off % 16 || in.raw_off + tiles * T != size)
      return DGT_E_CORRUPT;
  } else if (in.raw_off != 0 || streams_end != size) {
    return DGT_E_CORRUPT;
  }
  in.bits_per_weight = 8.0 * (double)size / ((double)in.n * (double)in.k);
  *out = in;
  return DGT_OK;
}

}  // extern "C"
