// Device building blocks of libdgt for gfx950 (CDNA4, wave64).
//
// Method: the page "arXiv'26 | 无损压缩逼近 Shannon 极限：你的 LLM 权重里一半以上的
// bit 是白存的" §3.1 -- every tile stream is split into R rANS lane sub-streams,
// one state per lane of the wavefront; decoded tiles go straight to on-chip
// storage and into the matrix multiply, never to global memory; decoding of the
// next tile overlaps the product of the current one.
//
// MI355X mapping used here:
//   * one wave64 holds the R lane states of one tile (R = 64), of two tiles
//     (R = 32, lanes 0-31 and 32-63) or two states of one tile per lane
//     (R = 128: states p and 64 + p, the tile's top and bottom row halves);
//   * the per-layer decode table lives in LDS: 4096 slots x 8 bytes
//     {f | symbol << 24, slot - c_s}, so one ds_read_b64 gives everything a
//     step needs and the state update is a single v_mad_u32_u24;
//   * renormalisation words are read from the tile's stream staged in LDS; the
//     lanes that need a word get consecutive words through a wave ballot and
//     mbcnt prefix count, in increasing lane order;
//   * the tile-local symbol order equals the 16x16x32 MFMA B-operand register
//     layout (lane p: row p % 16, k = 8 * (p / 16) + e), so after 8 steps a lane
//     holds exactly its B operand: decoded values go register -> matrix core.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dgt {
namespace dev {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr uint32_t kL = 1u << 16;
constexpr uint32_t kSlots = 4096;      // 2^prob_bits, prob_bits = 12 on the device
constexpr uint32_t kLutBytes = kSlots * 8;
constexpr uint32_t kCumBytes = 1040;   // (256 + 1) u32, padded
constexpr uint32_t kSlackWords = 64;   // u16 words of slack after each staged stream

enum Fmt : int { INT8 = 1, INT4 = 2, FP8 = 3, BF16 = 4, INT4P = 5, BF16E = 6, BF16P = 7,
                 BF16W = 8 };

// formats whose tiles carry one raw byte per weight next to the coded symbol
template <int FMT>
__host__ __device__ constexpr bool has_raw_bytes() {
  return FMT == BF16 || FMT == BF16E || FMT == BF16P;
}

// Decode steps per 16-row fragment: a lane's 8 weights of a fragment take 8
// symbols, or 4 when a symbol codes two weights.
template <int FMT>
__host__ __device__ constexpr int steps_per_frag() { return (FMT == INT4P || FMT == BF16P) ? 4 : 8; }

// 16-bit symbols (BF16P): the table lists the present symbols only and the
// decode table carries the symbol's high byte beside the slot offset.
template <int FMT>
__host__ __device__ constexpr bool wide_symbols() { return FMT == BF16P; }
constexpr uint32_t kCumBytesWide = 16400;  // (4096 + 1) u32 {c_s | symbol << 16}, padded
// Whole bf16 words (BF16W, 2^16 slots): no slot table.  The LDS holds, per
// 4 consecutive slots 4b .. 4b + 3, a 16-bit bucket word: the index of the
// entry holding slot 4b (13 bits) and, in bit 13 + k - 1, whether an entry
// starts at slot 4b + k (k = 1..3); after the buckets, the present symbols'
// entries {c_s, symbol | (f_s - 1) << 16} (up to kWordSymbols, plus the end
// entry {2^16, 0}), sized by the layer's alphabet.  The entry of slot 4b + j
// is the bucket's index plus the starts at offsets 1..j: one bucket read
// and one entry read per step.
constexpr uint32_t kWordSymbols = 8191;
constexpr uint32_t kWordEntryBytes = (kWordSymbols + 1) * 8;
constexpr uint32_t kWordBuckets = 16384;
constexpr uint32_t kWordBucketBytes = kWordBuckets * 2;
constexpr uint32_t kWordTabBytes = kWordBucketBytes + kWordEntryBytes;  // largest alphabet
// how a step finds its symbol: 0 the 12-bit slot table, 1 the slot table of
// 16-bit symbols (BF16P), 2 the bucket lookup of whole words (BF16W)
template <int FMT>
__host__ __device__ constexpr int sym_mode() { return FMT == BF16P ? 1 : FMT == BF16W ? 2 : 0; }
// LDS bytes of the decode table plus the cumulative table built with it
__host__ __device__ constexpr uint32_t tab_bytes_of(int fmt) {
  return fmt == BF16W ? kWordTabBytes : kLutBytes + (fmt == BF16P ? kCumBytesWide : kCumBytes);
}
template <int FMT>
__host__ __device__ constexpr uint32_t tab_bytes() { return tab_bytes_of(FMT); }
// LDS bytes of a layer's decode table (whole words: entries for its alphabet)
__host__ __device__ constexpr uint32_t tab_bytes_layer(int fmt, uint32_t alphabet) {
  return fmt == BF16W ? kWordBucketBytes + ((alphabet + 1) * 8 + 15) / 16 * 16 : tab_bytes_of(fmt);
}
// At most this many final steps of a tile decode the initial-state payload.
constexpr uint32_t kPayloadMax = 16;
// rANS states a wave lane holds for one chain: two when R = 128.
__host__ __device__ constexpr int states_per_lane(int R) { return R == 128 ? 2 : 1; }

// Everything a kernel needs to know about a layer (passed by value).
struct Layer {
  const uint16_t* table;    // f[alphabet]
  const uint32_t* index;    // off[tiles + 1], 4-byte units
  const uint8_t* ktab;      // k[tiles]
  const uint32_t* streams;  // streams section
  const uint8_t* raw;       // raw low bytes (BF16 split) or null
  uint32_t n, k, tile_n, tile_k, lanes, alphabet, tiles, kt, steps;
  uint32_t region_words;    // u16 capacity of one staged-stream region (even)
  uint32_t tab;             // LDS bytes of the decode table (tab_bytes_layer)
};

// Where the staged words start in LDS: after the decode table.
template <int FMT>
__device__ __forceinline__ uint32_t tab_of(const Layer& L) {
  if constexpr (FMT == BF16W) return L.tab;
  else return tab_bytes<FMT>();
}

__device__ __forceinline__ uint32_t lane_id() {
  return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
}
__device__ __forceinline__ uint32_t uniform(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_readfirstlane((int)v);
}

// Payload step count of tile t, t the same in every lane: a scalar load of
// the dword holding byte t (the k table starts 16-aligned and is padded to 16
// bytes, so the dword lies inside it).  A vector load of a value the code
// then makes uniform would be read back at once, waiting for every load
// issued before it.
__device__ __forceinline__ uint32_t ktab_scalar(const uint8_t* ktab, uint32_t t) {
  typedef __attribute__((address_space(4))) const uint32_t const_u32;
  const const_u32* w = reinterpret_cast<const_u32*>(reinterpret_cast<uintptr_t>(ktab) + (t & ~3u));
  return (*w >> (8u * (t & 3u))) & 0xFFu;
}

// Build the slot table in LDS from the shared frequency table: every slot r
// maps to the symbol s with c_s <= r < c_s + f_s.  Caller synchronises.
// The frequency load is split off so it can be issued before other loads
// (the vector-memory counter retires loads in order).
// The load is unconditional (a clamped index; build_lut drops the threads at
// or above the alphabet size), so no branch blurs the caller's wait counts.
__device__ __forceinline__ uint32_t lut_load_freq(const uint16_t* table, uint32_t alphabet) {
  return (uint32_t)table[min(threadIdx.x, alphabet - 1)];
}

__device__ inline void build_lut(uint32_t freq_of_thread, uint32_t alphabet, u32x2* lut,
                                 uint32_t* cum) {
  uint32_t t = threadIdx.x;
  asm volatile("" : "+v"(t));  // nothing derived from it is hoisted past a caller's loop
  const uint32_t lane = t & 63, wave = t >> 6;
  // inclusive scan of f over <= 256 symbols: wave scans plus wave totals
  uint32_t v = (t < alphabet) ? freq_of_thread : 0u;
  for (uint32_t d = 1; d < 64; d <<= 1) {
    uint32_t o = __shfl_up(v, d, 64);
    if (lane >= d) v += o;
  }
  if (t < 256) cum[1 + t] = v;
  if (t == 0) cum[0] = 0;
  __syncthreads();
  if (t < 256 && wave > 0) {
    uint32_t add = 0;
    for (uint32_t w = 0; w < wave; ++w) add += cum[1 + w * 64 + 63];
    v += add;
  }
  __syncthreads();
  if (t < 256) cum[1 + t] = v;
  __syncthreads();
  // each thread fills a contiguous run of slots, searching for the symbol of
  // a slot only when the slot leaves the current symbol's range
  const uint32_t per = (kSlots + blockDim.x - 1) / blockDim.x;
  const uint32_t r0 = t * per, r1 = min(r0 + per, kSlots);
  uint32_t s_cur = 0, c_lo = 0, c_hi = 0;  // empty range: forces the first search
  for (uint32_t r = r0; r < r1; ++r) {
    if (r >= c_hi) {
      uint32_t lo = 0, hi = alphabet;  // cum[lo] <= r < cum[hi]
      while (hi - lo > 1) {
        const uint32_t mid = (lo + hi) >> 1;
        if (cum[mid] <= r) lo = mid; else hi = mid;
      }
      s_cur = lo;
      c_lo = cum[lo];
      c_hi = cum[lo + 1];
    }
    u32x2 e;
    e.x = (c_hi - c_lo) | (s_cur << 24);
    e.y = r - c_lo;
    lut[r] = e;
  }
}

// Slot table from a sparse table of P entries {symbol | f << 16} in symbol
// order (16-bit symbols): entry .x = f | (symbol & 0xFF) << 24, .y = (slot -
// c_s) | (symbol >> 8) << 24, so the state update masks .y to 12 bits and the
// symbol's two bytes are the top bytes of .x and .y.  Every thread sums a
// contiguous run of entries; a block scan of the run sums gives each run's
// start; cum[e] = c_e | symbol_e << 16 (cum[P] = 2^12) is then searched per
// slot as in build_lut.  The decode table's memory serves as scratch for the
// per-wave sums before it is filled.  Caller synchronises.
__device__ inline void build_lut_sparse(const uint32_t* table, uint32_t P, u32x2* lut,
                                        uint32_t* cum) {
  uint32_t t = threadIdx.x;
  asm volatile("" : "+v"(t));  // nothing derived from it is hoisted past a caller's loop
  const uint32_t B = blockDim.x;
  const uint32_t lane = t & 63, wave = t >> 6;
  uint32_t* wsum = reinterpret_cast<uint32_t*>(lut);
  const uint32_t q = (P + B - 1) / B;
  const uint32_t e0 = min(t * q, P), e1 = min(e0 + q, P);
  uint32_t run = 0;
  for (uint32_t e = e0; e < e1; ++e) run += table[e] >> 16;
  uint32_t v = run;  // inclusive scan over the wave's threads
  for (uint32_t d = 1; d < 64; d <<= 1) {
    const uint32_t o = __shfl_up(v, d, 64);
    if (lane >= d) v += o;
  }
  if (lane == 63) wsum[wave] = v;
  __syncthreads();
  uint32_t c = v - run;
  for (uint32_t w = 0; w < wave; ++w) c += wsum[w];
  for (uint32_t e = e0; e < e1; ++e) {
    const uint32_t en = table[e];
    cum[e] = c | ((en & 0xFFFFu) << 16);
    c += en >> 16;
  }
  if (t == 0) cum[P] = kSlots;
  __syncthreads();  // cum complete and the scratch sums read: the table may be written
  const uint32_t per = (kSlots + B - 1) / B;
  const uint32_t r0 = t * per, r1 = min(r0 + per, kSlots);
  uint32_t s_cur = 0, c_lo = 0, c_hi = 0;  // empty range: forces the first search
  for (uint32_t r = r0; r < r1; ++r) {
    if (r >= c_hi) {
      uint32_t lo = 0, hi = P;  // (cum[lo] & 0xFFFF) <= r < (cum[hi] & 0xFFFF)
      while (hi - lo > 1) {
        const uint32_t mid = (lo + hi) >> 1;
        if ((cum[mid] & 0xFFFFu) <= r) lo = mid; else hi = mid;
      }
      s_cur = cum[lo] >> 16;
      c_lo = cum[lo] & 0xFFFFu;
      c_hi = cum[lo + 1] & 0xFFFFu;
    }
    u32x2 e;
    e.x = (c_hi - c_lo) | ((s_cur & 0xFFu) << 24);
    e.y = (r - c_lo) | ((s_cur >> 8) << 24);
    lut[r] = e;
  }
}

// Entries and bucket starts of whole-word symbols from the sparse table of P
// entries {symbol | (f - 1) << 16} in symbol order (see kWordSymbols): a
// block scan of per-thread runs gives every entry's start c, then bucket b
// (slots 16b .. 16b + 15) gets the last entry whose start is at most 16b.
// The entry memory serves as scratch for the per-wave sums before it is
// filled.  Caller synchronises.
__device__ inline void build_word_table(const uint32_t* table, uint32_t P, u32x2* ent,
                                        uint16_t* bucket) {
  uint32_t t = threadIdx.x;
  asm volatile("" : "+v"(t));  // nothing derived from it is hoisted past a caller's loop
  const uint32_t B = blockDim.x;
  const uint32_t lane = t & 63, wave = t >> 6;
  uint32_t* wsum = reinterpret_cast<uint32_t*>(bucket);  // before the buckets are written
  const uint32_t q = (P + B - 1) / B;
  const uint32_t e0 = min(t * q, P), e1 = min(e0 + q, P);
  uint32_t run = 0;
  for (uint32_t e = e0; e < e1; ++e) run += (table[e] >> 16) + 1;
  uint32_t v = run;  // inclusive scan over the wave's threads
  for (uint32_t d = 1; d < 64; d <<= 1) {
    const uint32_t o = __shfl_up(v, d, 64);
    if (lane >= d) v += o;
  }
  if (lane == 63) wsum[wave] = v;
  __syncthreads();
  uint32_t c = v - run;
  for (uint32_t w = 0; w < wave; ++w) c += wsum[w];
  __syncthreads();  // the sums are read before the entries overwrite them
  for (uint32_t e = e0; e < e1; ++e) {
    const uint32_t en = table[e];
    u32x2 x;
    x.x = c;
    x.y = en;
    ent[e] = x;
    const uint32_t f = (en >> 16) + 1;
    // the buckets whose first slot lies in [c, c + f) (each is written once)
    for (uint32_t b = (c + 3) >> 2; 4 * b < c + f; ++b) bucket[b] = (uint16_t)e;
    c += f;
  }
  if (t == 0) ent[P] = u32x2{1u << 16, 0u};
  __syncthreads();
  // starts inside each bucket: entries idx + 1, idx + 2, idx + 3 while they
  // begin at or below its last slot (the end entry begins past every slot,
  // so each read stays at or below entry P)
  for (uint32_t b = t; b < kWordBuckets; b += B) {
    const uint32_t idx = bucket[b], last = 4 * b + 3;
    uint32_t mask = 0;
    for (uint32_t j = 1; j <= 3; ++j) {
      const uint32_t cj = ent[idx + j].x;
      if (cj > last) break;
      mask |= 1u << (cj - 4 * b - 1);
    }
    bucket[b] = (uint16_t)(idx | (mask << 13));
  }
}

// Table load and decode-table build of a format: the dense table's
// frequency load is issued early (table_issue) and used by table_build.
template <int FMT>
__device__ __forceinline__ uint32_t table_issue(const Layer& L) {
  if constexpr (sym_mode<FMT>() != 0) return 0u;
  else return lut_load_freq(L.table, L.alphabet);
}
template <int FMT>
__device__ __forceinline__ void table_build(uint32_t fq, const Layer& L, u32x2* lut,
                                            uint32_t* cum) {
  if constexpr (sym_mode<FMT>() == 2)
    build_word_table(reinterpret_cast<const uint32_t*>(L.table), L.alphabet,
                     lut + kWordBucketBytes / 8, reinterpret_cast<uint16_t*>(lut));
  else if constexpr (sym_mode<FMT>() == 1)
    build_lut_sparse(reinterpret_cast<const uint32_t*>(L.table), L.alphabet, lut, cum);
  else
    build_lut(fq, L.alphabet, lut, cum);
}

// R lane states of one chain: one tile (R = 64 or 128) or two tiles (R = 32).
// Word positions are byte offsets into the workgroup's LDS; fields marked
// "uniform" hold the same value on every lane.
// A tile's words reach LDS either whole (staged before the first step) or
// through a ring of two chunks (R = 64 or 128, see Ring below).
struct Chain {
  uint32_t x;      // lane state (R = 128: state p, top half of the tile)
  uint32_t x2;     // R = 128: state 64 + p (bottom half)
  uint32_t lim;    // first payload step of the lane's tile (steps - k)
  uint32_t p0;     // uniform: next word of tile A: ring, 2 * words consumed;
                   //   whole stream, LDS byte offset (not clamped)
  uint32_t p1;     // uniform: next word of tile B (R = 32)
  uint32_t e0;     // uniform: ring, 2 * stream words; whole stream, end of A's words
  uint32_t e1;     // uniform: end of tile B's staged words
  uint32_t s0;     // uniform: ring, LDS byte offset of the ring; whole stream, start of A's words
  uint32_t s1;     // uniform: start of tile B's words
};

// Ring staging (R = 64 or 128).  8 steps of 64 states (4 steps of 128) read
// at most 512 words, so a tile's stream is cut into chunks of that size and a
// ring of two chunks holds the words any such group of steps can reach:
// before each group the chunk that covers the furthest word it could read is
// written to the ring (loaded one chunk ahead into registers), over the chunk
// two back, which is consumed.  Past the ring's end a mirror repeats the first
// 64 words of the even chunk in slot 0, so the (at most 64) consecutive words
// one state of every lane reads never wrap.
constexpr uint32_t kChunkWords = 8 * 64;
constexpr uint32_t kRingWords = 2 * kChunkWords;
constexpr uint32_t kRingRegionWords = kRingWords + 64 + 8;  // ring, mirror, slack
constexpr uint32_t kChunkDwords = kChunkWords / 2;          // 4 per lane
// steps between ring advances
__host__ __device__ constexpr int ring_group_steps(int R) { return (int)kChunkWords / R; }

// ILP chains advance one rANS step together, in three phases so that their
// LDS round trips overlap: (1) table reads for every state, (2) state update,
// wave ballot of the lanes that renormalise, word reads for every state,
// (3) merge.  Branch-free: every lane reads a word (in bounds: a pointer is clamped to its
// stream end and the region has kSlackWords of slack); only the lanes that
// renormalise take it.  The word of lane p is the next unread one plus the
// number of renormalising lanes below p (mbcnt of the ballot).  With two
// states per lane (R = 128) the first states' words come first, then the
// second states' (interleaving order j = s*128 + p).  CAREFUL also handles the
// payload switch (x -= L at step == lim, no reads from then on).
// Returns the table words (decoded symbol in the top byte) per state, or for
// 16-bit symbols (MODE 1, and the whole words of MODE 2) the symbol in the
// low half.  MODE 2 (2^16 slots): the bucket lookup of kWordBuckets.
template <int R, bool CAREFUL, int ILP, bool RING, int MODE = 0>
__device__ __forceinline__ void step_all(Chain (&c)[ILP], const u32x2* __restrict__ lut,
                                         const uint8_t* __restrict__ lds, uint32_t s,
                                         bool upper_half,
                                         uint32_t (&sym)[ILP][states_per_lane(R)]) {
  constexpr int NS = states_per_lane(R);
  constexpr bool SYM16 = MODE == 1;
  constexpr uint32_t NB = MODE == 2 ? 16u : 12u;  // frequency precision
  uint32_t x[ILP][NS];
  u32x2 e[ILP][NS];
  uint32_t wsym[ILP][NS];  // MODE 2: the whole word
#pragma unroll
  for (int i = 0; i < ILP; ++i)
#pragma unroll
    for (int h = 0; h < NS; ++h) {
      x[i][h] = h ? c[i].x2 : c[i].x;
      if (CAREFUL) x[i][h] = (s == c[i].lim) ? x[i][h] - kL : x[i][h];
      if constexpr (MODE == 2) {
        const uint32_t slot = x[i][h] & 0xFFFFu;
        const uint16_t* bucket = reinterpret_cast<const uint16_t*>(lut);
        const uint32_t bv = bucket[slot >> 2];
        const uint32_t starts = (bv >> 13) & ((1u << (slot & 3u)) - 1u);
        const u32x2 en =
            lut[kWordBucketBytes / 8 + (bv & 0x1FFFu) + (uint32_t)__builtin_popcount(starts)];
        // the step's operands: f, slot - c_s and the symbol
        e[i][h].x = (en.y >> 16) + 1u;
        e[i][h].y = slot - en.x;
        wsym[i][h] = en.y & 0xFFFFu;
      } else {
        e[i][h] = lut[x[i][h] & (kSlots - 1)];
      }
    }
  uint32_t xn[ILP][NS], w[ILP][NS];
  bool need[ILP][NS];
#pragma unroll
  for (int i = 0; i < ILP; ++i) {
    uint32_t pos = c[i].p0;  // uniform
#pragma unroll
    for (int h = 0; h < NS; ++h) {
      const uint32_t bias = SYM16 ? (e[i][h].y & 0xFFFu) : e[i][h].y;
      xn[i][h] = (e[i][h].x & 0xFFFFFFu) * (x[i][h] >> NB) + bias;  // v_mad_u32_u24
      need[i][h] = xn[i][h] < kL;
      if (CAREFUL) need[i][h] = need[i][h] && (s < c[i].lim);
      const uint64_t m = __builtin_amdgcn_ballot_w64(need[i][h]);
      const uint32_t mlo = (uint32_t)m, mhi = (uint32_t)(m >> 32);
      const uint32_t rank = __builtin_amdgcn_mbcnt_hi(mhi, __builtin_amdgcn_mbcnt_lo(mlo, 0u));
      uint32_t addr;
      if (R != 32 && RING) {
        addr = 2 * rank + (c[i].s0 + (pos & (2 * kRingWords - 1)));
        pos += 2 * (uint32_t)__builtin_popcountll(m);
        // keep the byte pointer itself in its scalar register (not a word
        // count the address is rebuilt from at every step)
        asm volatile("" : "+s"(pos));
      } else if (R != 32) {
        addr = 2 * rank + min(pos, c[i].e0);
        pos += 2 * (uint32_t)__builtin_popcountll(m);
      } else {
        const uint32_t pl = (uint32_t)__builtin_popcount(mlo);
        const uint32_t ph = (uint32_t)__builtin_popcount(mhi);
        // upper-half lanes count the lower half's bits too: start them pl lower
        const uint32_t b0 = min(c[i].p0, c[i].e0);
        const uint32_t b1 = min(c[i].p1, c[i].e1) - 2 * pl;
        addr = 2 * rank + (upper_half ? b1 : b0);
        pos += 2 * pl;
        c[i].p1 += 2 * ph;
      }
      w[i][h] = *reinterpret_cast<const uint16_t*>(lds + addr);
    }
    c[i].p0 = pos;
  }
#pragma unroll
  for (int i = 0; i < ILP; ++i)
#pragma unroll
    for (int h = 0; h < NS; ++h) {
      const uint32_t v = need[i][h] ? ((xn[i][h] << 16) | w[i][h]) : xn[i][h];
      if (h) c[i].x2 = v; else c[i].x = v;
      // 16-bit symbols: [low byte, high byte, 0, 0] from the entry's top bytes
      sym[i][h] = SYM16 ? __builtin_amdgcn_perm(e[i][h].y, e[i][h].x, 0x0c0c0703u)
                  : MODE == 2 ? wsym[i][h] : e[i][h].x;
    }
}

// Integrity flags of the chain's tile(s) after the last step, per lane's tile:
// 1 = a lane did not return to its initial value, 2 = words consumed != stream
// (a pad word may remain), 4 = read past the stream.
template <int R, bool RING>
__device__ __forceinline__ uint32_t final_flags(const Chain& c, uint32_t steps,
                                                bool upper_half) {
  const uint32_t want = (c.lim == steps) ? kL : 0u;
  const uint64_t bad = __builtin_amdgcn_ballot_w64(c.x != want || (R == 128 && c.x2 != want));
  uint32_t f = 0;
  const uint32_t half_bad = (R != 32) ? (bad != 0) : (upper_half ? (uint32_t)(bad >> 32)
                                                                 : (uint32_t)bad);
  if (half_bad) f |= 1u;
  const uint32_t p = (R == 32 && upper_half) ? c.p1 : c.p0;
  const uint32_t st = RING ? 0u : ((R == 32 && upper_half) ? c.s1 : c.s0);
  const uint32_t en = (R == 32 && upper_half) ? c.e1 : c.e0;
  const uint32_t used = (p - st) / 2, avail = (en - st) / 2;  // words
  if (!(used == avail || used + 1 == avail)) f |= 2u;
  if (used > avail) f |= 4u;
  return f;
}

// Staging of a tile's word stream into LDS in two phases, so the HBM latency
// of the loads overlaps other prologue work: stage_issue loads up to kPre
// dwords per lane into registers, stage_commit writes them to LDS and copies
// whatever the registers did not cover.
constexpr int kPre = 16;

struct Staged {
  uint32_t v[kPre];
  const uint32_t* src;   // the tile's words (after its states)
  const uint32_t* tile;  // the tile's stream (states first)
  int32_t last;          // last dword index of the tile's stream
  uint32_t words4;
};

// Locate tile t's stream (no word loads yet).
__device__ __forceinline__ void stage_begin(const Layer& L, uint32_t t, Staged& st) {
  const uint32_t o0 = L.index[t], o1 = L.index[t + 1];
  st.words4 = o1 - o0 - L.lanes;
  st.tile = L.streams + o0;
  st.src = st.tile + L.lanes;
  st.last = (int32_t)(o1 - o0) - 1;
}

// Load dwords j0 <= j < j1 of every lane's share into registers.  Every lane
// loads, without branches, so the vector-memory wait counts of the caller
// stay exact (a later wait for an earlier load does not have to drain these).
// Positions past the stream re-read the tile's last dword (the states come
// first, so the tile always has one); commits keep only the words below words4.
__device__ __forceinline__ void stage_load(Staged& st, uint32_t lanes, uint32_t sub_lane,
                                           uint32_t sub_size, int j0, int j1) {
#pragma unroll
  for (int j = j0; j < j1; ++j) {
    const int32_t i = (int32_t)(lanes + sub_lane + j * sub_size);
    st.v[j] = st.tile[min(i, st.last)];
  }
}

__device__ __forceinline__ void stage_issue(const Layer& L, uint32_t t, uint32_t sub_lane,
                                            uint32_t sub_size, Staged& st) {
  stage_begin(L, t, st);
  stage_load(st, L.lanes, sub_lane, sub_size, 0, kPre);
}

// Write staged dwords j0 <= j < j1 to LDS; REST also copies the dwords the
// registers did not cover straight from global memory.
__device__ __forceinline__ void stage_commit_part(const Staged& st, uint16_t* words,
                                                  uint32_t start, uint32_t sub_lane,
                                                  uint32_t sub_size, int j0, int j1, bool rest) {
  uint32_t* dst = reinterpret_cast<uint32_t*>(words + start) + sub_lane;
  const int32_t rem = (int32_t)st.words4 - (int32_t)sub_lane;
#pragma unroll
  for (int j = j0; j < j1; ++j)
    if (rem > (int32_t)(j * sub_size)) dst[j * sub_size] = st.v[j];
  if (rest) {
    const uint32_t* src = st.src + sub_lane;
    for (int32_t i = kPre * sub_size; i < rem; i += sub_size) dst[i] = src[i];
  }
}

// Returns the number of staged u16 words (including a possible pad word).
__device__ __forceinline__ uint32_t stage_commit(const Staged& st, uint16_t* words, uint32_t start,
                                                 uint32_t sub_lane, uint32_t sub_size) {
  stage_commit_part(st, words, start, sub_lane, sub_size, 0, kPre, true);
  return 2 * st.words4;
}

// A fragment reads fewer words than the first half of the staged registers
// hold (8 steps x at most one word per state: 512 words for R = 64, 1024 for
// R = 128, per tile 256 for R = 32, against kPre/2 * sub_size dwords), so the
// decode can start once that half is in LDS and the rest is written after
// the first fragment.
constexpr int kPreHalf = kPre / 2;

// One tile's ring: its stream, chunk count, committed chunks and the next
// chunk in flight (4 dwords per lane: dwords lane + 64 * i of the chunk).
struct Ring {
  const uint32_t* tile;  // the tile's stream (states first)
  uint32_t hdr;          // state dwords before the words (R)
  int32_t last;          // last dword index of the tile's stream
  uint32_t words4;       // uniform: stream dwords after the states
  uint32_t nchunks;      // uniform
  uint32_t cc;           // uniform: chunks written to the ring
  uint32_t nxt[4];
};

// Load chunk j of the ring's tile into v (every lane loads, clamped to the
// tile's own stream; dwords past the stream are never used).
__device__ __forceinline__ void ring_load(const Ring& r, uint32_t j, uint32_t lane,
                                          uint32_t (&v)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int32_t d = (int32_t)(r.hdr + j * kChunkDwords + lane + 64 * i);
    v[i] = r.tile[min(d, r.last)];
  }
}

// Start tile t: chunk 0 into c0, chunk 1 in flight.
__device__ __forceinline__ void ring_issue(const Layer& L, uint32_t t, uint32_t lane, Ring& r,
                                           uint32_t (&c0)[4]) {
  const uint32_t o0 = L.index[t], o1 = L.index[t + 1];
  r.tile = L.streams + o0;
  r.hdr = L.lanes;
  r.last = (int32_t)(o1 - o0) - 1;
  r.words4 = o1 - o0 - L.lanes;
  r.nchunks = (r.words4 + kChunkDwords - 1) / kChunkDwords;
  r.cc = 0;
  ring_load(r, 0, lane, c0);
  ring_load(r, 1, lane, r.nxt);
}

// Write chunk j (in v) to its ring slot; even chunks after the first also
// refresh the mirror.  base: LDS byte offset of the ring.
// (Ring setup for a chain: ring_issue, then after the LUT barrier ring_start.)
__device__ __forceinline__ void ring_write(uint8_t* lds, uint32_t base, uint32_t j, uint32_t lane,
                                           const uint32_t (&v)[4]) {
  uint32_t* d = reinterpret_cast<uint32_t*>(lds + base) + (j & 1) * kChunkDwords + lane;
#pragma unroll
  for (int i = 0; i < 4; ++i) d[64 * i] = v[i];
  if ((j & 1) == 0 && j >= 2 && lane < 32)
    reinterpret_cast<uint32_t*>(lds + base)[2 * kChunkDwords + lane] = v[0];
}

// Chunk 0 to the ring and the chain's word pointers.
__device__ __forceinline__ void ring_start(Ring& r, Chain& c, uint8_t* lds, uint32_t base,
                                           uint32_t lane, const uint32_t (&c0)[4]) {
  ring_write(lds, base, 0, lane, c0);
  r.cc = min(1u, r.nchunks);
  c.p0 = 0;
  c.s0 = base;
  c.e0 = 4 * r.words4;
  c.p1 = 0; c.s1 = base; c.e1 = c.e0;
}

// Before a group of steps whose first word is p (2 * words consumed): make
// sure the chunk holding the furthest word the group can read is in the ring.
// At most one chunk per group is needed.
__device__ __forceinline__ void ring_advance(Ring& r, uint8_t* lds, uint32_t base, uint32_t p,
                                             uint32_t lane) {
  const uint32_t need = ((p >> 1) + kChunkWords - 1) / kChunkWords;
  if (r.cc < r.nchunks && r.cc <= need) {
    ring_write(lds, base, r.cc, lane, r.nxt);
    r.cc += 1;
    if (r.cc < r.nchunks) ring_load(r, r.cc, lane, r.nxt);
  }
}

}  // namespace dev
}  // namespace dgt
