// C-ABI entry points of libdgt's device side, the fp8 activation-quantisation
// kernels and the static launch planner.
//
// Planner (the static tile schedule of "arXiv'26 | 无损压缩逼近 Shannon 极限" §3.1,
// fixed at launch, no run-time bookkeeping): Y is cut into strips of tile_n
// columns; a unit is ILP chains of consecutive k-tiles of one strip; units are
// numbered strip-major and dealt to workgroups in equal contiguous runs of W
// (one wave per unit), W chosen so the layer fills the CUs in as few rounds as
// registers and LDS allow.  Strips shared by several workgroups meet in the
// workspace (per-strip slots and counters).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "../../include/dgt.h"
#include "dgt_format.h"
#include "dgt_launch.h"

namespace dgt {
namespace dev {

// ---------------------------------------------------- fp8 activation quant
// Per-tensor e4m3 quantisation of X (bf16): amax, inv = fl32(448 / amax),
// sx = fl32(amax / 448), xq = e4m3_rne_satfinite(fl32(x * inv)).
struct QuantArgs {
  const uint16_t* x;
  uint16_t* xq;          // bf16 bits of the e4m3 value (exact: e4m3 is a subset of bf16)
  uint32_t* amax_bits;   // workspace: running max of |x| as fp32 bits
  uint32_t* done;        // workspace: finished-block counter
  float* sx;             // workspace: activation scale
  uint32_t count;
};

__global__ __launch_bounds__(256) void k_amax(QuantArgs q) {
  uint32_t mx = 0;
  for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < q.count; i += gridDim.x * blockDim.x)
    mx = max(mx, ((uint32_t)q.x[i] << 16) & 0x7FFFFFFFu);
  for (int d = 32; d > 0; d >>= 1) mx = max(mx, (uint32_t)__shfl_xor(mx, d, 64));
  if ((threadIdx.x & 63) == 0) atomicMax(q.amax_bits, mx);
}

__device__ __forceinline__ uint32_t f32_to_e4m3(float v) {
  // round to nearest even, saturate finite values to 448, NaN -> 0x7F
  const uint32_t u = __float_as_uint(v);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t au = u & 0x7FFFFFFFu;
  if (au > 0x7F800000u) return 0x7Fu;
  const float a = __uint_as_float(au);
  if (a >= 448.f) return sign | 0x7Eu;
  uint32_t mag;
  if (a < 0.015625f) {  // below 2^-6: subnormal grid of 2^-9
    const float q = a * 512.f;                   // exact scaling
    mag = (uint32_t)__builtin_rintf(q);          // ties to even, 0..8
  } else {
    const uint32_t exp = (au >> 23) - 127 + 7;   // 1..15
    const uint32_t man = au & 0x7FFFFFu;
    const uint32_t keep = man >> 20, rest = man & 0xFFFFFu;
    uint32_t m3 = keep;
    if (rest > 0x80000u || (rest == 0x80000u && (keep & 1u))) m3 += 1;
    mag = (exp << 3) + m3;                       // carry propagates into the exponent
  }
  return sign | mag;
}

__device__ __forceinline__ uint16_t e4m3_to_bf16(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, man = c & 7u;
  const float mag = e ? __uint_as_float(((e + 120u) << 23) | (man << 20))  // 2^(e-7) * 1.m
                      : (float)man * 0.001953125f;                       // m * 2^-9
  const uint32_t bits = __float_as_uint(mag) | ((c & 0x80u) << 24);
  return (uint16_t)(bits >> 16);
}

__global__ __launch_bounds__(256) void k_quant(QuantArgs q) {
  const float amax = __uint_as_float(
      __hip_atomic_load(q.amax_bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  float inv = 1.f, sx = 1.f;
  const bool zero = !(amax > 0.f) || amax > 3.4e38f;
  if (!zero) {
    inv = (float)(448.0 / (double)amax);
    sx = (float)((double)amax / 448.0);
  }
  for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < q.count; i += gridDim.x * blockDim.x) {
    const float v = __uint_as_float((uint32_t)q.x[i] << 16);
    q.xq[i] = zero ? (uint16_t)0 : e4m3_to_bf16(f32_to_e4m3(v * inv));
  }
  __shared__ bool last;
  __syncthreads();
  if (threadIdx.x == 0)
    last = __hip_atomic_fetch_add(q.done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
           gridDim.x - 1;
  __syncthreads();
  if (last && threadIdx.x == 0) {
    // every block has read amax by now; reset it for the next call
    __hip_atomic_store(q.sx, sx, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(q.amax_bits, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(q.done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}


// Small activations (count <= kQuantOneBlock): the maximum and the
// quantisation in one workgroup, one launch instead of two (same arithmetic
// as k_amax + k_quant; the shared maximum and counter stay at zero).
constexpr uint32_t kQuantOneBlock = 65536;

__global__ __launch_bounds__(1024) void k_amax_quant(QuantArgs q) {
  __shared__ uint32_t wmax[16];
  const uint32_t t = threadIdx.x, n8 = q.count / 8;  // count % 8 == 0 (K % 64 == 0)
  const u32x4* x8 = reinterpret_cast<const u32x4*>(q.x);
  uint32_t mx = 0;
  for (uint32_t i = t; i < n8; i += 1024) {
    const u32x4 v = x8[i];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      mx = max(mx, (v[j] << 16) & 0x7FFFFFFFu);
      mx = max(mx, v[j] & 0x7FFF0000u);
    }
  }
  for (int d = 32; d > 0; d >>= 1) mx = max(mx, (uint32_t)__shfl_xor(mx, d, 64));
  if ((t & 63) == 0) wmax[t >> 6] = mx;
  __syncthreads();
  uint32_t am = 0;
  for (uint32_t w = 0; w < (blockDim.x >> 6); ++w) am = max(am, wmax[w]);
  const float amax = __uint_as_float(am);
  float inv = 1.f, sx = 1.f;
  const bool zero = !(amax > 0.f) || amax > 3.4e38f;
  if (!zero) {
    inv = (float)(448.0 / (double)amax);
    sx = (float)((double)amax / 448.0);
  }
  u32x4* xq8 = reinterpret_cast<u32x4*>(q.xq);
  for (uint32_t i = t; i < n8; i += 1024) {
    const u32x4 v = x8[i];
    u32x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float lo = __uint_as_float(v[j] << 16), hi = __uint_as_float(v[j] & 0xFFFF0000u);
      const uint32_t ql = zero ? 0u : e4m3_to_bf16(f32_to_e4m3(lo * inv));
      const uint32_t qh = zero ? 0u : e4m3_to_bf16(f32_to_e4m3(hi * inv));
      o[j] = ql | (qh << 16);
    }
    xq8[i] = o;
  }
  if (t == 0) __hip_atomic_store(q.sx, sx, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace dev
}  // namespace dgt

// =================================================================== host side
namespace {

using namespace dgt::dev;

// u16 words of LDS per staged tile: the whole stream (longest tile + slack)
// or, for one tile per chain (R = 64, 128), a two-chunk ring (any length).
uint32_t region_words_of(const dgt_info* in, bool ring) {
  if (ring) return kRingRegionWords;
  const uint32_t words = 2 * (in->max_tile_words4 - in->lanes) + kSlackWords;
  return (words + 7) & ~7u;
}

bool layer_from_info(const void* d_blob, const dgt_info* in, Layer* L) {
  if (!d_blob || !in) return false;
  const uint8_t* b = static_cast<const uint8_t*>(d_blob);
  L->table = reinterpret_cast<const uint16_t*>(b + in->table_off);
  L->index = reinterpret_cast<const uint32_t*>(b + in->index_off);
  L->ktab = b + in->ktab_off;
  L->streams = reinterpret_cast<const uint32_t*>(b + in->streams_off);
  L->raw = in->raw_off ? b + in->raw_off : nullptr;
  L->n = in->n;
  L->k = in->k;
  L->tile_n = in->tile_n;
  L->tile_k = in->tile_k;
  L->lanes = in->lanes;
  L->alphabet = in->alphabet;
  L->tiles = in->tiles;
  L->kt = in->k / in->tile_k;
  L->steps = in->tile_n * in->tile_k / dgt::weights_per_symbol(in->fmt) / in->lanes;
  L->region_words = region_words_of(in, false);  // a plan using the ring overrides it
  L->tab = tab_bytes_layer((int)in->fmt, in->alphabet);
  return true;
}

int device_supported(const dgt_info* in) {
  if (!in) return DGT_E_ARG;
  if (in->fmt == DGT_FMT_BF16_WORD) {
    // whole words: 2^16 slots, 64 lanes, at most kWordSymbols distinct patterns
    if (in->prob_bits != 16 || in->lanes != 64 || in->alphabet > kWordSymbols)
      return DGT_E_UNSUPPORTED;
    return DGT_OK;
  }
  if (in->prob_bits != 12) return DGT_E_UNSUPPORTED;
  if (in->lanes != 32 && in->lanes != 64 && in->lanes != 128) return DGT_E_UNSUPPORTED;
  return DGT_OK;
}

struct FusedPlan {
  uint32_t ring, region_words;
  uint32_t mt, mix, waves, threads, cpw, n2, chains, cps, wgs, slots, strips, red_cols, lds;
  uint32_t rounds, red_off;
  uint32_t m_chunk;
  size_t part_off, part_bytes, quant_off, ws_bytes;
  // large-M variant (fragments shared through LDS): used when xm != 0;
  // xs > 1: its 16-wave subset form
  uint32_t xm, bps, bpw, batches, xbuf_off, xs;
};

constexpr uint32_t kCUs = 256;

// Units per workgroup so that the layer fills the CUs in as few rounds as the
// wave cap allows; a workgroup never spans more than two strips (W <= ups).
uint32_t pick_waves(uint32_t units, uint32_t ups, uint32_t cap) {
  uint32_t w = (units + kCUs - 1) / kCUs;
  w = std::min(std::max(w, 1u), cap);
  return std::min(w, ups);
}

// Packed accumulators for 2..8 rows (default); DGT_PACKED=0 plans the 16-row
// block kernels instead (the same products in the same order).
bool packed_from_env() {
  const char* v = std::getenv("DGT_PACKED");
  return !(v && std::strcmp(v, "0") == 0);
}

// Workgroups of the fused kernels take their work in XCD-major order
// (xcd_tile) when DGT_XCD_ORDER=1; results are identical.
bool xcd_order_from_env() {
  const char* v = std::getenv("DGT_XCD_ORDER");
  return v && std::strcmp(v, "1") == 0;
}

// One fragment buffer instead of two in the large-M kernel (the ablation rung
// without ping-pong, 64-lane layers), asked for by DGT_XM_SINGLE_BUFFER=1;
// results are identical.
bool xm_single_buffer_from_env() {
  const char* v = std::getenv("DGT_XM_SINGLE_BUFFER");
  return v && std::strcmp(v, "1") == 0;
}

// The 16-wave subset form of the large-M kernel for 256-row tiles at M <= 128
// (DGT_XM_SUBSETS=0 keeps the 8-wave kernel; results agree within rounding).
bool xm_subsets_from_env() {
  const char* v = std::getenv("DGT_XM_SUBSETS");
  return !(v && std::strcmp(v, "0") == 0);
}

// Large M: one launch in which every tile is decoded once and shared through
// LDS by waves that own disjoint row blocks, instead of one launch per chunk
// of rows that each decode the whole layer.  Needs R = 64 or 128 and k-tiles
// per strip divisible by the workgroup's wave count.  With 256-row tiles at
// 64 lanes and M <= 128 the subset form runs 16 decode chains per CU: 4
// subsets of 4 row groups (M <= 64) or 2 of 8 (M <= 128).
bool plan_fused_xm_xs(const dgt_info* in, uint32_t m, bool ring, uint32_t xs, FusedPlan* p);

// The subset form, where the layer and M allow it and it fits (k-tiles per
// strip, LDS) with the given staging.  int4 code pairs take it up to M = 64
// only: at M = 128 the 8-wave form measured faster (718 against 746 us on the
// 405B-scale FFN).
// allow: the subset form may be used (DGT_XM_SUBSETS at a call).
bool plan_fused_xm_sub(const dgt_info* in, uint32_t m, bool ring, bool allow, FusedPlan* p) {
  const uint32_t mmax = in->fmt == DGT_FMT_INT4_PAIR ? 64u : 128u;
  const bool sub = allow && in->tile_n == 256 && in->lanes == 64 && m <= mmax &&
                   !xm_single_buffer_from_env();
  return sub && plan_fused_xm_xs(in, m, ring, m <= 64 ? 4u : 2u, p);
}

// The 8-wave (or, for 128-row tiles, 16-wave) form.
bool plan_fused_xm(const dgt_info* in, uint32_t m, bool ring, FusedPlan* p) {
  return plan_fused_xm_xs(in, m, ring, 1u, p);
}

bool plan_fused_xm_xs(const dgt_info* in, uint32_t m, bool ring, uint32_t xs, FusedPlan* p) {
  p->rounds = 1;
  p->red_off = 0;
  const uint32_t fn = in->tile_n / 16;
  if (in->lanes == 32 || in->tile_k != 64 || (fn != 8 && fn != 16)) return false;
  const uint32_t ns = in->lanes == 128 ? 2 : 1;  // operands per wave and fragment
  if (m <= 16) return false;  // one register-resident pass (one 16-row block) covers M
  const uint32_t nw = xm_waves(fn, xs), mtw = xm_row_blocks(fn, xs), nt = xm_tiles(fn, xs);
  const uint32_t rows = xm_rows(fn, xs);
  if (m > rows) return false;
  const uint32_t kt = in->k / in->tile_k;
  if (kt % nt) return false;
  p->ring = ring ? 1 : 0;
  p->region_words = region_words_of(in, ring);
  const uint32_t region_bytes = p->region_words * 2;
  const uint32_t xbuf_off =
      (uint32_t)dgt::align_up((size_t)tab_bytes_layer((int)in->fmt, in->alphabet) + nt * region_bytes + 16, 16);
  const uint32_t fpb = xm_fpb(in->lanes == 128 ? 128 : 64, fn, (int)in->fmt, xs);
  const uint32_t lds = xbuf_off + 2 * fpb * nt * ns * 1024;
  if (lds > kMaxLds) return false;
  p->xm = 1;
  p->xs = xs;
  p->xbuf_off = xbuf_off;
  p->lds = lds;
  p->strips = in->n / in->tile_n;
  p->bps = kt / nt;
  p->batches = p->strips * p->bps;
  p->bpw = (p->batches + kCUs - 1) / kCUs;  // one workgroup per CU, one round
  p->wgs = (p->batches + p->bpw - 1) / p->bpw;
  p->slots = (p->bps + p->bpw - 1) / p->bpw + 1;
  p->threads = 64 * nw;
  p->m_chunk = m;
  p->mt = mtw;
  p->mix = 0;
  p->waves = nw;
  p->cpw = p->bpw;
  p->n2 = 0;
  p->chains = p->batches;
  p->cps = p->bps;
  p->red_cols = 0;
  size_t off = dgt::align_up((size_t)p->strips * 4, 256);
  p->part_off = off;
  // partial slots hold every row block of the workgroup (register layout)
  p->part_bytes = (size_t)p->strips * p->slots * rows * in->tile_n * 4;
  off = dgt::align_up(off + p->part_bytes, 256);
  p->quant_off = off;
  if (in->fmt == DGT_FMT_FP8_E4M3) off += dgt::align_up((size_t)m * in->k * 2, 256) + 256;
  p->ws_bytes = off;
  return true;
}

// Register-resident path: every wave keeps its rows' accumulators; M above
// one pass is handled in chunks of m_chunk rows.  Chains per workgroup C is
// the layer's chains over the CUs (one round) when the wave cap allows it;
// beyond the cap the first n2 waves take two chains each (MIX kernels).
// Workgroups of the multi-round kernel a CU holds at once (its registers and
// LDS decide, as the runtime reports for the current device); 1 when the
// runtime cannot tell.
uint32_t rounds_blocks_per_cu(const dgt_info* in, uint32_t fn, uint32_t mt, bool mix,
                              uint32_t threads, uint32_t lds) {
  GemmArgs a{};
  int n = 0, rc = DGT_E_ARG;
  switch (in->fmt) {
    case DGT_FMT_INT8: rc = launch_fused_rounds<INT8>(a, in->lanes, fn, mt, mix, 0, threads, lds, nullptr, &n); break;
    case DGT_FMT_INT4: rc = launch_fused_rounds<INT4>(a, in->lanes, fn, mt, mix, 0, threads, lds, nullptr, &n); break;
    case DGT_FMT_INT4_PAIR: rc = launch_fused_rounds<INT4P>(a, in->lanes, fn, mt, mix, 0, threads, lds, nullptr, &n); break;
    case DGT_FMT_BF16_EXP: rc = launch_fused_rounds<BF16E>(a, in->lanes, fn, mt, mix, 0, threads, lds, nullptr, &n); break;
    case DGT_FMT_BF16_PAIR: rc = launch_fused_rounds<BF16P>(a, in->lanes, fn, mt, mix, 0, threads, lds, nullptr, &n); break;
    case DGT_FMT_FP8_E4M3: rc = launch_fused_rounds<FP8>(a, in->lanes, fn, mt, mix, 0, threads, lds, nullptr, &n); break;
    case DGT_FMT_BF16_SPLIT: rc = launch_fused_rounds<BF16>(a, in->lanes, fn, mt, mix, 0, threads, lds, nullptr, &n); break;
    case DGT_FMT_BF16_WORD: rc = launch_fused_rounds<BF16W>(a, in->lanes, fn, mt, mix, 0, threads, lds, nullptr, &n); break;
    default: break;
  }
  return (rc == DGT_OK && n > 0) ? (uint32_t)n : 1u;
}

bool plan_fused_reg(const dgt_info* in, uint32_t m, bool ring, uint32_t rounds_env, FusedPlan* p,
                    bool* lds_bound) {
  p->xm = 0;
  p->ring = ring ? 1 : 0;
  p->region_words = region_words_of(in, ring);
  const uint32_t R = in->lanes, tpc = R == 32 ? 2 : 1;
  const uint32_t kt = in->k / in->tile_k;
  if (kt % tpc) return false;
  // Tn = 256 keeps 16 row bands of accumulators: 16-row chunks of X only
  p->m_chunk = std::min<uint32_t>(m, in->tile_n == 256 ? 16 : 64);
  // one row: the single-row mode (row bands packed into one accumulator);
  // up to 4 or 8 rows at 64 lanes: 4 or 2 bands per accumulator
  // (DGT_PACKED=0 takes the 16-row block instead)
  const bool pk = R == 64 && packed_from_env();
  p->mt = p->m_chunk == 1 ? 0u
          : (pk && p->m_chunk <= 4) ? (uint32_t)kPacked4
          : (pk && p->m_chunk <= 8) ? (uint32_t)kPacked8
          : p->m_chunk <= 16 ? 1u : 4u;
  p->strips = in->n / in->tile_n;
  p->chains = in->tiles / tpc;
  p->cps = kt / tpc;
  const uint32_t chain_lds = tpc * p->region_words * 2;
  const uint32_t tab = tab_bytes_layer((int)in->fmt, in->alphabet);
  if (tab + chain_lds > kMaxLds) return false;
  const uint32_t lds_cap = (kMaxLds - tab) / chain_lds;
  const uint32_t fn = in->tile_n / 16 == 8 ? 8 : 16;
  const uint32_t w1 = fused_max_threads(R, fn, p->mt, 1) / 64;  // one chain per wave
  const uint32_t w2 = fused_max_threads(R, fn, p->mt, 2) / 64;  // two-chain kernels
  uint32_t c = (p->chains + kCUs - 1) / kCUs;
  c = std::min(c, p->cps);
  *lds_bound = c > lds_cap && lds_cap < 2 * std::max(w1, w2);
  c = std::min(c, lds_cap);
  if (c > w1 && p->cps % 2) c = w1;
  if (c <= w1) {
    p->mix = 0;
    p->n2 = 0;
    p->waves = c;
  } else {
    c = std::min(c & ~1u, 2 * w2);
    p->mix = 1;
    p->n2 = c - w2;
    p->waves = w2;
    // More than one round of workgroups per CU: half-size workgroups (all
    // waves on two chains) so that two share a CU and one's prologue (table
    // and stream loads, LUT build) overlaps the other's decode.
    const uint64_t rounds = (p->chains + (uint64_t)c * kCUs - 1) / ((uint64_t)c * kCUs);
    const uint32_t half = w2 / 2;
    if (rounds > 1 && half >= 8 && p->cps % 2 == 0 &&
        2 * (tab + 2 * half * chain_lds) <= kMaxLds) {
      p->waves = half;
      p->n2 = half;
      c = 2 * half;
    }
  }
  p->cpw = c;
  p->threads = 64 * std::max(p->waves, 4u);       // the LUT build uses >= 4 waves
  p->wgs = (p->chains + c - 1) / c;
  p->slots = (p->cps + c - 1) / c + 1;
  p->rounds = 1;
  p->red_off = 0;
  p->lds = tab + c * chain_lds;
  uint32_t rc = in->tile_n;
  while (rc > 16 && (uint64_t)p->waves * p->m_chunk * rc * 4 > p->lds) rc /= 2;
  if ((uint64_t)p->waves * p->m_chunk * rc * 4 > p->lds) {
    p->lds = p->waves * p->m_chunk * rc * 4;
    if (p->lds > kMaxLds) return false;
  }
  p->red_cols = rc;
  // Layers that take several rounds of workgroups per CU run them inside
  // each workgroup (k_fused_rounds): the LUT is built once and a strip's
  // partial sums leave the workgroup once.  Ring staging, 16-row blocks of X,
  // full rounds inside one strip (cpw divides the units per strip).  The
  // reduction buffer then sits after the tables, over the rings.
  if (ring && (p->mt <= 1 || mt_packed((int)p->mt)) && R != 32 && p->cps % c == 0) {
    uint32_t rc2 = in->tile_n;
    while (rc2 > 16 && (uint64_t)p->waves * p->m_chunk * rc2 * 4 > c * chain_lds) rc2 /= 2;
    const uint32_t lds2 = tab + std::max<uint32_t>(c * chain_lds, p->waves * p->m_chunk * rc2 * 4);
    const uint32_t wg_rounds = p->wgs;
    uint32_t rounds = rounds_env;
    if (rounds == 0) {
      const uint32_t per_cu = rounds_blocks_per_cu(in, fn, p->mt, p->mix != 0, p->threads, lds2);
      rounds = (wg_rounds + kCUs * per_cu - 1) / (kCUs * per_cu);
    }
    if (rounds > 1 && lds2 <= kMaxLds) {
      const uint32_t cwg = c * rounds;
      p->rounds = rounds;
      p->wgs = (p->chains + cwg - 1) / cwg;
      p->slots = (p->cps + cwg - 1) / cwg + 1;
      p->red_off = tab;
      p->lds = lds2;
      p->red_cols = rc2;
    }
  }
  size_t off = dgt::align_up((size_t)p->strips * 4, 256);
  p->part_off = off;
  p->part_bytes = (size_t)p->strips * p->slots * p->m_chunk * in->tile_n * 4;
  off = dgt::align_up(off + p->part_bytes, 256);
  p->quant_off = off;
  if (in->fmt == DGT_FMT_FP8_E4M3) off += dgt::align_up((size_t)m * in->k * 2, 256) + 256;
  p->ws_bytes = off;
  return true;
}

// How tile streams reach LDS: chosen per layer, or forced by the environment
// variable DGT_STAGING ("whole" or "ring"; results are identical).
enum Staging { kAuto = 0, kWhole = 1, kRing = 2 };
Staging staging_from_env() {
  const char* v = std::getenv("DGT_STAGING");
  if (v && std::strcmp(v, "ring") == 0) return kRing;
  if (v && std::strcmp(v, "whole") == 0) return kWhole;
  return kAuto;
}

// Staging choice (one tile per chain: R = 64, 128): whole streams when they
// fit the planned chains in LDS and the launch is one round of workgroups;
// the ring when LDS would cap the chains per CU or workgroups come in several
// rounds (each waits for one chunk instead of its whole streams to decode).
// A forced staging that cannot serve the layer falls back to the choice.
// rounds: 0 = chosen per layer, else forced rounds per workgroup of the
// register path (where cpw divides the units per strip).
bool plan_fused(const dgt_info* in, uint32_t m, FusedPlan* p, Staging sg, uint32_t rounds,
                bool sub) {
  const bool r64 = in->lanes != 32;
  bool unused = false;
  if (sg == kRing && r64) {
    if (plan_fused_xm_sub(in, m, true, sub, p) || plan_fused_xm(in, m, true, p)) return true;
    if (plan_fused_reg(in, m, true, rounds, p, &unused)) return true;
  }
  if (sg == kWhole) {
    if (plan_fused_xm_sub(in, m, false, sub, p) || plan_fused_xm(in, m, false, p)) return true;
    if (plan_fused_reg(in, m, false, rounds, p, &unused)) return true;
  }
  // large M: the subset form (16 decode chains per CU) with either staging
  // before the 8-wave form
  if (plan_fused_xm_sub(in, m, false, sub, p)) return true;
  if (r64 && plan_fused_xm_sub(in, m, true, sub, p)) return true;
  if (plan_fused_xm(in, m, false, p)) return true;
  if (r64 && plan_fused_xm(in, m, true, p)) return true;
  bool lds_bound = false;
  const bool whole = plan_fused_reg(in, m, false, rounds, p, &lds_bound);
  if (!r64) return whole;
  if (whole && !lds_bound && p->wgs * p->rounds <= kCUs) return true;
  return plan_fused_reg(in, m, true, rounds, p, &unused);
}


// Rounds per workgroup of the register path, forced by the environment
// variable DGT_ROUNDS (a positive count; results are identical), else 0.
uint32_t rounds_from_env() {
  const char* v = std::getenv("DGT_ROUNDS");
  if (!v) return 0;
  const long r = std::strtol(v, nullptr, 10);
  return (r > 0 && r < 65536) ? (uint32_t)r : 0u;
}

int launch_quant(const uint16_t* d_x, uint32_t count, uint8_t* ws_q, hipStream_t st,
                 uint16_t** xq, float** sx) {
  QuantArgs q;
  q.x = d_x;
  q.xq = reinterpret_cast<uint16_t*>(ws_q + 256);
  q.amax_bits = reinterpret_cast<uint32_t*>(ws_q);
  q.done = reinterpret_cast<uint32_t*>(ws_q + 4);
  q.sx = reinterpret_cast<float*>(ws_q + 8);
  q.count = count;
  *xq = q.xq;
  *sx = q.sx;
  if (count <= kQuantOneBlock && count % 8 == 0) {
    hipLaunchKernelGGL(k_amax_quant, dim3(1), dim3(1024), 0, st, q);
    return hipGetLastError() == hipSuccess ? DGT_OK : DGT_E_HIP;
  }
  const uint32_t blocks = std::max<uint32_t>(1, std::min<uint32_t>(1024, (count + 2047) / 2048));
  hipLaunchKernelGGL(k_amax, dim3(blocks), dim3(256), 0, st, q);
  if (hipGetLastError() != hipSuccess) return DGT_E_HIP;
  hipLaunchKernelGGL(k_quant, dim3(blocks), dim3(256), 0, st, q);
  return hipGetLastError() == hipSuccess ? DGT_OK : DGT_E_HIP;
}

}  // namespace

namespace {

// Rows per launch of the fused kernels; larger M runs in passes of this many
// rows (each pass decodes the layer again).
constexpr uint32_t kPassRows = 256;
constexpr uint32_t kMaxRows = 1u << 16;

// Plans of the full passes and of the remainder pass, and the workspace both
// need: the partial region of the larger one and, for fp8, the quantised X of
// all rows (one per-tensor scale for the whole call).
struct CallPlan {
  FusedPlan full, rest;
  uint32_t n_full, rest_rows;
  size_t quant_off, ws_bytes;
};

bool plan_call(const dgt_info* in, uint32_t m, CallPlan* c, Staging sg, uint32_t rounds,
               bool sub) {
  c->n_full = m / kPassRows;
  c->rest_rows = m % kPassRows;
  size_t q = 0;
  if (c->n_full) {
    if (!plan_fused(in, kPassRows, &c->full, sg, rounds, sub)) return false;
    q = std::max(q, c->full.quant_off);
  }
  if (c->rest_rows) {
    if (!plan_fused(in, c->rest_rows, &c->rest, sg, rounds, sub)) return false;
    q = std::max(q, c->rest.quant_off);
  }
  c->quant_off = q;
  c->ws_bytes = q;
  if (in->fmt == DGT_FMT_FP8_E4M3) c->ws_bytes += dgt::align_up((size_t)m * in->k * 2, 256) + 256;
  return true;
}

// One pass of at most kPassRows rows with plan p.
int launch_pass(const FusedPlan& p, const dgt_info* info, const Layer& L0, const uint8_t* xsrc,
                uint32_t xrow, uint32_t m, const uint16_t* d_scales, float* sxp, float w_scale,
                float* d_y, uint8_t* ws, int32_t* d_status, hipStream_t st) {
  const uint32_t fn = info->tile_n / 16;
  const bool rg = p.ring != 0;
  Layer L = L0;
  L.region_words = p.region_words;
  if (p.xm) {
    // (the one-buffer rung exists for 64-lane layers)
    const bool pp = !(xm_single_buffer_from_env() && info->lanes == 64);
    XmArgs x;
    GemmArgs& a = x.g;
    a.L = L;
    a.x = xsrc;
    a.scales = d_scales;
    a.xscale = sxp;
    a.w_scale = w_scale;
    a.y = d_y;
    a.part = reinterpret_cast<float*>(ws + p.part_off);
    a.counters = reinterpret_cast<uint32_t*>(ws);
    a.status = d_status;
    a.m = m;
    a.x_row_bytes = xrow;
    a.y_row = info->n;
    a.waves = p.waves;
    a.tpw = 1;
    a.chains = p.chains;
    a.cps = p.cps;
    a.cpw = p.cpw;
    a.n2 = 0;
    a.slots = p.slots;
    a.red_cols = 0;
    a.rounds = 1;
    a.red_off = 0;
    a.swz = xcd_order_from_env() ? 1u : 0u;
    x.bps = p.bps;
    x.bpw = p.bpw;
    x.batches = p.batches;
    x.xbuf_off = p.xbuf_off;
    switch (info->fmt) {
      case DGT_FMT_INT8: return launch_fused_xm<INT8>(x, info->lanes, fn, rg, pp, p.xs, p.wgs, p.lds, st);
      case DGT_FMT_INT4: return launch_fused_xm<INT4>(x, info->lanes, fn, rg, pp, p.xs, p.wgs, p.lds, st);
      case DGT_FMT_INT4_PAIR: return launch_fused_xm<INT4P>(x, info->lanes, fn, rg, pp, p.xs, p.wgs, p.lds, st);
      case DGT_FMT_BF16_EXP: return launch_fused_xm<BF16E>(x, info->lanes, fn, rg, pp, p.xs, p.wgs, p.lds, st);
      case DGT_FMT_BF16_PAIR: return launch_fused_xm<BF16P>(x, info->lanes, fn, rg, pp, p.xs, p.wgs, p.lds, st);
      case DGT_FMT_FP8_E4M3: return launch_fused_xm<FP8>(x, info->lanes, fn, rg, pp, p.xs, p.wgs, p.lds, st);
      case DGT_FMT_BF16_SPLIT: return launch_fused_xm<BF16>(x, info->lanes, fn, rg, pp, p.xs, p.wgs, p.lds, st);
      case DGT_FMT_BF16_WORD: return launch_fused_xm<BF16W>(x, info->lanes, fn, rg, pp, p.xs, p.wgs, p.lds, st);
      default: return DGT_E_ARG;
    }
  }
  for (uint32_t m0 = 0; m0 < m; m0 += p.m_chunk) {
    GemmArgs a;
    a.L = L;
    a.x = xsrc + (size_t)m0 * xrow;
    a.scales = d_scales;
    a.xscale = sxp;
    a.w_scale = w_scale;
    a.y = d_y + (size_t)m0 * info->n;
    a.part = reinterpret_cast<float*>(ws + p.part_off);
    a.counters = reinterpret_cast<uint32_t*>(ws);
    a.status = d_status;
    a.m = std::min<uint32_t>(p.m_chunk, m - m0);
    a.x_row_bytes = xrow;
    a.y_row = info->n;
    a.waves = p.waves;
    a.tpw = info->lanes == 32 ? 2 : 1;
    a.chains = p.chains;
    a.cps = p.cps;
    a.cpw = p.cpw;
    a.n2 = p.n2;
    a.slots = p.slots;
    a.red_cols = p.red_cols;
    a.rounds = p.rounds;
    a.red_off = p.red_off;
    a.swz = xcd_order_from_env() ? 1u : 0u;
    const uint32_t grid = p.wgs, threads = p.threads;
    const bool mix = p.mix != 0;
    int rc;
    if (p.rounds > 1) {
      switch (info->fmt) {
        case DGT_FMT_INT8: rc = launch_fused_rounds<INT8>(a, info->lanes, fn, p.mt, mix, grid, threads, p.lds, st, nullptr); break;
        case DGT_FMT_INT4: rc = launch_fused_rounds<INT4>(a, info->lanes, fn, p.mt, mix, grid, threads, p.lds, st, nullptr); break;
        case DGT_FMT_INT4_PAIR: rc = launch_fused_rounds<INT4P>(a, info->lanes, fn, p.mt, mix, grid, threads, p.lds, st, nullptr); break;
        case DGT_FMT_BF16_EXP: rc = launch_fused_rounds<BF16E>(a, info->lanes, fn, p.mt, mix, grid, threads, p.lds, st, nullptr); break;
        case DGT_FMT_BF16_PAIR: rc = launch_fused_rounds<BF16P>(a, info->lanes, fn, p.mt, mix, grid, threads, p.lds, st, nullptr); break;
        case DGT_FMT_FP8_E4M3: rc = launch_fused_rounds<FP8>(a, info->lanes, fn, p.mt, mix, grid, threads, p.lds, st, nullptr); break;
        case DGT_FMT_BF16_SPLIT: rc = launch_fused_rounds<BF16>(a, info->lanes, fn, p.mt, mix, grid, threads, p.lds, st, nullptr); break;
        case DGT_FMT_BF16_WORD: rc = launch_fused_rounds<BF16W>(a, info->lanes, fn, p.mt, mix, grid, threads, p.lds, st, nullptr); break;
        default: return DGT_E_ARG;
      }
      if (rc) return rc;
      continue;
    }
    switch (info->fmt) {
      case DGT_FMT_INT8:
        rc = launch_fused<INT8>(a, info->lanes, fn, p.mt, mix, rg, grid, threads, p.lds, st);
        break;
      case DGT_FMT_INT4:
        rc = launch_fused<INT4>(a, info->lanes, fn, p.mt, mix, rg, grid, threads, p.lds, st);
        break;
      case DGT_FMT_INT4_PAIR:
        rc = launch_fused<INT4P>(a, info->lanes, fn, p.mt, mix, rg, grid, threads, p.lds, st);
        break;
      case DGT_FMT_BF16_EXP:
        rc = launch_fused<BF16E>(a, info->lanes, fn, p.mt, mix, rg, grid, threads, p.lds, st);
        break;
      case DGT_FMT_BF16_PAIR:
        rc = launch_fused<BF16P>(a, info->lanes, fn, p.mt, mix, rg, grid, threads, p.lds, st);
        break;
      case DGT_FMT_FP8_E4M3:
        rc = launch_fused<FP8>(a, info->lanes, fn, p.mt, mix, rg, grid, threads, p.lds, st);
        break;
      case DGT_FMT_BF16_SPLIT:
        rc = launch_fused<BF16>(a, info->lanes, fn, p.mt, mix, rg, grid, threads, p.lds, st);
        break;
      case DGT_FMT_BF16_WORD:
        rc = launch_fused<BF16W>(a, info->lanes, fn, p.mt, mix, rg, grid, threads, p.lds, st);
        break;
      default:
        rc = DGT_E_ARG;
    }
    if (rc) return rc;
  }
  return DGT_OK;
}

}  // namespace

extern "C" {

size_t dgt_gemm_workspace(const dgt_info* info, uint32_t m) {
  if (!info || m == 0 || m > kMaxRows) return 0;
  // enough for every staging, for one round per workgroup (the most partial
  // slots) and for either large-M form, so the environment may change
  // between calls
  size_t ws = 0;
  for (Staging sg : {kAuto, kWhole, kRing})
    for (uint32_t rounds : {0u, 1u})
      for (bool sub : {false, true}) {
        CallPlan c;
        if (!plan_call(info, m, &c, sg, rounds, sub)) return 0;
        ws = std::max(ws, c.ws_bytes);
      }
  return ws;
}

}  // extern "C"

namespace {

// Checks shared by the fused entry points; fills the call's plan.
int fused_prepare(const void* d_blob, const dgt_info* info, const uint16_t* d_x, uint32_t m,
                  const uint16_t* d_scales, float* d_y, CallPlan* c) {
  if (!d_blob || !info || !d_x || !d_y || m == 0 || m > kMaxRows) return DGT_E_ARG;
  if (((uintptr_t)d_blob & 15) || ((uintptr_t)d_x & 15)) return DGT_E_ARG;
  int rc = device_supported(info);
  if (rc) return rc;
  if ((info->fmt == DGT_FMT_INT4 || info->fmt == DGT_FMT_INT4_PAIR) &&
      (!d_scales || info->k % 128))
    return DGT_E_ARG;
  const uint32_t fn = info->tile_n / 16;
  if (fn != 8 && fn != 16) return DGT_E_UNSUPPORTED;
  if (info->lanes == 32 && (info->k / info->tile_k) % 2) return DGT_E_UNSUPPORTED;
  if (!plan_call(info, m, c, staging_from_env(), rounds_from_env(), xm_subsets_from_env()))
    return DGT_E_UNSUPPORTED;
  return DGT_OK;
}

// The launches of one fused call with plan c on workspace ws (counters at zero).
int fused_launch(const CallPlan& c, const void* d_blob, const dgt_info* info,
                 const uint16_t* d_x, uint32_t m, const uint16_t* d_scales, float w_scale,
                 float* d_y, uint8_t* ws, int32_t* d_status, hipStream_t st) {
  int rc = DGT_OK;
  Layer L;
  layer_from_info(d_blob, info, &L);
  const uint8_t* xsrc = reinterpret_cast<const uint8_t*>(d_x);
  const uint32_t xrow = info->k * 2;
  float* sxp = nullptr;
  if (info->fmt == DGT_FMT_FP8_E4M3) {
    uint16_t* xq = nullptr;
    float* sx = nullptr;
    rc = launch_quant(d_x, m * info->k, ws + c.quant_off, st, &xq, &sx);
    if (rc) return rc;
    xsrc = reinterpret_cast<const uint8_t*>(xq);
    sxp = sx;
  }
  // passes run in order on the stream and share the workspace (its counters
  // are back at zero after each)
  for (uint32_t pass = 0; pass <= c.n_full; ++pass) {
    const bool full = pass < c.n_full;
    const uint32_t rows = full ? kPassRows : c.rest_rows;
    if (rows == 0) break;
    const size_t r0 = (size_t)pass * kPassRows;
    rc = launch_pass(full ? c.full : c.rest, info, L, xsrc + r0 * xrow, xrow, rows, d_scales,
                     sxp, w_scale, d_y + r0 * info->n, ws, d_status, st);
    if (rc) return rc;
  }
  return DGT_OK;
}

// ------------------------------------------------ allocation-free workspace
// The workspace of dgt_fused_decode_gemm_noalloc: a static device array (each
// device holds its own copy from the library's load until the process ends).
// In host code `scratch` names a host-side stand-in; its device address comes
// from hipGetSymbolAddress, taken once per device and kept in g_scratch.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of the current device's scratch (set up on first use).
int scratch_of_current_device(uint8_t** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DGT_E_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return DGT_E_HIP;
    g_scratch[dev] = p;
  }
  *out = static_cast<uint8_t*>(g_scratch[dev]);
  return DGT_OK;
}

// Zero n dwords (a kernel rather than a memset node, so the call stays
// correct when a caller captures it into a graph).
__global__ __launch_bounds__(256) void k_zero(uint32_t* p, uint32_t n) {
  for (uint32_t i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) p[i] = 0u;
}

}  // namespace

extern "C" {

int dgt_fused_decode_gemm(const void* d_blob, const dgt_info* info, const uint16_t* d_x,
                          uint32_t m, const uint16_t* d_scales, float w_scale, float* d_y,
                          void* d_ws, size_t ws_bytes, int32_t* d_status, void* stream) {
  if (!d_ws || ((uintptr_t)d_ws & 255)) return DGT_E_ARG;
  CallPlan c;
  int rc = fused_prepare(d_blob, info, d_x, m, d_scales, d_y, &c);
  if (rc) return rc;
  if (ws_bytes < c.ws_bytes) return DGT_E_BUFSIZE;
  return fused_launch(c, d_blob, info, d_x, m, d_scales, w_scale, d_y,
                      static_cast<uint8_t*>(d_ws), d_status, static_cast<hipStream_t>(stream));
}

size_t dgt_noalloc_scratch_bytes(void) { return kScratchBytes; }

int dgt_fused_decode_gemm_noalloc(const void* d_blob, const dgt_info* info, const uint16_t* d_x,
                                  uint32_t m, const uint16_t* d_scales, float w_scale,
                                  float* d_y, int32_t* d_status, void* stream) {
  CallPlan c;
  int rc = fused_prepare(d_blob, info, d_x, m, d_scales, d_y, &c);
  if (rc) return rc;
  if (c.ws_bytes > kScratchBytes) return DGT_E_BUFSIZE;
  uint8_t* ws = nullptr;
  rc = scratch_of_current_device(&ws);
  if (rc) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  // the per-strip counters (and the fp8 quantisation's maximum and block
  // counter) must start at zero; the array keeps whatever the last call left
  const uint32_t strips = info->n / info->tile_n;
  const uint32_t counter_words = (uint32_t)(dgt::align_up((size_t)strips * 4, 256) / 4);
  hipLaunchKernelGGL(k_zero, dim3(std::min<uint32_t>((counter_words + 255) / 256, 64)),
                     dim3(256), 0, st, reinterpret_cast<uint32_t*>(ws), counter_words);
  if (hipGetLastError() != hipSuccess) return DGT_E_HIP;
  if (info->fmt == DGT_FMT_FP8_E4M3) {
    hipLaunchKernelGGL(k_zero, dim3(1), dim3(256), 0, st,
                       reinterpret_cast<uint32_t*>(ws + c.quant_off), 64u);
    if (hipGetLastError() != hipSuccess) return DGT_E_HIP;
  }
  return fused_launch(c, d_blob, info, d_x, m, d_scales, w_scale, d_y, ws, d_status, st);
}

int dgt_decode_tiles(const void* d_blob, const dgt_info* info, const uint32_t* d_tile_ids,
                     uint32_t n_ids, void* d_out, int32_t* d_status, void* stream) {
  if (!d_blob || !info || !d_out) return DGT_E_ARG;
  if ((uintptr_t)d_blob & 15) return DGT_E_ARG;
  int rc = device_supported(info);
  if (rc) return rc;
  if (!d_tile_ids) n_ids = info->tiles;
  if (n_ids == 0) return DGT_OK;
  DecodeArgs a;
  layer_from_info(d_blob, info, &a.L);
  a.ids = d_tile_ids;
  a.n_ids = n_ids;
  a.out = static_cast<uint8_t*>(d_out);
  a.status = d_status;
  const uint32_t R = info->lanes, tpc = R == 32 ? 2 : 1;
  // chains (tpc tiles each) over the CUs in one round of workgroups when the
  // wave cap allows: two chains per wave for large layers, 4..16 waves
  const uint32_t units = (n_ids + tpc - 1) / tpc;
  const uint32_t ilp = units >= kCUs * 16 ? 2 : 1;
  uint32_t waves = (units + kCUs * ilp - 1) / (kCUs * ilp);
  waves = std::min(std::max(waves, 4u), 16u);
  // whole streams when the workgroup's tiles fit LDS, else (R = 64, 128) the ring
  bool ring = false;
  auto lds_for = [&](uint32_t w) {
    return tab_bytes_layer((int)info->fmt, info->alphabet) + w * ilp * tpc * a.L.region_words * 2;
  };
  const Staging sg = staging_from_env();
  if (R != 32) {
    if (sg == kRing) ring = true;
    else if (sg == kWhole) ring = lds_for(4) > kMaxLds;
    else ring = lds_for(waves) > kMaxLds;
  }
  if (ring) a.L.region_words = region_words_of(info, true);
  while (waves > 4 && lds_for(waves) > kMaxLds) --waves;
  if (lds_for(waves) > kMaxLds) return DGT_E_UNSUPPORTED;
  a.waves = waves;
  const uint32_t per_wg = waves * ilp * tpc;
  const uint32_t grid = (n_ids + per_wg - 1) / per_wg;
  const uint32_t lds = lds_for(waves);
  hipStream_t st = static_cast<hipStream_t>(stream);
  switch (info->fmt) {
    case DGT_FMT_INT8: return launch_decode<INT8>(a, R, ilp, ring, grid, 64 * waves, lds, st);
    case DGT_FMT_INT4: return launch_decode<INT4>(a, R, ilp, ring, grid, 64 * waves, lds, st);
    case DGT_FMT_INT4_PAIR: return launch_decode<INT4P>(a, R, ilp, ring, grid, 64 * waves, lds, st);
    case DGT_FMT_BF16_EXP: return launch_decode<BF16E>(a, R, ilp, ring, grid, 64 * waves, lds, st);
    case DGT_FMT_BF16_PAIR: return launch_decode<BF16P>(a, R, ilp, ring, grid, 64 * waves, lds, st);
    case DGT_FMT_FP8_E4M3: return launch_decode<FP8>(a, R, ilp, ring, grid, 64 * waves, lds, st);
    case DGT_FMT_BF16_SPLIT: return launch_decode<BF16>(a, R, ilp, ring, grid, 64 * waves, lds, st);
    case DGT_FMT_BF16_WORD: return launch_decode<BF16W>(a, R, ilp, ring, grid, 64 * waves, lds, st);
    default: break;
  }
  return DGT_E_UNSUPPORTED;
}

namespace {
struct DensePlan {
  uint32_t strips, kt, tpw, ups, units, waves, wgs, slots, mc, mt;
  size_t part_off, quant_off, ws_bytes;
};
bool plan_dense(uint32_t fmt, uint32_t n, uint32_t k, uint32_t tile_n, uint32_t m, DensePlan* p) {
  if (m == 0 || (tile_n != 128 && tile_n != 256) || n % tile_n || k % 128) return false;
  p->strips = n / tile_n;
  p->kt = k / 64;
  p->tpw = 2;
  p->ups = p->kt / p->tpw;
  p->units = p->strips * p->ups;
  p->mc = std::min<uint32_t>(m, tile_n == 256 ? 16 : 64);
  p->mt = p->mc <= 16 ? 1 : 4;
  p->waves = pick_waves(p->units, p->ups, dense_max_threads(tile_n / 16, p->mt) / 64);
  p->wgs = (p->units + p->waves - 1) / p->waves;
  p->slots = (p->ups + p->waves - 1) / p->waves + 1;
  size_t off = dgt::align_up((size_t)p->strips * 4, 256);
  p->part_off = off;
  off += (size_t)p->strips * p->slots * p->mc * tile_n * 4;
  off = dgt::align_up(off, 256);
  p->quant_off = off;
  if (fmt == DGT_FMT_FP8_E4M3) off += dgt::align_up((size_t)m * k * 2, 256) + 256;
  p->ws_bytes = off;
  return true;
}
}  // namespace

size_t dgt_dense_workspace(uint32_t fmt, uint32_t n, uint32_t k, uint32_t tile_n, uint32_t m) {
  DensePlan p;
  return plan_dense(fmt, n, k, tile_n, m, &p) ? p.ws_bytes : 0;
}

int dgt_dense_gemm(uint32_t fmt, uint32_t n, uint32_t k, uint32_t tile_n, const void* d_w,
                   const uint16_t* d_x, uint32_t m, const uint16_t* d_scales, float w_scale,
                   float* d_y, void* d_ws, size_t ws_bytes, void* stream) {
  if (!d_w || !d_x || !d_y || !d_ws || m == 0 || m > 256) return DGT_E_ARG;
  if (fmt < DGT_FMT_INT8 || fmt > DGT_FMT_BF16_WORD) return DGT_E_ARG;
  // same decoded layout and values as the one-symbol-per-weight formats
  if (fmt == DGT_FMT_INT4_PAIR) fmt = DGT_FMT_INT4;
  if (fmt == DGT_FMT_BF16_EXP || fmt == DGT_FMT_BF16_PAIR || fmt == DGT_FMT_BF16_WORD)
    fmt = DGT_FMT_BF16_SPLIT;
  if ((tile_n != 128 && tile_n != 256) || n % tile_n || k % 64 || (k / 64) % 2)
    return DGT_E_SHAPE;
  if (fmt == DGT_FMT_INT4 && (!d_scales || k % 128)) return DGT_E_ARG;
  if (((uintptr_t)d_w & 15) || ((uintptr_t)d_x & 15) || ((uintptr_t)d_ws & 255))
    return DGT_E_ARG;
  DensePlan p;
  if (!plan_dense(fmt, n, k, tile_n, m, &p)) return DGT_E_SHAPE;
  if (ws_bytes < p.ws_bytes) return DGT_E_BUFSIZE;
  const uint32_t mc = p.mc, mt = p.mt, waves = p.waves;
  uint8_t* ws = static_cast<uint8_t*>(d_ws);
  const size_t part_off = p.part_off, quant_off = p.quant_off;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const uint8_t* xsrc = reinterpret_cast<const uint8_t*>(d_x);
  uint32_t xrow = k * 2;
  float* sxp = nullptr;
  if (fmt == DGT_FMT_FP8_E4M3) {
    uint16_t* xq = nullptr;
    float* sx = nullptr;
    int rc = launch_quant(d_x, m * k, ws + quant_off, st, &xq, &sx);
    if (rc) return rc;
    xsrc = reinterpret_cast<const uint8_t*>(xq);
    sxp = sx;
  }
  // one row: the streaming GEMV (X staged whole in LDS)
  if (m == 1 && (size_t)k * 2 <= 64 * 1024) {
    GemvArgs g;
    g.w = static_cast<const uint8_t*>(d_w);
    g.x = reinterpret_cast<const uint16_t*>(xsrc);
    g.scales = d_scales;
    g.xscale = sxp;
    g.w_scale = w_scale;
    g.y = d_y;
    g.n = n;
    g.k = k;
    switch (fmt) {
      case DGT_FMT_INT8: return launch_gemv<INT8>(g, st);
      case DGT_FMT_INT4: return launch_gemv<INT4>(g, st);
      case DGT_FMT_FP8_E4M3: return launch_gemv<FP8>(g, st);
      case DGT_FMT_BF16_SPLIT: return launch_gemv<BF16>(g, st);
      default: return DGT_E_UNSUPPORTED;
    }
  }
  // 32 rows and more: the LDS-tiled GEMM, all rows in one launch
  if (m >= 32) {
    DenseTiledArgs t;
    t.w = static_cast<const uint8_t*>(d_w);
    t.x = xsrc;
    t.scales = d_scales;
    t.xscale = sxp;
    t.w_scale = w_scale;
    t.y = d_y;
    t.m = m;
    t.n = n;
    t.k = k;
    t.x_row_bytes = xrow;
    t.nmb = (m + kDtRows - 1) / kDtRows;
    // 64-row blocks of W when 128-row ones would not give every CU two
    const uint32_t bn = t.nmb * (n / 128) >= 2 * kCUs ? 128u : 64u;
    t.nnb = n / bn;
    switch (fmt) {
      case DGT_FMT_INT8: return launch_dense_tiled<INT8>(t, bn, st);
      case DGT_FMT_INT4: return launch_dense_tiled<INT4>(t, bn, st);
      case DGT_FMT_FP8_E4M3: return launch_dense_tiled<FP8>(t, bn, st);
      case DGT_FMT_BF16_SPLIT: return launch_dense_tiled<BF16>(t, bn, st);
      default: return DGT_E_UNSUPPORTED;
    }
  }
  const uint32_t lds = 64 * 1024;
  for (uint32_t m0 = 0; m0 < m; m0 += mc) {
    DenseArgs d;
    GemmArgs& a = d.g;
    a.L = Layer{};
    a.x = xsrc + (size_t)m0 * xrow;
    a.scales = d_scales;
    a.xscale = sxp;
    a.w_scale = w_scale;
    a.y = d_y + (size_t)m0 * n;
    a.part = reinterpret_cast<float*>(ws + part_off);
    a.counters = reinterpret_cast<uint32_t*>(ws);
    a.status = nullptr;
    a.m = std::min<uint32_t>(mc, m - m0);
    a.x_row_bytes = xrow;
    a.y_row = n;
    a.waves = waves;
    a.tpw = p.tpw;
    a.chains = p.units;
    a.cps = p.ups;
    a.cpw = waves;
    a.n2 = 0;
    a.slots = p.slots;
    uint32_t rc_cols = tile_n;
    while (rc_cols > 16 && (uint64_t)waves * a.m * rc_cols * 4 > lds) rc_cols /= 2;
    a.red_cols = rc_cols;
    a.rounds = 1;
    a.red_off = 0;
    a.swz = 0;
    d.w = static_cast<const uint8_t*>(d_w);
    d.n = n;
    d.k = k;
    d.kt = p.kt;
    const uint32_t grid = p.wgs;
    int rc = DGT_E_UNSUPPORTED;
    const uint32_t fnv = tile_n / 16;
    switch (fmt) {
      case DGT_FMT_INT8: rc = launch_dense<INT8>(d, fnv, mt, grid, 64 * waves, lds, st); break;
      case DGT_FMT_INT4: rc = launch_dense<INT4>(d, fnv, mt, grid, 64 * waves, lds, st); break;
      case DGT_FMT_FP8_E4M3: rc = launch_dense<FP8>(d, fnv, mt, grid, 64 * waves, lds, st); break;
      case DGT_FMT_BF16_SPLIT:
        rc = launch_dense<BF16>(d, fnv, mt, grid, 64 * waves, lds, st);
        break;
      default: break;
    }
    if (rc) return rc;
  }
  return DGT_OK;
}

}  // extern "C"
