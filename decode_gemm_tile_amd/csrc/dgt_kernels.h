// HIP kernel templates of libdgt for gfx950 (instantiated per format in dgt_fmt.hip).
//
// The fused path follows the run-time stage of "arXiv'26 | 无损压缩逼近
// Shannon 极限" §3.1: tiles are decoded on chip and handed straight to the
// matrix multiply; the decompressed layer is never written to HBM.  §2.2
// (layer-level decompress-to-global then GEMM) is kept only as the
// dgt_decode_tiles + dgt_dense_gemm comparison path.
//
// Work decomposition (static schedule, fixed at launch): the output is cut into
// strips of tile_n columns of Y (one tile row band of W).  A strip's k-tiles are
// split over waves: each wave decodes ILP chains (ILP independent rANS chains
// interleaved step by step, so one wave keeps several LDS round trips in
// flight) and accumulates its partial Y[M, tile_n] in registers.  The waves of
// a workgroup cover consecutive k-tiles of one strip and reduce their partials
// through LDS in a fixed order; when a strip needs several workgroups, each
// writes its partial to the workspace and the last one to arrive (atomic
// counter per strip) sums them in workgroup order and writes Y.  Results are
// therefore deterministic run to run.
#pragma once
#include <hip/hip_runtime.h>

#include "dgt_device.h"

namespace dgt {
namespace dev {

// ------------------------------------------------------------ kernel params
struct GemmArgs {
  Layer L;
  const uint8_t* x;          // bf16 bits [M, K] (FP8: the quantised X as exact bf16)
  const uint16_t* scales;    // INT4: bf16 bits [N, K/128]
  float* xscale;             // FP8: device sx (per-tensor activation scale)
  float w_scale;             // FP8 weight scale
  float* y;                  // fp32 [M, N]
  float* part;               // workspace partials [strips][slots][M][tile_n]
  uint32_t* counters;        // workspace counters [strips]
  int32_t* status;           // per-tile status or null
  uint32_t m;                // rows of X / Y in this launch (<= 16 * MT)
  uint32_t x_row_bytes;      // row stride of x in bytes
  uint32_t y_row;            // row stride of y in floats (= N)
  uint32_t waves;            // waves per workgroup
  uint32_t tpw;              // dense path: k-tiles per unit (one wave's work)
  uint32_t chains;           // schedule units in the layer (fused: chains; dense: units)
  uint32_t cps;              // units per strip
  uint32_t cpw;              // units per workgroup
  uint32_t n2;               // waves that take two units (the first n2 waves)
  uint32_t slots;            // partial slots per strip in the workspace
  uint32_t red_cols;         // tile_n columns reduced per LDS pass
  uint32_t rounds;           // k_fused_rounds: rounds of cpw units per workgroup
  uint32_t red_off;          // k_fused_rounds: LDS byte offset of the reduction buffer
  uint32_t swz;              // 1: workgroups take their work in XCD-major order (wg_of)
};

// Workgroup g of T runs on XCD g mod 8 under round-robin dispatch.  xcd_tile
// numbers the workgroups XCD-major, so that consecutive numbers (work that
// shares data: the row blocks of one block of Y, the workgroups of one strip)
// run on one XCD and share its L2.  A bijection of [0, T) for any T.
__host__ __device__ constexpr uint32_t xcd_tile(uint32_t g, uint32_t T) {
  return (g % 8) < T % 8 ? (g % 8) * (T / 8 + 1) + g / 8
                         : (T % 8) * (T / 8 + 1) + ((g % 8) - T % 8) * (T / 8) + g / 8;
}
__device__ __forceinline__ uint32_t wg_of(const GemmArgs& a) {
  return a.swz ? xcd_tile(blockIdx.x, gridDim.x) : blockIdx.x;
}

// Static schedule: units (a chain of TPC consecutive k-tiles of one strip for
// the fused path) are numbered strip-major; workgroup b takes units
// [b*C, b*C + C), C <= units per strip, so it covers the tail of one strip and
// the head of the next at most.  Its first n2 waves take two units each, the
// others one (n2 > 0 only with C and the units per strip even, so a wave's
// pair never straddles a strip): this evens the per-SIMD work when C is not a
// multiple of the wave count.  The workgroups touching strip s are
// floor(s*cps/C) .. floor(((s+1)*cps-1)/C).
__device__ __forceinline__ uint32_t strip_first_wg(uint32_t s, uint32_t cps, uint32_t C) {
  return (uint32_t)(((uint64_t)s * cps) / C);
}
__device__ __forceinline__ uint32_t strip_last_wg(uint32_t s, uint32_t cps, uint32_t C) {
  return (uint32_t)(((uint64_t)(s + 1) * cps - 1) / C);
}
// first unit of wave w inside its workgroup's range, and how many waves hold
// the first r units of the range
__device__ __forceinline__ uint32_t wave_first_unit(uint32_t w, uint32_t n2) {
  return w < n2 ? 2 * w : n2 + w;
}
__device__ __forceinline__ uint32_t waves_covering(uint32_t r, uint32_t n2) {
  return r <= 2 * n2 ? (r + 1) / 2 : n2 + (r - 2 * n2);
}

template <int FMT>
struct OperandTraits;
template <>
struct OperandTraits<INT8> { static constexpr int xbytes = 2; };
template <>
struct OperandTraits<INT4> { static constexpr int xbytes = 2; };
template <>
struct OperandTraits<INT4P> { static constexpr int xbytes = 2; };
template <>
struct OperandTraits<BF16E> { static constexpr int xbytes = 2; };
template <>
struct OperandTraits<BF16P> { static constexpr int xbytes = 2; };
template <>
struct OperandTraits<BF16> { static constexpr int xbytes = 2; };
template <>
struct OperandTraits<FP8> { static constexpr int xbytes = 2; };  // e4m3 widened to bf16
template <>
struct OperandTraits<BF16W> { static constexpr int xbytes = 2; };

// B operand of one fragment from 8 decoded LUT words (+ raw bytes / scales).
struct BOp {
  u32x4 v;  // bf16 path: 8 bf16; fp8 path: v.x, v.y hold 8 bytes
};

__device__ __forceinline__ uint32_t pack_hi_bytes(uint32_t e1, uint32_t e0) {
  return __builtin_amdgcn_perm(e1, e0, 0x0c0c0703u);  // [s0, s1, 0, 0]
}

// The B operand is built in two stages so that a fragment in flight holds 4
// registers per state rather than 8: pair_b reduces two consecutive decoded
// symbols (LUT words, symbol in the top byte) to one register as soon as both
// exist; finish_b adds raw bytes or scales and yields the operand.  Formats
// whose symbol already codes two weights (int4 pairs) keep one symbol per
// register and skip pair_b.
template <int FMT>
__device__ __forceinline__ uint32_t pair_b(uint32_t e0, uint32_t e1) {
  if constexpr (FMT == BF16 || FMT == INT4) {
    return pack_hi_bytes(e1, e0);  // [s0, s1, 0, 0]
  } else if constexpr (FMT == BF16E) {
    // exponents into bits 14..7 and 30..23 of the pair
    return (e0 >> 17) | ((e1 >> 1) & 0x7F800000u);
  } else if constexpr (FMT == INT8) {
    const uint32_t f0 = __float_as_uint((float)((int32_t)e0 >> 24));
    const uint32_t f1 = __float_as_uint((float)((int32_t)e1 >> 24));
    return __builtin_amdgcn_perm(f1, f0, 0x07060302u);  // two bf16 (exact integers)
  } else if constexpr (FMT == FP8) {
    return __builtin_amdgcn_perm(e1, e0, 0x07030c0cu);  // e4m3 bytes in the high half
  } else if constexpr (FMT == BF16W) {
    return e0 | (e1 << 16);  // the two weights' bf16 patterns
  } else {
    return e0;
  }
}

template <int FMT>
__device__ __forceinline__ BOp finish_b(const uint32_t (&q)[4], u32x2 raw, float sc,
                                        float nsc8) {
  BOp b;
  if constexpr (FMT == BF16 || FMT == BF16P) {  // q[i]: the high bytes of weights 2i, 2i+1
    b.v.x = __builtin_amdgcn_perm(q[0], raw.x, 0x05010400u);
    b.v.y = __builtin_amdgcn_perm(q[1], raw.x, 0x05030402u);
    b.v.z = __builtin_amdgcn_perm(q[2], raw.y, 0x05010400u);
    b.v.w = __builtin_amdgcn_perm(q[3], raw.y, 0x05030402u);
  } else if constexpr (FMT == BF16E) {
    // sign and mantissa from the raw bytes, each copied into both bytes of
    // its half by the byte permute, exponents from the pair
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t r = i < 2 ? raw.x : raw.y;
      const uint32_t sm = __builtin_amdgcn_perm(0u, r, (i & 1) ? 0x03030202u : 0x01010000u);
      o[i] = (sm & 0x807F807Fu) | (q[i] & ~0x807F807Fu);
    }
    b.v.x = o[0]; b.v.y = o[1]; b.v.z = o[2]; b.v.w = o[3];
  } else if constexpr (FMT == INT8 || FMT == BF16W) {
    b.v.x = q[0]; b.v.y = q[1]; b.v.z = q[2]; b.v.w = q[3];
  } else if constexpr (FMT == INT4) {
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      floatx2 w;
      w.x = __builtin_fmaf((float)(q[i] & 0xFFu), sc, nsc8);
      w.y = __builtin_fmaf((float)((q[i] >> 8) & 0xFFu), sc, nsc8);
      const bf16x2 h = __builtin_convertvector(w, bf16x2);
      o[i] = __builtin_bit_cast(uint32_t, h);
    }
    b.v.x = o[0]; b.v.y = o[1]; b.v.z = o[2]; b.v.w = o[3];
  } else if constexpr (FMT == INT4P) {  // symbol i: weights 2i (low nibble), 2i+1
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      floatx2 w;
      w.x = __builtin_fmaf((float)((q[i] >> 24) & 15u), sc, nsc8);
      w.y = __builtin_fmaf((float)(q[i] >> 28), sc, nsc8);
      const bf16x2 h = __builtin_convertvector(w, bf16x2);
      o[i] = __builtin_bit_cast(uint32_t, h);
    }
    b.v.x = o[0]; b.v.y = o[1]; b.v.z = o[2]; b.v.w = o[3];
  } else {  // FP8: e4m3 bytes widened exactly to bf16 (e4m3 is a subset of bf16)
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const floatx2 f = __builtin_amdgcn_cvt_pk_f32_fp8((int)q[i], true);
      o[i] = __builtin_amdgcn_perm(__float_as_uint(f.y), __float_as_uint(f.x), 0x07060302u);
    }
    b.v.x = o[0]; b.v.y = o[1]; b.v.z = o[2]; b.v.w = o[3];
  }
  return b;
}

// Collects a fragment's decoded symbols step by step into the 4 registers
// finish_b takes.
template <int FMT>
struct FragAcc {
  uint32_t q[4];
  uint32_t prev;
  __device__ __forceinline__ void put(int i, uint32_t e) {
    if constexpr (steps_per_frag<FMT>() == 8) {
      if (i & 1) q[i >> 1] = pair_b<FMT>(prev, e);
      else prev = e;
    } else {
      q[i] = e;
    }
  }
};

template <int FMT>
__device__ __forceinline__ BOp make_b(const uint32_t (&e)[steps_per_frag<FMT>()], u32x2 raw,
                                      float sc, float nsc8) {
  FragAcc<FMT> f;
#pragma unroll
  for (int i = 0; i < steps_per_frag<FMT>(); ++i) f.put(i, e[i]);
  return finish_b<FMT>(f.q, raw, sc, nsc8);
}

// All formats multiply on the bf16 matrix cores with fp32 accumulation.  The
// fp8 x fp8 matrix instructions sum each 32-term dot product with only about
// 16 bits relative to the sum of |products|, short of a 1e-5 output bound, so
// e4m3 operands are widened (exactly) to bf16 instead.
template <int FMT>
__device__ __forceinline__ floatx4 mfma(const u32x4& a, const BOp& b, floatx4 acc) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b.v), acc, 0, 0, 0);
}

// A operand (X) for lane l: row m, 8 consecutive k starting at k0.
template <int FMT>
__device__ __forceinline__ u32x4 load_a(const GemmArgs& a, uint32_t m, uint32_t k0) {
  u32x4 r = {0u, 0u, 0u, 0u};
  if (m < a.m) {
    const uint8_t* p = a.x + (size_t)m * a.x_row_bytes + (size_t)k0 * OperandTraits<FMT>::xbytes;
    r = *reinterpret_cast<const u32x4*>(p);
  }
  return r;
}

// ---------------------------------------------------------------- reduction
// Sum the per-wave partials acc[FN][MT] of a workgroup through LDS in wave
// order, separately for the (at most two) strips the workgroup covers.  A strip
// covered by one workgroup is written to Y directly; otherwise each workgroup
// stores its partial in its slot and the last one to arrive (per-strip
// counter) sums the slots in order, so results are deterministic.
// Units [u0, u1) of workgroup blockIdx.x are reduced: C units per workgroup
// in the strip numbering above; the waves holding units are those of the
// first min(u1 - u0, cpw) units of a round.
// MT = 0 is the single-row mode (M = 1): instead of one accumulator per row
// band, row band b of the tile is multiplied with an A operand holding X in
// row b only, so accumulator row b collects band b and one 16x16 accumulator
// holds all <= 16 bands (4 VGPRs instead of 4 per band).
// The same packing holds up to PR = 4 or 8 rows of X (MT = packed_mt(PR)):
// an accumulator then takes 16 / PR bands, its row PR * (b % (16 / PR)) + m
// collecting row m of band b, so PR rows cost 4 VGPRs per 16 / PR bands
// instead of 4 per band.  MT codes: 0 and 16 + PR packed, 1 and 4 the number
// of 16-row blocks of X.
__host__ __device__ constexpr int packed_mt(int rows) { return 16 + rows; }
constexpr int kPacked4 = packed_mt(4), kPacked8 = packed_mt(8);
__host__ __device__ constexpr bool mt_packed(int MT) { return MT == 0 || MT > 16; }
__host__ __device__ constexpr int packed_rows(int MT) { return MT > 16 ? MT - 16 : 1; }
__host__ __device__ constexpr int packed_bands(int MT) { return 16 / packed_rows(MT); }
__host__ __device__ constexpr int acc_bands(int FN, int MT) {
  return mt_packed(MT) ? (FN + packed_bands(MT) - 1) / packed_bands(MT) : FN;
}
__host__ __device__ constexpr int acc_blocks(int MT) { return mt_packed(MT) ? 1 : MT; }

template <int FN, int MT>
__device__ __forceinline__ void reduce_range(const GemmArgs& a,
                                             floatx4 (&acc)[acc_bands(FN, MT)][acc_blocks(MT)],
                                             float* red, float out_scale, uint32_t u0,
                                             uint32_t u1, uint32_t C, uint32_t t) {
  const uint32_t lane = t & 63, wave = t >> 6;
  const uint32_t M = a.m, TN = FN * 16, RC = a.red_cols;
  const uint32_t wg = wg_of(a);
  const uint32_t nw = waves_covering(min(u1 - u0, a.cpw), a.n2);  // active waves
  const uint32_t sA = u0 / a.cps, sB = (u1 - 1) / a.cps;
  const uint32_t split =                                         // waves in strip A
      (sA == sB) ? nw : waves_covering((sA + 1) * a.cps - u0, a.n2);
  const uint32_t nstrips = (sA == sB) ? 1u : 2u;
  __syncthreads();  // LUT / staged streams are no longer needed
  for (uint32_t c0 = 0; c0 < TN; c0 += RC) {
    if (mt_packed(MT) && wave < nw) {
      // accumulator j, row s = 4 * (lane / 16) + i: row s % PR of band
      // j * PB + s / PR
      constexpr uint32_t PR = packed_rows(MT), PB = packed_bands(MT);
#pragma unroll
      for (int j = 0; j < acc_bands(FN, MT); ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t s = 4 * (lane >> 4) + i, band = j * PB + s / PR, m = s % PR;
          const uint32_t col = band * 16 + (lane & 15);
          if (band < (uint32_t)FN && m < M && col >= c0 && col < c0 + RC)
            red[((size_t)wave * M + m) * RC + (col - c0)] = acc[j][0][i];
        }
    } else if (wave < nw) {
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        const uint32_t col = fn * 16 + (lane & 15);
        if (col >= c0 && col < c0 + RC) {
#pragma unroll
          for (int mt = 0; mt < acc_blocks(MT); ++mt) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const uint32_t m = mt * 16 + 4 * (lane >> 4) + i;
              if (m < M) red[((size_t)wave * M + m) * RC + (col - c0)] = acc[acc_bands(FN, MT) > 1 ? fn : 0][mt][i];
            }
          }
        }
      }
    }
    __syncthreads();
    for (uint32_t idx = t; idx < M * RC; idx += blockDim.x) {
      const uint32_t m = idx / RC, col = c0 + idx % RC;
      for (uint32_t k = 0; k < nstrips; ++k) {
        const uint32_t s = k ? sB : sA;
        const uint32_t w0 = k ? split : 0u, w1 = k ? nw : split;
        float v = 0.f;
        for (uint32_t w = w0; w < w1; ++w) v += red[(size_t)w * M * RC + idx];
        const uint32_t f = strip_first_wg(s, a.cps, C), l = strip_last_wg(s, a.cps, C);
        if (f == l) {
          a.y[(size_t)m * a.y_row + s * TN + col] = v * out_scale;
        } else {
          // agent-scope store: coherent across XCDs without an L2 writeback
          __hip_atomic_store(&a.part[(((size_t)s * a.slots + (wg - f)) * M + m) * TN + col], v,
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
    __syncthreads();
  }
  // Hand-off to the last workgroup of a shared strip.  The partials are
  // agent-scope atomic stores; waiting for their completion before the counter
  // update (and reading them back with agent-scope atomic loads) orders them
  // without the device-wide cache writeback/invalidate a full fence costs on a
  // multi-XCD part.
  uint32_t* last_flag = reinterpret_cast<uint32_t*>(red);  // reduction buffer is free now
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (t < nstrips) {
    const uint32_t s = t ? sB : sA;
    const uint32_t f = strip_first_wg(s, a.cps, C), l = strip_last_wg(s, a.cps, C);
    uint32_t last = 0;
    if (f != l) {
      const uint32_t old = __hip_atomic_fetch_add(&a.counters[s], 1u, __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT);
      last = (old == l - f) ? 1u : 0u;
    }
    last_flag[t] = last;
  }
  __syncthreads();
  for (uint32_t k = 0; k < nstrips; ++k) {
    if (!last_flag[k]) continue;
    const uint32_t s = k ? sB : sA;
    const uint32_t n = strip_last_wg(s, a.cps, C) - strip_first_wg(s, a.cps, C) + 1;
    for (uint32_t idx = t; idx < M * TN; idx += blockDim.x) {
      const uint32_t m = idx / TN, col = idx % TN;
      float v = 0.f;
      for (uint32_t g = 0; g < n; ++g)
        v += __hip_atomic_load(&a.part[(((size_t)s * a.slots + g) * M + m) * TN + col],
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      a.y[(size_t)m * a.y_row + s * TN + col] = v * out_scale;
    }
    if (t == 0)
      __hip_atomic_store(&a.counters[s], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// One round per workgroup: units [b*C, b*C + C).
template <int FN, int MT>
__device__ __forceinline__ void reduce_and_store(const GemmArgs& a,
                                                 floatx4 (&acc)[acc_bands(FN, MT)][acc_blocks(MT)],
                                                 float* red, float out_scale) {
  const uint32_t u0 = wg_of(a) * a.cpw;
  reduce_range<FN, MT>(a, acc, red, out_scale, u0, min(u0 + a.cpw, a.chains), a.cpw, threadIdx.x);
}

// --------------------------------------------------------------- fused GEMM
// FN = tile_n / 16 row bands per tile, MT = 16-row blocks of X.  A wave runs
// one or two chains (a chain is one tile for R = 64, two for R = 32); MIX
// kernels hold both code paths and the first n2 waves take two chains
// interleaved step by step.  LDS: LUT | cumulative table | staged stream
// regions (one per tile of the workgroup).
// Workgroup size cap per variant: kernels whose registers fit in 128 VGPRs run
// up to 16 waves per workgroup; the others (more row bands or row blocks of
// accumulators) stay at 8 waves with up to 256 VGPRs.
template <bool V>
struct BoolC { static constexpr bool value = V; };
template <int V>
struct IntC { static constexpr int value = V; };
// f(IntC<I>{}) for I = B .. E-1, unrolled at compile time
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(IntC<B>{});
    static_for<B + 1, E>(f);
  }
}

__host__ __device__ constexpr uint32_t fused_max_threads(int R, int FN, int MT, int ILP) {
  // (the packed kernels are held to 128 VGPRs: 16 waves per CU)
  return mt_packed(MT) ? ((R != 32 || ILP == 1) ? 1024u : 512u)
                       : ((MT == 1 && FN <= 8 && (R != 32 || ILP == 1)) ? 1024u : 512u);
}
__host__ __device__ constexpr uint32_t dense_max_threads(int FN, int MT) {
  return (MT == 1 && FN <= 8) ? 1024u : 512u;
}

// Decode and multiply ILP chains (ch[0..ILP)) of one strip into acc.  With
// two states per lane (R = 128) a fragment step yields the same 16x32 block
// position in both row halves of the tile: two products that share X.
// after_first() runs once the first fragment has been decoded (it writes the
// rest of whole-staged streams to LDS).
template <int FMT, int R, int FN, int MT, int ILP, bool RING, typename AfterFirst>
__device__ __forceinline__ void fused_chains(const GemmArgs& a, const u32x2* lut, uint8_t* smem,
                                             Chain (&chs)[2], Ring (&rgs)[2],
                                             const uint32_t (&tile_lane)[2],
                                             const uint32_t (&k0_lane)[2], uint32_t strip,
                                             floatx4 (&acc)[acc_bands(FN, MT)][acc_blocks(MT)],
                                             AfterFirst&& after_first) {
  const Layer& L = a.L;
  constexpr int NS = states_per_lane(R);
  constexpr uint32_t FW = (R == 128 ? 64 : R) / 2;  // fragment width (columns)
  constexpr int FNH = FN / NS;                        // row bands per state
  constexpr int SPF = steps_per_frag<FMT>();
  constexpr int ADV = ring_group_steps(R);
  Chain (&ch)[ILP] = *reinterpret_cast<Chain(*)[ILP]>(&chs[0]);
  Ring (&rg)[ILP] = *reinterpret_cast<Ring(*)[ILP]>(&rgs[0]);
  const uint32_t lane = lane_id();
  const bool upper = lane >= 32;
  // the word pointers are wave-uniform: keep them (and their updates) scalar
#pragma unroll
  for (int c = 0; c < ILP; ++c) {
    ch[c].p0 = uniform(ch[c].p0); ch[c].e0 = uniform(ch[c].e0); ch[c].s0 = uniform(ch[c].s0);
    ch[c].p1 = uniform(ch[c].p1); ch[c].e1 = uniform(ch[c].e1); ch[c].s1 = uniform(ch[c].s1);
    if (RING) {
      rg[c].cc = uniform(rg[c].cc);
      rg[c].nchunks = uniform(rg[c].nchunks);
    }
  }
  uint32_t lim_min = ch[0].lim;
#pragma unroll
  for (int c = 0; c < ILP; ++c) {
    lim_min = min(lim_min, uniform(ch[c].lim));
    if (R == 32) lim_min = min(lim_min, (uint32_t)__builtin_amdgcn_readlane((int)ch[c].lim, 32));
  }
  const uint32_t FK = L.tile_k / FW;
  const uint32_t G = FK * FNH;
  const uint32_t kgroups = L.k / 128;
  // one tile per chain: the tile and its first column are wave-uniform, so
  // only the lane's offsets stay in vector registers
  uint32_t tl[ILP], kb[ILP];
  const uint32_t koff = (R == 32) ? 0u : 8 * (lane >> 4);
#pragma unroll
  for (int c = 0; c < ILP; ++c) {
    tl[c] = (R == 32) ? tile_lane[c] : uniform(tile_lane[c]);
    kb[c] = (R == 32) ? k0_lane[c] : uniform(k0_lane[c] - koff);
  }
  // operands that come from global memory are fetched one fragment (raw
  // bytes, scales) or one column block (X) ahead of their use
  auto load_raw = [&](int c, uint32_t g, int h) __attribute__((always_inline)) -> u32x2 {
    const uint32_t p = (R == 128) ? 64 * h + lane : lane % R;
    const uint8_t* rp = L.raw + (size_t)tl[c] * L.tile_n * L.tile_k +
                        (size_t)g * 8 * R + p * 8;
    return *reinterpret_cast<const u32x2*>(rp);
  };
  auto load_scale = [&](int c, uint32_t g, int h) __attribute__((always_inline)) -> float {
    const uint32_t fkg = g / FNH, fng = g % FNH;
    const uint32_t row = strip * L.tile_n + (h * FNH + fng) * 16 + (lane & 15);
    const uint16_t sb = a.scales[(size_t)row * kgroups + (kb[c] + koff + fkg * FW) / 128];
    return __uint_as_float((uint32_t)sb << 16);
  };
  u32x2 raw_n[ILP][NS];
  float sc_n[ILP][NS];
#pragma unroll
  for (int c = 0; c < ILP; ++c)
#pragma unroll
    for (int h = 0; h < NS; ++h) {
      raw_n[c][h] = u32x2{0u, 0u};
      sc_n[c][h] = 0.f;
      if constexpr (has_raw_bytes<FMT>()) raw_n[c][h] = load_raw(c, 0, h);
      if constexpr (FMT == INT4 || FMT == INT4P) sc_n[c][h] = load_scale(c, 0, h);
    }
  constexpr bool kPrefetchA = mt_packed(MT) || MT == 1;
  constexpr int MB = acc_blocks(MT);
  // the X row of this lane (packed modes: the row its accumulator slot collects)
  const uint32_t xrow = mt_packed(MT) ? (lane & 15) % packed_rows(MT) : (lane & 15);
  u32x4 A_n[ILP][MB];
  if constexpr (kPrefetchA) {
#pragma unroll
    for (int c = 0; c < ILP; ++c)
#pragma unroll
      for (int mt = 0; mt < MB; ++mt)
        A_n[c][mt] = load_a<FMT>(a, mt * 16 + xrow, kb[c] + koff);
  }
  // A operands of column block fk (X is fetched one block ahead in the packed
  // modes and at MT = 1)
  u32x4 A[ILP][MB];
  auto take_a = [&](uint32_t fk) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < ILP; ++c)
#pragma unroll
      for (int mt = 0; mt < MB; ++mt) {
        if constexpr (kPrefetchA)
          A[c][mt] = A_n[c][mt];
        else
          A[c][mt] = load_a<FMT>(a, mt * 16 + xrow, kb[c] + fk * FW + koff);
      }
  };
  auto prefetch_a = [&](uint32_t fk) __attribute__((always_inline)) {
    if constexpr (kPrefetchA) {
      if (fk + 1 < FK) {
#pragma unroll
        for (int c = 0; c < ILP; ++c)
#pragma unroll
          for (int mt = 0; mt < MB; ++mt)
            A_n[c][mt] = load_a<FMT>(a, mt * 16 + xrow, kb[c] + (fk + 1) * FW + koff);
      }
    }
  };
  // Loads for later fragments are issued after the fragment's last ring
  // advance: a chunk written to the ring waits for the loads issued before it,
  // and these are then one fragment old instead of just issued.
  constexpr int kPrefetchStep = RING ? ((SPF - 1) / ADV) * ADV : 0;
  // one fragment: row band fn of every state, column block fk
  auto frag = [&](uint32_t fk, auto fnc) __attribute__((always_inline)) {
    constexpr int fn = decltype(fnc)::value;
    const uint32_t g = fk * FNH + fn;
    const uint32_t s0 = g * SPF;
    const uint32_t gn = min(g + 1, G - 1);
    u32x2 raw[ILP][NS];
    float sc[ILP][NS], nsc8[ILP][NS];
#pragma unroll
    for (int c = 0; c < ILP; ++c)
#pragma unroll
      for (int h = 0; h < NS; ++h) {
        raw[c][h] = raw_n[c][h];
        sc[c][h] = sc_n[c][h];
        nsc8[c][h] = -8.f * sc[c][h];
      }
    auto prefetch = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int c = 0; c < ILP; ++c)
#pragma unroll
        for (int h = 0; h < NS; ++h) {
          if constexpr (has_raw_bytes<FMT>()) raw_n[c][h] = load_raw(c, gn, h);
          if constexpr (FMT == INT4 || FMT == INT4P) sc_n[c][h] = load_scale(c, gn, h);
        }
      if (fn == 0) prefetch_a(fk);
    };
    FragAcc<FMT> e[ILP][NS];
    auto steps = [&](auto careful) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < SPF; ++i) {
        if constexpr (RING) {
          if (i % ADV == 0) {
#pragma unroll
            for (int c = 0; c < ILP; ++c) ring_advance(rg[c], smem, ch[c].s0, ch[c].p0, lane);
          }
        }
        if (i == kPrefetchStep) prefetch();
        uint32_t sy[ILP][NS];
        step_all<R, decltype(careful)::value, ILP, RING, sym_mode<FMT>()>(ch, lut, smem, s0 + i, upper, sy);
#pragma unroll
        for (int c = 0; c < ILP; ++c)
#pragma unroll
          for (int h = 0; h < NS; ++h) e[c][h].put(i, sy[c][h]);
      }
    };
    // payload steps (at most the last kPayloadMax) fall in the last fragments
    if (fn < FNH - (int)(kPayloadMax / SPF) || s0 + SPF - 1 < lim_min)
      steps(BoolC<false>{});
    else
      steps(BoolC<true>{});
#pragma unroll
    for (int c = 0; c < ILP; ++c)
#pragma unroll
      for (int h = 0; h < NS; ++h) {
        const BOp b = finish_b<FMT>(e[c][h].q, raw[c][h], sc[c][h], nsc8[c][h]);
        if constexpr (mt_packed(MT)) {
          // band h * FNH + fn: X in that band's rows of the A operand only
          constexpr int PR = packed_rows(MT), PB = packed_bands(MT);
          const int band = h * FNH + fn;
          const bool row = (lane & 15) / PR == (uint32_t)(band % PB);
          u32x4 ap;
          ap.x = row ? A[c][0].x : 0u;
          ap.y = row ? A[c][0].y : 0u;
          ap.z = row ? A[c][0].z : 0u;
          ap.w = row ? A[c][0].w : 0u;
          acc[band / PB][0] = mfma<FMT>(ap, b, acc[band / PB][0]);
        } else {
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
            acc[h * FNH + fn][mt] = mfma<FMT>(A[c][mt], b, acc[h * FNH + fn][mt]);
        }
      }
  };
  // The first fragment runs ahead of the loop, so that whatever after_first()
  // consumes is dead inside the loop (whose copy of it skips block 0).
  take_a(0);
  frag(0u, IntC<0>{});
  after_first();
  for (uint32_t fk = 0; fk < FK; ++fk) {
    if (fk > 0) take_a(fk);
    static_for<0, FNH>([&](auto fnc) __attribute__((always_inline)) {
      if (decltype(fnc)::value > 0 || fk > 0) frag(fk, fnc);
    });
  }
  if (a.status) {
    const uint32_t half_lane = lane & 31;
#pragma unroll
    for (int c = 0; c < ILP; ++c) {
      const uint32_t f = final_flags<R, RING>(ch[c], L.steps, upper);
      if (R != 32 ? lane == 0 : half_lane == 0) a.status[tl[c]] = (int32_t)f;
    }
  }
}

// RING (R = 64 or 128): stream the tile words through a two-chunk ring
// instead of staging them whole (any stream length; less LDS per chain).
template <int FMT, int R, int FN, int MT, bool MIX, bool RING>
__global__ __launch_bounds__(fused_max_threads(R, FN, MT, MIX ? 2 : 1)) void k_fused(GemmArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  u32x2* lut = reinterpret_cast<u32x2*>(smem);
  uint32_t* cum = reinterpret_cast<uint32_t*>(smem + kLutBytes);
  uint16_t* words = reinterpret_cast<uint16_t*>(smem + tab_of<FMT>(a.L));
  const Layer& L = a.L;
  constexpr uint32_t TPC = R == 32 ? 2 : 1;  // tiles per chain

  const uint32_t lane = lane_id();
  const uint32_t wave = uniform(threadIdx.x >> 6);
  const uint32_t u0 = wg_of(a) * a.cpw, u1 = min(u0 + a.cpw, a.chains);
  const uint32_t cw = wave_first_unit(wave, a.n2);
  // chains of this wave: 2 for the first n2 waves, else 1; none past the range
  uint32_t nch = (MIX && wave < a.n2) ? 2u : 1u;
  if (u0 + cw >= u1) nch = 0;
  else nch = min(nch, u1 - u0 - cw);
  const uint32_t chain0 = u0 + cw;
  const uint32_t strip = nch ? chain0 / a.cps : 0u;
  const uint32_t kt_first = nch ? (chain0 % a.cps) * TPC : 0u;
  const bool upper = lane >= 32;
  const uint32_t half_lane = lane & 31;

  Chain ch[2];
  uint32_t tile_lane[2] = {0u, 0u};
  uint32_t k0_lane[2] = {0u, 0u};
  Staged stg[2];   // whole streams
  Ring rg[2];      // ring: chunk 0 (c0) now, later chunks through the ring
  uint32_t c0[2][4];
  uint32_t kq[2];  // payload step counts, loaded before the streams
  const uint32_t fq = table_issue<FMT>(L);
  const uint32_t sub_lane = R != 32 ? lane : half_lane, sub_size = R != 32 ? 64u : 32u;
  // 1) issue the stream loads, 2) build the LUT while they are in flight,
  // 3) write the first words to LDS.  Both chain slots always load (a missing
  // second chain repeats the first) so that every wave has the same loads in
  // flight and the LUT build waits for the table alone.  Whole streams load
  // in two halves, the first halves of both chains first: decoding starts
  // once they are in LDS and the second halves follow after one fragment.
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const uint32_t cc = (c < (int)nch) ? (uint32_t)c : 0u;
    const uint32_t ta = strip * L.kt + kt_first + cc * TPC;
    const uint32_t t_l = (R == 32 && upper) ? ta + 1 : ta;
    tile_lane[c] = t_l;
    kq[c] = (R == 32) ? (uint32_t)L.ktab[t_l] : ktab_scalar(L.ktab, t_l);
    if constexpr (RING)
      ring_issue(L, t_l, lane, rg[c], c0[c]);
    else
      stage_begin(L, t_l, stg[c]);
    ch[c].x = L.streams[L.index[t_l] + (R == 32 ? half_lane : lane)];
    ch[c].x2 = (R == 128) ? L.streams[L.index[t_l] + 64 + lane] : 0u;
    const uint32_t kt_l = kt_first + cc * TPC + ((R == 32 && upper) ? 1u : 0u);
    k0_lane[c] = kt_l * L.tile_k + 8 * ((lane % R) >> 4);
  }
  if constexpr (!RING) {
#pragma unroll
    for (int c = 0; c < 2; ++c) stage_load(stg[c], L.lanes, sub_lane, sub_size, 0, kPreHalf);
#pragma unroll
    for (int c = 0; c < 2; ++c) stage_load(stg[c], L.lanes, sub_lane, sub_size, kPreHalf, kPre);
  }
  table_build<FMT>(fq, L, lut, cum);
  // the payload counts were loaded before the streams: waiting for them does
  // not wait for the stream loads (the counter retires loads in order)
#pragma unroll
  for (int c = 0; c < 2; ++c)
    if (c < (int)nch) ch[c].lim = L.steps - kq[c];
  __syncthreads();  // LUT complete; each wave's staged streams are private to it
  uint32_t cstart[2] = {0u, 0u};  // this lane's tile region (u16 words)
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    if (c < (int)nch) {
      const uint32_t ra = (cw + c) * TPC * L.region_words;
      if constexpr (RING) {
        ring_start(rg[c], ch[c], smem, tab_of<FMT>(a.L) + 2 * ra, lane, c0[c]);
      } else {
        const uint32_t rb = (R == 32) ? ra + L.region_words : ra;
        cstart[c] = (R == 32 && upper) ? rb : ra;
        stage_commit_part(stg[c], words, cstart[c], sub_lane, sub_size, 0, kPreHalf, false);
        const uint32_t mine = 2 * stg[c].words4;
        const uint32_t na = uniform(mine);
        const uint32_t nb = (R == 32) ? (uint32_t)__builtin_amdgcn_readlane((int)mine, 32) : na;
        const uint32_t ba = tab_of<FMT>(a.L) + 2 * ra, bb = tab_of<FMT>(a.L) + 2 * rb;
        ch[c].p0 = ba; ch[c].s0 = ba; ch[c].e0 = ba + 2 * na;
        ch[c].p1 = bb; ch[c].s1 = bb; ch[c].e1 = bb + 2 * nb;
      }
    }
  }
  auto commit_rest = [&]() __attribute__((always_inline)) {
    if constexpr (!RING) {
#pragma unroll
      for (int c = 0; c < 2; ++c)
        if (c < (int)nch)
          stage_commit_part(stg[c], words, cstart[c], sub_lane, sub_size, kPreHalf, kPre, true);
    }
  };

  floatx4 acc[acc_bands(FN, MT)][acc_blocks(MT)];
#pragma unroll
  for (int fn = 0; fn < acc_bands(FN, MT); ++fn)
#pragma unroll
    for (int mt = 0; mt < acc_blocks(MT); ++mt) acc[fn][mt] = floatx4{0.f, 0.f, 0.f, 0.f};
  if constexpr (MIX) {
    if (nch == 2)
      fused_chains<FMT, R, FN, MT, 2, RING>(a, lut, smem, ch, rg, tile_lane, k0_lane, strip, acc,
                                            commit_rest);
    else if (nch == 1)
      fused_chains<FMT, R, FN, MT, 1, RING>(a, lut, smem, ch, rg, tile_lane, k0_lane, strip, acc,
                                            commit_rest);
  } else {
    if (nch == 1)
      fused_chains<FMT, R, FN, MT, 1, RING>(a, lut, smem, ch, rg, tile_lane, k0_lane, strip, acc,
                                            commit_rest);
  }
  float out_scale = 1.f;
  if constexpr (FMT == FP8)
    out_scale = __hip_atomic_load(a.xscale, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) * a.w_scale;
  reduce_and_store<FN, MT>(a, acc, reinterpret_cast<float*>(smem), out_scale);
}

// Layers with more chains than the CUs hold at once: a workgroup runs
// a.rounds rounds of a.cpw units (a.cpw divides the units per strip and the
// units of the layer, so every round is full and lies in one strip).  The LUT
// is built once; a wave's accumulators carry over the rounds of a strip and
// are reduced when the next round starts another strip or the range ends,
// through a buffer at a.red_off that leaves the LUT intact.  Streams come
// through the ring.  Each wave holds the same number of chains (ILP) in every
// round, so its rounds are one loop with one decode path.
template <int FMT, int R, int FN, int MT, int ILP>
__device__ __forceinline__ void fused_rounds(const GemmArgs& a, uint8_t* smem, uint32_t fq,
                                             uint32_t cw) {
  const Layer& L = a.L;
  const u32x2* lut = reinterpret_cast<const u32x2*>(smem);
  uint32_t* cum = reinterpret_cast<uint32_t*>(smem + kLutBytes);
  float* red = reinterpret_cast<float*>(smem + a.red_off);
  const uint32_t C = a.cpw, CW = a.cpw * a.rounds;
  const uint32_t U0 = wg_of(a) * CW, U1 = min(U0 + CW, a.chains);
  floatx4 acc[acc_bands(FN, MT)][acc_blocks(MT)];
  for (uint32_t u0 = U0; u0 < U1; u0 += C) {
    const uint32_t lane = lane_id();
    const bool first = u0 == U0;
    const uint32_t chain0 = u0 + cw;
    const uint32_t strip = chain0 / a.cps;
    const uint32_t kt_first = chain0 % a.cps;
    Chain ch[2];
    Ring rg[2];
    uint32_t tile_lane[2] = {0u, 0u};
    uint32_t k0_lane[2] = {0u, 0u};
    uint32_t c0[2][4];
    uint32_t kq[2];  // payload step counts, loaded before the streams
#pragma unroll
    for (int c = 0; c < ILP; ++c) {
      const uint32_t t = strip * L.kt + kt_first + c;
      tile_lane[c] = t;
      kq[c] = ktab_scalar(L.ktab, t);
      ring_issue(L, t, lane, rg[c], c0[c]);
      ch[c].x = L.streams[L.index[t] + lane];
      ch[c].x2 = (R == 128) ? L.streams[L.index[t] + 64 + lane] : 0u;
      k0_lane[c] = (kt_first + c) * L.tile_k + 8 * (lane >> 4);
    }
    if (first) {
      table_build<FMT>(fq, L, const_cast<u32x2*>(lut), cum);
      __syncthreads();
    }
#pragma unroll
    for (int c = 0; c < ILP; ++c) {
      ch[c].lim = L.steps - kq[c];
      ring_start(rg[c], ch[c], smem, tab_of<FMT>(a.L) + 2 * (cw + c) * L.region_words, lane, c0[c]);
    }
    if (first) {
#pragma unroll
      for (int fn = 0; fn < acc_bands(FN, MT); ++fn)
#pragma unroll
        for (int mt = 0; mt < acc_blocks(MT); ++mt) acc[fn][mt] = floatx4{0.f, 0.f, 0.f, 0.f};
    }
    if constexpr (ILP > 0)
      fused_chains<FMT, R, FN, MT, ILP, true>(a, lut, smem, ch, rg, tile_lane, k0_lane, strip,
                                              acc, []() {});
    // reduce at the end of the range or before a round in another strip
    const uint32_t un = u0 + C;
    if (un >= U1 || un / a.cps != u0 / a.cps) {
      float out_scale = 1.f;
      if constexpr (FMT == FP8)
        out_scale = __hip_atomic_load(a.xscale, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) * a.w_scale;
      reduce_range<FN, MT>(a, acc, red, out_scale, max(U0, (u0 / a.cps) * a.cps), u0 + C, CW,
                           threadIdx.x);
      if (un < U1) {
#pragma unroll
        for (int fn = 0; fn < acc_bands(FN, MT); ++fn)
#pragma unroll
          for (int mt = 0; mt < acc_blocks(MT); ++mt) acc[fn][mt] = floatx4{0.f, 0.f, 0.f, 0.f};
        __syncthreads();  // the reduction buffer overlaps the next round's rings
      }
    }
  }
}

template <int FMT, int R, int FN, int MT, bool MIX>
__global__ __launch_bounds__(fused_max_threads(R, FN, MT, MIX ? 2 : 1)) void k_fused_rounds(GemmArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  const uint32_t wave = uniform(threadIdx.x >> 6);
  const uint32_t cw = wave_first_unit(wave, a.n2);
  const uint32_t fq = table_issue<FMT>(a.L);
  // chains per wave: 2 for the first n2 waves, else 1; none past the round
  if (MIX && wave < a.n2)
    fused_rounds<FMT, R, FN, MT, 2>(a, smem, fq, cw);
  else if (cw < a.cpw)
    fused_rounds<FMT, R, FN, MT, 1>(a, smem, fq, cw);
  else
    fused_rounds<FMT, R, FN, MT, 0>(a, smem, fq, cw);
}

// ------------------------------------------------- fused GEMM, large M (LDS)
// When M is too large for one wave to hold every row's accumulators, decoded
// fragments are shared through an LDS ping-pong buffer (the double-buffered
// decode/compute overlap of [P1 §3.1]).  A workgroup of NW waves works on
// batches of NT = NW * ILP consecutive k-tiles of one strip; each wave decodes
// ILP of them as interleaved chains.  After every group of FPB fragments (8
// steps each) each wave publishes its finished 16x32 B operands (two per
// fragment with two states per lane) into buffer (group & 1); after one
// barrier every wave multiplies all the group's operands with its own MTW
// 16-row blocks of X (A operands of the NT k-ranges stay in registers for the
// fragments that share them).  Each weight is decoded once for all
// M <= NW * MTW * 16 rows.  Registers bound the shape: A takes
// rows * NT / 4 and the accumulators rows * 2 VGPRs per wave, so a CU holds
// 16 decode chains at most (tile_n 128: 16 waves x 16 rows, one chain each;
// tile_n 256: 8 waves x 32 rows).  A workgroup runs bpw consecutive batches;
// each wave owns distinct rows, so accumulators go straight to Y (or to the
// strip's workspace slot) when the strip changes, with no LDS reduction.

struct XmArgs {
  GemmArgs g;
  uint32_t bps;        // batches per strip (k-tiles / NT)
  uint32_t bpw;        // batches per workgroup
  uint32_t batches;    // total batches (strips * bps)
  uint32_t xbuf_off;   // byte offset of the fragment buffers in LDS (16-aligned)
};

// XS = 1: every wave multiplies every tile of the batch into its own row
// blocks (8 waves x 32 rows for 256-row tiles, 16 x 16 for 128-row tiles).
// XS > 1 (256-row tiles, M <= 256 / XS): 16 waves in XS subsets of 16 / XS
// row groups; a wave multiplies only its subset's tiles, so its accumulators
// and A operands fit 128 VGPRs and a CU runs 16 decode chains instead of 8;
// the subsets' partial sums are added through LDS before the hand-off.
__host__ __device__ constexpr int xm_waves(int FN, int XS = 1) {
  return (FN == 8 || XS > 1) ? 16 : 8;
}
__host__ __device__ constexpr int xm_row_blocks(int FN, int XS = 1) {
  return (FN == 8 || XS > 1) ? 1 : 2;
}
__host__ __device__ constexpr int xm_ilp(int FN) { return 1; }
__host__ __device__ constexpr int xm_tiles(int FN, int XS = 1) {
  return xm_waves(FN, XS) * xm_ilp(FN);
}
// rows a workgroup holds
__host__ __device__ constexpr int xm_rows(int FN, int XS = 1) {
  return xm_waves(FN, XS) / XS * xm_row_blocks(FN, XS) * 16;
}
// fragments published per barrier: the most (4, 2 or 1) whose doubled buffers
// stay within 64 KiB of LDS (operands of 1 KiB: tiles x states per lane per
// fragment), 32 KiB beside the larger table of whole bf16 words
__host__ __device__ constexpr int xm_fpb(int R, int FN, int fmt, int XS = 1) {
  const int budget = (fmt == BF16W ? 32 : 64) * 1024;
  return 2 * 4 * xm_tiles(FN, XS) * states_per_lane(R) * 1024 <= budget   ? 4
         : 2 * 2 * xm_tiles(FN, XS) * states_per_lane(R) * 1024 <= budget ? 2
                                                                           : 1;
}

// Partials of a strip shared by several workgroups are kept in the
// accumulators' register layout (slot, wave, row block, fragment, float pair,
// lane), so every 8-byte store and load of a wave covers 512 contiguous bytes.
// A slot holds the full NW * MTW * 16 rows.
// owner = false: a wave whose sums another wave holds (XS > 1); it takes part
// in the barriers only.  NW: the waves that own row blocks (waves 0..NW-1).
template <int FN, int MTW, int NW = xm_waves(FN)>
__device__ __forceinline__ void xm_flush(const XmArgs& x, floatx4 (&acc)[FN][MTW],
                                         uint32_t strip, uint32_t* flag, float out_scale,
                                         bool owner = true) {
  constexpr uint32_t kSlotPairs = NW * MTW * FN * 2 * 64;  // float pairs per slot
  const GemmArgs& a = x.g;
  const uint32_t lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t M = a.m, TN = FN * 16, wg = wg_of(a);
  const uint32_t f = strip_first_wg(strip, x.bps, x.bpw), l = strip_last_wg(strip, x.bps, x.bpw);
  // waves whose rows all lie at or past M hold nothing to hand over
  const bool rows = owner && wave * MTW * 16 < M;
  auto store_y = [&](int fn, int mt, floatx4 v) __attribute__((always_inline)) {
    const uint32_t col = strip * TN + fn * 16 + (lane & 15);
    const uint32_t m0 = (wave * MTW + mt) * 16 + 4 * (lane >> 4);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (m0 + i < M) a.y[(size_t)(m0 + i) * a.y_row + col] = v[i] * out_scale;
  };
  auto pair_ptr = [&](uint32_t slot, int fn, int mt, int h) __attribute__((always_inline)) {
    return reinterpret_cast<uint64_t*>(a.part) + ((size_t)strip * a.slots + slot) * kSlotPairs +
           ((((wave * MTW + mt) * FN + fn) * 2 + h) * 64 + lane);
  };
  if (f == l) {
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
      for (int mt = 0; mt < MTW; ++mt) {
        if (rows) store_y(fn, mt, acc[fn][mt]);
        acc[fn][mt] = floatx4{0.f, 0.f, 0.f, 0.f};
      }
    return;
  }
#pragma unroll
  for (int fn = 0; fn < FN; ++fn)
#pragma unroll
    for (int mt = 0; mt < MTW; ++mt) {
      // agent-scope stores: coherent across XCDs without an L2 writeback
      if (rows) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint64_t bits = (uint64_t)__float_as_uint(acc[fn][mt][2 * h]) |
                                ((uint64_t)__float_as_uint(acc[fn][mt][2 * h + 1]) << 32);
          __hip_atomic_store(pair_ptr(wg - f, fn, mt, h), bits, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
        }
      }
      acc[fn][mt] = floatx4{0.f, 0.f, 0.f, 0.f};
    }
  // hand-off to the last workgroup of the strip, ordered as in reduce_and_store
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t old = __hip_atomic_fetch_add(&a.counters[strip], 1u, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
    *flag = (old == l - f) ? 1u : 0u;
  }
  __syncthreads();
  const bool last = *flag != 0;
  __syncthreads();  // flag is rewritten by the next flush
  if (!last || !rows) return;  // (wave 0 always has rows: it resets the counter)
  const uint32_t n = l - f + 1;
#pragma unroll
  for (int fn = 0; fn < FN; ++fn)
#pragma unroll
    for (int mt = 0; mt < MTW; ++mt) {
      floatx4 v = floatx4{0.f, 0.f, 0.f, 0.f};
      for (uint32_t g = 0; g < n; ++g) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint64_t bits =
              __hip_atomic_load(pair_ptr(g, fn, mt, h), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          v[2 * h] += __uint_as_float((uint32_t)bits);
          v[2 * h + 1] += __uint_as_float((uint32_t)(bits >> 32));
        }
      }
      store_y(fn, mt, v);
    }
  if (threadIdx.x == 0)
    __hip_atomic_store(&a.counters[strip], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// XS > 1: the waves of subsets 1..XS-1 hand their sums to the wave of subset
// 0 that owns the same row group, through the (idle) fragment buffers, BP
// row bands at a time; fixed order, so the result is deterministic.  Every
// wave ends with zeroed accumulators except the owners.
template <int FN, int XS, int G, int BP>
__device__ __forceinline__ void xm_subset_reduce(floatx4 (&acc)[FN][1], uint8_t* xbuf,
                                                 uint32_t wave, bool has_rows) {
  const uint32_t lane = lane_id(), sub = wave / G, rg = wave % G;
#pragma unroll
  for (int f0 = 0; f0 < FN; f0 += BP) {
    __syncthreads();  // the buffers' previous readers are done
    if (sub > 0 && has_rows) {
      floatx4* slot = reinterpret_cast<floatx4*>(xbuf) + ((sub - 1) * G + rg) * BP * 64 + lane;
#pragma unroll
      for (int b = 0; b < BP; ++b) slot[b * 64] = acc[f0 + b][0];
    }
    __syncthreads();
    if (sub == 0 && has_rows) {
#pragma unroll
      for (int s2 = 1; s2 < XS; ++s2) {
        const floatx4* slot =
            reinterpret_cast<const floatx4*>(xbuf) + ((s2 - 1) * G + rg) * BP * 64 + lane;
#pragma unroll
        for (int b = 0; b < BP; ++b) {
          const floatx4 v = slot[b * 64];
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[f0 + b][0][i] += v[i];
        }
      }
    }
  }
  __syncthreads();  // the buffers are free for the next batch
  if (sub > 0) {
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) acc[fn][0] = floatx4{0.f, 0.f, 0.f, 0.f};
  }
}

// R = 64 or 128 (one tile per chain) and tile_k = 64 only.  With two states
// per lane a wave publishes two operands per fragment (the tile's two row
// halves at the same k), multiplied into the two halves' accumulators.
// PP = false keeps one fragment buffer (a barrier after the products, before
// the next group is published): the rung without ping-pong of the ablation.
template <int FMT, int R, int FN, bool RING, bool PP = true, int XS = 1>
__global__ __launch_bounds__(64 * xm_waves(FN, XS)) void k_fused_xm(XmArgs x) {
  constexpr int NW = xm_waves(FN, XS), MTW = xm_row_blocks(FN, XS), ILP = xm_ilp(FN);
  constexpr int NT = NW * ILP;
  constexpr int NG = NW / XS;  // row groups (waves of one subset)
  constexpr int TJ = NT / XS;  // tiles a wave multiplies
  constexpr int NS = states_per_lane(R), FNH = FN / NS, NO = NT * NS;  // operands per fragment
  constexpr int NOW = TJ * NS;                                         // ... a wave multiplies
  constexpr int FPB = xm_fpb(R, FN, FMT, XS);
  static_assert(FNH % FPB == 0 && (NO * FPB) % 4 == 0, "fragment groups");
  static_assert(XS == 1 || (MTW == 1 && NS == 1 && ILP == 1 && NOW % (4 / FPB) == 0),
                "subsets: one row block per wave, one state per lane");
  // row bands per pass of the subset reduction: its slots fit the fragment buffers
  constexpr int BP = (XS - 1) * NG * 4 * 1024 <= 2 * FPB * NO * 1024   ? 4
                     : (XS - 1) * NG * 2 * 1024 <= 2 * FPB * NO * 1024 ? 2
                                                                      : 1;
  static_assert(FNH % 2 == 0, "fragment parity slots");
  constexpr uint32_t FW = 32, TK = 64, FK = TK / FW, G = FK * FNH;
  constexpr int SPF = steps_per_frag<FMT>();
  constexpr int ADV = ring_group_steps(R);
  extern __shared__ __align__(16) uint8_t smem[];
  const GemmArgs& a = x.g;
  const Layer& L = a.L;
  u32x2* lut = reinterpret_cast<u32x2*>(smem);
  uint32_t* cum = reinterpret_cast<uint32_t*>(smem + kLutBytes);
  uint16_t* words = reinterpret_cast<uint16_t*>(smem + tab_of<FMT>(a.L));
  uint8_t* xbuf = smem + x.xbuf_off;
  uint32_t* flag = reinterpret_cast<uint32_t*>(smem + x.xbuf_off - 16);
  const uint32_t lane = lane_id();
  const uint32_t wave = uniform(threadIdx.x >> 6);
  const uint32_t sub = wave / NG;  // subset: tiles [sub * TJ, (sub + 1) * TJ) of a batch
  const uint32_t row0 = (wave % NG) * MTW * 16;
  const bool has_rows = row0 < a.m;
  const uint32_t kgroups = L.k / 128;
  float out_scale = 1.f;
  if constexpr (FMT == FP8)
    out_scale = __hip_atomic_load(a.xscale, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) * a.w_scale;
  const uint32_t fq = table_issue<FMT>(L);
  const uint32_t b0 = wg_of(a) * x.bpw, b1 = min(b0 + x.bpw, x.batches);
  floatx4 acc[FN][MTW];
#pragma unroll
  for (int fn = 0; fn < FN; ++fn)
#pragma unroll
    for (int mt = 0; mt < MTW; ++mt) acc[fn][mt] = floatx4{0.f, 0.f, 0.f, 0.f};
  for (uint32_t b = b0; b < b1; ++b) {
    const uint32_t strip = b / x.bps, kt0 = (b % x.bps) * NT;
    // chain c of this wave decodes batch tile j = c * NW + wave
    uint32_t tj[ILP];
    Chain ch[ILP];
    Ring rg[ILP];
    uint32_t c0[ILP][4];
    Staged stg[ILP];
    uint32_t kq[ILP];  // payload step counts, loaded before the streams
#pragma unroll
    for (int c = 0; c < ILP; ++c) {
      tj[c] = strip * L.kt + kt0 + c * NW + wave;
      kq[c] = ktab_scalar(L.ktab, tj[c]);
      if constexpr (RING)
        ring_issue(L, tj[c], lane, rg[c], c0[c]);
      else
        stage_issue(L, tj[c], lane, 64u, stg[c]);
      ch[c].x = L.streams[L.index[tj[c]] + lane];
      ch[c].x2 = (R == 128) ? L.streams[L.index[tj[c]] + 64 + lane] : 0u;
    }
    if (b == b0) table_build<FMT>(fq, L, lut, cum);
#pragma unroll
    for (int c = 0; c < ILP; ++c) ch[c].lim = L.steps - kq[c];
    __syncthreads();  // LUT complete; the previous batch's fragment reads are done
    uint32_t lim_min = 0xFFFFFFFFu;
#pragma unroll
    for (int c = 0; c < ILP; ++c) {
      const uint32_t region = (wave * ILP + c) * L.region_words;
      const uint32_t base = tab_of<FMT>(a.L) + 2 * region;
      if constexpr (RING) {
        ring_start(rg[c], ch[c], smem, base, lane, c0[c]);
        ch[c].p0 = uniform(ch[c].p0); ch[c].s0 = uniform(ch[c].s0); ch[c].e0 = uniform(ch[c].e0);
        rg[c].cc = uniform(rg[c].cc);
        rg[c].nchunks = uniform(rg[c].nchunks);
      } else {
        const uint32_t n = uniform(stage_commit(stg[c], words, region, lane, 64u));
        ch[c].p0 = base; ch[c].s0 = base; ch[c].e0 = base + 2 * n;
        ch[c].p1 = base; ch[c].s1 = base; ch[c].e1 = base + 2 * n;
      }
      lim_min = min(lim_min, uniform(ch[c].lim));
    }
    auto load_raw = [&](int c, uint32_t g, int h) __attribute__((always_inline)) -> u32x2 {
      const uint8_t* rp = L.raw + (size_t)tj[c] * FN * 16 * TK + (size_t)g * 8 * R +
                          (64 * h + lane) * 8;
      return *reinterpret_cast<const u32x2*>(rp);
    };
    // the scale of the lane's row in band fng: a tile's 64 columns lie in one
    // 128-column group, so it is the lane's first-band index plus a uniform
    // band offset.  In the subset form the offset is added where the load is
    // issued (the empty asm keeps the compiler from computing and loading
    // every fragment's scale early and holding them all in registers, which
    // spilled the accumulators inside the decode loop); the 8-wave form has
    // the registers, and its early loads measured faster
    size_t sidx[ILP];
#pragma unroll
    for (int c = 0; c < ILP; ++c)
      sidx[c] = (size_t)(strip * L.tile_n + (lane & 15)) * kgroups +
                (kt0 + c * NW + wave) * TK / 128;
    auto load_scale = [&](int c, uint32_t g, int h) __attribute__((always_inline)) -> float {
      const uint32_t fkg = g / FNH, fng = g % FNH;
      if constexpr (XS > 1) {
        size_t i0 = sidx[c];
        asm volatile("" : "+v"(i0));
        const uint16_t sb = a.scales[i0 + (size_t)((h * FNH + fng) * 16) * kgroups];
        return __uint_as_float((uint32_t)sb << 16);
      } else {
        const uint32_t row = strip * L.tile_n + (h * FNH + fng) * 16 + (lane & 15);
        const uint32_t k0 = (kt0 + c * NW + wave) * TK + 8 * (lane >> 4) + fkg * FW;
        const uint16_t sb = a.scales[(size_t)row * kgroups + k0 / 128];
        return __uint_as_float((uint32_t)sb << 16);
      }
    };
    // raw bytes and scales of a fragment are loaded one fragment ahead (a
    // fragment's 8 steps then cover their latency), in the slot of the
    // fragment's parity (FNH is even, so the parity of g is that of fn)
    u32x2 rawq[2][ILP][NS];
    float scq[2][ILP][NS];
    auto prefetch = [&](uint32_t g, int slot) __attribute__((always_inline)) {
#pragma unroll
      for (int c = 0; c < ILP; ++c)
#pragma unroll
        for (int h = 0; h < NS; ++h) {
          rawq[slot][c][h] = u32x2{0u, 0u};
          scq[slot][c][h] = 0.f;
          if constexpr (has_raw_bytes<FMT>()) rawq[slot][c][h] = load_raw(c, g, h);
          if constexpr (FMT == INT4 || FMT == INT4P) scq[slot][c][h] = load_scale(c, g, h);
        }
    };
    prefetch(0, 0);
    // X rows of this wave; rows >= M repeat row M - 1 (their sums are never stored)
    const uint8_t* xp[MTW];
#pragma unroll
    for (int mt = 0; mt < MTW; ++mt) {
      const uint32_t row = row0 + mt * 16 + (lane & 15);
      xp[mt] = a.x + (size_t)min(row, a.m - 1) * a.x_row_bytes +
               ((size_t)kt0 * TK + 8 * (lane >> 4)) * 2;
    }
    for (uint32_t fk = 0; fk < FK; ++fk) {
      // X for this wave's rows and the k-ranges of its TJ tiles, column block fk
      u32x4 A[TJ][MTW];
      if (has_rows) {
#pragma unroll
        for (int j = 0; j < TJ; ++j)
#pragma unroll
          for (int mt = 0; mt < MTW; ++mt)
            A[j][mt] = *reinterpret_cast<const u32x4*>(xp[mt] + fk * FW * 2 +
                                                       (sub * TJ + j) * TK * 2);
      }
      // FPB fragments per barrier: each wave decodes and publishes them, then
      // every wave multiplies all of them (alternating accumulators, so
      // consecutive matrix operations do not wait for each other)
#pragma unroll
      for (int f0 = 0; f0 < FNH; f0 += FPB) {
        const uint32_t gq = (fk * FNH + f0) / FPB;
        uint8_t* buf = xbuf + (PP ? (gq & 1) : 0u) * (FPB * NO * 1024);
#pragma unroll
        for (int d = 0; d < FPB; ++d) {
        const int fn = f0 + d;
        const uint32_t g = fk * FNH + fn;
        const uint32_t s0 = g * SPF;
        // the next fragment's raw bytes and scales: issued after this
        // fragment's last ring advance (a chunk written to the ring waits for
        // the loads issued before it)
        constexpr int kPrefetchStep = RING ? ((SPF - 1) / ADV) * ADV : 0;
        const int cur = fn & 1;  // compile-time once the loops are unrolled
        const bool has_next = g + 1 < FK * FNH;
        FragAcc<FMT> e[ILP][NS];
        auto steps = [&](auto careful) __attribute__((always_inline)) {
#pragma unroll
          for (int i = 0; i < SPF; ++i) {
            if constexpr (RING) {
              if (i % ADV == 0) {
#pragma unroll
                for (int c = 0; c < ILP; ++c)
                  ring_advance(rg[c], smem, ch[c].s0, ch[c].p0, lane);
              }
            }
            if (i == kPrefetchStep && has_next) prefetch(g + 1, cur ^ 1);
            uint32_t sy[ILP][NS];
            step_all<R, decltype(careful)::value, ILP, RING, sym_mode<FMT>()>(ch, lut, smem, s0 + i, false, sy);
#pragma unroll
            for (int c = 0; c < ILP; ++c)
#pragma unroll
              for (int h = 0; h < NS; ++h) e[c][h].put(i, sy[c][h]);
          }
        };
        // payload steps (at most the last kPayloadMax) fall in the last fragments
        if (fn < FNH - (int)(kPayloadMax / SPF) || s0 + SPF - 1 < lim_min)
          steps(BoolC<false>{});
        else
          steps(BoolC<true>{});
        // operand o = j * NS + h of fragment d: batch tile j = c * NW + wave, row half h
#pragma unroll
        for (int c = 0; c < ILP; ++c)
#pragma unroll
          for (int h = 0; h < NS; ++h) {
            const BOp bop = finish_b<FMT>(e[c][h].q, rawq[cur][c][h], scq[cur][c][h],
                                          -8.f * scq[cur][c][h]);
            *reinterpret_cast<u32x4*>(buf + (d * NO + (c * NW + wave) * NS + h) * 1024 +
                                      lane * 16) = bop.v;
          }
        }
        __syncthreads();
        if (has_rows) {
          // operands are read kXB at a time so their LDS latencies overlap;
          // this wave's operands are o = sub * NOW + (0 .. NOW - 1)
          constexpr int kXB = 4;
          const uint8_t* bufw = buf + sub * NOW * 1024 + lane * 16;
#pragma unroll
          for (int o0 = 0; o0 < NOW; o0 += kXB / FPB) {
            BOp bq[kXB];
#pragma unroll
            for (int q = 0; q < kXB; ++q) {
              const int d = q % FPB, o = o0 + q / FPB;
              bq[q].v = *reinterpret_cast<const u32x4*>(bufw + (d * NO + o) * 1024);
            }
#pragma unroll
            for (int q = 0; q < kXB; ++q) {
              const int d = q % FPB, o = o0 + q / FPB, h = o % NS, ai = h * FNH + f0 + d;
#pragma unroll
              for (int mt = 0; mt < MTW; ++mt)
                acc[ai][mt] = mfma<FMT>(A[o / NS][mt], bq[q], acc[ai][mt]);
            }
          }
          // keep each group of reads ahead of its products
#pragma unroll
          for (int o0 = 0; o0 < NOW; o0 += kXB / FPB) {
            __builtin_amdgcn_sched_group_barrier(0x100, kXB, 0);        // LDS reads
            __builtin_amdgcn_sched_group_barrier(0x008, kXB * MTW, 0);  // MFMA
          }
        }
        if constexpr (!PP) __syncthreads();  // one buffer: every read done before the next publish
      }
    }
    if (a.status) {
#pragma unroll
      for (int c = 0; c < ILP; ++c) {
        const uint32_t fl = final_flags<R, RING>(ch[c], L.steps, false);
        if (lane == 0) a.status[tj[c]] = (int32_t)fl;
      }
    }
    if (b + 1 == b1 || (b + 1) / x.bps != strip) {
      if constexpr (XS > 1) {
        xm_subset_reduce<FN, XS, NG, BP>(acc, xbuf, wave, has_rows);
        xm_flush<FN, MTW, NG>(x, acc, strip, flag, out_scale, sub == 0);
      } else {
        xm_flush<FN, MTW>(x, acc, strip, flag, out_scale);
      }
    }
  }
}

// --------------------------------------------------------------- decode only
struct DecodeArgs {
  Layer L;
  const uint32_t* ids;  // tile ids or null (all)
  uint32_t n_ids;
  uint8_t* out;         // [N, K] of u8 or u16
  int32_t* status;
  uint32_t waves;
};

template <int FMT, int R, int ILP, bool RING>
__global__ __launch_bounds__(1024) void k_decode(DecodeArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  u32x2* lut = reinterpret_cast<u32x2*>(smem);
  uint32_t* cum = reinterpret_cast<uint32_t*>(smem + kLutBytes);
  uint16_t* words = reinterpret_cast<uint16_t*>(smem + tab_of<FMT>(a.L));
  const Layer& L = a.L;
  constexpr uint32_t TPC = R == 32 ? 2 : 1;
  constexpr int NS = states_per_lane(R);
  constexpr int ADV = ring_group_steps(R);
  const uint32_t lane = lane_id();
  const uint32_t wave = uniform(threadIdx.x >> 6);
  const bool upper = lane >= 32;
  const uint32_t half_lane = lane & 31;
  const uint32_t first = uniform((blockIdx.x * a.waves + wave) * ILP * TPC);
  const bool active = first < a.n_ids;

  Chain ch[ILP];
  uint32_t tile_lane[ILP];
  bool id_ok[ILP];  // the lane's tile id names a tile of the layer
  Staged stg[ILP];  // whole streams
  Ring rg[ILP];     // ring
  uint32_t c0[ILP][4];
  const uint32_t region0 = wave * ILP * TPC * L.region_words;
  const uint32_t fq = table_issue<FMT>(L);
  // every wave issues the same loads (an idle wave repeats the last id) so
  // the LUT build waits for the table alone
#pragma unroll
  for (int c = 0; c < ILP; ++c) {
    // slots past the end repeat the last id (same tile decoded twice, same output)
    const uint32_t ia = min(first + c * TPC, a.n_ids - 1);
    const uint32_t ib = min(first + c * TPC + 1, a.n_ids - 1);
    const uint32_t ta = a.ids ? a.ids[ia] : ia;
    const uint32_t tb = (R == 32) ? (a.ids ? a.ids[ib] : ib) : ta;
    const uint32_t t_id = (R == 32 && upper) ? tb : ta;
    // an id past the layer decodes tile 0 in its place and writes nothing
    id_ok[c] = t_id < L.tiles;
    const uint32_t t_l = id_ok[c] ? t_id : 0u;
    tile_lane[c] = t_l;
    if constexpr (RING)
      ring_issue(L, t_l, lane, rg[c], c0[c]);
    else
      stage_issue(L, t_l, R != 32 ? lane : half_lane, R != 32 ? 64u : 32u, stg[c]);
    ch[c].x = L.streams[L.index[t_l] + (R == 32 ? half_lane : lane)];
    ch[c].x2 = (R == 128) ? L.streams[L.index[t_l] + 64 + lane] : 0u;
  }
  table_build<FMT>(fq, L, lut, cum);
  // the payload counts are read after the LUT build (read before the
  // streams they slowed this kernel down, 66 -> 76 us on the bf16 MLP layer)
#pragma unroll
  for (int c = 0; c < ILP; ++c) ch[c].lim = L.steps - (uint32_t)L.ktab[tile_lane[c]];
  __syncthreads();  // LUT complete; each wave's staged stream is private to it
  if (!active) return;
#pragma unroll
  for (int c = 0; c < ILP; ++c) {
    const uint32_t ra = region0 + c * TPC * L.region_words;
    if constexpr (RING) {
      ring_start(rg[c], ch[c], smem, tab_of<FMT>(a.L) + 2 * ra, lane, c0[c]);
      ch[c].p0 = uniform(ch[c].p0); ch[c].s0 = uniform(ch[c].s0); ch[c].e0 = uniform(ch[c].e0);
      rg[c].cc = uniform(rg[c].cc);
      rg[c].nchunks = uniform(rg[c].nchunks);
    } else {
      const uint32_t rb = (R == 32) ? ra + L.region_words : ra;
      const uint32_t mine = stage_commit(stg[c], words, (R == 32 && upper) ? rb : ra,
                                         R != 32 ? lane : half_lane, R != 32 ? 64u : 32u);
      const uint32_t na = uniform(mine);
      const uint32_t nb = (R == 32) ? (uint32_t)__builtin_amdgcn_readlane((int)mine, 32) : na;
      const uint32_t ba = tab_of<FMT>(a.L) + 2 * ra, bb = tab_of<FMT>(a.L) + 2 * rb;
      ch[c].p0 = ba; ch[c].s0 = ba; ch[c].e0 = ba + 2 * na;
      ch[c].p1 = bb; ch[c].s1 = bb; ch[c].e1 = bb + 2 * nb;
    }
  }
  uint32_t lim_min = L.steps;
#pragma unroll
  for (int c = 0; c < ILP; ++c) {
    lim_min = min(lim_min, uniform(ch[c].lim));
    if (R == 32) lim_min = min(lim_min, (uint32_t)__builtin_amdgcn_readlane((int)ch[c].lim, 32));
  }
  constexpr int SPF = steps_per_frag<FMT>();
  constexpr uint32_t FW = (R == 128 ? 64 : R) / 2;  // fragment width (columns)
  const uint32_t FNH = L.tile_n / 16 / NS;            // row bands per state
  const uint32_t G = L.steps / SPF;
  const uint32_t p = lane % R;
  auto steps = [&](uint32_t s0, auto careful, uint32_t (&e)[ILP][NS][SPF]) {
#pragma unroll
    for (int i = 0; i < SPF; ++i) {
      if constexpr (RING) {
        if (i % ADV == 0) {
#pragma unroll
          for (int c = 0; c < ILP; ++c) ring_advance(rg[c], smem, ch[c].s0, ch[c].p0, lane);
        }
      }
      uint32_t sy[ILP][NS];
      step_all<R, decltype(careful)::value, ILP, RING, sym_mode<FMT>()>(ch, lut, smem, s0 + i, upper, sy);
#pragma unroll
      for (int c = 0; c < ILP; ++c)
#pragma unroll
        for (int h = 0; h < NS; ++h) e[c][h][i] = sy[c][h];
    }
  };
  for (uint32_t g = 0; g < G; ++g) {
    const uint32_t s0 = g * SPF;
    uint32_t e[ILP][NS][SPF];
    if (s0 + SPF - 1 < lim_min)
      steps(s0, BoolC<false>{}, e);
    else
      steps(s0, BoolC<true>{}, e);
    const uint32_t fk = g / FNH, fn = g % FNH;
#pragma unroll
    for (int c = 0; c < ILP; ++c)
#pragma unroll
      for (int h = 0; h < NS; ++h) {
        if (!id_ok[c]) continue;
        const uint32_t t = tile_lane[c];
        const uint32_t row = (t / L.kt) * L.tile_n + (h * FNH + fn) * 16 + (p & 15);
        const uint32_t col = (t % L.kt) * L.tile_k + fk * FW + 8 * (p >> 4);
        if constexpr (FMT == BF16W) {
          const BOp b = make_b<FMT>(e[c][h], u32x2{0u, 0u}, 0.f, 0.f);
          *reinterpret_cast<u32x4*>(a.out + ((size_t)row * L.k + col) * 2) = b.v;
        } else if constexpr (has_raw_bytes<FMT>()) {
          const uint8_t* rp = L.raw + (size_t)t * L.tile_n * L.tile_k + (size_t)g * 8 * R +
                              (64 * h + p) * 8;
          const u32x2 raw = *reinterpret_cast<const u32x2*>(rp);
          const BOp b = make_b<FMT>(e[c][h], raw, 0.f, 0.f);
          *reinterpret_cast<u32x4*>(a.out + ((size_t)row * L.k + col) * 2) = b.v;
        } else if constexpr (FMT == INT4P) {
          // symbol i -> code bytes 2i (low nibble) and 2i+1 (high nibble)
          uint32_t q[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t sy = e[c][h][i] >> 24;
            q[i] = (sy & 0x0Fu) | ((sy & 0xF0u) << 4);
          }
          u32x2 v;
          v.x = q[0] | (q[1] << 16);
          v.y = q[2] | (q[3] << 16);
          *reinterpret_cast<u32x2*>(a.out + (size_t)row * L.k + col) = v;
        } else {
          const uint32_t(&ec)[SPF] = e[c][h];
          u32x2 v;
          v.x = pack_hi_bytes(ec[1], ec[0]) | (pack_hi_bytes(ec[3], ec[2]) << 16);
          v.y = pack_hi_bytes(ec[5], ec[4]) | (pack_hi_bytes(ec[7], ec[6]) << 16);
          *reinterpret_cast<u32x2*>(a.out + (size_t)row * L.k + col) = v;
        }
      }
  }
  if (a.status) {
#pragma unroll
    for (int c = 0; c < ILP; ++c) {
      const uint32_t f = final_flags<R, RING>(ch[c], L.steps, upper);
      if ((R != 32 ? lane == 0 : half_lane == 0) && id_ok[c]) a.status[tile_lane[c]] = (int32_t)f;
    }
  }
}

// -------------------------------------------------------------- dense GEMM
// Same strip / wave decomposition and reduction as k_fused, W read from HBM
// in the layout dgt_decode_tiles writes (row-major [N, K] elements).
struct DenseArgs {
  GemmArgs g;
  const uint8_t* w;
  uint32_t n, k, kt;   // kt: 64-column k-tiles per strip
};

template <int FMT, int FN, int MT>
__global__ __launch_bounds__(dense_max_threads(FN, MT)) void k_dense(DenseArgs d) {
  extern __shared__ __align__(16) uint8_t smem[];
  const GemmArgs& a = d.g;
  const uint32_t lane = lane_id();
  const uint32_t wave = uniform(threadIdx.x >> 6);
  const uint32_t unit = uniform(blockIdx.x * a.cpw + wave);
  const bool active = wave < a.cpw && unit < a.chains;
  const uint32_t strip = active ? unit / a.cps : 0u;
  const uint32_t kt_first = active ? (unit % a.cps) * a.tpw : d.kt;
  floatx4 acc[FN][MT];
#pragma unroll
  for (int fn = 0; fn < FN; ++fn)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[fn][mt] = floatx4{0.f, 0.f, 0.f, 0.f};
  const uint32_t kgroups = d.k / 128;
  for (uint32_t kt = kt_first; kt < min(kt_first + a.tpw, d.kt); ++kt) {
#pragma unroll
    for (uint32_t fk = 0; fk < 2; ++fk) {
      const uint32_t k0 = kt * 64 + fk * 32 + 8 * (lane >> 4);
      u32x4 A[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) A[mt] = load_a<FMT>(a, mt * 16 + (lane & 15), k0);
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        const uint32_t row = strip * FN * 16 + fn * 16 + (lane & 15);
        BOp b;
        if constexpr (FMT == BF16) {
          b.v = *reinterpret_cast<const u32x4*>(d.w + ((size_t)row * d.k + k0) * 2);
        } else {
          const u32x2 v = *reinterpret_cast<const u32x2*>(d.w + (size_t)row * d.k + k0);
          uint32_t e[8];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            e[i] = v.x << (24 - 8 * i);
            e[4 + i] = v.y << (24 - 8 * i);
          }
          float sc = 0.f, nsc8 = 0.f;
          if constexpr (FMT == INT4) {
            sc = __uint_as_float((uint32_t)a.scales[(size_t)row * kgroups + k0 / 128] << 16);
            nsc8 = -8.f * sc;
          }
          b = make_b<FMT>(e, u32x2{0u, 0u}, sc, nsc8);
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[fn][mt] = mfma<FMT>(A[mt], b, acc[fn][mt]);
      }
    }
  }
  float out_scale = 1.f;
  if constexpr (FMT == FP8)
    out_scale = __hip_atomic_load(a.xscale, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) * a.w_scale;
  reduce_and_store<FN, MT>(a, acc, reinterpret_cast<float*>(smem), out_scale);
}

// ------------------------------------------- dense GEMM, LDS-tiled (large M)
// The uncompressed baseline at larger M: a plain tiled GEMM that reads each
// BN x 64 block of W once per 128 rows of X.  Workgroups of 4 waves compute
// 128 x BN blocks of Y (each wave a 64 x BN/2 quarter of 16 x 16 MFMA tiles);
// k advances 64 at a time through two LDS stages of X and W (bf16, rows
// padded to 144 bytes so the 16 rows an operand read touches fall in distinct
// banks), the next stage's global loads in flight while the current one is
// multiplied.  Byte formats are widened to bf16 as they enter LDS, with the
// fused path's own conversion (the same values).  Blocks are numbered
// XCD-major (xcd_tile), so the row blocks that read one W block share an L2.
struct DenseTiledArgs {
  const uint8_t* w;
  const uint8_t* x;          // bf16 rows of x_row_bytes (fp8: the quantised X)
  const uint16_t* scales;    // INT4: bf16 [N, K / 128]
  const float* xscale;       // FP8: activation scale on the device
  float w_scale;
  float* y;                  // fp32 [M, N]
  uint32_t m, n, k, x_row_bytes;
  uint32_t nmb, nnb;         // 128-row blocks of M, BN-row blocks of N
};
constexpr uint32_t kDtRows = 128, kDtPitch = 144;
__host__ __device__ constexpr uint32_t dense_tiled_lds(int BN) {
  return 2 * (kDtRows + BN) * kDtPitch;  // two stages of X block then W block
}

template <int FMT, int BN>
__global__ __launch_bounds__(256) void k_dense_tiled(DenseTiledArgs d) {
  constexpr int NB = BN / 32;  // W chunks per thread and 16-column blocks per wave
  constexpr uint32_t kStage = (kDtRows + BN) * kDtPitch;
  extern __shared__ __align__(16) uint8_t smem[];
  const uint32_t tid = threadIdx.x, lane = tid & 63u;
  const uint32_t wave = uniform(tid >> 6), wm = wave & 1u, wn = wave >> 1;
  const uint32_t tile = xcd_tile(blockIdx.x, d.nmb * d.nnb);
  const uint32_t m0 = (tile % d.nmb) * kDtRows, n0 = (tile / d.nmb) * BN;
  const uint32_t kgroups = d.k / 128, kt_end = d.k / 64;
  // global chunks of this thread: c = tid + 256 i -> row c / 8, elements 8 (c % 8) ..
  constexpr bool WIDE = FMT == BF16;
  u32x4 ra[4], rb[NB];
  u32x2 rbb[NB];
  float sc[NB];
  auto gload = [&](uint32_t kt) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t c = tid + 256u * i, row = c >> 3, kk = kt * 64u + (c & 7u) * 8u;
      ra[i] = u32x4{0u, 0u, 0u, 0u};
      if (m0 + row < d.m)
        ra[i] = *reinterpret_cast<const u32x4*>(d.x + (size_t)(m0 + row) * d.x_row_bytes + kk * 2);
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const uint32_t c = tid + 256u * i, row = c >> 3, kk = kt * 64u + (c & 7u) * 8u;
      const size_t wr = (size_t)(n0 + row) * d.k + kk;
      if constexpr (WIDE) {
        rb[i] = *reinterpret_cast<const u32x4*>(d.w + wr * 2);
      } else {
        rbb[i] = *reinterpret_cast<const u32x2*>(d.w + wr);
        sc[i] = 0.f;
        if constexpr (FMT == INT4)
          sc[i] = __uint_as_float((uint32_t)d.scales[(size_t)(n0 + row) * kgroups + kk / 128] << 16);
      }
    }
  };
  auto lstore = [&](uint32_t stage) __attribute__((always_inline)) {
    uint8_t* xs = smem + stage * kStage;
    uint8_t* ws = xs + kDtRows * kDtPitch;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t c = tid + 256u * i;
      *reinterpret_cast<u32x4*>(xs + (c >> 3) * kDtPitch + (c & 7u) * 16u) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const uint32_t c = tid + 256u * i, off = (c >> 3) * kDtPitch + (c & 7u) * 16u;
      if constexpr (WIDE) {
        *reinterpret_cast<u32x4*>(ws + off) = rb[i];
      } else {
        uint32_t e[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          e[j] = rbb[i].x << (24 - 8 * j);
          e[4 + j] = rbb[i].y << (24 - 8 * j);
        }
        *reinterpret_cast<u32x4*>(ws + off) = make_b<FMT>(e, u32x2{0u, 0u}, sc[i], -8.f * sc[i]).v;
      }
    }
  };
  floatx4 acc[NB][4];
#pragma unroll
  for (int fn = 0; fn < NB; ++fn)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) acc[fn][mt] = floatx4{0.f, 0.f, 0.f, 0.f};
  const uint32_t lrow = (lane & 15u) * kDtPitch, lk = (lane >> 4) * 16u;
  gload(0);
  lstore(0);
  __syncthreads();
  for (uint32_t kt = 0; kt < kt_end; ++kt) {
    const bool more = kt + 1 < kt_end;
    if (more) gload(kt + 1);
    const uint8_t* xs = smem + (kt & 1u) * kStage;
    const uint8_t* ws = xs + kDtRows * kDtPitch;
#pragma unroll
    for (uint32_t ks = 0; ks < 2; ++ks) {
      u32x4 A[4];
      BOp B[NB];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        A[mt] = *reinterpret_cast<const u32x4*>(xs + (wm * 64u + mt * 16u) * kDtPitch + lrow +
                                                ks * 64u + lk);
#pragma unroll
      for (int fn = 0; fn < NB; ++fn)
        B[fn].v = *reinterpret_cast<const u32x4*>(ws + (wn * (BN / 2) + fn * 16u) * kDtPitch +
                                                  lrow + ks * 64u + lk);
#pragma unroll
      for (int fn = 0; fn < NB; ++fn)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) acc[fn][mt] = mfma<FMT>(A[mt], B[fn], acc[fn][mt]);
    }
    // the other stage was last read before the previous barrier
    if (more) lstore((kt + 1) & 1u);
    __syncthreads();
  }
  float out_scale = 1.f;
  if constexpr (FMT == FP8)
    out_scale = __hip_atomic_load(d.xscale, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) * d.w_scale;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint32_t row = m0 + wm * 64u + mt * 16u + 4u * (lane >> 4) + r;
      if (row < d.m) {
#pragma unroll
        for (int fn = 0; fn < NB; ++fn)
          d.y[(size_t)row * d.n + n0 + wn * (BN / 2) + fn * 16u + (lane & 15u)] =
              acc[fn][mt][r] * out_scale;
      }
    }
}

// ------------------------------------------------- dense GEMV (M = 1)
// One row of X against W streamed once: X in LDS, each wave takes kGvRows
// rows of W, every lane 8 consecutive k per load (16 bytes of bf16, 8 of the
// byte formats), the next loads in flight while the current ones are summed
// in fp32; one wave reduction per row.  Byte formats are widened to bf16
// with the fused path's conversion, then to fp32.
struct GemvArgs {
  const uint8_t* w;
  const uint16_t* x;
  const uint16_t* scales;
  const float* xscale;
  float w_scale;
  float* y;
  uint32_t n, k;
};
constexpr uint32_t kGvRows = 4, kGvWaves = 8;

template <int FMT>
__global__ __launch_bounds__(64 * kGvWaves) void k_gemv(GemvArgs g) {
  extern __shared__ __align__(16) uint8_t smem[];
  uint16_t* xs = reinterpret_cast<uint16_t*>(smem);
  const uint32_t tid = threadIdx.x, lane = tid & 63u, wave = uniform(tid >> 6);
  for (uint32_t i = tid; i < g.k / 8; i += blockDim.x)
    reinterpret_cast<u32x4*>(xs)[i] = reinterpret_cast<const u32x4*>(g.x)[i];
  __syncthreads();
  const uint32_t r0 = (blockIdx.x * kGvWaves + wave) * kGvRows;
  if (r0 >= g.n) return;
  const uint32_t kgroups = g.k / 128;
  constexpr bool WIDE = FMT == BF16;
  float sum[kGvRows];
#pragma unroll
  for (uint32_t r = 0; r < kGvRows; ++r) sum[r] = 0.f;
  auto widen = [&](uint32_t row, uint32_t kk, u32x4 wv, u32x2 wb) __attribute__((always_inline)) -> u32x4 {
    if constexpr (WIDE) {
      return wv;
    } else {
      float s = 0.f;
      if constexpr (FMT == INT4)
        s = __uint_as_float((uint32_t)g.scales[(size_t)row * kgroups + kk / 128] << 16);
      uint32_t e[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        e[j] = wb.x << (24 - 8 * j);
        e[4 + j] = wb.y << (24 - 8 * j);
      }
      return make_b<FMT>(e, u32x2{0u, 0u}, s, -8.f * s).v;
    }
  };
  auto dot8 = [&](u32x4 wv, u32x4 xv, float acc) __attribute__((always_inline)) -> float {
    const uint32_t wq[4] = {wv.x, wv.y, wv.z, wv.w}, xq[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc = __builtin_fmaf(__uint_as_float(wq[j] << 16), __uint_as_float(xq[j] << 16), acc);
      acc = __builtin_fmaf(__uint_as_float(wq[j] & 0xFFFF0000u), __uint_as_float(xq[j] & 0xFFFF0000u), acc);
    }
    return acc;
  };
  // 4 chunks of 512 k per row in flight
  constexpr uint32_t U = 4;
  for (uint32_t k0 = 0; k0 < g.k; k0 += 512u * U) {
    u32x4 wv[kGvRows][U];
    u32x2 wb[kGvRows][U];
#pragma unroll
    for (uint32_t r = 0; r < kGvRows; ++r)
#pragma unroll
      for (uint32_t u = 0; u < U; ++u) {
        const uint32_t kk = k0 + u * 512u + lane * 8u;
        const uint32_t row = min(r0 + r, g.n - 1u);
        wv[r][u] = u32x4{0u, 0u, 0u, 0u};
        wb[r][u] = u32x2{0u, 0u};
        if (kk < g.k) {
          if constexpr (WIDE)
            wv[r][u] = *reinterpret_cast<const u32x4*>(g.w + ((size_t)row * g.k + kk) * 2);
          else
            wb[r][u] = *reinterpret_cast<const u32x2*>(g.w + (size_t)row * g.k + kk);
        }
      }
#pragma unroll
    for (uint32_t u = 0; u < U; ++u) {
      const uint32_t kk = k0 + u * 512u + lane * 8u;
      if (kk < g.k) {
        const u32x4 xv = *reinterpret_cast<const u32x4*>(xs + kk);
#pragma unroll
        for (uint32_t r = 0; r < kGvRows; ++r)
          sum[r] = dot8(widen(min(r0 + r, g.n - 1u), kk, wv[r][u], wb[r][u]), xv, sum[r]);
      }
    }
  }
  float out_scale = 1.f;
  if constexpr (FMT == FP8)
    out_scale = __hip_atomic_load(g.xscale, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) * g.w_scale;
#pragma unroll
  for (uint32_t r = 0; r < kGvRows; ++r) {
    float v = sum[r];
#pragma unroll
    for (uint32_t o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    if (lane == 0 && r0 + r < g.n) g.y[r0 + r] = v * out_scale;
  }
}

}  // namespace dev
}  // namespace dgt
