// Instantiates the kernels of one weight format (compiled once per format with
// -DDGT_FMT=<dgt_format>) so the formats build in parallel.
#include "../../include/dgt.h"
#include "dgt_launch.h"

#ifndef DGT_FMT
#error "DGT_FMT must be defined"
#endif

namespace dgt {
namespace dev {
namespace {

template <typename K>
bool set_lds(K kernel, uint32_t bytes) {
  if (bytes <= 64 * 1024) return true;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes) ==
         hipSuccess;
}

template <int R, int FN, int MT, bool MIX, bool RING>
int fused_t(const GemmArgs& a, uint32_t grid, uint32_t threads, uint32_t lds, hipStream_t st) {
  auto k = k_fused<DGT_FMT, R, FN, MT, MIX, RING>;
  if (!set_lds(k, lds)) return DGT_E_HIP;
  hipLaunchKernelGGL(k, dim3(grid), dim3(threads), lds, st, a);
  return hipGetLastError() == hipSuccess ? DGT_OK : DGT_E_HIP;
}

template <int R, int FN, bool RING>
int fused_r(const GemmArgs& a, uint32_t mt, bool mix, uint32_t grid, uint32_t threads,
            uint32_t lds, hipStream_t st) {
  if (mt == 0 && !mix) return fused_t<R, FN, 0, false, RING>(a, grid, threads, lds, st);
  if (mt == 0 && mix) return fused_t<R, FN, 0, true, RING>(a, grid, threads, lds, st);
  if (mt == 1 && !mix) return fused_t<R, FN, 1, false, RING>(a, grid, threads, lds, st);
  if (mt == 1 && mix) return fused_t<R, FN, 1, true, RING>(a, grid, threads, lds, st);
  if constexpr (R == 64) {  // up to 4 or 8 rows packed: 64 lanes
    if (mt == kPacked4 && !mix) return fused_t<R, FN, kPacked4, false, RING>(a, grid, threads, lds, st);
    if (mt == kPacked4 && mix) return fused_t<R, FN, kPacked4, true, RING>(a, grid, threads, lds, st);
    if (mt == kPacked8 && !mix) return fused_t<R, FN, kPacked8, false, RING>(a, grid, threads, lds, st);
    if (mt == kPacked8 && mix) return fused_t<R, FN, kPacked8, true, RING>(a, grid, threads, lds, st);
  }
  if constexpr (FN <= 8) {
    if (mt == 4 && !mix) return fused_t<R, FN, 4, false, RING>(a, grid, threads, lds, st);
    if (mt == 4 && mix) return fused_t<R, FN, 4, true, RING>(a, grid, threads, lds, st);
  }
  return DGT_E_UNSUPPORTED;
}

template <int R, int FN, int MT, bool MIX>
int rounds_t(const GemmArgs& a, uint32_t grid, uint32_t threads, uint32_t lds, hipStream_t st,
             int* blocks_per_cu) {
  auto k = k_fused_rounds<DGT_FMT, R, FN, MT, MIX>;
  if (!set_lds(k, lds)) return DGT_E_HIP;
  if (blocks_per_cu) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void*>(k),
                                                     (int)threads, lds) != hipSuccess)
      return DGT_E_HIP;
    *blocks_per_cu = n;
    return DGT_OK;
  }
  hipLaunchKernelGGL(k, dim3(grid), dim3(threads), lds, st, a);
  return hipGetLastError() == hipSuccess ? DGT_OK : DGT_E_HIP;
}

}  // namespace

// Ring staging exists for R = 64 and 128 (one tile per chain).
template <>
int launch_fused<DGT_FMT>(const GemmArgs& a, uint32_t lanes, uint32_t fn, uint32_t mt, bool mix,
                          bool ring, uint32_t grid, uint32_t threads, uint32_t lds,
                          hipStream_t st) {
#define DGT_FUSED_CASE(RR, FNV)                                                      \
  if (lanes == RR && fn == FNV)                                                      \
    return ring ? fused_r<RR, FNV, true>(a, mt, mix, grid, threads, lds, st)         \
                : fused_r<RR, FNV, false>(a, mt, mix, grid, threads, lds, st);
  DGT_FUSED_CASE(64, 8)
  DGT_FUSED_CASE(64, 16)
  if constexpr (DGT_FMT != BF16W) {  // whole bf16 words: 64 lanes only
    DGT_FUSED_CASE(128, 8)
    DGT_FUSED_CASE(128, 16)
    if (ring) return DGT_E_UNSUPPORTED;
    if (lanes == 32 && fn == 8) return fused_r<32, 8, false>(a, mt, mix, grid, threads, lds, st);
    if (lanes == 32 && fn == 16) return fused_r<32, 16, false>(a, mt, mix, grid, threads, lds, st);
  }
#undef DGT_FUSED_CASE
  return DGT_E_UNSUPPORTED;
}

// Multi-round register path (ring staging, one 16-row block of X, or the
// single-row mode mt = 0): launches, or with blocks_per_cu set only reports
// how many workgroups a CU holds at once.
template <>
int launch_fused_rounds<DGT_FMT>(const GemmArgs& a, uint32_t lanes, uint32_t fn, uint32_t mt,
                                 bool mix, uint32_t grid, uint32_t threads, uint32_t lds,
                                 hipStream_t st, int* blocks_per_cu) {
#define DGT_ROUNDS_CASE(RR, FNV)                                                              \
  if (lanes == RR && fn == FNV && mt == 0)                                                    \
    return mix ? rounds_t<RR, FNV, 0, true>(a, grid, threads, lds, st, blocks_per_cu)         \
               : rounds_t<RR, FNV, 0, false>(a, grid, threads, lds, st, blocks_per_cu);       \
  if (lanes == RR && fn == FNV && mt == 1)                                                    \
    return mix ? rounds_t<RR, FNV, 1, true>(a, grid, threads, lds, st, blocks_per_cu)         \
               : rounds_t<RR, FNV, 1, false>(a, grid, threads, lds, st, blocks_per_cu);
  DGT_ROUNDS_CASE(64, 8)
  DGT_ROUNDS_CASE(64, 16)
  // up to 4 or 8 rows packed (64 lanes)
#define DGT_PACKED_CASE(FNV, MTV)                                                             \
  if (lanes == 64 && fn == FNV && mt == MTV)                                                  \
    return mix ? rounds_t<64, FNV, MTV, true>(a, grid, threads, lds, st, blocks_per_cu)       \
               : rounds_t<64, FNV, MTV, false>(a, grid, threads, lds, st, blocks_per_cu);
  DGT_PACKED_CASE(8, kPacked4)
  DGT_PACKED_CASE(16, kPacked4)
  DGT_PACKED_CASE(8, kPacked8)
  DGT_PACKED_CASE(16, kPacked8)
#undef DGT_PACKED_CASE
  if constexpr (DGT_FMT != BF16W) {
    DGT_ROUNDS_CASE(128, 8)
    DGT_ROUNDS_CASE(128, 16)
  }
#undef DGT_ROUNDS_CASE
  return DGT_E_UNSUPPORTED;
}

// pingpong = false: one fragment buffer (ablation; 64 lanes only).
// xs > 1: the 16-wave subset kernel (256-row tiles, 64 lanes, M <= 256 / xs).
template <>
int launch_fused_xm<DGT_FMT>(const XmArgs& x, uint32_t lanes, uint32_t fn, bool ring,
                             bool pingpong, uint32_t xs, uint32_t grid, uint32_t lds,
                             hipStream_t st) {
#define DGT_XM_CASE(RR, FNV, RG, PPV)                                           \
  if (lanes == RR && fn == FNV && ring == RG && pingpong == PPV && xs == 1) {   \
    auto k = k_fused_xm<DGT_FMT, RR, FNV, RG, PPV>;                             \
    if (!set_lds(k, lds)) return DGT_E_HIP;                                     \
    hipLaunchKernelGGL(k, dim3(grid), dim3(64 * xm_waves(FNV)), lds, st, x);    \
    return hipGetLastError() == hipSuccess ? DGT_OK : DGT_E_HIP;                \
  }
#define DGT_XS_CASE(RG, XSV)                                                    \
  if (lanes == 64 && fn == 16 && ring == RG && pingpong && xs == XSV) {         \
    auto k = k_fused_xm<DGT_FMT, 64, 16, RG, true, XSV>;                        \
    if (!set_lds(k, lds)) return DGT_E_HIP;                                     \
    hipLaunchKernelGGL(k, dim3(grid), dim3(64 * xm_waves(16, XSV)), lds, st, x); \
    return hipGetLastError() == hipSuccess ? DGT_OK : DGT_E_HIP;                \
  }
  DGT_XS_CASE(false, 2)
  DGT_XS_CASE(true, 2)
  DGT_XS_CASE(false, 4)
  DGT_XS_CASE(true, 4)
#undef DGT_XS_CASE
  DGT_XM_CASE(64, 8, false, true)
  DGT_XM_CASE(64, 8, true, true)
  DGT_XM_CASE(64, 16, false, true)
  DGT_XM_CASE(64, 16, true, true)
  DGT_XM_CASE(64, 8, false, false)
  DGT_XM_CASE(64, 8, true, false)
  DGT_XM_CASE(64, 16, false, false)
  DGT_XM_CASE(64, 16, true, false)
  if constexpr (DGT_FMT != BF16W) {  // whole bf16 words: 64 lanes only
    DGT_XM_CASE(128, 8, false, true)
    DGT_XM_CASE(128, 8, true, true)
    DGT_XM_CASE(128, 16, false, true)
    DGT_XM_CASE(128, 16, true, true)
  }
#undef DGT_XM_CASE
  return DGT_E_UNSUPPORTED;
}

template <>
int launch_decode<DGT_FMT>(const DecodeArgs& a, uint32_t lanes, uint32_t ilp, bool ring,
                           uint32_t grid, uint32_t threads, uint32_t lds, hipStream_t st) {
#define DGT_DECODE_CASE(RR, II, RG)                                            \
  if (lanes == RR && ilp == II && ring == RG) {                                \
    auto k = k_decode<DGT_FMT, RR, II, RG>;                                    \
    if (!set_lds(k, lds)) return DGT_E_HIP;                                    \
    hipLaunchKernelGGL(k, dim3(grid), dim3(threads), lds, st, a);              \
    return hipGetLastError() == hipSuccess ? DGT_OK : DGT_E_HIP;               \
  }
  DGT_DECODE_CASE(64, 1, false)
  DGT_DECODE_CASE(64, 2, false)
  DGT_DECODE_CASE(64, 1, true)
  DGT_DECODE_CASE(64, 2, true)
  if constexpr (DGT_FMT != BF16W) {
    DGT_DECODE_CASE(128, 1, false)
    DGT_DECODE_CASE(128, 2, false)
    DGT_DECODE_CASE(128, 1, true)
    DGT_DECODE_CASE(128, 2, true)
    DGT_DECODE_CASE(32, 1, false)
    DGT_DECODE_CASE(32, 2, false)
  }
#undef DGT_DECODE_CASE
  return DGT_E_UNSUPPORTED;
}

template <>
int launch_dense<DGT_FMT>(const DenseArgs& d, uint32_t fn, uint32_t mt, uint32_t grid,
                          uint32_t threads, uint32_t lds, hipStream_t st) {
  if constexpr (DGT_FMT == INT4P || DGT_FMT == BF16E || DGT_FMT == BF16P || DGT_FMT == BF16W) {
    return DGT_E_UNSUPPORTED;  // their decoded weights are read as INT4 / BF16_SPLIT
  } else {
#define DGT_DENSE_CASE(FNV, MTV)                                                        \
  if (fn == FNV && mt == MTV) {                                                         \
    auto k = k_dense<DGT_FMT, FNV, MTV>;                                                \
    if (!set_lds(k, lds)) return DGT_E_HIP;                                             \
    hipLaunchKernelGGL(k, dim3(grid), dim3(threads), lds, st, d);                       \
    return hipGetLastError() == hipSuccess ? DGT_OK : DGT_E_HIP;                        \
  }
  DGT_DENSE_CASE(8, 1)
  DGT_DENSE_CASE(8, 4)
  DGT_DENSE_CASE(16, 1)
#undef DGT_DENSE_CASE
  return DGT_E_UNSUPPORTED;
  }
}

template <>
int launch_dense_tiled<DGT_FMT>(const DenseTiledArgs& d, uint32_t bn, hipStream_t st) {
  if constexpr (DGT_FMT == INT4P || DGT_FMT == BF16E || DGT_FMT == BF16P || DGT_FMT == BF16W) {
    return DGT_E_UNSUPPORTED;
  } else {
    auto run = [&](auto k, uint32_t lds) {
      if (!set_lds(k, lds)) return DGT_E_HIP;
      hipLaunchKernelGGL(k, dim3(d.nmb * d.nnb), dim3(256), lds, st, d);
      return hipGetLastError() == hipSuccess ? DGT_OK : DGT_E_HIP;
    };
    if (bn == 128) return run(k_dense_tiled<DGT_FMT, 128>, dense_tiled_lds(128));
    if (bn == 64) return run(k_dense_tiled<DGT_FMT, 64>, dense_tiled_lds(64));
    return DGT_E_UNSUPPORTED;
  }
}

template <>
int launch_gemv<DGT_FMT>(const GemvArgs& g, hipStream_t st) {
  if constexpr (DGT_FMT == INT4P || DGT_FMT == BF16E || DGT_FMT == BF16P || DGT_FMT == BF16W) {
    return DGT_E_UNSUPPORTED;
  } else {
    auto k = k_gemv<DGT_FMT>;
    const uint32_t lds = g.k * 2;
    if (!set_lds(k, lds)) return DGT_E_HIP;
    const uint32_t rows = kGvRows * kGvWaves;
    hipLaunchKernelGGL(k, dim3((g.n + rows - 1) / rows), dim3(64 * kGvWaves), lds, st, g);
    return hipGetLastError() == hipSuccess ? DGT_OK : DGT_E_HIP;
  }
}

}  // namespace dev
}  // namespace dgt
