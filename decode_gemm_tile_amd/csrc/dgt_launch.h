// Per-format kernel launchers (defined in dgt_fmt.hip, one object per format).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dgt_kernels.h"

namespace dgt {
namespace dev {

constexpr uint32_t kMaxLds = 160 * 1024;

template <int FMT>
int launch_fused(const GemmArgs& a, uint32_t lanes, uint32_t fn, uint32_t mt, bool mix,
                 bool ring, uint32_t grid, uint32_t threads, uint32_t lds, hipStream_t st);
template <int FMT>
int launch_fused_rounds(const GemmArgs& a, uint32_t lanes, uint32_t fn, uint32_t mt, bool mix,
                        uint32_t grid, uint32_t threads, uint32_t lds, hipStream_t st,
                        int* blocks_per_cu);
template <int FMT>
int launch_fused_xm(const XmArgs& x, uint32_t lanes, uint32_t fn, bool ring, bool pingpong,
                    uint32_t xs, uint32_t grid, uint32_t lds, hipStream_t st);
template <int FMT>
int launch_decode(const DecodeArgs& a, uint32_t lanes, uint32_t ilp, bool ring, uint32_t grid,
                  uint32_t threads, uint32_t lds, hipStream_t st);
template <int FMT>
int launch_dense(const DenseArgs& d, uint32_t fn, uint32_t mt, uint32_t grid, uint32_t threads,
                 uint32_t lds, hipStream_t st);
template <int FMT>
int launch_dense_tiled(const DenseTiledArgs& d, uint32_t bn, hipStream_t st);
template <int FMT>
int launch_gemv(const GemvArgs& g, hipStream_t st);

}  // namespace dev
}  // namespace dgt
