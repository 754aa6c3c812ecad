// Precision probe of the matrix instructions the fp8 format could use (test
// infrastructure, not part of libdgt): one wave multiplies a 16 x K by a
// K x 16 matrix of e4m3 values, chained over K in steps of 32 into fp32
// accumulators, once with the fp8 x fp8 16x16x32 instruction and once with
// the operands widened exactly to bf16 and the bf16 16x16x32 instruction.
// Both operands are given as 16 rows of K bytes (B transposed), K % 32 == 0.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx2 __attribute__((ext_vector_type(2)));

// 8 e4m3 bytes -> 8 bf16 values (e4m3 is a subset of bf16: exact)
__device__ bf16x8 widen(uint64_t v) {
  uint32_t o[4];
  for (int i = 0; i < 4; ++i) {
    const uint32_t pair = (uint32_t)(v >> (16 * i)) & 0xFFFFu;
    const floatx2 f = __builtin_amdgcn_cvt_pk_f32_fp8((int)pair, false);
    o[i] = (__float_as_uint(f.x) >> 16) | (__float_as_uint(f.y) & 0xFFFF0000u);
  }
  bf16x8 r;
  __builtin_memcpy(&r, o, 16);
  return r;
}

__global__ __launch_bounds__(64) void k_probe(const uint8_t* a, const uint8_t* b, uint32_t k,
                                              float* d_fp8, float* d_bf16) {
  const uint32_t lane = threadIdx.x;
  const uint32_t row = lane & 15, kq = 8 * (lane >> 4);
  floatx4 acc8 = {0.f, 0.f, 0.f, 0.f}, acc16 = {0.f, 0.f, 0.f, 0.f};
  for (uint32_t k0 = 0; k0 < k; k0 += 32) {
    const uint64_t av = *reinterpret_cast<const uint64_t*>(a + (size_t)row * k + k0 + kq);
    const uint64_t bv = *reinterpret_cast<const uint64_t*>(b + (size_t)row * k + k0 + kq);
    acc8 = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8((long)av, (long)bv, acc8, 0, 0, 0);
    acc16 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(widen(av), widen(bv), acc16, 0, 0, 0);
  }
  // lane l holds D[4 (l / 16) + i][l % 16]
  for (int i = 0; i < 4; ++i) {
    const uint32_t r = 4 * (lane >> 4) + i;
    d_fp8[r * 16 + row] = acc8[i];
    d_bf16[r * 16 + row] = acc16[i];
  }
}

}  // namespace

// 0 on success, else the HIP error code.  a, b: device [16][k] e4m3 bytes,
// 8-byte aligned; d_fp8, d_bf16: device [16][16] fp32 outputs.
extern "C" int probe_fp8_mfma(const uint8_t* a, const uint8_t* b, uint32_t k, float* d_fp8,
                              float* d_bf16, void* stream) {
  if (!a || !b || !d_fp8 || !d_bf16 || k == 0 || k % 32) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(k_probe, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream), a, b, k,
                     d_fp8, d_bf16);
  return (int)hipGetLastError();
}
