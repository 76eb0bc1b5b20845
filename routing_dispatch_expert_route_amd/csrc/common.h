// common.h -- internal helpers shared by the HIP kernels of libmoe (not part
// of the C ABI).  gfx950 only: wave64, bf16 MFMA.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;

typedef uint16_t bf16_t;  // raw bfloat16 bits (upper half of a binary32)

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint32_t h) {
  return __uint_as_float(h << 16);
}
// low / high bf16 of a packed pair
__device__ __forceinline__ float bf16lo(uint32_t p) { return __uint_as_float(p << 16); }
__device__ __forceinline__ float bf16hi(uint32_t p) { return __uint_as_float(p & 0xffff0000u); }

// Two fp32 values -> packed bf16 pair (lo in bits 0-15), round to nearest
// even: one v_cvt_pk_bf16_f32.  For every finite or infinite input it gives
// the bits of the integer rounding (u + 0x7fff + lsb) >> 16 (checked over all
// 2^32 patterns on gfx950); a NaN stays a NaN.
typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
typedef float f32x2_v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_v f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_v));
}

template <typename T>
__host__ __device__ __forceinline__ T ceil_div(T a, T b) { return (a + b - 1) / b; }

}  // namespace moe
