// combine.hip -- gate-weighted un-permute back to token order.
//
// "271,104 Routes", section 1: y(x) = sum over the selected experts of
// p_i(x) E_i(x); section 3: undo the grouping, apply the gate weights, add,
// original token order.  "Session 19", "Top-k and mixture": the always-on
// shared expert is added outside the gate normalisation; the full trace: a
// dropped route contributes nothing and the kept gates stay as they are.
//
// One wave per token; each lane owns 16-byte column chunks.  The k rows of a
// token are gathered with vector loads, summed in fp32 in slot order j = 0..k-1
// (fused multiply-add by the gate), the shared row added last, and the sum
// rounded once to the output type.  No atomics: the order is fixed.
#include "common.h"
#include "launch.h"

namespace moe {

template <bool BF16>
__global__ __launch_bounds__(256) void combine_kernel(const void* __restrict__ yp,
                                                      const int32_t* __restrict__ route_pos,
                                                      const float* __restrict__ gates,
                                                      const void* __restrict__ ysh, int T, int k,
                                                      int d, void* __restrict__ y) {
  constexpr int G = BF16 ? 8 : 4;  // elements per 16-byte chunk
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
  if (t >= T) return;
  const int nch = d / G;
  int pos[8];
  float g[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    pos[j] = j < k ? route_pos[(size_t)t * k + j] : -1;
    g[j] = j < k ? gates[(size_t)t * k + j] : 0.0f;
  }
  const u32x4_t* Y = reinterpret_cast<const u32x4_t*>(yp);
  const u32x4_t* S = reinterpret_cast<const u32x4_t*>(ysh);
  u32x4_t* O = reinterpret_cast<u32x4_t*>(y);
  for (int c = lane; c < nch; c += 64) {
    float acc[G];
#pragma unroll
    for (int q = 0; q < G; ++q) acc[q] = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (pos[j] < 0) continue;
      const u32x4_t v = Y[(size_t)pos[j] * nch + c];
      if constexpr (BF16) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc[2 * q] = __builtin_fmaf(g[j], bf16lo(v[q]), acc[2 * q]);
          acc[2 * q + 1] = __builtin_fmaf(g[j], bf16hi(v[q]), acc[2 * q + 1]);
        }
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[q] = __builtin_fmaf(g[j], __uint_as_float(v[q]), acc[q]);
      }
    }
    if (ysh) {
      const u32x4_t v = S[(size_t)t * nch + c];
      if constexpr (BF16) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc[2 * q] += bf16lo(v[q]);
          acc[2 * q + 1] += bf16hi(v[q]);
        }
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[q] += __uint_as_float(v[q]);
      }
    }
    u32x4_t o;
    if constexpr (BF16) {
#pragma unroll
      for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(acc[2 * q], acc[2 * q + 1]);
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) o[q] = __float_as_uint(acc[q]);
    }
    O[(size_t)t * nch + c] = o;
  }
}

hipError_t launch_combine(bool bf16, const void* y_packed, const int32_t* route_pos,
                          const float* gates, const void* y_shared, int T, int k, int d, void* y,
                          hipStream_t st) {
  if (T == 0) return hipSuccess;
  dim3 grid(ceil_div(T, 4)), block(256);
  if (bf16)
    hipLaunchKernelGGL(combine_kernel<true>, grid, block, 0, st, y_packed, route_pos, gates,
                       y_shared, T, k, d, y);
  else
    hipLaunchKernelGGL(combine_kernel<false>, grid, block, 0, st, y_packed, route_pos, gates,
                       y_shared, T, k, d, y);
  return hipGetLastError();
}

}  // namespace moe
