// combine.hip -- gate-weighted un-permute back to token order.
//
// "271,104 Routes", section 1: y(x) = sum over the selected experts of
// p_i(x) E_i(x); section 3: undo the grouping, apply the gate weights, add,
// original token order.  "Session 19", "Top-k and mixture": the always-on
// shared expert is added outside the gate normalisation; the full trace: a
// dropped route contributes nothing and the kept gates stay as they are.
//
// One wave per (token, slice of 64 column chunks); each lane owns one chunk
// of 8 (bf16) or 4 (fp32) output columns.  The k rows of a token (any k;
// expert choice passes one slot per expert) are gathered with vector loads,
// summed in fp32 in slot order j = 0..k-1 (fused multiply-add by the gate), the shared
// row added last, and the sum rounded once to the output type.  When the
// down GEMM split K, a row is first the sum of its fp32 partial planes in
// plane order.  No atomics: every order is fixed.
#include "common.h"
#include "launch.h"

namespace moe {

// Load G consecutive values of row p starting at column col as fp32.
// Partial planes (at most 8) are summed in plane order; the loop is fully
// unrolled so the loads of all planes are in flight together.
template <bool BF16, bool PARTIAL, int G>
__device__ __forceinline__ void load_row(const void* yp, int splits, long stride, size_t p,
                                         int d, int col, float* v) {
  if constexpr (PARTIAL) {
    const float* P = reinterpret_cast<const float*>(yp) + p * d + col;
    f32x4_t part[8][G / 4];
#pragma unroll
    for (int s = 0; s < 8; ++s)
#pragma unroll
      for (int q = 0; q < G / 4; ++q)
        part[s][q] = s < splits ? *reinterpret_cast<const f32x4_t*>(P + (size_t)s * stride + 4 * q)
                                : f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int q = 0; q < G / 4; ++q) {
      f32x4_t s4 = part[0][q];
#pragma unroll
      for (int s = 1; s < 8; ++s)
        if (s < splits) s4 += part[s][q];
#pragma unroll
      for (int t = 0; t < 4; ++t) v[4 * q + t] = s4[t];
    }
  } else if constexpr (BF16) {
    const u32x4_t u = *reinterpret_cast<const u32x4_t*>(reinterpret_cast<const bf16_t*>(yp) +
                                                       p * d + col);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[2 * q] = bf16lo(u[q]);
      v[2 * q + 1] = bf16hi(u[q]);
    }
  } else {
    const f32x4_t u = *reinterpret_cast<const f32x4_t*>(reinterpret_cast<const float*>(yp) +
                                                       p * d + col);
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] = u[q];
  }
}

template <bool BF16>
__device__ __forceinline__ void store_out(void* y, size_t idx, const float* acc) {
  if constexpr (BF16) {
    u32x4_t o;
#pragma unroll
    for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(acc[2 * q], acc[2 * q + 1]);
    *reinterpret_cast<u32x4_t*>(reinterpret_cast<bf16_t*>(y) + idx) = o;
  } else {
    f32x4_t o = {acc[0], acc[1], acc[2], acc[3]};
    *reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(y) + idx) = o;
  }
}

// grid: (token groups of 4, column slices of 64 chunks); one wave per
// (token, slice), one chunk per lane
template <bool BF16, bool PARTIAL>
__global__ __launch_bounds__(256) void combine_kernel(const void* __restrict__ yp, int splits,
                                                      long split_stride,
                                                      const int32_t* __restrict__ route_pos,
                                                      const float* __restrict__ gates,
                                                      long s_tok, long s_slot,
                                                      const void* __restrict__ ysh, int T, int k,
                                                      int d, void* __restrict__ y) {
  constexpr int G = BF16 ? 8 : 4;  // output elements per 16-byte chunk
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
  const int col = (blockIdx.y * 64 + lane) * G;
  if (t >= T || col >= d) return;
  float acc[G];
#pragma unroll
  for (int q = 0; q < G; ++q) acc[q] = 0.0f;
  // slots in groups of eight (one group when k <= 8; expert choice passes
  // one slot per expert)
  for (int j0 = 0; j0 < k; j0 += 8) {
    int pos[8];
    float g[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const size_t at = (size_t)t * s_tok + (size_t)(j0 + j) * s_slot;
      pos[j] = j0 + j < k ? route_pos[at] : -1;
      g[j] = j0 + j < k ? gates[at] : 0.0f;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (pos[j] < 0) continue;
      float v[G];
      load_row<BF16, PARTIAL, G>(yp, splits, split_stride, (size_t)pos[j], d, col, v);
#pragma unroll
      for (int q = 0; q < G; ++q) acc[q] = __builtin_fmaf(g[j], v[q], acc[q]);
    }
  }
  if (ysh) {
    float v[G];
    load_row<BF16, false, G>(ysh, 1, 0, (size_t)t, d, col, v);
#pragma unroll
    for (int q = 0; q < G; ++q) acc[q] += v[q];
  }
  store_out<BF16>(y, (size_t)t * d + col, acc);
}

// The same sum for direct rows and k <= KS slots (KS = 2, 4 or 8): a wave
// holds one token, so its route positions are wave-uniform and the KS rows
// load without a branch -- a dropped slot loads the token's first kept row
// and adds nothing -- all in flight before the first sum, which keeps slot
// order (the kernel above issues one row at a time behind its branches).
template <bool BF16, int KS>
__global__ __launch_bounds__(256) void combine_rows_kernel(const void* __restrict__ yp,
                                                           const int32_t* __restrict__ route_pos,
                                                           const float* __restrict__ gates,
                                                           const void* __restrict__ ysh, int T,
                                                           int k, int d, void* __restrict__ y) {
  constexpr int G = BF16 ? 8 : 4;  // output elements per 16-byte chunk
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
  const int col = (blockIdx.y * 64 + lane) * G;
  if (t >= T || col >= d) return;
  int pos[KS];
  float g[KS];
#pragma unroll
  for (int j = 0; j < KS; ++j) {  // all of the token's slots in flight together
    const size_t at = (size_t)t * k + (j < k ? j : 0);
    pos[j] = route_pos[at];
    g[j] = gates[at];
  }
  int any = -1;
#pragma unroll
  for (int j = 0; j < KS; ++j) {
    pos[j] = j < k ? __builtin_amdgcn_readfirstlane(pos[j]) : -1;
    if (any < 0 && pos[j] >= 0) any = pos[j];
  }
  float acc[G];
#pragma unroll
  for (int q = 0; q < G; ++q) acc[q] = 0.0f;
  if (any >= 0) {
    float v[KS][G];
#pragma unroll
    for (int j = 0; j < KS; ++j)
      load_row<BF16, false, G>(yp, 1, 0, (size_t)(pos[j] >= 0 ? pos[j] : any), d, col, v[j]);
#pragma unroll
    for (int j = 0; j < KS; ++j) {
      if (pos[j] < 0) continue;
#pragma unroll
      for (int q = 0; q < G; ++q) acc[q] = __builtin_fmaf(g[j], v[j][q], acc[q]);
    }
  }
  if (ysh) {
    float v[G];
    load_row<BF16, false, G>(ysh, 1, 0, (size_t)t, d, col, v);
#pragma unroll
    for (int q = 0; q < G; ++q) acc[q] += v[q];
  }
  store_out<BF16>(y, (size_t)t * d + col, acc);
}

// Slot-major route tables (expert choice: slot e of token t at e*T + t, one
// slot per expert, a handful of them taken): a wave holds one token and its
// lanes read 64 slots at once; the taken ones (a ballot, in increasing e)
// are summed in batches of up to 8 rows, each batch's rows in flight
// together, in slot order -- the generic kernel's sums, without reading the
// E slots eight at a time.
template <bool BF16>
__global__ __launch_bounds__(256) void combine_slots_kernel(const void* __restrict__ yp,
                                                            const int32_t* __restrict__ route_pos,
                                                            const float* __restrict__ gates,
                                                            const void* __restrict__ ysh, int T,
                                                            int E, int d, void* __restrict__ y) {
  constexpr int G = BF16 ? 8 : 4;  // output elements per 16-byte chunk
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
  const int col = (blockIdx.y * 64 + lane) * G;
  if (t >= T) return;  // whole waves: the column test comes after the ballots
  const bool colok = col < d;
  float acc[G];
#pragma unroll
  for (int q = 0; q < G; ++q) acc[q] = 0.0f;
  for (int e0 = 0; e0 < E; e0 += 64) {
    const int e = e0 + lane;
    const int p = e < E ? route_pos[(size_t)e * T + t] : -1;
    const float gv = e < E ? gates[(size_t)e * T + t] : 0.0f;
    uint64_t m = __ballot(p >= 0);
    while (m) {  // wave-uniform
      constexpr int B = 8;
      int pos[B];
      float g[B];
#pragma unroll
      for (int j = 0; j < B; ++j) {  // the next (up to) B taken slots, in order
        const int src = m ? __builtin_ctzll(m) : 0;
        pos[j] = m ? __builtin_amdgcn_readlane(p, src) : -1;
        g[j] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gv), src));
        m &= m - 1;  // 0 stays 0
      }
      if (colok) {
        float v[B][G];
#pragma unroll
        for (int j = 0; j < B; ++j)
          load_row<BF16, false, G>(yp, 1, 0, (size_t)(pos[j] >= 0 ? pos[j] : pos[0]), d, col, v[j]);
#pragma unroll
        for (int j = 0; j < B; ++j) {
          if (pos[j] < 0) continue;
#pragma unroll
          for (int q = 0; q < G; ++q) acc[q] = __builtin_fmaf(g[j], v[j][q], acc[q]);
        }
      }
    }
  }
  if (!colok) return;
  if (ysh) {
    float v[G];
    load_row<BF16, false, G>(ysh, 1, 0, (size_t)t, d, col, v);
#pragma unroll
    for (int q = 0; q < G; ++q) acc[q] += v[q];
  }
  store_out<BF16>(y, (size_t)t * d + col, acc);
}

// y[p][:] = sum_s parts[s][p][:] for the valid rows, rounded once.
template <bool BF16>
__global__ __launch_bounds__(256) void reduce_splits_kernel(const float* __restrict__ parts,
                                                            int splits, long stride,
                                                            const int32_t* __restrict__ offsets,
                                                            int E, long R_max, int N,
                                                            void* __restrict__ y) {
  constexpr int G = BF16 ? 8 : 4;
  const long rows = offsets ? (long)offsets[E] : R_max;
  const long per_row = N / G;
  const long total = (rows < R_max ? rows : R_max) * per_row;
  for (long g = (long)blockIdx.x * blockDim.x + threadIdx.x; g < total;
       g += (long)gridDim.x * blockDim.x) {
    const long p = g / per_row;
    const int col = (int)(g - p * per_row) * G;
    float v[G];
    load_row<BF16, true, G>(parts, splits, stride, (size_t)p, N, col, v);
    store_out<BF16>(y, (size_t)p * N + col, v);
  }
}

static hipError_t combine_strided(bool bf16, const void* y_packed, int splits, long split_stride,
                                  const int32_t* route_pos, const float* gates, long s_tok,
                                  long s_slot, const void* y_shared, int T, int k, int d, void* y,
                                  hipStream_t st) {
  if (T == 0) return hipSuccess;
  dim3 grid(ceil_div(T, 4), ceil_div(d, 64 * (bf16 ? 8 : 4))), block(256);
  const bool part = splits > 1;
#define CB(B, P)                                                                           \
  hipLaunchKernelGGL((combine_kernel<B, P>), grid, block, 0, st, y_packed, splits, split_stride, \
                     route_pos, gates, s_tok, s_slot, y_shared, T, k, d, y)
  if (bf16) {
    if (part) CB(true, true);
    else CB(true, false);
  } else {
    if (part) CB(false, true);
    else CB(false, false);
  }
#undef CB
  return hipGetLastError();
}

hipError_t launch_combine(bool bf16, const void* y_packed, int splits, long split_stride,
                          const int32_t* route_pos, const float* gates, const void* y_shared,
                          int T, int k, int d, void* y, hipStream_t st) {
  if (splits <= 1 && k <= 8 && T > 0) {
    dim3 grid(ceil_div(T, 4), ceil_div(d, 64 * (bf16 ? 8 : 4))), block(256);
#define CR(B, K)                                                                                \
  hipLaunchKernelGGL((combine_rows_kernel<B, K>), grid, block, 0, st, y_packed, route_pos, gates, \
                     y_shared, T, k, d, y)
    const int ks = k <= 2 ? 2 : (k <= 4 ? 4 : 8);
    if (bf16) {
      if (ks == 2) CR(true, 2);
      else if (ks == 4) CR(true, 4);
      else CR(true, 8);
    } else {
      if (ks == 2) CR(false, 2);
      else if (ks == 4) CR(false, 4);
      else CR(false, 8);
    }
#undef CR
    return hipGetLastError();
  }
  return combine_strided(bf16, y_packed, splits, split_stride, route_pos, gates, k, 1, y_shared,
                         T, k, d, y, st);
}

hipError_t launch_combine_slot_major(bool bf16, const void* y_packed, int splits,
                                     long split_stride, const int32_t* route_pos,
                                     const float* gates, const void* y_shared, int T, int k,
                                     int d, void* y, hipStream_t st) {
  if (splits <= 1 && T > 0) {
    dim3 grid(ceil_div(T, 4), ceil_div(d, 64 * (bf16 ? 8 : 4))), block(256);
    if (bf16)
      hipLaunchKernelGGL(combine_slots_kernel<true>, grid, block, 0, st, y_packed, route_pos, gates,
                         y_shared, T, k, d, y);
    else
      hipLaunchKernelGGL(combine_slots_kernel<false>, grid, block, 0, st, y_packed, route_pos,
                         gates, y_shared, T, k, d, y);
    return hipGetLastError();
  }
  return combine_strided(bf16, y_packed, splits, split_stride, route_pos, gates, 1, T, y_shared,
                         T, k, d, y, st);
}

hipError_t launch_reduce_splits(bool bf16, const float* parts, int splits, long split_stride,
                                const int32_t* offsets, int E, long R_max, int N, void* y,
                                hipStream_t st) {
  const long total = R_max * (N / (bf16 ? 8 : 4));
  if (total == 0) return hipSuccess;
  long blocks = (total + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (bf16)
    hipLaunchKernelGGL(reduce_splits_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, st, parts,
                       splits, split_stride, offsets, E, R_max, N, y);
  else
    hipLaunchKernelGGL(reduce_splits_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, st,
                       parts, splits, split_stride, offsets, E, R_max, N, y);
  return hipGetLastError();
}

}  // namespace moe
