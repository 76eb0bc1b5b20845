// permute.hip -- counting-sort dispatch ("pack") with capacity.
//
// "271,104 Routes", section 3: flatten the routes r = t*k + j, order them by
// expert with a stable sort, bincount + cumsum for the per-expert ends, and
// duplicate the token rows with index_select.  "Session 19", "Capacity" and
// the full trace: each expert seats C = ceil(phi*T*k/E) routes; arrivals past
// C are dropped in arrival order.
//
// A stable sort by a small key is a counting sort, built here from three
// passes over fixed chunks of 256 consecutive routes (one wave per chunk):
//   hist     per-chunk demand of every expert            -> cnt[e][chunk]
//   scan     per expert, exclusive prefix over chunks (the arrival base of
//            each chunk), demand n_e, kept m_e = min(n_e, C), offsets
//   scatter  each route's slot = chunk base + rank among earlier routes of
//            its chunk with the same expert (wave ballots: no atomics decide
//            an order), kept iff slot < C; writes route_pos and row_token
// and one copy pass for the packed rows:
//   gather   x_packed[p] = x[row_token[p]], 16-byte vector copies.
// Every slot equals the number of earlier routes to the same expert, so the
// result is identical to a sequential stable counting sort, bit for bit.
// Expert ids outside [0, E) are treated as dropped routes (never counted).
#include "common.h"
#include "launch.h"

namespace moe {

constexpr int kChunk = 256;  // routes per chunk (4 wave iterations)

__global__ __launch_bounds__(64) void hist_kernel(const int32_t* __restrict__ ids, int R, int E,
                                                  int nchunks, int32_t* __restrict__ cnt) {
  __shared__ int s_cnt[256];
  const int lane = threadIdx.x;
  const int c = blockIdx.x;
  for (int e = lane; e < E; e += kWave) s_cnt[e] = 0;
  __syncthreads();
  const int r0 = c * kChunk;
  constexpr int NIT = kChunk / kWave;
  int ev[NIT];  // all of the lane's ids in flight together
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int r = r0 + it * kWave + lane;
    ev[it] = r < R ? ids[r] : -1;
  }
#pragma unroll
  for (int it = 0; it < NIT; ++it)
    if (ev[it] >= 0 && ev[it] < E) atomicAdd(&s_cnt[ev[it]], 1);
  __syncthreads();
  for (int e = lane; e < E; e += kWave) cnt[(size_t)e * nchunks + c] = s_cnt[e];
}

__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int s = 1; s < kWave; s <<= 1) {
    int o = __shfl_up(v, s, kWave);
    if (lane >= s) v += o;
  }
  return v;
}

// One block of 1024 threads.  cnt[e][c] becomes the exclusive prefix over c.
__global__ __launch_bounds__(1024) void scan_kernel(int32_t* __restrict__ cnt, int E, int nchunks,
                                                    int C, int32_t* __restrict__ counts,
                                                    int32_t* __restrict__ kept,
                                                    int32_t* __restrict__ offsets) {
  __shared__ int s_kept[256];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int nwaves = blockDim.x / kWave;
  for (int e = wave; e < E; e += nwaves) {
    int32_t* row = cnt + (size_t)e * nchunks;
    int carry = 0;
    constexpr int NB = 8;  // groups of 64 chunks loaded together
    for (int c1 = 0; c1 < nchunks; c1 += NB * kWave) {
      int v[NB];
#pragma unroll
      for (int q = 0; q < NB; ++q) {
        const int c = c1 + q * kWave + lane;
        v[q] = c < nchunks ? row[c] : 0;
      }
#pragma unroll
      for (int q = 0; q < NB; ++q) {
        const int c = c1 + q * kWave + lane;
        const int incl = wave_incl_scan(v[q], lane);
        if (c < nchunks) row[c] = carry + incl - v[q];
        carry += __shfl(incl, kWave - 1, kWave);
      }
    }
    if (lane == 0) {
      const int m = (C < 0 || carry <= C) ? carry : C;
      counts[e] = carry;
      kept[e] = m;
      s_kept[e] = m;
    }
  }
  __syncthreads();
  if (wave == 0) {
    int carry = 0;
    if (lane == 0) offsets[0] = 0;
    for (int e0 = 0; e0 < E; e0 += kWave) {
      const int e = e0 + lane;
      const int v = e < E ? s_kept[e] : 0;
      const int incl = wave_incl_scan(v, lane);
      if (e < E) offsets[e + 1] = carry + incl;
      carry += __shfl(incl, kWave - 1, kWave);
    }
  }
}

__global__ __launch_bounds__(64) void scatter_kernel(const int32_t* __restrict__ ids, int R, int k,
                                                     int E, int nchunks, int C,
                                                     const int32_t* __restrict__ base,
                                                     const int32_t* __restrict__ offsets,
                                                     int32_t* __restrict__ route_pos,
                                                     int32_t* __restrict__ row_token) {
  __shared__ int s_run[256];
  __shared__ int s_off[256];
  const int lane = threadIdx.x;
  const int c = blockIdx.x;
  for (int e = lane; e < E; e += kWave) {
    s_run[e] = base[(size_t)e * nchunks + c];
    s_off[e] = offsets[e];
  }
  __syncthreads();
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  const int r0 = c * kChunk;
  constexpr int NIT = kChunk / kWave;
  int ev[NIT];  // all of the lane's ids in flight together
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int r = r0 + it * kWave + lane;
    ev[it] = r < R ? ids[r] : -1;
  }
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int r = r0 + it * kWave + lane;
    const int e = ev[it];
    const bool valid = r < R && e >= 0 && e < E;
    // lanes holding the same expert id: match on all 8 bits (E <= 256)
    uint64_t m = __ballot(valid);
#pragma unroll
    for (int bit = 0; bit < 8; ++bit) {
      const bool on = (e >> bit) & 1;
      const uint64_t bb = __ballot(on);
      m &= on ? bb : ~bb;
    }
    const int rank = __popcll(m & lt_mask);
    int slot = 0;
    if (valid) slot = s_run[e] + rank;
    __syncthreads();  // every lane has read its running count
    // the last lane of each expert group advances that expert's count
    if (valid && (m >> lane) == 1ull) s_run[e] = slot + 1;
    __syncthreads();
    if (r < R) {
      if (valid && (C < 0 || slot < C)) {
        const int p = s_off[e] + slot;
        route_pos[r] = p;
        row_token[p] = r / k;
      } else {
        route_pos[r] = -1;
      }
    }
  }
}

// x_packed[p][:] = x[row_token[p]][:] for p < offsets[E]; 16-byte chunks.
__global__ __launch_bounds__(256) void gather_rows_kernel(const u32x4_t* __restrict__ x,
                                                          const int32_t* __restrict__ row_token,
                                                          const int32_t* __restrict__ offsets,
                                                          int E, int chunks_per_row, long total,
                                                          u32x4_t* __restrict__ out) {
  const long n = (long)offsets[E] * chunks_per_row;
  const long lim = n < total ? n : total;
  for (long g = (long)blockIdx.x * blockDim.x + threadIdx.x; g < lim;
       g += (long)gridDim.x * blockDim.x) {
    const long p = g / chunks_per_row;
    const int ch = (int)(g - p * chunks_per_row);
    out[g] = x[(long)row_token[p] * chunks_per_row + ch];
  }
}

int permute_nchunks(long R) { return (int)((R + kChunk - 1) / kChunk); }

hipError_t launch_permute_index(const int32_t* ids, int T, int k, int E, int C, int32_t* cnt_ws,
                                int32_t* counts, int32_t* kept, int32_t* offsets,
                                int32_t* route_pos, int32_t* row_token, hipStream_t st) {
  const int R = T * k;
  const int nch = permute_nchunks(R);
  if (nch > 0) {
    hipLaunchKernelGGL(hist_kernel, dim3(nch), dim3(kWave), 0, st, ids, R, E, nch, cnt_ws);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, st, cnt_ws, E, nch, C, counts, kept,
                     offsets);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || nch == 0) return err;
  hipLaunchKernelGGL(scatter_kernel, dim3(nch), dim3(kWave), 0, st, ids, R, k, E, nch, C, cnt_ws,
                     offsets, route_pos, row_token);
  return hipGetLastError();
}

hipError_t launch_gather_rows(const void* x, const int32_t* row_token, const int32_t* offsets,
                              int E, long R_max, long row_bytes, void* x_packed,
                              hipStream_t st) {
  const int cpr = (int)(row_bytes / 16);
  const long total = R_max * cpr;
  if (total == 0) return hipSuccess;
  long blocks = (total + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(gather_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, st,
                     reinterpret_cast<const u32x4_t*>(x), row_token, offsets, E, cpr, total,
                     reinterpret_cast<u32x4_t*>(x_packed));
  return hipGetLastError();
}

}  // namespace moe
