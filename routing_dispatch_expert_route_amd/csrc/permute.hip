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

// Whole permute in one workgroup of 1024 threads (16 waves), for route counts
// small enough that one CU finishes them faster than three dependent
// launches: histogram by LDS atomics, capacity and the exclusive prefix by
// one wave, then the routes in chunks of 1024 in route order -- the rank of
// a route is the running count of its expert before the chunk, plus the
// routes of the same expert in earlier waves of the chunk, plus its rank
// among the lanes of its own wave (ballots).  Same result as the chunked
// kernels above, bit for bit.
constexpr int kSmallThreads = 1024;
constexpr int kSmallWaves = kSmallThreads / kWave;
constexpr long kSmallMaxRoutes = 4096;

__global__ __launch_bounds__(kSmallThreads) void permute_small_kernel(
    const int32_t* __restrict__ ids, int R, int k, int E, int C, int32_t* __restrict__ counts,
    int32_t* __restrict__ kept, int32_t* __restrict__ offsets, int32_t* __restrict__ route_pos,
    int32_t* __restrict__ row_token) {
  __shared__ int s_cnt[256];
  __shared__ int s_off[256];
  __shared__ int s_run[256];
  __shared__ int s_w[kSmallWaves][256];  // per-wave counts of the chunk, then their prefix
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  for (int e = tid; e < E; e += kSmallThreads) {
    s_cnt[e] = 0;
    s_run[e] = 0;
  }
  __syncthreads();
  for (int r = tid; r < R; r += kSmallThreads) {
    const int e = ids[r];
    if (e >= 0 && e < E) atomicAdd(&s_cnt[e], 1);
  }
  __syncthreads();
  if (wave == 0) {
    int carry = 0;
    if (lane == 0) offsets[0] = 0;
    for (int e0 = 0; e0 < E; e0 += kWave) {
      const int e = e0 + lane;
      const int n = e < E ? s_cnt[e] : 0;
      const int m = (C < 0 || n <= C) ? n : C;
      const int incl = wave_incl_scan(m, lane);
      if (e < E) {
        counts[e] = n;
        kept[e] = m;
        s_off[e] = carry + incl - m;
        offsets[e + 1] = carry + incl;
      }
      carry += __shfl(incl, kWave - 1, kWave);
    }
  }
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  for (int base = 0; base < R; base += kSmallThreads) {
    for (int e = lane; e < E; e += kWave) s_w[wave][e] = 0;
    const int r = base + tid;
    const int e = r < R ? ids[r] : -1;
    const bool valid = r < R && e >= 0 && e < E;
    uint64_t m = __ballot(valid);
#pragma unroll
    for (int bit = 0; bit < 8; ++bit) {
      const bool on = (e >> bit) & 1;
      const uint64_t bb = __ballot(on);
      m &= on ? bb : ~bb;
    }
    const int rank = __popcll(m & lt_mask);
    __syncthreads();  // s_w cleared (and s_off written, first chunk)
    // the first lane of each expert group records the group's size
    if (valid && rank == 0) s_w[wave][e] = __popcll(m);
    __syncthreads();
    // per expert: exclusive prefix over the waves, and the running count
    for (int x = tid; x < E; x += kSmallThreads) {
      int acc = s_run[x];
      for (int w = 0; w < kSmallWaves; ++w) {
        const int c = s_w[w][x];
        s_w[w][x] = acc;
        acc += c;
      }
      s_run[x] = acc;
    }
    __syncthreads();
    if (r < R) {
      const int slot = valid ? s_w[wave][e] + rank : 0;
      if (valid && (C < 0 || slot < C)) {
        const int p = s_off[e] + slot;
        route_pos[r] = p;
        row_token[p] = r / k;
      } else {
        route_pos[r] = -1;
      }
    }
    __syncthreads();  // s_w is reused by the next chunk
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

// Fixed-shape dispatch buffer [E, C, d] ("Session 19", "Capacity": capacity
// is a tensor dimension; slot table of "Visual support -- Capacity").  From
// the packed dispatch: a kept route r of expert e at packed row p sits in
// slot p - offsets[e] of e, i.e. row e*C + slot of the buffer.
__global__ __launch_bounds__(256) void padded_index_kernel(const int32_t* __restrict__ route_pos,
                                                           const int32_t* __restrict__ ids,
                                                           const int32_t* __restrict__ offsets,
                                                           int R, int C,
                                                           int32_t* __restrict__ pad_pos) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= R) return;
  const int p = route_pos[r];
  if (p < 0) {
    pad_pos[r] = -1;
    return;
  }
  const int e = ids[r];
  pad_pos[r] = e * C + (p - offsets[e]);
}

// x_pad[e*C + c] = x[row_token[offsets[e] + c]] for c < kept[e], zero rows
// for the empty slots; offsets_pad[e] = e*C (the buffer's row groups).
__global__ __launch_bounds__(256) void fill_padded_kernel(const u32x4_t* __restrict__ x,
                                                          const int32_t* __restrict__ row_token,
                                                          const int32_t* __restrict__ offsets,
                                                          const int32_t* __restrict__ kept, int E,
                                                          int C, int cpr, long total,
                                                          u32x4_t* __restrict__ x_pad,
                                                          int32_t* __restrict__ offsets_pad) {
  const long g0 = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (g0 <= E) offsets_pad[g0] = (int32_t)(g0 * C);
  const u32x4_t zero = {0u, 0u, 0u, 0u};
  for (long g = g0; g < total; g += (long)gridDim.x * blockDim.x) {
    const long p = g / cpr;
    const int ch = (int)(g - p * cpr);
    const int e = (int)(p / C);
    const int c = (int)(p - (long)e * C);
    x_pad[g] = c < kept[e] ? x[(long)row_token[offsets[e] + c] * cpr + ch] : zero;
  }
}

hipError_t launch_padded(const void* x, const int32_t* ids, const int32_t* route_pos,
                         const int32_t* offsets, const int32_t* kept, const int32_t* row_token,
                         int T, int k, int E, int C, long row_bytes, int32_t* pad_pos,
                         void* x_pad, int32_t* offsets_pad, hipStream_t st) {
  const int R = T * k;
  if (R > 0) {
    hipLaunchKernelGGL(padded_index_kernel, dim3(ceil_div(R, 256)), dim3(256), 0, st, route_pos,
                       ids, offsets, R, C, pad_pos);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  const int cpr = (int)(row_bytes / 16);
  const long total = (long)E * C * cpr;
  long blocks = (total + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  // offsets_pad (E + 1 entries) is written by the first threads, even when
  // the buffer has no rows
  if (blocks < (E + 256) / 256) blocks = (E + 256) / 256;
  hipLaunchKernelGGL(fill_padded_kernel, dim3((unsigned)blocks), dim3(256), 0, st,
                     reinterpret_cast<const u32x4_t*>(x), row_token, offsets, kept, E, C, cpr, total,
                     reinterpret_cast<u32x4_t*>(x_pad), offsets_pad);
  return hipGetLastError();
}

int permute_nchunks(long R) { return (int)((R + kChunk - 1) / kChunk); }

hipError_t launch_permute_index(const int32_t* ids, int T, int k, int E, int C, int32_t* cnt_ws,
                                int32_t* counts, int32_t* kept, int32_t* offsets,
                                int32_t* route_pos, int32_t* row_token, hipStream_t st) {
  const int R = T * k;
  if (R <= kSmallMaxRoutes) {
    hipLaunchKernelGGL(permute_small_kernel, dim3(1), dim3(kSmallThreads), 0, st, ids, R, k, E, C,
                       counts, kept, offsets, route_pos, row_token);
    return hipGetLastError();
  }
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
