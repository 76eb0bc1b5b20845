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
#include "topk.h"

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
  // wave w scans experts w, w + nwaves, ...; NE of them and NB groups of 64
  // chunks each are loaded together, so their loads are in flight at once
  constexpr int NE = 4, NB = 4;
  for (int e0 = wave; e0 < E; e0 += NE * nwaves) {
    int carry[NE];
#pragma unroll
    for (int j = 0; j < NE; ++j) carry[j] = 0;
    for (int c1 = 0; c1 < nchunks; c1 += NB * kWave) {
      int v[NE][NB];
#pragma unroll
      for (int j = 0; j < NE; ++j) {
        const int e = e0 + j * nwaves;
#pragma unroll
        for (int q = 0; q < NB; ++q) {
          const int c = c1 + q * kWave + lane;
          v[j][q] = e < E && c < nchunks ? cnt[(size_t)e * nchunks + c] : 0;
        }
      }
#pragma unroll
      for (int j = 0; j < NE; ++j) {
        const int e = e0 + j * nwaves;  // the same in every lane
        if (e >= E) break;
#pragma unroll
        for (int q = 0; q < NB; ++q) {
          if (c1 + q * kWave >= nchunks) break;  // the same in every lane
          const int c = c1 + q * kWave + lane;
          const int incl = wave_incl_scan(v[j][q], lane);
          if (c < nchunks) cnt[(size_t)e * nchunks + c] = carry[j] + incl - v[j][q];
          carry[j] += __shfl(incl, kWave - 1, kWave);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < NE; ++j) {
      const int e = e0 + j * nwaves;
      if (lane == 0 && e < E) {
        const int m = (C < 0 || carry[j] <= C) ? carry[j] : C;
        counts[e] = carry[j];
        kept[e] = m;
        s_kept[e] = m;
      }
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
// launches.  Route r = q * 1024 + tid lies in group (q, wave): the groups
// in route order are g = q * 16 + wave, 64 of them.  The ballots on the
// expert-id bits give each route its rank among the lanes of its wave and
// each group its size per expert; one wave per expert then scans the 64
// group sizes, which gives every group its expert's running count before it
// and the expert's demand; one wave clips the demands to the capacity and
// forms the offsets.  A route's slot is its group's running count plus its
// rank -- the number of routes of its expert before it, as the chunked
// kernels above count them, so the same result bit for bit.
constexpr int kSmallThreads = 1024;
constexpr int kSmallWaves = kSmallThreads / kWave;
constexpr long kSmallMaxRoutes = 4096;

constexpr int kSmallPerThread = kSmallMaxRoutes / kSmallThreads;
static_assert(kSmallPerThread * kSmallWaves <= kWave, "one lane per group in the per-expert scan");

// The body, over the routes' experts already in registers: thread tid holds
// route q * kSmallThreads + tid in idv[q] (-1 past R), loaded together by
// the caller, so no pass waits on memory.  PT: routes per thread the caller
// covers (R <= PT * 1024), which sizes the group table.
template <int PT>
__device__ __forceinline__ void permute_small_body(const int (&idv)[PT], int R, int k,
                                                   int E, int C, int32_t* __restrict__ counts,
                                                   int32_t* __restrict__ kept,
                                                   int32_t* __restrict__ offsets,
                                                   int32_t* __restrict__ route_pos,
                                                   int32_t* __restrict__ row_token) {
  static_assert(PT >= 1 && PT <= kSmallPerThread, "at most 4096 routes");
  constexpr int kGroups = PT * kSmallWaves;
  __shared__ int s_off[256];
  __shared__ int s_g[kGroups][256];  // group sizes per expert, then their prefix
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  for (int i = tid; i < kGroups * E; i += kSmallThreads) s_g[i / E][i % E] = 0;
  __syncthreads();
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  int rank[PT];
#pragma unroll
  for (int q = 0; q < PT; ++q) {
    const int r = q * kSmallThreads + tid;
    const int e = idv[q];
    const bool valid = r < R && e >= 0 && e < E;
    // lanes holding the same expert id: match on all 8 bits (E <= 256)
    uint64_t m = __ballot(valid);
#pragma unroll
    for (int bit = 0; bit < 8; ++bit) {
      const bool on = (e >> bit) & 1;
      const uint64_t bb = __ballot(on);
      m &= on ? bb : ~bb;
    }
    rank[q] = __popcll(m & lt_mask);
    // the first lane of each expert's lanes records the group's size
    if (valid && rank[q] == 0) s_g[q * kSmallWaves + wave][e] = __popcll(m);
  }
  __syncthreads();
  // per expert (a wave each): exclusive prefix over the groups in route order
  for (int e = wave; e < E; e += kSmallWaves) {
    const int c = lane < kGroups ? s_g[lane][e] : 0;
    const int incl = wave_incl_scan(c, lane);
    if (lane < kGroups) s_g[lane][e] = incl - c;
    if (lane == kWave - 1) s_off[e] = incl;  // the expert's demand, for now
  }
  __syncthreads();
  if (wave == 0) {
    int carry = 0;
    if (lane == 0) offsets[0] = 0;
    for (int e0 = 0; e0 < E; e0 += kWave) {
      const int e = e0 + lane;
      const int n = e < E ? s_off[e] : 0;
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
  __syncthreads();
#pragma unroll
  for (int q = 0; q < PT; ++q) {
    const int r = q * kSmallThreads + tid;
    if (r < R) {
      const int e = idv[q];
      const bool valid = e >= 0 && e < E;
      const int slot = valid ? s_g[q * kSmallWaves + wave][e] + rank[q] : 0;
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

template <int PT>
__global__ __launch_bounds__(kSmallThreads) void permute_small_kernel(
    const int32_t* __restrict__ ids, int R, int k, int E, int C, int32_t* __restrict__ counts,
    int32_t* __restrict__ kept, int32_t* __restrict__ offsets, int32_t* __restrict__ route_pos,
    int32_t* __restrict__ row_token) {
  int idv[PT];
#pragma unroll
  for (int q = 0; q < PT; ++q) {
    const int r = q * kSmallThreads + (int)threadIdx.x;
    idv[q] = r < R ? ids[r] : -1;
  }
  permute_small_body(idv, R, k, E, C, counts, kept, offsets, route_pos, row_token);
}

// Top-k and the whole permute in one workgroup, for few tokens (at most
// kFusedMaxT; the top-k of many tokens is faster spread over many CUs, as
// topk_rank_kernel does) and at most kFusedMaxE experts: topk_token (the
// same selection and gate sums as topk_rank_kernel, so the same ids and
// gates bit for bit) runs first, a thread per token, and leaves the ids in
// LDS for the permute.  One launch and its gap fewer than top-k followed by
// the permute: about 5 us of a decode step.
constexpr int kFusedMaxE = 16;
constexpr int kFusedMaxT = 256;

template <int KMAX>
__global__ __launch_bounds__(kSmallThreads) void topk_permute_small_kernel(
    const float* __restrict__ logits, int T, int E, int k, int renorm, int C,
    int32_t* __restrict__ ids, float* __restrict__ gates, int32_t* __restrict__ counts,
    int32_t* __restrict__ kept, int32_t* __restrict__ offsets, int32_t* __restrict__ route_pos,
    int32_t* __restrict__ row_token) {
  static_assert(kFusedMaxT <= kSmallThreads, "a thread per token");
  __shared__ int s_ids[kFusedMaxT * 8];
  const int t = threadIdx.x;
  if (t < T) {
    float v[kFusedMaxE];
    const float* lr = logits + (size_t)t * E;
#pragma unroll
    for (int e = 0; e < kFusedMaxE; ++e) v[e] = e < E ? lr[e] : 0.0f;
    int bi[KMAX];
    float gate[KMAX];
    topk_token<KMAX, kFusedMaxE>([&](int e) { return v[e]; }, E, k, renorm, bi, gate);
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      if (j < k) {
        ids[(size_t)t * k + j] = bi[j];
        gates[(size_t)t * k + j] = gate[j];
        s_ids[t * k + j] = bi[j];
      }
    }
  }
  __syncthreads();
  constexpr int PT = kFusedMaxT * KMAX <= kSmallThreads ? 1 : 2;
  static_assert(kFusedMaxT * KMAX <= PT * kSmallThreads, "every route in a thread");
  int idv[PT];
#pragma unroll
  for (int q = 0; q < PT; ++q) {
    const int r = q * kSmallThreads + t;
    idv[q] = r < T * k ? s_ids[r] : -1;
  }
  permute_small_body(idv, T * k, k, E, C, counts, kept, offsets, route_pos, row_token);
}

bool topk_permute_fused(int T, int k, int E) {
  return T <= kFusedMaxT && k <= 8 && E <= kFusedMaxE;
}

hipError_t launch_topk_permute(const float* logits, int T, int E, int k, int renorm, int C,
                               int32_t* ids, float* gates, int32_t* counts, int32_t* kept,
                               int32_t* offsets, int32_t* route_pos, int32_t* row_token,
                               hipStream_t st) {
  if (!topk_permute_fused(T, k, E)) return hipErrorInvalidValue;
#define TP(KM)                                                                                 \
  hipLaunchKernelGGL(topk_permute_small_kernel<KM>, dim3(1), dim3(kSmallThreads), 0, st, logits, \
                     T, E, k, renorm, C, ids, gates, counts, kept, offsets, route_pos, row_token)
  if (k <= 1) TP(1);
  else if (k <= 2) TP(2);
  else if (k <= 4) TP(4);
  else TP(8);
#undef TP
  return hipGetLastError();
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
// x_pad[e*C + c] = x[row_token[offsets[e] + c]] for c < kept[e], zero rows
// for the empty slots; offsets_pad[e] = e*C (the buffer's row groups); and,
// in the same launch, every route's pad_pos = e*C + slot, or -1 when dropped
// (both read only the packed dispatch).
__global__ __launch_bounds__(256) void fill_padded_kernel(const u32x4_t* __restrict__ x,
                                                          const int32_t* __restrict__ row_token,
                                                          const int32_t* __restrict__ offsets,
                                                          const int32_t* __restrict__ kept, int E,
                                                          int C, int cpr, long total,
                                                          u32x4_t* __restrict__ x_pad,
                                                          int32_t* __restrict__ offsets_pad,
                                                          const int32_t* __restrict__ route_pos,
                                                          const int32_t* __restrict__ ids, int R,
                                                          int32_t* __restrict__ pad_pos) {
  const long g0 = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const long stride = (long)gridDim.x * blockDim.x;
  if (g0 <= E) offsets_pad[g0] = (int32_t)(g0 * C);
  for (long r = g0; r < R; r += stride) {
    const int p = route_pos[r];
    pad_pos[r] = p < 0 ? -1 : ids[r] * C + (p - offsets[ids[r]]);
  }
  const u32x4_t zero = {0u, 0u, 0u, 0u};
  for (long g = g0; g < total; g += stride) {
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
  const int cpr = (int)(row_bytes / 16);
  const long total = (long)E * C * cpr;
  long blocks = (total + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  // offsets_pad (E + 1 entries) is written by the first threads, even when
  // the buffer has no rows
  if (blocks < (E + 256) / 256) blocks = (E + 256) / 256;
  hipLaunchKernelGGL(fill_padded_kernel, dim3((unsigned)blocks), dim3(256), 0, st,
                     reinterpret_cast<const u32x4_t*>(x), row_token, offsets, kept, E, C, cpr, total,
                     reinterpret_cast<u32x4_t*>(x_pad), offsets_pad, route_pos, ids, R, pad_pos);
  return hipGetLastError();
}

// Overflow policy "reroute" ("Session 19", "Overflow policies": the
// overflowing route is handled by the token's next-best expert).  Routes
// keep the seats of the drop policy; then the dropped ones, in arrival
// order, each take the best-ranked expert of their token (logit descending,
// lower index first) that the token does not hold and that still has room.
// That is a greedy in arrival order -- every choice depends on the earlier
// ones.  Up to 64 experts, reroute_da_kernel below reaches the same result
// in parallel rounds while its per-expert bitmaps fit LDS; beyond that one
// wave walks the dropped routes one by one (reroute_kernel here, or
// reroute_wide_kernel, four experts per lane, past 64 experts).  A parallel kernel first writes, for every dropped
// route, the rank of each expert (one byte each; the walk) or the experts
// in preference order (the parallel rounds).  The walk stages a 64-route
// chunk's rank rows in LDS (the next chunk's are loaded while this one is
// walked); for a route, lane e reads
// its expert's rank and the choice is the lowest rank among the lanes with
// room that the token does not hold -- six ballots over the rank bits, no
// branches; lane e keeps expert e's seat count (E <= 64).
//   ids_out   final expert of every route; slot  seat at that expert, or -1
//   offsets   exclusive prefix of the seats used per expert
constexpr int kRerouteMaxE = 64;

// The rank of expert e in dropped route r's preference order (experts
// ahead: larger logit, or equal logit and lower index), one thread per
// (r, e), stored as rank[r][e] (the walk) or inverted, order[r][rank] = e
// (ORDER: the parallel rounds read the experts in preference order).
// RS: bytes per route (64, or 256 for the wide walk).
template <bool ORDER, int RS>
__device__ __forceinline__ void reroute_rank_at(long g, const float* __restrict__ logits,
                                                const int32_t* __restrict__ route_pos0,
                                                const int32_t* __restrict__ offsets0, int R,
                                                int k, int E, int C, uint8_t* __restrict__ rank) {
  const int r = (int)(g / RS), e = (int)(g % RS);
  if (r >= R || e >= E || route_pos0[r] >= 0) return;
  if (ORDER && offsets0[E] >= (long)E * C) return;  // every seat taken: nothing moves
  const float* l = logits + (size_t)(r / k) * E;
  const float le = l[e];
  int rk = 0;
  for (int e2 = 0; e2 < E; ++e2) {
    const float l2 = l[e2];
    rk += (l2 > le) | ((l2 == le) & (e2 < e));
  }
  if (ORDER)
    rank[(size_t)r * RS + rk] = (uint8_t)e;
  else
    rank[(size_t)r * RS + e] = (uint8_t)rk;
}
template <bool ORDER, int RS>
__global__ __launch_bounds__(256) void reroute_rank_kernel(const float* __restrict__ logits,
                                                           const int32_t* __restrict__ route_pos0,
                                                           const int32_t* __restrict__ offsets0,
                                                           int R, int k, int E, int C,
                                                           uint8_t* __restrict__ rank) {
  reroute_rank_at<ORDER, RS>((long)blockIdx.x * blockDim.x + threadIdx.x, logits, route_pos0,
                             offsets0, R, k, E, C, rank);
}

__global__ __launch_bounds__(64) void reroute_kernel(
    const uint8_t* __restrict__ rank, const int32_t* __restrict__ ids_in,
    const int32_t* __restrict__ route_pos0, const int32_t* __restrict__ offsets0,
    const int32_t* __restrict__ kept, int T, int k, int E, int C, int32_t* __restrict__ ids_out,
    int32_t* __restrict__ slot, int32_t* __restrict__ offsets) {
  __shared__ __attribute__((aligned(16))) uint8_t s_rank[kWave][kRerouteMaxE];
  const int lane = threadIdx.x;
  const int R = T * k;
  int fill = lane < E ? kept[lane] : 0;  // lane e: seats used at expert e
  uint64_t avail = __ballot(lane < E && fill < C);  // experts with room
  int cur_t = -1;
  uint64_t cur_mask[8];  // final experts of token cur_t's slots, one bit each
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) cur_mask[jj] = 0;
  // chunk data of lane i: its route's drop-policy position and expert, and,
  // when dropped, its rank row and its token's experts
  int p0, e0, tid[8];
  uint4 rw[4];
  auto load = [&](int base) {
    const int rr = base + lane;
    p0 = rr < R ? route_pos0[rr] : 0;
    e0 = rr < R ? ids_in[rr] : 0;
    const bool drop = rr < R && p0 < 0;
    const uint4* src = reinterpret_cast<const uint4*>(rank + (size_t)(drop ? rr : 0) * kRerouteMaxE);
#pragma unroll
    for (int w = 0; w < 4; ++w) rw[w] = (drop && 16 * w < E) ? src[w] : uint4{0u, 0u, 0u, 0u};
    const int t = drop ? rr / k : 0;
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) tid[jj] = (drop && jj < k) ? ids_in[t * k + jj] : 0;
  };
  load(0);
  for (int base = 0; base < R; base += kWave) {
    const int cp0 = p0, ce0 = e0;
    int ctid[8];
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) ctid[jj] = tid[jj];
    __syncthreads();  // the previous chunk's rank rows are no longer read
#pragma unroll
    for (int w = 0; w < 4; ++w) *reinterpret_cast<uint4*>(&s_rank[lane][16 * w]) = rw[w];
    __syncthreads();
    if (base + kWave < R) load(base + kWave);  // in flight during this chunk's walk
    const int rr = base + lane;
    if (rr < R && cp0 >= 0) {  // kept by the drop policy: same expert, same seat
      ids_out[rr] = ce0;
      slot[rr] = cp0 - offsets0[ce0];
    }
    uint64_t m = __ballot(rr < R && cp0 < 0);
    int b = m ? __builtin_amdgcn_readfirstlane(__builtin_ctzll(m)) : 0;
    int key = s_rank[b][lane & (kRerouteMaxE - 1)];
    while (m) {
      m &= m - 1;
      const int bn = m ? __builtin_amdgcn_readfirstlane(__builtin_ctzll(m)) : b;
      const int key_next = s_rank[bn][lane & (kRerouteMaxE - 1)];  // issued ahead
      const int r = base + b;
      const int t = r / k, j = r - t * k;
      if (t != cur_t) {
        cur_t = t;
#pragma unroll
        for (int jj = 0; jj < 8; ++jj)
          cur_mask[jj] = (jj < k) ? (1ull << __builtin_amdgcn_readlane(ctid[jj], b)) : 0ull;
      }
      uint64_t held = 0;
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) held |= (jj != j) ? cur_mask[jj] : 0ull;
      // lowest rank among the experts with room the token does not hold:
      // ranks are distinct, six ballots over their bits leave one lane
      uint64_t alive = avail & ~held & __ballot(lane < E);
#pragma unroll
      for (int bit = 5; bit >= 0; --bit) {
        const uint64_t zeros = __ballot(((key >> bit) & 1) == 0) & alive;
        alive = zeros ? zeros : alive;
      }
      if (alive) {
        const int best = __builtin_ctzll(alive);
        const int seat = __builtin_amdgcn_readlane(fill, best);
        if (lane == best) fill = seat + 1;
        if (lane == 0) {
          slot[r] = seat;
          ids_out[r] = best;
        }
        if (seat + 1 >= C) avail &= ~(1ull << best);
#pragma unroll
        for (int jj = 0; jj < 8; ++jj)
          if (jj == j) cur_mask[jj] = 1ull << best;
      } else {  // no expert with room: dropped after all (lane b's own expert)
        const int orig = __builtin_amdgcn_readlane(ce0, b);
        if (lane == 0) {
          ids_out[r] = orig;
          slot[r] = -1;
        }
      }
      b = bn;
      key = key_next;
    }
  }
  const int f = lane < E ? fill : 0;
  const int incl = wave_incl_scan(f, lane);
  if (lane == 0) offsets[0] = 0;
  if (lane < E) offsets[lane + 1] = incl;
}

// The walk for 64 < E <= 256: lane l keeps the seat counts of experts l,
// l + 64, l + 128 and l + 192, and a dropped route takes the smallest
// (rank, expert) key among the experts with room that its token does not
// hold -- a wave minimum in place of reroute_kernel's ballots over one
// expert per lane.  Ranks are distinct, so the key names one expert: the
// same choice as the walk above, one route at a time in arrival order.
constexpr int kRerouteWideE = 256;
__global__ __launch_bounds__(64) void reroute_wide_kernel(
    const uint8_t* __restrict__ rank, const int32_t* __restrict__ ids_in,
    const int32_t* __restrict__ route_pos0, const int32_t* __restrict__ offsets0,
    const int32_t* __restrict__ kept, int T, int k, int E, int C, int32_t* __restrict__ ids_out,
    int32_t* __restrict__ slot, int32_t* __restrict__ offsets) {
  constexpr int G = kRerouteWideE / kWave;  // experts per lane
  constexpr int NW = kRerouteWideE / 16;    // 16-byte words of a rank row
  __shared__ __attribute__((aligned(16))) uint8_t s_rank[kWave][kRerouteWideE];
  const int lane = threadIdx.x;
  const int R = T * k;
  int fill[G];  // seats used at expert lane + 64 * g
#pragma unroll
  for (int g = 0; g < G; ++g) fill[g] = lane + kWave * g < E ? kept[lane + kWave * g] : 0;
  int cur_t = -1;
  int cur_e[8];  // final experts of token cur_t's slots (wave-uniform)
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) cur_e[jj] = -1;
  int p0, e0, tid[8];
  uint4 rw[NW];
  auto load = [&](int base) {
    const int rr = base + lane;
    p0 = rr < R ? route_pos0[rr] : 0;
    e0 = rr < R ? ids_in[rr] : 0;
    const bool drop = rr < R && p0 < 0;
    const uint4* src = reinterpret_cast<const uint4*>(rank + (size_t)(drop ? rr : 0) * kRerouteWideE);
#pragma unroll
    for (int w = 0; w < NW; ++w) rw[w] = (drop && 16 * w < E) ? src[w] : uint4{0u, 0u, 0u, 0u};
    const int t = drop ? rr / k : 0;
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) tid[jj] = (drop && jj < k) ? ids_in[t * k + jj] : 0;
  };
  load(0);
  for (int base = 0; base < R; base += kWave) {
    const int cp0 = p0, ce0 = e0;
    int ctid[8];
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) ctid[jj] = tid[jj];
    __syncthreads();  // the previous chunk's rank rows are no longer read
#pragma unroll
    for (int w = 0; w < NW; ++w) *reinterpret_cast<uint4*>(&s_rank[lane][16 * w]) = rw[w];
    __syncthreads();
    if (base + kWave < R) load(base + kWave);  // in flight during this chunk's walk
    const int rr = base + lane;
    if (rr < R && cp0 >= 0) {  // kept by the drop policy: same expert, same seat
      ids_out[rr] = ce0;
      slot[rr] = cp0 - offsets0[ce0];
    }
    uint64_t m = __ballot(rr < R && cp0 < 0);
    while (m) {
      const int b = __builtin_amdgcn_readfirstlane(__builtin_ctzll(m));
      m &= m - 1;
      const int r = base + b;
      const int t = r / k, j = r - t * k;
      if (t != cur_t) {
        cur_t = t;
#pragma unroll
        for (int jj = 0; jj < 8; ++jj)
          cur_e[jj] = jj < k ? __builtin_amdgcn_readlane(ctid[jj], b) : -1;
      }
      uint32_t key = 0xffffffffu;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const int e = lane + kWave * g;
        bool ok = e < E && fill[g] < C;
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) ok = ok && !(jj != j && cur_e[jj] == e);
        const uint32_t kk = ((uint32_t)s_rank[b][e] << 8) | (uint32_t)e;
        if (ok && kk < key) key = kk;
      }
#pragma unroll
      for (int o = kWave / 2; o >= 1; o >>= 1) {
        const uint32_t other = (uint32_t)__shfl_xor((int)key, o, kWave);
        key = other < key ? other : key;
      }
      key = (uint32_t)__builtin_amdgcn_readfirstlane((int)key);
      if (key != 0xffffffffu) {
        const int best = (int)(key & 255u);
        const int owner = best % kWave, gb = best / kWave;
        int mine = fill[0];
#pragma unroll
        for (int g = 1; g < G; ++g) mine = g == gb ? fill[g] : mine;
        const int seat = __builtin_amdgcn_readlane(mine, owner);
        if (lane == owner) {
#pragma unroll
          for (int g = 0; g < G; ++g)
            if (g == gb) fill[g] = seat + 1;
        }
        if (lane == 0) {
          slot[r] = seat;
          ids_out[r] = best;
        }
#pragma unroll
        for (int jj = 0; jj < 8; ++jj)
          if (jj == j) cur_e[jj] = best;
      } else {  // no expert with room: dropped after all (lane b's own expert)
        const int orig = __builtin_amdgcn_readlane(ce0, b);
        if (lane == 0) {
          ids_out[r] = orig;
          slot[r] = -1;
        }
      }
    }
  }
  int carry = 0;
  if (lane == 0) offsets[0] = 0;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int e = lane + kWave * g;
    const int f = e < E ? fill[g] : 0;
    const int incl = wave_incl_scan(f, lane);
    if (e < E) offsets[e + 1] = carry + incl;
    carry += __shfl(incl, kWave - 1, kWave);
  }
}

// Packed rows of the rerouted dispatch: route_pos[r] = offsets[ids[r]] +
// slot[r] (or -1), row_token[route_pos[r]] = r / k.
__global__ __launch_bounds__(256) void reroute_rows_kernel(const int32_t* __restrict__ ids,
                                                           const int32_t* __restrict__ slot,
                                                           const int32_t* __restrict__ offsets,
                                                           int R, int k,
                                                           int32_t* __restrict__ route_pos,
                                                           int32_t* __restrict__ row_token) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= R) return;
  const int sl = slot[r];
  if (sl < 0) {
    route_pos[r] = -1;
    return;
  }
  const int p = offsets[ids[r]] + sl;
  route_pos[r] = p;
  row_token[p] = r / k;
}

// The same result in parallel rounds.  A token's dropped routes are
// consecutive in arrival order and must take distinct experts, so the walk is
// a serial dictatorship over tokens: in token order, each token with n_t
// dropped routes takes its n_t best experts that still have a seat (its own
// experts excluded), its i-th dropped route the i-th best of them.  When every
// expert ranks tokens by one common priority, deferred acceptance with the
// tokens proposing ends in exactly that assignment (a standard property of
// matching under a common priority), and each of its rounds is parallel:
//   1. every token drops the experts that rejected it, then proposes along its
//      preference list (experts it holds originally and experts without a
//      free seat after the drop policy are skipped) until it holds n_t
//      experts again or the list ends;
//   2. every expert keeps the earliest tokens it holds, up to its free seats,
//      and rejects the rest.
// It ends after a round without proposals (each proposal moves a token's
// list pointer, so that round comes).  Seats follow token order among an
// expert's accepted routes, as in the walk.  One block of 1024 threads, laid
// out for T tokens (the bound on the tokens with drops), W = ceil(T / 32):
//   held  [E][W] uint32   bit a: token a holds (or is proposed to) expert e
//   dirty [W] uint32      bit a: token a was cut in the last round
// in a fixed LDS arena, shared by every wave, and the per-token state
//   hold  [T] uint64      experts token a holds
//   own   [T] uint64      experts token a had from the router (skipped)
//   first [T] int32       its first dropped route (its preference list is
//                         that route's row of experts in preference order)
//   tok   [T] uint16      token index of token a (token order)
//   need  [T] uint8       its dropped routes n_t
//   next  [T] uint8       next position of its preference list
// in the arena too when it fits (TOK_LDS), else in a global workspace region:
// each token's state is read and written only by the thread that owns the
// token, so it needs no sharing, only room.  Preference rows are read 16
// bytes at a time (a row is 64 bytes, 64-byte aligned); experts the token
// had and experts without a free seat are skipped as they come up.
constexpr int kDaThreads = 1024;
constexpr int kDaWaves = kDaThreads / kWave;
constexpr long kDaArena = 144L * 1024;
constexpr int kDaMaxT = 65535;  // token indices and seat prefixes fit uint16

// held and dirty from the arena's start; the per-token arrays from the
// arena's next byte (TOK_LDS) or from 0 in a global region.  lds_bytes and
// tok_bytes are the two footprints.
struct DaLayout {
  long held, dirty, hold, own, first, tok, need, next, lds_bytes, tok_bytes;
};
__host__ __device__ inline DaLayout da_layout(int T, int E, bool tok_lds) {
  const long W = (T + 31) / 32;
  DaLayout L;
  L.held = 0;
  L.dirty = L.held + (long)E * W * 4;
  const long shared_end = L.dirty + 4L * W;
  const long tb = tok_lds ? (shared_end + 7) & ~7L : 0;
  L.hold = tb;
  L.own = L.hold + 8L * T;
  L.first = L.own + 8L * T;
  L.tok = L.first + 4L * T;
  L.need = L.tok + ((2L * T + 3) & ~3L);
  L.next = L.need + T;
  const long end = L.next + T;
  L.tok_bytes = end - tb;
  L.lds_bytes = tok_lds ? end : shared_end;
  return L;
}

// The parallel reroute's workspace region: token-indexed arrays written by
// reroute_tok_at (tneed: dropped routes of token t, 0 for none; town:
// the experts the router gave it; tfirst: its first dropped route) and by
// reroute_da_kernel (tidx: its index among the tokens with drops; thold: the
// experts it holds at the end; gheld / gpre: the final per-expert bitmaps and
// seat prefixes), which reroute_seat_kernel reads; then, when the per-token
// state of the rounds does not fit LDS, that state (tok_bytes of da_layout).
struct RrLayout {
  long town, thold, tfirst, tidx, tneed, gheld, gpre, state, bytes;
};
__host__ __device__ inline RrLayout rr_layout(int T, int E, bool tok_lds) {
  const long W = (T + 31) / 32;
  RrLayout L;
  L.tneed = 0;  // read 16 bytes at a time
  L.town = (T + 15L) & ~15L;
  L.thold = L.town + 8L * T;
  L.tfirst = L.thold + 8L * T;
  L.tidx = L.tfirst + 4L * T;
  L.gheld = (L.tidx + 4L * T + 15) & ~15L;
  L.gpre = L.gheld + 4L * E * W;
  L.state = (L.gpre + 2L * E * W + 15) & ~15L;
  L.bytes = L.state + (tok_lds ? 0 : da_layout(T, E, false).tok_bytes);
  return L;
}

// byte p of a 16-byte chunk
__device__ __forceinline__ int chunk_byte(const u32x4_t& c, int p) {
  const int q = (p >> 2) & 3;
  const uint32_t w = q == 0 ? c[0] : q == 1 ? c[1] : q == 2 ? c[2] : c[3];
  return (int)((w >> ((p & 3) * 8)) & 0xFFu);
}

template <bool TOK_LDS>
__global__ __launch_bounds__(kDaThreads) void reroute_da_kernel(
    const uint8_t* __restrict__ order, const int32_t* __restrict__ offsets0,
    const int32_t* __restrict__ kept, int T, int E, int C, int32_t* __restrict__ offsets,
    uint8_t* __restrict__ region) {
  __shared__ __attribute__((aligned(16))) uint8_t arena[kDaArena];
  __shared__ int s_kept[kRerouteMaxE], s_free[kRerouteMaxE], s_new[kRerouteMaxE],
      s_fill[kRerouteMaxE];
  __shared__ int s_wsum[kDaWaves];
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wv = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int W = (T + 31) / 32;
  const DaLayout L = da_layout(T, E, TOK_LDS);
  const RrLayout G = rr_layout(T, E, TOK_LDS);
  const uint8_t* tneed = region + G.tneed;
  const uint64_t* town = reinterpret_cast<const uint64_t*>(region + G.town);
  const int32_t* tfirst = reinterpret_cast<const int32_t*>(region + G.tfirst);
  uint64_t* thold = reinterpret_cast<uint64_t*>(region + G.thold);
  int32_t* tidx = reinterpret_cast<int32_t*>(region + G.tidx);
  uint32_t* gheld = reinterpret_cast<uint32_t*>(region + G.gheld);
  uint16_t* gpre = reinterpret_cast<uint16_t*>(region + G.gpre);
  uint8_t* tok_state = region + G.state;
  uint32_t* held = reinterpret_cast<uint32_t*>(arena + L.held);
  // bit a: token a lost an expert in the last cut (or the rounds just began);
  // the others have nothing to do (they hold n_t experts or their list ran
  // out)
  uint32_t* dirty = reinterpret_cast<uint32_t*>(arena + L.dirty);
  uint8_t* const tb = TOK_LDS ? arena : tok_state;
  uint64_t* hold = reinterpret_cast<uint64_t*>(tb + L.hold);
  uint64_t* own = reinterpret_cast<uint64_t*>(tb + L.own);
  int32_t* first = reinterpret_cast<int32_t*>(tb + L.first);
  uint16_t* tok = reinterpret_cast<uint16_t*>(tb + L.tok);
  uint8_t* need = tb + L.need;
  uint8_t* next = tb + L.next;

  if (offsets0[E] >= (long)E * C) {  // every seat taken: the seats stay the drop policy's
    if (wv == 0) {
      const int inc = wave_incl_scan(lane < E ? kept[lane] : 0, lane);
      if (lane == 0) offsets[0] = 0;
      if (lane < E) offsets[lane + 1] = inc;
    }
    return;
  }
  if (tid < E) {
    const int kp = kept[tid];
    s_kept[tid] = kp;
    s_free[tid] = C > kp ? C - kp : 0;
    s_new[tid] = 0;
  }
  for (int i = tid; i < E * W; i += kDaThreads) held[i] = 0;
  for (int i = tid; i < W; i += kDaThreads) dirty[i] = ~0u;

  // tokens with dropped routes in token order: each thread a run of cpt
  // tokens (a multiple of 16, <= 64 as T <= 65535) read as 16-byte chunks of
  // tneed; a block scan of the run counts places them
  const int cpt = ((T + kDaThreads - 1) / kDaThreads + 15) & ~15;
  const int t0 = tid * cpt;
  uint64_t amask = 0;
  for (int q = 0; q < cpt; q += 16) {
    if (t0 + q >= T) break;
    const u32x4_t c = *reinterpret_cast<const u32x4_t*>(tneed + t0 + q);
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (chunk_byte(c, i) && t0 + q + i < T) amask |= 1ull << (q + i);
  }
  const int na = __popcll(amask);
  const int incl = wave_incl_scan(na, lane);
  if (lane == kWave - 1) s_wsum[wv] = incl;
  __syncthreads();
  int at = incl - na, an = 0;
  for (int w = 0; w < kDaWaves; ++w) {
    const int s = s_wsum[w];
    at += w < wv ? s : 0;
    an += s;
  }
  const int A = __builtin_amdgcn_readfirstlane(an);
  while (amask) {
    const int t = t0 + __builtin_ctzll(amask);
    tok[at] = (uint16_t)t;
    tidx[t] = at++;
    amask &= amask - 1;
  }
  __syncthreads();

  // per token: the experts it had, its first dropped route (every route of
  // a token shares the logits, so that route's order row is the token's
  // preference list) and n_t, from the token-indexed arrays
  for (int a0 = 0; a0 < A; a0 += kDaThreads) {
    const int a = a0 + tid;
    if (a >= A) continue;
    const int t = tok[a];
    own[a] = town[t];
    first[a] = tfirst[t];
    need[a] = tneed[t];
    next[a] = 0;
    hold[a] = 0;
  }
  __syncthreads();

  // Every branch around the round's barriers is wave-uniform: the per-token
  // loops run the same trip count on every lane (a lane past A idles in the
  // body), and the exit reads the block-wide OR as a scalar.  With per-lane
  // loop bounds (a = tid; a < A) the compiler may route the lanes that have
  // no token straight from one round's barriers to the next's, and a wave
  // holding both kinds of lane then meets the barriers out of step.
  const int wpl = (W + kWave - 1) / kWave;
  for (;;) {
    // rejections of the last round, then proposals up to n_t held experts
    int proposed = 0;
    for (int a0 = 0; a0 < A; a0 += kDaThreads) {
      const int a = a0 + tid;
      if (a >= A) continue;
      const int word = a >> 5;
      const uint32_t bit = 1u << (a & 31);
      if (!(dirty[word] & bit)) continue;
      atomicAnd(&dirty[word], ~bit);
      uint64_t h = hold[a];
      for (uint64_t m = h; m; m &= m - 1) {
        const int e = __builtin_ctzll(m);
        if (!(held[e * W + word] & bit)) h &= ~(1ull << e);
      }
      const int nd = need[a];
      int p = next[a];
      const uint8_t* pa = order + (size_t)first[a] * kRerouteMaxE;
      const uint64_t om = own[a];
      u32x4_t c = {0u, 0u, 0u, 0u};
      int cbase = -1;
      while ((int)__popcll(h) < nd && p < E) {
        if ((p & ~15) != cbase) {
          cbase = p & ~15;
          c = *reinterpret_cast<const u32x4_t*>(pa + cbase);
        }
        const int e = chunk_byte(c, p++);
        if (((om >> e) & 1) || s_free[e] <= 0) continue;  // had it, or no seat
        atomicOr(&held[e * W + word], bit);
        h |= 1ull << e;
        s_new[e] = 1;
        proposed = 1;
      }
      hold[a] = h;
      next[a] = (uint8_t)p;
    }
    if (!__builtin_amdgcn_readfirstlane(__syncthreads_or(proposed))) break;
    // each expert with proposals keeps its earliest s_free[e] tokens; lane i
    // of the expert's wave owns words [i*wpl, (i+1)*wpl)
    for (int e = wv; e < E; e += kDaWaves) {
      if (!__builtin_amdgcn_readfirstlane(s_new[e])) continue;
      uint32_t* row = held + e * W;
      const int cap = s_free[e];
      const int w0 = lane * wpl, w1 = min(W, w0 + wpl);
      int c = 0;
      for (int w = w0; w < w1; ++w) c += __popc(row[w]);
      const int inc = wave_incl_scan(c, lane);
      if (__shfl(inc, kWave - 1, kWave) > cap) {
        int before = inc - c;
        for (int w = w0; w < w1; ++w) {
          uint32_t v = row[w];
          const int pc = __popc(v);
          if (before >= cap) {
            v = 0;
          } else if (before + pc > cap) {  // keep the lowest cap - before bits
            uint32_t keep = 0;
            for (int q = cap - before; q > 0; --q) {
              const uint32_t low = v & (0u - v);
              keep |= low;
              v ^= low;
            }
            v = keep;
          }
          if (before + pc > cap) {
            const uint32_t cut = row[w] & ~v;
            row[w] = v;
            if (cut) atomicOr(&dirty[w], cut);  // these tokens propose again
          }
          before += pc;
        }
      }
      if (lane == 0) s_new[e] = 0;
    }
    __syncthreads();
  }

  // seats: per expert, the exclusive prefix of its words' popcounts; the
  // bitmaps, prefixes and final holdings go out to reroute_seat_kernel
  for (int e = wv; e < E; e += kDaWaves) {
    const uint32_t* row = held + e * W;
    const int w0 = lane * wpl, w1 = min(W, w0 + wpl);
    int c = 0;
    for (int w = w0; w < w1; ++w) c += __popc(row[w]);
    const int inc = wave_incl_scan(c, lane);
    int before = inc - c;
    for (int w = w0; w < w1; ++w) {
      const uint32_t v = row[w];
      gheld[e * W + w] = v;
      gpre[e * W + w] = (uint16_t)before;  // < T <= 65535
      before += __popc(v);
    }
    if (lane == kWave - 1) s_fill[e] = s_kept[e] + inc;
  }
  for (int a0 = 0; a0 < A; a0 += kDaThreads) {
    const int a = a0 + tid;
    if (a < A) thold[tok[a]] = hold[a];
  }
  __syncthreads();
  if (wv == 0) {
    const int f = lane < E ? s_fill[lane] : 0;
    const int inc = wave_incl_scan(f, lane);
    if (lane == 0) offsets[0] = 0;
    if (lane < E) offsets[lane + 1] = inc;
  }
}

// One thread per token, before the rounds: its kept routes keep expert and
// seat; its dropped routes are counted, its first one and its router
// experts noted (the rounds' input, token-indexed).
__device__ __forceinline__ void reroute_tok_at(
    int t, const int32_t* __restrict__ ids_in, const int32_t* __restrict__ route_pos0,
    const int32_t* __restrict__ offsets0, int T, int k, int E, int32_t* __restrict__ ids_out,
    int32_t* __restrict__ slot, uint8_t* __restrict__ region) {
  if (t >= T) return;
  const RrLayout G = rr_layout(T, E, true);
  uint64_t om = 0;
  int nd = 0, rf = -1;
  for (int j = 0; j < k; ++j) {
    const int r = t * k + j;
    const int p = route_pos0[r];
    const int e = ids_in[r];
    om |= 1ull << e;
    if (p >= 0) {
      ids_out[r] = e;
      slot[r] = p - offsets0[e];
    } else {
      if (rf < 0) rf = r;
      ++nd;
    }
  }
  region[G.tneed + t] = (uint8_t)nd;
  reinterpret_cast<uint64_t*>(region + G.town)[t] = om;
  reinterpret_cast<int32_t*>(region + G.tfirst)[t] = rf;
}

// The set-up before the rounds, in one launch: blocks below n_rank write the
// dropped routes' experts in preference order (reroute_rank_at), the rest
// the token arrays (reroute_tok_at); the two read only the dispatch.
__global__ __launch_bounds__(256) void reroute_prep_kernel(
    int n_rank, const float* __restrict__ logits, const int32_t* __restrict__ ids_in,
    const int32_t* __restrict__ route_pos0, const int32_t* __restrict__ offsets0, int T, int k,
    int E, int C, uint8_t* __restrict__ order, int32_t* __restrict__ ids_out,
    int32_t* __restrict__ slot, uint8_t* __restrict__ region) {
  const int b = blockIdx.x;
  if (b < n_rank)
    reroute_rank_at<true, kRerouteMaxE>((long)b * blockDim.x + threadIdx.x, logits, route_pos0,
                                        offsets0, T * k, k, E, C, order);
  else
    reroute_tok_at((b - n_rank) * blockDim.x + threadIdx.x, ids_in, route_pos0, offsets0, T, k, E,
                   ids_out, slot, region);
}

// One thread per token, after the rounds: a token with drops gives its i-th
// dropped route the i-th best expert it holds, at seat kept[e] + the number
// of accepted tokens before it (token order), or leaves it dropped when none
// is left.  With route_pos set, every route of the token also gets its
// packed row, route_pos[r] = offsets[e] + seat, and row_token of that row
// (reroute_rows_kernel's work, done per token: one launch fewer, worth it
// for a route or two per token; with k = 8 the per-thread stores of 8
// consecutive positions cost more than the launch).
__global__ __launch_bounds__(256) void reroute_seat_kernel(
    const uint8_t* __restrict__ order, const int32_t* __restrict__ ids_in,
    const int32_t* __restrict__ route_pos0, const int32_t* __restrict__ offsets0,
    const int32_t* __restrict__ kept, int T, int k, int E, int C, int32_t* __restrict__ ids_out,
    int32_t* __restrict__ slot, const uint8_t* __restrict__ region,
    const int32_t* __restrict__ offsets, int32_t* __restrict__ route_pos,
    int32_t* __restrict__ row_token) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= T) return;
  const RrLayout G = rr_layout(T, E, true);
  auto place = [&](int r, int e, int sl) {
    if (!route_pos) return;
    if (sl < 0) {
      route_pos[r] = -1;
      return;
    }
    const int p = offsets[e] + sl;
    route_pos[r] = p;
    row_token[p] = t;
  };
  if (region[G.tneed + t] == 0) {  // every route kept: the seats of the drop policy
    if (!route_pos) return;
    for (int j = 0; j < k; ++j) {
      const int r = t * k + j;
      const int e = ids_in[r];
      place(r, e, route_pos0[r] - offsets0[e]);
    }
    return;
  }
  const int W = (T + 31) / 32;
  // every seat taken: the rounds wrote nothing and every dropped route stays
  const bool full = offsets0[E] >= (long)E * C;
  const int a = full ? 0 : reinterpret_cast<const int32_t*>(region + G.tidx)[t];
  uint64_t h = full ? 0 : reinterpret_cast<const uint64_t*>(region + G.thold)[t];
  const int rf = reinterpret_cast<const int32_t*>(region + G.tfirst)[t];
  const uint32_t* gheld = reinterpret_cast<const uint32_t*>(region + G.gheld);
  const uint16_t* gpre = reinterpret_cast<const uint16_t*>(region + G.gpre);
  const int word = a >> 5;
  const uint32_t below = (1u << (a & 31)) - 1u;
  const uint8_t* pa = order + (size_t)rf * kRerouteMaxE;
  u32x4_t c = {0u, 0u, 0u, 0u};
  int cbase = -1;
  int p = 0;
  for (int j = 0; j < k; ++j) {
    const int r = t * k + j;
    const int p0 = route_pos0[r];
    if (p0 >= 0) {  // kept by the drop policy
      const int e0 = ids_in[r];
      place(r, e0, p0 - offsets0[e0]);
      continue;
    }
    int e = -1;
    while (h && p < E) {  // the next best held expert
      if ((p & ~15) != cbase) {
        cbase = p & ~15;
        c = *reinterpret_cast<const u32x4_t*>(pa + cbase);
      }
      const int x = chunk_byte(c, p++);
      if ((h >> x) & 1) {
        e = x;
        h &= ~(1ull << x);
        break;
      }
    }
    if (e < 0) {  // no expert with room: dropped after all
      ids_out[r] = ids_in[r];
      slot[r] = -1;
      place(r, 0, -1);
    } else {
      const int sl = kept[e] + gpre[e * W + word] + __popc(gheld[e * W + word] & below);
      ids_out[r] = e;
      slot[r] = sl;
      place(r, e, sl);
    }
  }
}

// The three reroute kernels by footprint: all state in LDS, the per-token
// state in the workspace, or the serial walk.
enum class RerouteKind { kDaLds, kDaGlobal, kWalk };
static RerouteKind reroute_kind(int T, int E) {
  if (T <= kDaMaxT && da_layout(T, E, true).lds_bytes <= kDaArena) return RerouteKind::kDaLds;
  if (T <= kDaMaxT && da_layout(T, E, false).lds_bytes <= kDaArena) return RerouteKind::kDaGlobal;
  return RerouteKind::kWalk;
}

long reroute_state_bytes(int T, int E) {
  const RerouteKind kind = reroute_kind(T, E);
  return kind == RerouteKind::kWalk ? 0 : rr_layout(T, E, kind == RerouteKind::kDaLds).bytes;
}

hipError_t launch_reroute(const float* logits, const int32_t* ids_in, const int32_t* route_pos0,
                          const int32_t* offsets0, const int32_t* kept, int T, int k, int E,
                          int C, int32_t* ids_out, int32_t* slot, int32_t* offsets,
                          int32_t* route_pos, int32_t* row_token, uint8_t* pref,
                          uint8_t* da_state, hipStream_t st) {
  const int R = T * k;
  if (E > kRerouteMaxE) {  // beyond one expert per lane: the wide walk
    if (R > 0) {
      const long threads = (long)R * kRerouteWideE;
      hipLaunchKernelGGL((reroute_rank_kernel<false, kRerouteWideE>),
                         dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st, logits,
                         route_pos0, offsets0, R, k, E, C, pref);
      hipError_t err = hipGetLastError();
      if (err != hipSuccess) return err;
    }
    hipLaunchKernelGGL(reroute_wide_kernel, dim3(1), dim3(kWave), 0, st, pref, ids_in, route_pos0,
                       offsets0, kept, T, k, E, C, ids_out, slot, offsets);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || R == 0) return err;
    hipLaunchKernelGGL(reroute_rows_kernel, dim3(ceil_div(R, 256)), dim3(256), 0, st, ids_out,
                       slot, offsets, R, k, route_pos, row_token);
    return hipGetLastError();
  }
  const RerouteKind kind = reroute_kind(T, E);
  if (kind == RerouteKind::kWalk) {
    if (R > 0) {
      const long threads = (long)R * kRerouteMaxE;
      hipLaunchKernelGGL((reroute_rank_kernel<false, kRerouteMaxE>),
                         dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st, logits,
                         route_pos0, offsets0, R, k, E, C, pref);
      hipError_t err = hipGetLastError();
      if (err != hipSuccess) return err;
    }
    hipLaunchKernelGGL(reroute_kernel, dim3(1), dim3(kWave), 0, st, pref, ids_in, route_pos0,
                       offsets0, kept, T, k, E, C, ids_out, slot, offsets);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || R == 0) return err;
    hipLaunchKernelGGL(reroute_rows_kernel, dim3(ceil_div(R, 256)), dim3(256), 0, st, ids_out,
                       slot, offsets, R, k, route_pos, row_token);
    return hipGetLastError();
  }
  // preference lists and token set-up in one launch, the rounds in one
  // workgroup, then the seats and packed rows per token
  const dim3 tgrid(ceil_div(T, 256));
  if (T > 0) {
    const int n_rank = (int)(((long)R * kRerouteMaxE + 255) / 256);
    hipLaunchKernelGGL(reroute_prep_kernel, dim3((unsigned)(n_rank + ceil_div(T, 256))),
                       dim3(256), 0, st, n_rank, logits, ids_in, route_pos0, offsets0, T, k, E, C,
                       pref, ids_out, slot, da_state);
  }
  if (kind == RerouteKind::kDaLds)
    hipLaunchKernelGGL(reroute_da_kernel<true>, dim3(1), dim3(kDaThreads), 0, st, pref, offsets0,
                       kept, T, E, C, offsets, da_state);
  else
    hipLaunchKernelGGL(reroute_da_kernel<false>, dim3(1), dim3(kDaThreads), 0, st, pref,
                       offsets0, kept, T, E, C, offsets, da_state);
  const bool rows_here = k <= 2;  // see reroute_seat_kernel
  if (T > 0)
    hipLaunchKernelGGL(reroute_seat_kernel, tgrid, dim3(256), 0, st, pref, ids_in, route_pos0,
                       offsets0, kept, T, k, E, C, ids_out, slot, da_state, offsets,
                       rows_here ? route_pos : nullptr, row_token);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || R == 0 || rows_here) return err;
  hipLaunchKernelGGL(reroute_rows_kernel, dim3(ceil_div(R, 256)), dim3(256), 0, st, ids_out, slot,
                     offsets, R, k, route_pos, row_token);
  return hipGetLastError();
}

// seats[e] = offsets[e+1] - offsets[e]
__global__ __launch_bounds__(256) void seats_kernel(const int32_t* __restrict__ offsets, int E,
                                                    int32_t* __restrict__ seats) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e < E) seats[e] = offsets[e + 1] - offsets[e];
}

hipError_t launch_seats(const int32_t* offsets, int E, int32_t* seats, hipStream_t st) {
  hipLaunchKernelGGL(seats_kernel, dim3(ceil_div(E, 256)), dim3(256), 0, st, offsets, E, seats);
  return hipGetLastError();
}

// Overflow policy "queue to the next micro-batch" ("Session 19", "Overflow
// policies": the overflowing route is processed in the next micro-batch).
// The dispatch is the drop policy over the arrival sequence -- the Q queued
// routes first, then the call's T*k routes -- run by the counting sort above
// with one route per arrival, so a packed row holds an arrival index a.  The
// row of arrival a is its carried row q_x[a] (a < Q) or its token's row
// x[(a - Q) / k].

// rows[p] = row of arrival arr[p] for p < count[0]; 16-byte chunks
__global__ __launch_bounds__(256) void queue_gather_kernel(const u32x4_t* __restrict__ x,
                                                           const u32x4_t* __restrict__ qx,
                                                           const int32_t* __restrict__ arr,
                                                           const int32_t* __restrict__ count,
                                                           int Q, int k, int cpr, long total,
                                                           u32x4_t* __restrict__ rows) {
  const long n = (long)count[0] * cpr;
  const long lim = n < total ? n : total;
  for (long g = (long)blockIdx.x * blockDim.x + threadIdx.x; g < lim;
       g += (long)gridDim.x * blockDim.x) {
    const long p = g / cpr;
    const int ch = (int)(g - p * cpr);
    const int a = arr[p];
    rows[g] = a < Q ? qx[(long)a * cpr + ch] : x[(long)((a - Q) / k) * cpr + ch];
  }
}

// The outgoing queue: the arrivals with pos < 0, in arrival order, by a
// stream compaction in one workgroup (ballots per wave, a prefix over the
// waves, a running count over chunks of 1024 arrivals).  Writes n_out, each
// entry's arrival, expert, gate and tag (queued: carried; new: tag_base +
// token).
__global__ __launch_bounds__(1024) void queue_compact_kernel(
    const int32_t* __restrict__ pos, int N, int Q, int k, const int32_t* __restrict__ q_ids,
    const float* __restrict__ q_gates, const int64_t* __restrict__ q_tags,
    const int32_t* __restrict__ ids, const float* __restrict__ gates, int64_t tag_base,
    int32_t* __restrict__ n_out, int32_t* __restrict__ arr, int32_t* __restrict__ out_ids,
    float* __restrict__ out_gates, int64_t* __restrict__ out_tags) {
  constexpr int NW = 1024 / kWave;
  __shared__ int s_wsum[NW];
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wv = __builtin_amdgcn_readfirstlane(tid / kWave);
  const uint64_t lt = lane ? (~0ull >> (kWave - lane)) : 0ull;
  int carry = 0;
  for (int base = 0; base < N; base += 1024) {  // same trip count on every lane
    const int a = base + tid;
    const bool wait = a < N && pos[a] < 0;
    const uint64_t m = __ballot(wait);
    if (lane == 0) s_wsum[wv] = __popcll(m);
    __syncthreads();
    int before = carry, chunk = 0;
    for (int w = 0; w < NW; ++w) {
      const int c = s_wsum[w];
      before += w < wv ? c : 0;
      chunk += c;
    }
    if (wait) {
      const int p = before + __popcll(m & lt);
      arr[p] = a;
      if (a < Q) {
        out_ids[p] = q_ids[a];
        out_gates[p] = q_gates[a];
        out_tags[p] = q_tags[a];
      } else {
        const int r = a - Q;
        out_ids[p] = ids[r];
        out_gates[p] = gates[r];
        out_tags[p] = tag_base + r / k;
      }
    }
    carry += chunk;
    __syncthreads();  // s_wsum is rewritten by the next chunk
  }
  if (tid == 0) n_out[0] = carry;
}

hipError_t launch_queue_gather(const void* x, const void* q_x, const int32_t* arr,
                               const int32_t* count, int Q, int k, long max_rows, long row_bytes,
                               void* rows, hipStream_t st) {
  const int cpr = (int)(row_bytes / 16);
  const long total = max_rows * cpr;
  if (total == 0) return hipSuccess;
  long blocks = (total + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(queue_gather_kernel, dim3((unsigned)blocks), dim3(256), 0, st,
                     reinterpret_cast<const u32x4_t*>(x), reinterpret_cast<const u32x4_t*>(q_x),
                     arr, count, Q, k, cpr, total, reinterpret_cast<u32x4_t*>(rows));
  return hipGetLastError();
}

hipError_t launch_queue_compact(const int32_t* pos, long N, int Q, int k, const int32_t* q_ids,
                                const float* q_gates, const int64_t* q_tags, const int32_t* ids,
                                const float* gates, int64_t tag_base, int32_t* n_out,
                                int32_t* arr, int32_t* out_ids, float* out_gates,
                                int64_t* out_tags, hipStream_t st) {
  hipLaunchKernelGGL(queue_compact_kernel, dim3(1), dim3(1024), 0, st, pos, (int)N, Q, k, q_ids,
                     q_gates, q_tags, ids, gates, tag_base, n_out, arr, out_ids, out_gates,
                     out_tags);
  return hipGetLastError();
}

int permute_nchunks(long R) { return (int)((R + kChunk - 1) / kChunk); }

hipError_t launch_permute_index(const int32_t* ids, int T, int k, int E, int C, int32_t* cnt_ws,
                                int32_t* counts, int32_t* kept, int32_t* offsets,
                                int32_t* route_pos, int32_t* row_token, hipStream_t st) {
  const int R = T * k;
  if (R <= kSmallMaxRoutes) {
#define PS(PT)                                                                                \
  hipLaunchKernelGGL(permute_small_kernel<PT>, dim3(1), dim3(kSmallThreads), 0, st, ids, R, k, E, \
                     C, counts, kept, offsets, route_pos, row_token)
    if (R <= kSmallThreads) PS(1);
    else if (R <= 2 * kSmallThreads) PS(2);
    else PS(4);
#undef PS
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
