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

// Overflow policy "reroute" ("Session 19", "Overflow policies": the
// overflowing route is handled by the token's next-best expert).  Routes
// keep the seats of the drop policy; then the dropped ones, in arrival
// order, each take the best-ranked expert of their token (logit descending,
// lower index first) that the token does not hold and that still has room.
// That is a greedy in arrival order -- every choice depends on the earlier
// ones -- so one wave walks the dropped routes one by one, after a parallel
// kernel has written every dropped route's rank of each expert (one byte
// each).  The walk stages a 64-route chunk's rank rows in LDS (the next
// chunk's are loaded while this one is walked); for a route, lane e reads
// its expert's rank and the choice is the lowest rank among the lanes with
// room that the token does not hold -- six ballots over the rank bits, no
// branches; lane e keeps expert e's seat count (E <= 64).
//   ids_out   final expert of every route; slot  seat at that expert, or -1
//   offsets   exclusive prefix of the seats used per expert
constexpr int kRerouteMaxE = 64;

// rank[r][e] = rank of expert e in dropped route r's preference order
// (experts ahead: larger logit, or equal logit and lower index); one thread
// per (r, e)
__global__ __launch_bounds__(256) void reroute_rank_kernel(const float* __restrict__ logits,
                                                           const int32_t* __restrict__ route_pos0,
                                                           int R, int k, int E,
                                                           uint8_t* __restrict__ rank) {
  const long g = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const int r = (int)(g / kRerouteMaxE), e = (int)(g % kRerouteMaxE);
  if (r >= R || e >= E || route_pos0[r] >= 0) return;
  const float* l = logits + (size_t)(r / k) * E;
  const float le = l[e];
  int rk = 0;
  for (int e2 = 0; e2 < E; ++e2) {
    const float l2 = l[e2];
    rk += (l2 > le) | ((l2 == le) & (e2 < e));
  }
  rank[(size_t)r * kRerouteMaxE + e] = (uint8_t)rk;
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

// Top-1 routing (k = 1) in parallel.  A token then holds no other expert, so
// the greedy above is a serial dictatorship: the dropped routes choose in
// arrival order, and every expert in effect ranks routes by that one order.
// When all experts share one priority order, deferred acceptance with the
// routes proposing ends in exactly the assignment of the serial dictatorship
// in that order, and each of its rounds is parallel: every unplaced route
// proposes to its next preferred expert among those with a free seat after
// the drop policy, each expert keeps the earliest routes it holds or was
// proposed, up to its free seats, and rejects the rest, and the rejected
// routes move one rank on.  It ends after a round without proposals (each
// proposal moves a route's rank or places it, so that round comes).  Seats
// follow arrival order among an expert's accepted routes, as in the walk.
// One block of 1024 threads; the state sits in dynamic LDS, sized for R
// routes (the bound on the dropped ones), W = ceil(R / 32):
//   held  [E][W] uint32   bit j: dropped route j is held by / proposed to e
//   drop  [R] uint16      route index of dropped route j (arrival order)
//   pref  [R][E] uint8    expert at each preference rank of route j, or
//                         kNoExpert where that expert had no free seat (after
//                         the rounds the area holds [E][W] int seat prefixes)
//   next  [R] uint8       next rank route j tries
//   cur   [R] uint8       expert route j is proposed to or held by, or kNoExpert
constexpr int kDaThreads = 1024;
constexpr int kDaWaves = kDaThreads / kWave;
constexpr uint8_t kNoExpert = 0xFF;
constexpr long kDaMaxLds = 60L * 1024;  // with the static arrays, under 64 KB
constexpr int kDaMaxR = 65535;          // route indices fit uint16

struct DaLayout {
  long held, drop, pref, next, cur, bytes;
};
__host__ __device__ inline DaLayout da_layout(int R, int E) {
  const long W = (R + 31) / 32;
  DaLayout L;
  L.held = 0;
  L.drop = (long)E * W * 4;
  L.pref = L.drop + ((2L * R + 3) & ~3L);
  const long pref_bytes = (long)R * E > (long)E * W * 4 ? (long)R * E : (long)E * W * 4;
  L.next = L.pref + ((pref_bytes + 3) & ~3L);
  L.cur = L.next + R;
  L.bytes = L.cur + R;
  return L;
}

__global__ __launch_bounds__(kDaThreads) void reroute_da_kernel(
    const uint8_t* __restrict__ rank, const int32_t* __restrict__ ids_in,
    const int32_t* __restrict__ route_pos0, const int32_t* __restrict__ offsets0,
    const int32_t* __restrict__ kept, int R, int E, int C, int32_t* __restrict__ ids_out,
    int32_t* __restrict__ slot, int32_t* __restrict__ offsets) {
  extern __shared__ __attribute__((aligned(16))) uint32_t s_dyn[];
  __shared__ int s_kept[kRerouteMaxE], s_free[kRerouteMaxE], s_new[kRerouteMaxE],
      s_fill[kRerouteMaxE];
  __shared__ int s_wsum[kDaWaves];
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wv = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int W = (R + 31) / 32;
  const DaLayout L = da_layout(R, E);
  uint8_t* base = reinterpret_cast<uint8_t*>(s_dyn);
  uint32_t* held = reinterpret_cast<uint32_t*>(base + L.held);
  uint16_t* drop = reinterpret_cast<uint16_t*>(base + L.drop);
  uint8_t* pref = base + L.pref;
  uint8_t* next = base + L.next;
  uint8_t* cur = base + L.cur;

  if (tid < E) {
    const int kp = kept[tid];
    s_kept[tid] = kp;
    s_free[tid] = C > kp ? C - kp : 0;
    s_new[tid] = 0;
  }
  for (int i = tid; i < E * W; i += kDaThreads) held[i] = 0;

  // dropped routes in arrival order (each thread a run of cpt routes; block
  // scan of the run counts); kept routes keep expert and seat
  const int cpt = (R + kDaThreads - 1) / kDaThreads;  // <= 64
  const int r0 = tid * cpt, r1 = min(R, r0 + cpt);
  int nd = 0;
  uint64_t dmask = 0;
  for (int r = r0; r < r1; ++r) {
    const int p = route_pos0[r];
    if (p < 0) {
      dmask |= 1ull << (r - r0);
      ++nd;
    } else {
      const int e = ids_in[r];
      ids_out[r] = e;
      slot[r] = p - offsets0[e];
    }
  }
  const int incl = wave_incl_scan(nd, lane);
  if (lane == kWave - 1) s_wsum[wv] = incl;
  __syncthreads();
  int at = incl - nd, rd = 0;
  for (int w = 0; w < kDaWaves; ++w) {
    const int s = s_wsum[w];
    at += w < wv ? s : 0;
    rd += s;
  }
  const int Rd = __builtin_amdgcn_readfirstlane(rd);
  while (dmask) {
    drop[at++] = (uint16_t)(r0 + __builtin_ctzll(dmask));
    dmask &= dmask - 1;
  }
  __syncthreads();

  // preference lists: pref[j][rank of e] = e when e has a free seat
  for (int i = tid; i < Rd * E; i += kDaThreads) {
    const int j = i / E, e = i - j * E;
    const int rk = rank[(size_t)drop[j] * kRerouteMaxE + e];
    pref[j * E + rk] = s_free[e] > 0 ? (uint8_t)e : kNoExpert;
  }
  for (int j = tid; j < Rd; j += kDaThreads) {
    next[j] = 0;
    cur[j] = kNoExpert;
  }
  __syncthreads();

  // The round loop keeps every branch around its barriers wave-uniform: the
  // per-route loops run the same trip count on every lane (a lane past Rd
  // idles in the body), and the exit reads the block-wide OR as a scalar.
  // With a per-lane loop bound (j = tid; j < Rd) the compiler may route the
  // lanes that have no route straight from one round's barriers to the
  // next's, and a wave holding both kinds of lane then meets the barriers
  // out of step with the others.
  for (;;) {
    // proposals of the unplaced routes
    int proposed = 0;
    for (int j0 = 0; j0 < Rd; j0 += kDaThreads) {
      const int j = j0 + tid;
      if (j >= Rd || cur[j] != kNoExpert) continue;
      const uint8_t* pj = pref + j * E;
      int p = next[j];
      while (p < E && pj[p] == kNoExpert) ++p;
      next[j] = (uint8_t)p;
      if (p < E) {
        const int e = pj[p];
        atomicOr(&held[e * W + (j >> 5)], 1u << (j & 31));
        cur[j] = (uint8_t)e;
        s_new[e] = 1;
        proposed = 1;
      }
    }
    if (!__builtin_amdgcn_readfirstlane(__syncthreads_or(proposed))) break;
    // each expert with proposals keeps its earliest s_free[e] routes; lane i
    // of the expert's wave owns words [i*wpl, (i+1)*wpl)
    const int wpl = (W + kWave - 1) / kWave;
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
          if (before + pc > cap) row[w] = v;
          before += pc;
        }
      }
      if (lane == 0) s_new[e] = 0;
    }
    __syncthreads();
    // rejected routes (their bit cleared) move one rank on
    for (int j0 = 0; j0 < Rd; j0 += kDaThreads) {
      const int j = j0 + tid;
      if (j >= Rd) continue;
      const int e = cur[j];
      if (e != kNoExpert && !((held[e * W + (j >> 5)] >> (j & 31)) & 1u)) {
        cur[j] = kNoExpert;
        next[j] = (uint8_t)(next[j] + 1);
      }
    }
  }

  // seats: per expert, the exclusive prefix of its words' popcounts (into
  // the preference area, no longer read), then each route's rank among the
  // accepted ones
  int32_t* pre = reinterpret_cast<int32_t*>(pref);
  {
    const int wpl = (W + kWave - 1) / kWave;
    for (int e = wv; e < E; e += kDaWaves) {
      const uint32_t* row = held + e * W;
      const int w0 = lane * wpl, w1 = min(W, w0 + wpl);
      int c = 0;
      for (int w = w0; w < w1; ++w) c += __popc(row[w]);
      const int inc = wave_incl_scan(c, lane);
      int before = inc - c;
      for (int w = w0; w < w1; ++w) {
        pre[e * W + w] = before;
        before += __popc(row[w]);
      }
      if (lane == kWave - 1) s_fill[e] = s_kept[e] + inc;
    }
  }
  __syncthreads();
  for (int j = tid; j < Rd; j += kDaThreads) {
    const int r = drop[j], e = cur[j];
    if (e == kNoExpert) {  // no expert with room: dropped after all
      ids_out[r] = ids_in[r];
      slot[r] = -1;
    } else {
      const int w = j >> 5;
      ids_out[r] = e;
      slot[r] = s_kept[e] + pre[e * W + w] + __popc(held[e * W + w] & ((1u << (j & 31)) - 1u));
    }
  }
  if (wv == 0) {
    const int f = lane < E ? s_fill[lane] : 0;
    const int inc = wave_incl_scan(f, lane);
    if (lane == 0) offsets[0] = 0;
    if (lane < E) offsets[lane + 1] = inc;
  }
}

hipError_t launch_reroute(const float* logits, const int32_t* ids_in, const int32_t* route_pos0,
                          const int32_t* offsets0, const int32_t* kept, int T, int k, int E,
                          int C, int32_t* ids_out, int32_t* slot, int32_t* offsets,
                          int32_t* route_pos, int32_t* row_token, uint8_t* pref,
                          hipStream_t st) {
  const int R = T * k;
  if (R > 0) {
    const long threads = (long)R * kRerouteMaxE;
    hipLaunchKernelGGL(reroute_rank_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                       st, logits, route_pos0, R, k, E, pref);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  const long da_bytes = da_layout(R, E).bytes;
  if (k == 1 && R <= kDaMaxR && da_bytes <= kDaMaxLds) {
    hipLaunchKernelGGL(reroute_da_kernel, dim3(1), dim3(kDaThreads), (unsigned)da_bytes, st, pref,
                       ids_in, route_pos0, offsets0, kept, R, E, C, ids_out, slot, offsets);
  } else {
    hipLaunchKernelGGL(reroute_kernel, dim3(1), dim3(kWave), 0, st, pref, ids_in, route_pos0,
                       offsets0, kept, T, k, E, C, ids_out, slot, offsets);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || R == 0) return err;
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
// with one route per arrival, so a packed row holds an arrival index a.
// These kernels turn that into source rows of the row buffer [token rows;
// queued rows] and build the outgoing queue.

// row_token[p] = a  ->  the row of arrival a in [x (T rows); queued rows]
__global__ __launch_bounds__(256) void queue_src_kernel(const int32_t* __restrict__ offsets, int E,
                                                        int Q, int T, int k, long R_max,
                                                        int32_t* __restrict__ row_token) {
  const long p = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (p >= R_max || p >= offsets[E]) return;
  const int a = row_token[p];
  row_token[p] = a < Q ? T + a : (a - Q) / k;
}

// flags[a] = 0 for an arrival that waits again (pos < 0), -1 (no key) else
__global__ __launch_bounds__(256) void queue_flags_kernel(const int32_t* __restrict__ pos, long N,
                                                          int32_t* __restrict__ flags) {
  const long a = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (a < N) flags[a] = pos[a] < 0 ? 0 : -1;
}

// Entry p < n_out of the outgoing queue from its arrival arr[p]: expert,
// gate, tag and the source row of its token row.
__global__ __launch_bounds__(256) void queue_out_kernel(
    const int32_t* __restrict__ arr, const int32_t* __restrict__ n_out, long N, int Q, int T, int k,
    const int32_t* __restrict__ q_ids, const float* __restrict__ q_gates,
    const int64_t* __restrict__ q_tags, const int32_t* __restrict__ ids,
    const float* __restrict__ gates, int64_t tag_base, int32_t* __restrict__ out_ids,
    float* __restrict__ out_gates, int64_t* __restrict__ out_tags, int32_t* __restrict__ src) {
  const long p = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (p >= N || p >= n_out[0]) return;
  const int a = arr[p];
  if (a < Q) {
    out_ids[p] = q_ids[a];
    out_gates[p] = q_gates[a];
    out_tags[p] = q_tags[a];
    src[p] = T + a;
  } else {
    const int r = a - Q;
    out_ids[p] = ids[r];
    out_gates[p] = gates[r];
    out_tags[p] = tag_base + r / k;
    src[p] = r / k;
  }
}

hipError_t launch_queue_src(const int32_t* offsets, int E, int Q, int T, int k, long R_max,
                            int32_t* row_token, hipStream_t st) {
  if (R_max <= 0) return hipSuccess;
  hipLaunchKernelGGL(queue_src_kernel, dim3((unsigned)((R_max + 255) / 256)), dim3(256), 0, st,
                     offsets, E, Q, T, k, R_max, row_token);
  return hipGetLastError();
}

hipError_t launch_queue_out(const int32_t* pos, long N, int Q, int T, int k, const int32_t* q_ids,
                            const float* q_gates, const int64_t* q_tags, const int32_t* ids,
                            const float* gates, int64_t tag_base, int32_t* flags, int32_t* cnt_ws,
                            int32_t* n_out, int32_t* kept1, int32_t* off1, int32_t* qpos,
                            int32_t* arr, int32_t* out_ids, float* out_gates, int64_t* out_tags,
                            int32_t* src, hipStream_t st) {
  if (N <= 0) {
    // an empty arrival sequence still reports an empty queue
    return launch_permute_index(flags, 0, 1, 1, -1, cnt_ws, n_out, kept1, off1, qpos, arr, st);
  }
  const unsigned blocks = (unsigned)((N + 255) / 256);
  hipLaunchKernelGGL(queue_flags_kernel, dim3(blocks), dim3(256), 0, st, pos, N, flags);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  // one key: the waiting arrivals in arrival order (counting sort, no capacity)
  err = launch_permute_index(flags, (int)N, 1, 1, -1, cnt_ws, n_out, kept1, off1, qpos, arr, st);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(queue_out_kernel, dim3(blocks), dim3(256), 0, st, arr, n_out, N, Q, T, k,
                     q_ids, q_gates, q_tags, ids, gates, tag_base, out_ids, out_gates, out_tags,
                     src);
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
