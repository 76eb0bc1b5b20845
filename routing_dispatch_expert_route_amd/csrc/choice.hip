// choice.hip -- expert-choice routing: the experts pick their tokens.
//
// "MoE Inference Visualized", "Why MoE Matters for Infrastructure": against
// load imbalance the experts can choose the tokens instead of the tokens
// choosing experts; every expert then receives the same number of rows.
// The page names the idea only.  Reading used here: the score of (t, e) is
// the full softmax probability of the router logits; expert e keeps the
// Ce = min(C, T) tokens of largest score, the lower token index first among
// equal scores; a kept pair's gate is its score; a token may be kept by any
// number of experts, none included.
//
// ec_scores_kernel  softmax of each token's logits -> scores [T][E] (when
//                   asked for) and keys [E][T] (the score's bits,
//                   expert-major so that one expert's column is contiguous;
//                   scores are >= +0, so their bits order like the values;
//                   read back as floats they are also the gates).
// ec_select_kernel  one block per expert, the column in registers (thread i
//                   holds tokens c*NT + i).  The Ce-th largest key is found
//                   two bits per round (the largest thr with count(key >=
//                   thr) >= Ce; each round counts three candidates: per-lane
//                   counts, a wave sum by DPP, a block sum through LDS) and
//                   stops early once a candidate splits off exactly Ce keys.
//                   Seating then takes the keys above thr and the first
//                   Ce - count(key > thr) keys equal to it in token order
//                   (per-chunk wave counts, one barrier, prefixes), so
//                   expert e's rows e*Ce .. e*Ce+Ce-1 list its tokens in
//                   increasing index; the route table is written
//                   expert-major [E][T] (coalesced).  No atomics: the result
//                   is unique.
// ec_transpose_kernel  the [T][E] route table for callers that ask for it.
#include "common.h"
#include "launch.h"

namespace moe {

constexpr int kScoreTok = 32;   // tokens per block of the score kernel
constexpr int kScoreLanes = 8;  // threads per token

__global__ __launch_bounds__(256) void ec_scores_kernel(const float* __restrict__ logits, int T,
                                                        int E, float* __restrict__ scores,
                                                        uint32_t* __restrict__ keys) {
  extern __shared__ float s_l[];  // [kScoreTok][E+1]
  const int t0 = blockIdx.x * kScoreTok;
  const int nt = min(kScoreTok, T - t0);
  const int stride = E + 1;
  const int n = nt * E;
  const float* src = logits + (size_t)t0 * E;
  for (int i = threadIdx.x; i < n; i += blockDim.x) s_l[(i / E) * stride + i % E] = src[i];
  __syncthreads();
  const int j = threadIdx.x / kScoreLanes;  // token of this thread
  const int q = threadIdx.x % kScoreLanes;  // its share of the experts
  if (j < nt) {
    float* row = s_l + j * stride;
    float m = -INFINITY;
    for (int e = q; e < E; e += kScoreLanes) m = fmaxf(m, row[e]);
#pragma unroll
    for (int o = 1; o < kScoreLanes; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, kScoreLanes));
    float sum = 0.0f;
    for (int e = q; e < E; e += kScoreLanes) {
      const float v = expf(row[e] - m);
      row[e] = v;
      sum += v;
    }
#pragma unroll
    for (int o = 1; o < kScoreLanes; o <<= 1) sum += __shfl_xor(sum, o, kScoreLanes);
    const float inv = 1.0f / sum;
    for (int e = q; e < E; e += kScoreLanes) row[e] *= inv;
  }  // the shuffles stay inside groups of kScoreLanes lanes, all on one token
  __syncthreads();
  if (scores) {
    float* dst = scores + (size_t)t0 * E;
    for (int i = threadIdx.x; i < n; i += blockDim.x) dst[i] = s_l[(i / E) * stride + i % E];
  }
  // expert-major keys: consecutive threads take consecutive tokens
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const int e = i / nt, jj = i % nt;
    keys[(size_t)e * T + t0 + jj] = __float_as_uint(s_l[jj * stride + e]);
  }
}

// Sum of v over the 64 lanes of the wave, in every lane: pairs and quads by
// quad permutes, the 16-lane row by rotations of 4 and 8 (every source lane
// is valid, so no lane is masked), then the four rows.
__device__ __forceinline__ uint32_t wave_sum(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xf, 0xf, false);   // quad [1,0,3,2]
  v += (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xf, 0xf, false);   // quad [2,3,0,1]
  v += (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x124, 0xf, 0xf, false);  // row_ror:4
  v += (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x128, 0xf, 0xf, false);  // row_ror:8
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 0) +
         (uint32_t)__builtin_amdgcn_readlane((int)v, 16) +
         (uint32_t)__builtin_amdgcn_readlane((int)v, 32) +
         (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
}

// NT threads, KPT keys per thread (T <= NT * KPT); thread i holds tokens
// c*NT + i (coalesced loads and stores).  Writes the expert-major route
// table pos_et[e][t] (row e*Ce + i, or -1), row_token and offsets.
template <int NT, int KPT>
__global__ __launch_bounds__(NT) void ec_select_kernel(const uint32_t* __restrict__ keys, int T,
                                                       int E, int Ce,
                                                       int32_t* __restrict__ pos_et,
                                                       int32_t* __restrict__ row_token,
                                                       int32_t* __restrict__ offsets) {
  constexpr int NW = NT / 64;
  // per-wave counts, two 16-bit counts to a dword
  __shared__ uint32_t s_a[2][NW], s_b[2][NW];
  __shared__ uint32_t s_c[KPT][NW];  // seating: per-chunk, per-wave counts
  const int e = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const uint32_t* col = keys + (size_t)e * T;
  uint32_t key[KPT];
#pragma unroll
  for (int c = 0; c < KPT; ++c) {
    const int t = c * NT + tid;
    key[c] = t < T ? col[t] : 0u;
  }
  // Consecutive rounds use the two halves of s_a / s_b in turn: a round's
  // writes follow the previous round's barrier, which every thread reaches
  // only after reading the half written two rounds before.
  int par = 0;
  auto block_sum = [&](uint32_t wa, uint32_t wb, uint32_t* ta, uint32_t* tb) {
    if (lane == 0) {
      s_a[par][wid] = wa;
      s_b[par][wid] = wb;
    }
    __syncthreads();
    uint32_t a = 0, b = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      a += s_a[par][w];
      b += s_b[par][w];
    }
    *ta = a;
    *tb = b;
    par ^= 1;
  };
  // Block counts of the keys >= v[0..nv-1].  Padding keys are 0 and every
  // candidate is >= 1, so they never count.  Counts travel two to a dword
  // (at most T <= 32768 each).
  auto count_ge = [&](const uint32_t* v, int nv, int* total) {
    uint32_t n01 = 0, n2 = 0;
#pragma unroll
    for (int c = 0; c < KPT; ++c) {
      n01 += (uint32_t)(key[c] >= v[0]);
      if (nv > 1) n01 += (uint32_t)(key[c] >= v[1]) << 16;
      if (nv > 2) n2 += (uint32_t)(key[c] >= v[2]);
    }
    uint32_t ta = 0, tb = 0;
    block_sum(wave_sum(n01), nv > 2 ? wave_sum(n2) : 0u, &ta, &tb);
    total[0] = (int)(ta & 0xffffu);
    total[1] = (int)(ta >> 16);
    total[2] = (int)tb;
  };
  // thr = the Ce-th largest key: the largest value with count(key >= thr)
  // >= Ce (count(key >= 0) = T >= Ce), two bits per round, largest bits
  // first.  When a candidate splits off exactly Ce keys the set is known:
  // every key >= it, and none equal to the boundary is needed.
  uint32_t thr = 0;
  int n_gt = -1;
  for (int lo = 30; lo >= 0 && n_gt < 0; lo -= 2) {
    uint32_t v[3];
#pragma unroll
    for (int j = 0; j < 3; ++j) v[j] = thr | (uint32_t)(j + 1) << lo;
    int tot[3];
    count_ge(v, 3, tot);
    // counts fall as the candidate grows: take the largest that keeps Ce
    int jj = 0;
#pragma unroll
    for (int j = 0; j < 3; ++j)
      if (tot[j] >= Ce) jj = j + 1;
    if (jj > 0) {
      thr = v[jj - 1];
      if (tot[jj - 1] == Ce) {  // block-uniform
        thr -= 1u;              // "key > thr" is now exactly "key >= v"
        n_gt = Ce;
      }
    }
  }
  if (n_gt < 0) {
    if (thr == 0xffffffffu) {
      n_gt = 0;
    } else {
      uint32_t v[1] = {thr + 1u};
      int tot[3];
      count_ge(v, 1, tot);
      n_gt = tot[0];
    }
  }
  const int need = Ce - n_gt;  // tokens equal to thr to seat, in token order
  // Seating in token order: every wave's counts above / equal to thr per
  // chunk (ballots), one barrier, then each chunk's prefix over the earlier
  // chunks and the earlier waves of this one.
  const int nch = (T + NT - 1) / NT;  // chunks holding tokens
  const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
  for (int c = 0; c < KPT; ++c) {
    if (c >= nch) break;  // block-uniform
    const bool valid = c * NT + tid < T;
    const uint64_t mg = __ballot(valid && key[c] > thr);
    const uint64_t me = __ballot(valid && key[c] == thr);
    if (lane == 0) s_c[c][wid] = (uint32_t)__popcll(mg) | (uint32_t)__popcll(me) << 16;
  }
  __syncthreads();
  uint32_t run = 0;  // above | equal << 16 over the earlier chunks
#pragma unroll
  for (int c = 0; c < KPT; ++c) {
    if (c >= nch) break;  // block-uniform
    const int t = c * NT + tid;
    const bool valid = t < T;
    const bool gt = valid && key[c] > thr;
    const bool eq = valid && key[c] == thr;
    const uint64_t mg = __ballot(gt), me = __ballot(eq);
    uint32_t before = run, total = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const uint32_t x = s_c[c][w];
      if (w < wid) before += x;
      total += x;
    }
    run += total;
    const int gb = (int)(before & 0xffffu) + __popcll(mg & below);
    const int eb = (int)(before >> 16) + __popcll(me & below);
    // seated: above thr, or among the first `need` equal to it; the row
    // index is the number of seated tokens before t (< Ce by the choice of
    // thr; the bound is kept for arbitrary key bits)
    const int pos = gb + min(eb, need);
    const bool sel = (gt || (eq && eb < need)) && pos < Ce;
    if (valid) pos_et[(size_t)e * T + t] = sel ? e * Ce + pos : -1;
    if (sel) row_token[e * Ce + pos] = t;
  }
  if (tid == 0) {
    offsets[e] = e * Ce;
    if (e == E - 1) offsets[E] = E * Ce;
  }
}

// route_pos[t][e] = pos_et[e][t], through a tile of kTrTok tokens in LDS
// (E * (kTrTok + 1) ints: 33 KiB at E = 256).
constexpr int kTrTok = 32;
__global__ __launch_bounds__(256) void ec_transpose_kernel(const int32_t* __restrict__ pos_et,
                                                           int T, int E,
                                                           int32_t* __restrict__ route_pos) {
  extern __shared__ int32_t s_t[];  // [E][kTrTok + 1]
  const int t0 = blockIdx.x * kTrTok;
  const int nt = min(kTrTok, T - t0);
  for (int i = threadIdx.x; i < E * kTrTok; i += blockDim.x) {
    const int e = i / kTrTok, j = i % kTrTok;
    if (j < nt) s_t[e * (kTrTok + 1) + j] = pos_et[(size_t)e * T + t0 + j];
  }
  __syncthreads();
  for (int i = threadIdx.x; i < nt * E; i += blockDim.x) {
    const int j = i / E, e = i % E;
    route_pos[(size_t)(t0 + j) * E + e] = s_t[e * (kTrTok + 1) + j];
  }
}

hipError_t launch_expert_choice(const float* logits, int T, int E, int Ce, float* scores,
                                uint32_t* keys, int32_t* pos_et, int32_t* route_pos,
                                int32_t* row_token, int32_t* offsets, hipStream_t st) {
  // T = 0: no scores; the select blocks still write offsets (all zero)
  if (T > 0) {
    const size_t lds = (size_t)kScoreTok * (E + 1) * sizeof(float);
    hipLaunchKernelGGL(ec_scores_kernel, dim3(ceil_div(T, kScoreTok)),
                       dim3(kScoreTok * kScoreLanes), lds, st, logits, T, E, scores, keys);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  // 256 threads (a wave per SIMD: no repeated reductions) up to 4096
  // tokens, 1024 above (more waves to hide the per-round latency)
#define SEL(NT_, K)                                                                        \
  hipLaunchKernelGGL((ec_select_kernel<NT_, K>), dim3(E), dim3(NT_), 0, st, keys, T, E, Ce, \
                     pos_et, row_token, offsets)
  if (T <= 512) SEL(256, 2);
  else if (T <= 1024) SEL(256, 4);
  else if (T <= 2048) SEL(256, 8);
  else if (T <= 4096) SEL(256, 16);
  else if (T <= 8192) SEL(1024, 8);
  else if (T <= 16384) SEL(1024, 16);
  else if (T <= 32768) SEL(1024, 32);
  else return hipErrorInvalidValue;
#undef SEL
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || !route_pos || T == 0) return err;
  hipLaunchKernelGGL(ec_transpose_kernel, dim3(ceil_div(T, kTrTok)), dim3(256),
                     (size_t)E * (kTrTok + 1) * sizeof(int32_t), st, pos_et, T, E, route_pos);
  return hipGetLastError();
}

}  // namespace moe
