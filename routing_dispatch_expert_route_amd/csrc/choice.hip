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
// ec_scores_kernel  softmax of each token's logits -> scores [T][E] (the
//                   combine's gates) and keys [E][T] (the score's bits,
//                   expert-major so that one expert's column is contiguous;
//                   scores are >= +0, so their bits order like the values).
// ec_select_kernel  one block of 1024 threads per expert, the column in
//                   registers.  The Ce-th largest key is found bit by bit
//                   (the largest thr with count(key >= thr) >= Ce, 32 counts
//                   over the block, each by wave ballots); one ordered pass
//                   then seats the keys above it and the first
//                   Ce - count(key > thr) keys equal to it, in token order,
//                   so expert e's rows e*Ce .. e*Ce+Ce-1 list its tokens in
//                   increasing index.  No atomics: the result is unique.
#include "common.h"
#include "launch.h"

namespace moe {

constexpr int kScoreTok = 32;   // tokens per block of the score kernel
constexpr int kScoreLanes = 8;  // threads per token
constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;

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
  float* dst = scores + (size_t)t0 * E;
  for (int i = threadIdx.x; i < n; i += blockDim.x) dst[i] = s_l[(i / E) * stride + i % E];
  // expert-major keys: consecutive threads take consecutive tokens
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const int e = i / nt, jj = i % nt;
    keys[(size_t)e * T + t0 + jj] = __float_as_uint(s_l[jj * stride + e]);
  }
}

// KPT keys per thread: T <= 1024 * KPT
template <int KPT>
__global__ __launch_bounds__(kSelThreads) void ec_select_kernel(
    const uint32_t* __restrict__ keys, int T, int E, int Ce, int32_t* __restrict__ route_pos,
    int32_t* __restrict__ row_token, int32_t* __restrict__ offsets) {
  __shared__ int s_w[2][2][kSelWaves];  // [round parity][count kind][wave]
  const int e = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const uint32_t* col = keys + (size_t)e * T;
  uint32_t key[KPT];
#pragma unroll
  for (int c = 0; c < KPT; ++c) {
    const int t = c * kSelThreads + tid;
    key[c] = t < T ? col[t] : 0u;
  }
  if (tid == 0) {
    offsets[e] = e * Ce;
    if (e == E - 1) offsets[E] = E * Ce;
  }
  // Block-wide count of the valid keys >= v.  Consecutive rounds use the
  // two halves of s_w in turn: a round's writes follow the previous
  // round's barrier, which every thread reaches only after reading the
  // half written two rounds before.
  int par = 0;
  auto count_ge = [&](uint32_t v) {
    int cnt = 0;
#pragma unroll
    for (int c = 0; c < KPT; ++c)
      cnt += __popcll(__ballot(c * kSelThreads + tid < T && key[c] >= v));
    if (lane == 0) s_w[par][0][wid] = cnt;
    __syncthreads();
    int total = 0;
#pragma unroll
    for (int w = 0; w < kSelWaves; ++w) total += s_w[par][0][w];
    par ^= 1;
    return total;
  };
  // thr = the Ce-th largest key (count(key >= 0) = T >= Ce)
  uint32_t thr = 0;
  for (int b = 31; b >= 0; --b) {
    const uint32_t cand = thr | (1u << b);
    if (count_ge(cand) >= Ce) thr = cand;
  }
  const int n_gt = thr == 0xffffffffu ? 0 : count_ge(thr + 1u);
  const int need = Ce - n_gt;  // >= 1 tokens equal to thr to seat
  const uint64_t below = (1ull << lane) - 1ull;
  int gt_run = 0, eq_run = 0;  // counts over the earlier chunks
#pragma unroll
  for (int c = 0; c < KPT; ++c) {
    if (c * kSelThreads >= T) break;  // block-uniform: no chunk left
    const int t = c * kSelThreads + tid;
    const bool valid = t < T;
    const bool gt = valid && key[c] > thr;
    const bool eq = valid && key[c] == thr;
    const uint64_t mg = __ballot(gt), me = __ballot(eq);
    if (lane == 0) {
      s_w[par][0][wid] = __popcll(mg);
      s_w[par][1][wid] = __popcll(me);
    }
    __syncthreads();
    int gb = gt_run, eb = eq_run, gtot = 0, etot = 0;
#pragma unroll
    for (int w = 0; w < kSelWaves; ++w) {
      const int a = s_w[par][0][w], b = s_w[par][1][w];
      if (w < wid) {
        gb += a;
        eb += b;
      }
      gtot += a;
      etot += b;
    }
    par ^= 1;
    gb += __popcll(mg & below);
    eb += __popcll(me & below);
    // seated: above thr, or among the first `need` equal to it
    const bool sel = gt || (eq && eb < need);
    const int pos = gb + min(eb, need);
    if (valid) route_pos[(size_t)t * E + e] = sel ? e * Ce + pos : -1;
    if (sel) row_token[e * Ce + pos] = t;
    gt_run += gtot;
    eq_run += etot;
  }
}

hipError_t launch_expert_choice(const float* logits, int T, int E, int Ce, float* scores,
                                uint32_t* keys, int32_t* route_pos, int32_t* row_token,
                                int32_t* offsets, hipStream_t st) {
  // T = 0: no scores; the select blocks still write offsets (all zero)
  if (T > 0) {
    const size_t lds = (size_t)kScoreTok * (E + 1) * sizeof(float);
    hipLaunchKernelGGL(ec_scores_kernel, dim3(ceil_div(T, kScoreTok)),
                       dim3(kScoreTok * kScoreLanes), lds, st, logits, T, E, scores, keys);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  const int chunks = ceil_div(T, kSelThreads);
#define SEL(K)                                                                                  \
  hipLaunchKernelGGL(ec_select_kernel<K>, dim3(E), dim3(kSelThreads), 0, st, keys, T, E, Ce, \
                     route_pos, row_token, offsets)
  if (chunks <= 1) SEL(1);
  else if (chunks <= 2) SEL(2);
  else if (chunks <= 4) SEL(4);
  else if (chunks <= 8) SEL(8);
  else if (chunks <= 16) SEL(16);
  else if (chunks <= 32) SEL(32);
  else return hipErrorInvalidValue;  // T > 32768: 64 keys per thread would spill
#undef SEL
  return hipGetLastError();
}

}  // namespace moe
