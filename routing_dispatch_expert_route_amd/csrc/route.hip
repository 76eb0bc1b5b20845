// route.hip -- router projection, softmax and top-k.
//
// "Mixture of Experts: Routing, Dispatch, and Load Balancing", section 1:
// the router is a linear projection x W^T + b to one logit per expert,
// followed by softmax.  "271,104 Routes", section 2: topk on the logits, then
// softmax over the k selected logits (the renormalised gate); "MoE Inference
// Visualized", "Expert Execution": the top-1 output is scaled by its full
// softmax probability (no renormalisation).
//
// Two kernels:
//   router_r64_kernel  a wave per (tokens, experts) group: each logit is a
//       dot product in the fixed fp32 order R64 (partial sums over
//       granules of eight elements, one per lane, folded by halving; bias
//       added last).  That fixed order is what makes the logits -- and so
//       the selected expert ids at near ties -- bit-reproducible.
//   topk_rank_kernel  one lane per (token, expert): an expert's rank among
//       its token's logits (logit desc, index asc) is its slot when below k;
//       then the gates.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace moe {

// Calls f(integral_constant<int, I>) for I = B .. E-1 (compile-time unrolled).
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// Router logits in the fixed summation order R64: hidden index i lies in
// granule i / 8 (eight consecutive elements, one 16-byte load in bf16) and
// granule q belongs to partial sum q mod 64 -- lane q mod 64 of a wave, which
// runs a chain of fused multiply-adds over its granules' elements in
// increasing i from +0.  The 64 partial sums of a dot product are then
// folded by halving, p[l] = p[l] + p[l + s] for l < s, s = 32, ..., 1, and
// the bias is added to p[0].  Each wave-level load covers 64 consecutive
// granules (1 KiB of a row), so a row is read once, coalesced.
//
// One wave computes TPW tokens x EPW experts (C = TPW*EPW dot products, each
// lane holding C partial sums); weights are reused across the TPW tokens and
// token rows across the EPW experts.  The fold works on all C dot products
// at once: at each halving step the two lanes of a pair (l, l ^ s) each keep
// half of their dot products and exchange the other half, so each step
// moves half as many values as the last and every lane finishes with the
// result of dot product lane / (64 / C) -- the same sums as the fold above
// (a pair's sum is p[l] + p[l + s], and fp32 addition commutes).
template <int C>
__device__ __forceinline__ void r64_fold(float (&v)[C], int lane) {
  static_for<0, 6>([&](auto L) {
    constexpr int lev = decltype(L)::value;
    constexpr int s = 32 >> lev;
    constexpr int n = (C >> lev) > 1 ? (C >> lev) : 1;  // dot products held
    constexpr int half = n / 2;
    const bool up = (lane & s) != 0;  // this lane holds partial sum l + s
    if constexpr (half >= 1) {
#pragma unroll
      for (int i = 0; i < half; ++i) {
        const float keep = up ? v[half + i] : v[i];
        const float send = up ? v[i] : v[half + i];
        v[i] = keep + __shfl_xor(send, s, kWave);
      }
    } else {
      v[0] = v[0] + __shfl_xor(v[0], s, kWave);
    }
  });
}

template <bool BF16, int TPW, int EPW>
__global__ __launch_bounds__(64) void router_r64_kernel(const void* __restrict__ x,
                                                        const void* __restrict__ w,
                                                        const float* __restrict__ b, int T, int d,
                                                        int E, float* __restrict__ logits) {
  constexpr int C = TPW * EPW;
  static_assert(C >= 1 && C <= 64 && (C & (C - 1)) == 0, "a power of two up to 64");
  constexpr int NL = BF16 ? 1 : 2;  // 16-byte loads per granule
  const int lane = threadIdx.x;
  const int n_eg = (E + EPW - 1) / EPW;
  const int eg = blockIdx.x % n_eg;
  const int t0 = (blockIdx.x / n_eg) * TPW, e0 = eg * EPW;
  const int Q = d / 8;
  const size_t rowb = (size_t)d * (BF16 ? 2 : 4);
  const char* xr[TPW];
  const char* wr[EPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t)
    xr[t] = reinterpret_cast<const char*>(x) + (size_t)min(t0 + t, T - 1) * rowb;
#pragma unroll
  for (int e = 0; e < EPW; ++e)
    wr[e] = reinterpret_cast<const char*>(w) + (size_t)min(e0 + e, E - 1) * rowb;

  struct Granule {
    u32x4_t x[TPW][NL];
    u32x4_t w[EPW][NL];
  };
  auto load = [&](int q, Granule& g) {
    const size_t o = (size_t)q * 16 * NL;
#pragma unroll
    for (int t = 0; t < TPW; ++t)
#pragma unroll
      for (int h = 0; h < NL; ++h) g.x[t][h] = *reinterpret_cast<const u32x4_t*>(xr[t] + o + 16 * h);
#pragma unroll
    for (int e = 0; e < EPW; ++e)
#pragma unroll
      for (int h = 0; h < NL; ++h) g.w[e][h] = *reinterpret_cast<const u32x4_t*>(wr[e] + o + 16 * h);
  };
  // element j (0..7) of a granule as fp32
  auto elem = [&](const u32x4_t (&v)[NL], int j) -> float {
    if constexpr (BF16) return (j & 1) ? bf16hi(v[0][j >> 1]) : bf16lo(v[0][j >> 1]);
    else return __uint_as_float(v[j >> 2][j & 3]);
  };
  float acc[C];
#pragma unroll
  for (int c = 0; c < C; ++c) acc[c] = 0.0f;
  auto consume = [&](const Granule& g) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float xv[TPW];
#pragma unroll
      for (int t = 0; t < TPW; ++t) xv[t] = elem(g.x[t], j);
#pragma unroll
      for (int e = 0; e < EPW; ++e) {
        const float wv = elem(g.w[e], j);
#pragma unroll
        for (int t = 0; t < TPW; ++t) acc[t * EPW + e] = __builtin_fmaf(xv[t], wv, acc[t * EPW + e]);
      }
    }
  };
  // a lane's granules q = lane, lane + 64, ... (in increasing i), the next
  // granule's loads in flight while the current one is consumed
  Granule g0, g1;
  int q = lane;
  if (q < Q) load(q, g0);
  while (q < Q) {
    if (q + 64 < Q) load(q + 64, g1);
    consume(g0);
    q += 64;
    if (q >= Q) break;
    if (q + 64 < Q) load(q + 64, g0);
    consume(g1);
    q += 64;
  }
  r64_fold<C>(acc, lane);
  constexpr int LPC = 64 / C;  // lanes holding each result
  if (lane % LPC == 0) {
    const int c = lane / LPC;
    const int t = t0 + c / EPW, e = e0 + c % EPW;
    if (t < T && e < E) {
      float v = acc[0];
      if (b) v = v + b[e];
      logits[(size_t)t * E + e] = v;
    }
  }
}

// Top-k by rank, one lane per (token, expert): expert e's rank is the number
// of experts that precede it (larger logit, or an equal one at a lower
// index); it is selected iff rank < k, into slot rank -- the same selection
// as the insertion pass of topk_token, in E comparisons per lane instead of
// E*k serial steps per token.  The gates are topk_token's too: exp(l - max)
// summed in slot order (renormalised) or in expert order, then divided, so
// the same bits.  EP: lanes per token, a power of two >= E.
template <int EP>
__global__ __launch_bounds__(256) void topk_rank_kernel(const float* __restrict__ logits, int T,
                                                        int E, int k, int renorm,
                                                        int32_t* __restrict__ ids,
                                                        float* __restrict__ gates) {
  constexpr int TPB = 256 / EP;  // tokens per block
  __shared__ float s_l[TPB][EP + 1];
  __shared__ float s_ex[TPB][EP + 1];
  __shared__ float s_m[TPB];
  const int tid = threadIdx.x;
  const int tl = tid / EP, e = tid % EP;
  const int t0 = blockIdx.x * TPB;
  const int nt = min(TPB, T - t0);
  // the block's logits are nt*E consecutive floats
  for (int i = tid; i < nt * E; i += 256) s_l[i / E][i % E] = logits[(size_t)t0 * E + i];
  __syncthreads();
  const bool active = tl < nt && e < E;
  float l = 0.0f;
  int rank = E;
  if (active) {
    l = s_l[tl][e];
    rank = 0;
    for (int e2 = 0; e2 < E; ++e2) {
      const float l2 = s_l[tl][e2];
      rank += (l2 > l) | ((l2 == l) & (e2 < e));
    }
    if (rank == 0) s_m[tl] = l;
  }
  __syncthreads();
  float ex = 0.0f;
  if (active) {
    ex = expf(l - s_m[tl]);
    if (!renorm) s_ex[tl][e] = ex;
    else if (rank < k) s_ex[tl][rank] = ex;
  }
  __syncthreads();
  if (active && rank < k) {
    const int n = renorm ? k : E;
    float denom = 0.0f;
    for (int j = 0; j < n; ++j) denom += s_ex[tl][j];
    const size_t o = (size_t)(t0 + tl) * k + rank;
    ids[o] = e;
    gates[o] = ex / denom;
  }
}

hipError_t launch_route(bool bf16, const void* x, const void* w, const float* b, int T, int d,
                        int E, int k, int renorm, float* logits, int32_t* ids, float* gates,
                        hipStream_t st) {
  if (T == 0) return hipSuccess;
  // a wave per TPW tokens x EPW experts: the most reuse (up to 4 tokens x 16
  // experts) that still leaves about 2048 waves, fewer tokens first, then
  // fewer experts
  int EPW = 1;
  while (EPW < E && EPW < 16) EPW *= 2;
  int TPW = 4;
  auto waves = [&](int tpw, int epw) { return (long)ceil_div(T, tpw) * ceil_div(E, epw); };
  while (TPW > 1 && waves(TPW, EPW) < 2048) TPW /= 2;
  while (EPW > 1 && waves(TPW, EPW) < 2048) EPW /= 2;
  const dim3 grid((unsigned)waves(TPW, EPW)), block(64);
#define RL(BF, TP, EP)                                                                        \
  if (TPW == TP && EPW == EP)                                                                 \
  hipLaunchKernelGGL((router_r64_kernel<BF, TP, EP>), grid, block, 0, st, x, w, b, T, d, E, \
                     logits)
#define RL_E(BF, TP) \
  RL(BF, TP, 1); RL(BF, TP, 2); RL(BF, TP, 4); RL(BF, TP, 8); RL(BF, TP, 16)
  if (bf16) {
    RL_E(true, 1); RL_E(true, 2); RL_E(true, 4);
  } else {
    RL_E(false, 1); RL_E(false, 2); RL_E(false, 4);
  }
#undef RL_E
#undef RL
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || !ids) return err;  // logits only
  int ep = 4;
  while (ep < E) ep *= 2;  // E <= 256
  const dim3 tb(256);
#define TR(EP_)                                                                        \
  hipLaunchKernelGGL(topk_rank_kernel<EP_>, dim3(ceil_div(T, 256 / EP_)), tb, 0, st, logits, T, \
                     E, k, renorm, ids, gates)
  switch (ep) {
    case 4: TR(4); break;
    case 8: TR(8); break;
    case 16: TR(16); break;
    case 32: TR(32); break;
    case 64: TR(64); break;
    case 128: TR(128); break;
    default: TR(256); break;
  }
#undef TR
  return hipGetLastError();
}

}  // namespace moe
