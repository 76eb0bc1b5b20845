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
//   router_logits_kernel  one lane per (token, expert) chain: each logit is a
//       sequential fp32 fused multiply-add over the hidden index in
//       increasing order, bias added after the sum.  That fixed order is what
//       makes the logits -- and so the selected expert ids at near ties --
//       bit-reproducible.  Token and expert rows are staged through LDS as
//       fp32 tiles (see the kernel).
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

// Router logits.  Block = 64 tokens x (4 * EPW) experts; lane = token, wave
// w owns experts e0 + w*EPW + j.  The hidden dimension advances in chunks of
// RKC (128 when the chains are few and latency-bound, 64 when many blocks
// share a CU): the block stages the x tile [64][RKC] and the W tile
// [4*EPW][RKC] in LDS as fp32 (converted once per element), then every lane
// runs its EPW fused-multiply-add chains in increasing hidden index, reading
// its own x row and broadcast W rows.  Chunks are prefetched two ahead into
// two register sets while the current one is consumed.
template <bool BF16, int EPW, int RKC>
__global__ __launch_bounds__(256) void router_logits_kernel(
    const void* __restrict__ x, const void* __restrict__ w, const float* __restrict__ b, int T,
    int d, int E, float* __restrict__ logits) {
  constexpr int EB = 4 * EPW;             // experts per block
  constexpr int G = BF16 ? 8 : 4;         // elements per 16-byte chunk
  constexpr int CPR = RKC / G;            // 16-byte chunks per tile row
  constexpr int XPT = 64 * CPR / 256;     // x chunks per thread
  constexpr int WPT = (EB * CPR + 255) / 256;  // W chunks per thread (upper bound)
  constexpr int XS = RKC + 4;             // padded fp32 row (conflict-free b128 reads)
  __shared__ __attribute__((aligned(16))) float sx[64 * XS];
  __shared__ __attribute__((aligned(16))) float sw[EB * RKC];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int t0 = blockIdx.x * 64;
  const int e0 = blockIdx.y * EB;
  const char* xb = reinterpret_cast<const char*>(x);
  const char* wb = reinterpret_cast<const char*>(w);
  constexpr int esz = BF16 ? 2 : 4;
  const u32x4_t zero = {0u, 0u, 0u, 0u};

  u32x4_t rx[2][XPT], rw[2][WPT];
  auto fetch = [&](int set, int k0) {
#pragma unroll
    for (int q = 0; q < XPT; ++q) {
      const int c = q * 256 + tid;
      const int row = c / CPR, col = (c % CPR) * G;
      const int t = min(t0 + row, T - 1);
      rx[set][q] = (k0 + col < d)
                       ? *reinterpret_cast<const u32x4_t*>(xb + ((size_t)t * d + k0 + col) * esz)
                       : zero;
    }
#pragma unroll
    for (int q = 0; q < WPT; ++q) {
      const int c = q * 256 + tid;
      const int row = c / CPR, col = (c % CPR) * G;
      const int e = min(e0 + row, E - 1);
      rw[set][q] = (c < EB * CPR && k0 + col < d)
                       ? *reinterpret_cast<const u32x4_t*>(wb + ((size_t)e * d + k0 + col) * esz)
                       : zero;
    }
  };
  auto put = [&](float* dst, const u32x4_t v) {
    if constexpr (BF16) {
      f32x4_t lo = {bf16lo(v[0]), bf16hi(v[0]), bf16lo(v[1]), bf16hi(v[1])};
      f32x4_t hi = {bf16lo(v[2]), bf16hi(v[2]), bf16lo(v[3]), bf16hi(v[3])};
      *reinterpret_cast<f32x4_t*>(dst) = lo;
      *reinterpret_cast<f32x4_t*>(dst + 4) = hi;
    } else {
      *reinterpret_cast<u32x4_t*>(dst) = v;
    }
  };
  auto stage = [&](int set) {
#pragma unroll
    for (int q = 0; q < XPT; ++q) {
      const int c = q * 256 + tid;
      put(sx + (c / CPR) * XS + (c % CPR) * G, rx[set][q]);
    }
#pragma unroll
    for (int q = 0; q < WPT; ++q) {
      const int c = q * 256 + tid;
      if (c < EB * CPR) put(sw + (c / CPR) * RKC + (c % CPR) * G, rw[set][q]);
    }
  };

  float acc[EPW];
#pragma unroll
  for (int j = 0; j < EPW; ++j) acc[j] = 0.0f;
  const float* xr = sx + lane * XS;
  // One k step = 4 hidden indices: this lane's x values and each expert's
  // W values, then 4 FMAs per chain in increasing index.
  struct Step {
    f32x4_t x;
    f32x4_t w[EPW];
  };
  auto read_step = [&](int kk, Step& q) {
    q.x = *reinterpret_cast<const f32x4_t*>(xr + kk);
#pragma unroll
    for (int j = 0; j < EPW; ++j)
      q.w[j] = *reinterpret_cast<const f32x4_t*>(sw + (wave * EPW + j) * RKC + kk);
  };
  auto fma_step = [&](const Step& q) {
#pragma unroll
    for (int j = 0; j < EPW; ++j) {
      acc[j] = __builtin_fmaf(q.x[0], q.w[j][0], acc[j]);
      acc[j] = __builtin_fmaf(q.x[1], q.w[j][1], acc[j]);
      acc[j] = __builtin_fmaf(q.x[2], q.w[j][2], acc[j]);
      acc[j] = __builtin_fmaf(q.x[3], q.w[j][3], acc[j]);
    }
  };
  // A full chunk: the LDS reads run P steps ahead of the FMAs (a ring of P
  // register sets), so their latency hides behind (P-1) steps of FMAs even
  // with one or two waves per SIMD; the schedule keeps each step's FMAs
  // before the refill it allows.
  constexpr int P = EPW == 4 ? 3 : 8 / EPW;
  constexpr int NSTEP = RKC / 4;
  static_assert(P <= NSTEP, "read-ahead within a chunk");
  auto consume_full = [&]() {
    Step q[P];
    static_for<0, P>([&](auto i) { read_step(decltype(i)::value * 4, q[decltype(i)::value]); });
    static_for<0, NSTEP>([&](auto si) {
      constexpr int st = decltype(si)::value;
      fma_step(q[st % P]);
      if constexpr (st + P < NSTEP) {
        read_step((st + P) * 4, q[st % P]);
        __builtin_amdgcn_sched_group_barrier(0x002, 4 * EPW, 0);  // the FMAs
        __builtin_amdgcn_sched_group_barrier(0x100, 1 + EPW, 0);  // then the refill
      }
    });
  };
  auto consume = [&](int k0) {
    const int kc = min(RKC, d - k0);  // a multiple of 8
    if (kc == RKC) {
      consume_full();
    } else {
      for (int kk = 0; kk < kc; kk += 4) {
        Step q;
        read_step(kk, q);
        fma_step(q);
      }
    }
  };
  const int nc = (d + RKC - 1) / RKC;
  fetch(0, 0);
  if (nc > 1) fetch(1, RKC);
  for (int c = 0; c < nc; c += 2) {
    __syncthreads();  // previous chunk fully consumed
    stage(0);
    if (c + 2 < nc) fetch(0, (c + 2) * RKC);
    __syncthreads();
    consume(c * RKC);
    if (c + 1 >= nc) break;
    __syncthreads();
    stage(1);
    if (c + 3 < nc) fetch(1, (c + 3) * RKC);
    __syncthreads();
    consume((c + 1) * RKC);
  }
  const int t = t0 + lane;
  if (t >= T) return;
#pragma unroll
  for (int j = 0; j < EPW; ++j) {
    const int e = e0 + wave * EPW + j;
    if (e < E) {
      float v = acc[j];
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
  // experts per wave: the most register reuse that still leaves about
  // 2048 waves (two per SIMD) of independent chains
  const long waves_at1 = (long)ceil_div(T, kWave) * E;
  int EPW = 1;
  if (waves_at1 >= 8192) EPW = 4;
  else if (waves_at1 >= 4096) EPW = 2;
  dim3 grid(ceil_div(T, kWave), ceil_div(E, 4 * EPW));
  dim3 block(256);
#define RL(BF, EPW_)                                                                            \
  hipLaunchKernelGGL((router_logits_kernel<BF, EPW_, (EPW_ == 4 ? 64 : 128)>), grid, block, 0, st, \
                     x, w, b, T, d, E, logits)
  if (bf16) {
    if (EPW == 1) RL(true, 1);
    else if (EPW == 2) RL(true, 2);
    else RL(true, 4);
  } else {
    if (EPW == 1) RL(false, 1);
    else if (EPW == 2) RL(false, 2);
    else RL(false, 4);
  }
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
