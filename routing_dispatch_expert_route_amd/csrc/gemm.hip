// gemm.hip -- expert FFN as variable-size grouped GEMMs.
//
// "271,104 Routes", section 3: rows of one expert are packed into a batch so
// the expert runs one dense matmul; "Mixture-of-experts routing": dropless
// variable-size grouped matmuls; "MoE Inference Visualized", "Expert
// Execution": down_proj(SiLU(gate_proj(x)) * up_proj(x)).
//
// GEMM 1:  h[p, :]  = SiLU(A[p] Wg[e]^T) * (A[p] Wu[e]^T)   (SwiGLU epilogue)
// GEMM 2:  y[p, :]  = h[p] Wd[e]^T
// for every packed row p of expert e (rows [offsets[e], offsets[e+1])).
// Both operands are K-contiguous ([rows][K] activations, [N][K] weights), so
// every MFMA fragment is one 16-byte LDS read.
//
// Tile scheduling needs no host readback: the grid is an upper bound on the
// number of (row tile, column tile) pairs; each workgroup finds its expert by
// a wave-wide prefix scan over ceil(m_e / BM) read from the device offsets,
// and workgroups past the last tile exit at once.
//
// GEMM 1 can read its A rows through an index (a_rows[p] = source token), so
// the whole-layer path never materialises the packed copy of x.
#include "common.h"
#include "launch.h"

namespace moe {

struct GemmArgs {
  const void* A;          // [rows][K] activations (packed rows, or tokens via a_rows)
  const int32_t* a_rows;  // optional row index: A row of packed row p is a_rows[p]
  const int32_t* offsets; // [E+1] device offsets, or nullptr: one group of M_dense rows
  int E;
  int M_dense;
  const void* B0;  // gate (SwiGLU) or down weights [E][N][K]
  const void* B1;  // up weights [E][N][K] (SwiGLU only)
  int N;
  int K;
  void* C;  // [rows][N]
  int n_tiles;
};

// Find the (expert, first row, row count) of row-tile mt.  Executed by one
// wave; lane 0 of the finding lane group writes the result to info[0..2]
// (info[0] stays -1 when mt is past the last tile).
template <int BM>
__device__ __forceinline__ void find_row_tile(const GemmArgs& a, int mt, int lane, int* info) {
  if (a.offsets == nullptr) {
    if (lane == 0) {
      const int r0 = mt * BM;
      if (r0 < a.M_dense) {
        info[0] = 0;
        info[1] = r0;
        info[2] = min(BM, a.M_dense - r0);
      } else {
        info[0] = -1;
      }
    }
    return;
  }
  if (lane == 0) info[0] = -1;
  int carry = 0;
  for (int e0 = 0; e0 < a.E; e0 += kWave) {
    const int e = e0 + lane;
    int m = 0, off = 0;
    if (e < a.E) {
      off = a.offsets[e];
      m = a.offsets[e + 1] - off;
    }
    const int tiles = (m + BM - 1) / BM;
    int incl = tiles;
#pragma unroll
    for (int s = 1; s < kWave; s <<= 1) {
      const int o = __shfl_up(incl, s, kWave);
      if (lane >= s) incl += o;
    }
    const int excl = carry + incl - tiles;
    if (e < a.E && mt >= excl && mt < excl + tiles) {
      const int local = mt - excl;
      info[0] = e;
      info[1] = off + local * BM;
      info[2] = min(BM, m - local * BM);
    }
    carry += __shfl(incl, kWave - 1, kWave);
  }
}

// ---------------------------------------------------------------------------
// bf16 MFMA kernel.  256 threads = WGM x WGN waves; block tile BM x BNO
// outputs; BK = 64 per LDS stage, two stages.  LDS rows hold 8 chunks of 16
// bytes; chunk c of row r is stored at c ^ (r & 7) so that the 8 lanes that
// read one column chunk of 8 consecutive rows hit 8 different bank groups.
// ---------------------------------------------------------------------------
template <int BM, int BNO, int WGM, int WGN, bool SWIGLU, bool GATHER>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(GemmArgs a) {
  constexpr int BK = 64;
  constexpr int CH = BK / 8;  // 16-byte chunks per LDS row
  constexpr int NREG = SWIGLU ? 2 : 1;
  constexpr int BNB = BNO * NREG;  // weight rows in the B tile
  constexpr int WTM = BM / WGM, WTN = BNO / WGN;
  constexpr int TM = WTM / 32, TN = WTN / 32;
  constexpr int A_LD = BM * CH / 256;   // A chunks per thread per stage
  constexpr int B_LD = BNB * CH / 256;  // B chunks per thread per stage
  static_assert(WGM * WGN == 4, "four waves");
  static_assert(TM >= 1 && TN >= 1 && A_LD >= 1 && B_LD >= 1, "tile shape");

  __shared__ __attribute__((aligned(16))) u32x4_t sA[2][BM * CH];
  __shared__ __attribute__((aligned(16))) u32x4_t sB[2][BNB * CH];
  __shared__ int s_info[3];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
  const int mt = blockIdx.x / a.n_tiles;
  const int nt = blockIdx.x % a.n_tiles;

  if (wave == 0) find_row_tile<BM>(a, mt, lane, s_info);
  __syncthreads();
  const int e = s_info[0];
  if (e < 0) return;
  const int row0 = s_info[1];
  const int rows = s_info[2];
  const int K = a.K, N = a.N;

  // per-thread global sources (fixed over the K loop)
  const bf16_t* a_src[A_LD];
  int a_lds[A_LD];
  int a_k[A_LD];
#pragma unroll
  for (int q = 0; q < A_LD; ++q) {
    const int idx = q * 256 + tid;
    const int r = idx / CH, c = idx % CH;
    const int p = row0 + (r < rows ? r : rows - 1);
    const int src = GATHER ? a.a_rows[p] : p;
    a_src[q] = reinterpret_cast<const bf16_t*>(a.A) + (size_t)src * K + c * 8;
    a_k[q] = c * 8;
    a_lds[q] = r * CH + (c ^ (r & 7));
  }
  const bf16_t* b_src[B_LD];
  int b_lds[B_LD];
  int b_k[B_LD];
#pragma unroll
  for (int q = 0; q < B_LD; ++q) {
    const int idx = q * 256 + tid;
    const int r = idx / CH, c = idx % CH;
    const int reg = r / BNO;
    int n = nt * BNO + (r % BNO);
    n = n < N ? n : N - 1;
    const bf16_t* base = reinterpret_cast<const bf16_t*>(reg == 0 ? a.B0 : a.B1);
    b_src[q] = base + ((size_t)e * N + n) * K + c * 8;
    b_k[q] = c * 8;
    b_lds[q] = r * CH + (c ^ (r & 7));
  }

  f32x16_t acc[NREG][TM][TN];
#pragma unroll
  for (int g = 0; g < NREG; ++g)
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[g][i][j][v] = 0.0f;

  u32x4_t ra[A_LD], rb[B_LD];
  const u32x4_t zero = {0u, 0u, 0u, 0u};
  auto gload = [&](int k0) {
#pragma unroll
    for (int q = 0; q < A_LD; ++q)
      ra[q] = (k0 + a_k[q] < K) ? *reinterpret_cast<const u32x4_t*>(a_src[q] + k0) : zero;
#pragma unroll
    for (int q = 0; q < B_LD; ++q)
      rb[q] = (k0 + b_k[q] < K) ? *reinterpret_cast<const u32x4_t*>(b_src[q] + k0) : zero;
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int q = 0; q < A_LD; ++q) sA[buf][a_lds[q]] = ra[q];
#pragma unroll
    for (int q = 0; q < B_LD; ++q) sB[buf][b_lds[q]] = rb[q];
  };

  const int nk = (K + BK - 1) / BK;
  gload(0);
  sstore(0);
  __syncthreads();
  const int lrow = lane & 31;
  const int lk = lane >> 5;
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * BK);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int ch = ks * 2 + lk;
      bf16x8_t af[TM];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int r = wm * WTM + i * 32 + lrow;
        af[i] = __builtin_bit_cast(bf16x8_t, sA[buf][r * CH + (ch ^ (r & 7))]);
      }
#pragma unroll
      for (int g = 0; g < NREG; ++g) {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int r = g * BNO + wn * WTN + j * 32 + lrow;
          const bf16x8_t bf = __builtin_bit_cast(bf16x8_t, sB[buf][r * CH + (ch ^ (r & 7))]);
#pragma unroll
          for (int i = 0; i < TM; ++i)
            acc[g][i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf, acc[g][i][j], 0, 0, 0);
        }
      }
    }
    if (kt + 1 < nk) sstore(buf ^ 1);
    __syncthreads();
  }

  // epilogue: accumulator element v of lane l is (row 8*(v/4) + 4*(l/32) + v%4, col l%32)
  bf16_t* Cp = reinterpret_cast<bf16_t*>(a.C);
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int col = nt * BNO + wn * WTN + j * 32 + lrow;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = wm * WTM + i * 32 + 8 * (v >> 2) + 4 * lk + (v & 3);
        float o;
        if constexpr (SWIGLU) {
          const float gv = acc[0][i][j][v];
          const float uv = acc[1][i][j][v];
          o = gv / (1.0f + expf(-gv)) * uv;
        } else {
          o = acc[0][i][j][v];
        }
        if (r < rows && col < N) Cp[(size_t)(row0 + r) * N + col] = (bf16_t)f32_to_bf16(o);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 kernel (plain fp32 FMA, one output element per thread, K ascending).
// Serves the fp32 dtype, whose shapes here are small.
// ---------------------------------------------------------------------------
template <bool SWIGLU, bool GATHER>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs a) {
  constexpr int BM = 16, BNO = 16;
  __shared__ int s_info[3];
  const int tid = threadIdx.x;
  const int mt = blockIdx.x / a.n_tiles;
  const int nt = blockIdx.x % a.n_tiles;
  if (tid < 64) find_row_tile<BM>(a, mt, tid, s_info);
  __syncthreads();
  const int e = s_info[0];
  if (e < 0) return;
  const int row0 = s_info[1], rows = s_info[2];
  const int r = tid / BNO, c = tid % BNO;
  const int col = nt * BNO + c;
  if (r >= rows || col >= a.N) return;
  const int p = row0 + r;
  const int src = GATHER ? a.a_rows[p] : p;
  const float* Ar = reinterpret_cast<const float*>(a.A) + (size_t)src * a.K;
  const float* B0 = reinterpret_cast<const float*>(a.B0) + ((size_t)e * a.N + col) * a.K;
  float s0 = 0.0f, s1 = 0.0f;
  if constexpr (SWIGLU) {
    const float* B1 = reinterpret_cast<const float*>(a.B1) + ((size_t)e * a.N + col) * a.K;
    for (int kk = 0; kk < a.K; ++kk) {
      s0 = __builtin_fmaf(Ar[kk], B0[kk], s0);
      s1 = __builtin_fmaf(Ar[kk], B1[kk], s1);
    }
    s0 = s0 / (1.0f + expf(-s0)) * s1;
  } else {
    for (int kk = 0; kk < a.K; ++kk) s0 = __builtin_fmaf(Ar[kk], B0[kk], s0);
  }
  reinterpret_cast<float*>(a.C)[(size_t)p * a.N + col] = s0;
}

// Upper bound on the number of row tiles of size BM over all groups.
static long row_tile_bound(const GemmPlan& pl, int BM) {
  if (pl.offsets == nullptr) return (pl.M_dense + BM - 1) / BM;
  const long by_rows = (pl.R_max + (long)pl.E * (BM - 1)) / BM;
  const long by_cap = (long)pl.E * ((pl.m_cap + BM - 1) / BM);
  return by_rows < by_cap ? by_rows : by_cap;
}

template <int BM, int BNO, int WGM, int WGN, bool SWIGLU>
static hipError_t run_bf16(const GemmPlan& pl, GemmArgs a, hipStream_t st) {
  a.n_tiles = (a.N + BNO - 1) / BNO;
  const long mtb = row_tile_bound(pl, BM);
  const long blocks = mtb * a.n_tiles;
  if (blocks == 0) return hipSuccess;
  if (a.a_rows)
    hipLaunchKernelGGL((gemm_bf16_kernel<BM, BNO, WGM, WGN, SWIGLU, true>), dim3((unsigned)blocks),
                       dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((gemm_bf16_kernel<BM, BNO, WGM, WGN, SWIGLU, false>),
                       dim3((unsigned)blocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <bool SWIGLU>
static hipError_t run_f32(const GemmPlan& pl, GemmArgs a, hipStream_t st) {
  a.n_tiles = (a.N + 15) / 16;
  const long blocks = row_tile_bound(pl, 16) * a.n_tiles;
  if (blocks == 0) return hipSuccess;
  if (a.a_rows)
    hipLaunchKernelGGL((gemm_f32_kernel<SWIGLU, true>), dim3((unsigned)blocks), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((gemm_f32_kernel<SWIGLU, false>), dim3((unsigned)blocks), dim3(256), 0, st,
                       a);
  return hipGetLastError();
}

hipError_t launch_gemm_swiglu(const GemmPlan& pl, const void* A, const int32_t* a_rows,
                              const void* Wg, const void* Wu, int N, int K, void* H,
                              hipStream_t st) {
  GemmArgs a{A, a_rows, pl.offsets, pl.E, pl.M_dense, Wg, Wu, N, K, H, 0};
  if (!pl.bf16) return run_f32<true>(pl, a, st);
  return run_bf16<128, 128, 2, 2, true>(pl, a, st);
}

hipError_t launch_gemm_down(const GemmPlan& pl, const void* H, const void* Wd, int N, int K,
                            void* Y, hipStream_t st) {
  GemmArgs a{H, nullptr, pl.offsets, pl.E, pl.M_dense, Wd, nullptr, N, K, Y, 0};
  if (!pl.bf16) return run_f32<false>(pl, a, st);
  return run_bf16<128, 128, 2, 2, false>(pl, a, st);
}

}  // namespace moe
