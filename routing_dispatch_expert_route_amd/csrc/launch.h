// launch.h -- host-side launchers of the HIP kernels (internal to libmoe).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// router_r64_kernel + topk_rank_kernel (the projection only when ids
// is null)
hipError_t launch_route(bool bf16, const void* x, const void* w, const float* b, int T, int d,
                        int E, int k, int renorm, float* logits, int32_t* ids, float* gates,
                        hipStream_t st);

// hist + scan + scatter.  cnt_ws holds E * permute_nchunks(T*k) ints.
int permute_nchunks(long R);
hipError_t launch_permute_index(const int32_t* ids, int T, int k, int E, int C, int32_t* cnt_ws,
                                int32_t* counts, int32_t* kept, int32_t* offsets,
                                int32_t* route_pos, int32_t* row_token, hipStream_t st);
// Top-k (as launch_route's) and the counting-sort permute in one launch, from
// router logits [T][E], when topk_permute_fused(T, k, E) (T <= 256, E <= 16):
// ids and gates as launch_route writes them, then the outputs of
// launch_permute_index.
bool topk_permute_fused(int T, int k, int E);
hipError_t launch_topk_permute(const float* logits, int T, int E, int k, int renorm, int C,
                               int32_t* ids, float* gates, int32_t* counts, int32_t* kept,
                               int32_t* offsets, int32_t* route_pos, int32_t* row_token,
                               hipStream_t st);
hipError_t launch_gather_rows(const void* x, const int32_t* row_token, const int32_t* offsets,
                              int E, long R_max, long row_bytes, void* x_packed, hipStream_t st);
// Overflow policy "reroute" after a drop-policy dispatch (route_pos0,
// offsets0, kept from launch_permute_index); E <= 256, k <= 8, C >= 0.
// Writes the final experts, the packed positions and rows of the result.
// pref: scratch of T*k*64 bytes, T*k*256 when E > 64 (per dropped route,
// its experts' ranks or its experts in preference order);
// da_state: scratch of reroute_state_bytes(T, E) bytes, 16-byte aligned (the
// parallel kernel's token arrays, final bitmaps and, when it does not fit
// LDS, its per-token state; 0 bytes where the walk runs).
long reroute_state_bytes(int T, int E);
hipError_t launch_reroute(const float* logits, const int32_t* ids_in, const int32_t* route_pos0,
                          const int32_t* offsets0, const int32_t* kept, int T, int k, int E,
                          int C, int32_t* ids_out, int32_t* slot, int32_t* offsets,
                          int32_t* route_pos, int32_t* row_token, uint8_t* pref,
                          uint8_t* da_state, hipStream_t st);
// Queue policy ("queue to the next micro-batch"), after launch_permute_index
// over the arrival sequence (Q queued routes, then T*k routes, one route per
// arrival).  launch_queue_gather copies, for p < count[0] (at most max_rows),
// the row of arrival arr[p] -- q_x[a] for a < Q, else x[(a - Q) / k] -- into
// rows[p].  launch_queue_compact lists the arrivals with pos < 0 in arrival
// order (n_out[0] of them, arrivals in arr) with their expert, gate and tag
// (queued: carried; new: tag_base + token).
hipError_t launch_queue_gather(const void* x, const void* q_x, const int32_t* arr,
                               const int32_t* count, int Q, int k, long max_rows, long row_bytes,
                               void* rows, hipStream_t st);
hipError_t launch_queue_compact(const int32_t* pos, long N, int Q, int k, const int32_t* q_ids,
                                const float* q_gates, const int64_t* q_tags, const int32_t* ids,
                                const float* gates, int64_t tag_base, int32_t* n_out,
                                int32_t* arr, int32_t* out_ids, float* out_gates,
                                int64_t* out_tags, hipStream_t st);
// seats[e] = offsets[e+1] - offsets[e]
hipError_t launch_seats(const int32_t* offsets, int E, int32_t* seats, hipStream_t st);
// Fixed-shape [E, C, d] buffer from a packed dispatch (needs C >= 1): padded
// route positions, the buffer's rows (zero for empty slots) and its row
// groups offsets_pad[e] = e*C.
hipError_t launch_padded(const void* x, const int32_t* ids, const int32_t* route_pos,
                         const int32_t* offsets, const int32_t* kept, const int32_t* row_token,
                         int T, int k, int E, int C, long row_bytes, int32_t* pad_pos,
                         void* x_pad, int32_t* offsets_pad, hipStream_t st);

// Expert-choice routing from router logits [T][E]: scores [T][E] (softmax;
// may be null), keys [E][T] (the scores' bits, expert-major), pos_et [E][T]
// (row e*Ce + i or -1), route_pos [T][E] (the same table token-major; may be
// null), row_token [E*Ce] and offsets[e] = e*Ce.  Needs 1 <= Ce <= T (Ce =
// 0 when T = 0) and E*T < 2^29.
hipError_t launch_expert_choice(const float* logits, int T, int E, int Ce, float* scores,
                                uint32_t* keys, int32_t* pos_et, int32_t* route_pos,
                                int32_t* row_token, int32_t* offsets, hipStream_t st);

// Row groups of a grouped GEMM: device offsets[E+1] (never read on the
// host), or one dense group of M_dense rows when offsets is null.
struct GemmPlan {
  bool bf16;
  bool grouped;  // rows come in E groups given by offsets (else one dense group)
  const int32_t* offsets;
  int E;
  int M_dense;
  long R_max;  // bound on offsets[E]
  long m_cap;  // bound on any one group's rows
  // fp32 scratch of gemm_tail_floats(plan, N, K) floats for the down GEMM's
  // last-round tiles split along K (nullptr: no split)
  float* tail = nullptr;
  // rows GEMM 1's tile shape is chosen for, when R_max overstates them
  // (the queue policy: E*C bounds its seats, T*k routes arrive per call);
  // 0: R_max.  The grid still covers R_max rows.
  long R_tile = 0;
};
// True when GEMM 1 of this plan should read packed rows rather than gather
// token rows: the 256x256 tile with a wide output (a pure function of the
// plan and shape).
bool gemm_swiglu_prefers_packed(const GemmPlan& pl, int N, int K);
// fp32 scratch the down GEMM of this plan uses to split its last round of
// 256x256 tiles along K (0 when it does not): a pure function of the plan.
long gemm_tail_floats(const GemmPlan& pl, int N, int K);
// a_nrows: rows of A (its byte extent bounds the activation loads)
hipError_t launch_gemm_swiglu(const GemmPlan& pl, const void* A, const int32_t* a_rows,
                              long a_nrows, const void* Wg, const void* Wu, int N, int K, void* H,
                              hipStream_t st);
// K splits the down GEMM uses for this plan (1 = direct dtype output;
// more = fp32 partial planes [splits][R_max][N] summed in a fixed order by
// the consumer).  A pure function of the plan, so workspace sizing and the
// launch agree.
int gemm_down_splits(const GemmPlan& pl, int N, int K);
hipError_t launch_gemm_down(const GemmPlan& pl, const void* H, const void* Wd, int N, int K,
                            void* Y, int splits, long split_stride, hipStream_t st);
// The down GEMM with the combine of one route per token (no shared expert,
// no K split, bf16, N % 8 == 0) fused: packed row p, of token row_token[p],
// is scaled by gates[token] and written to row token of y [T][N]; tokens
// with route_pos[t] < 0 get zero rows.  Bit-identical to launch_gemm_down
// followed by launch_combine with k = 1.
hipError_t launch_gemm_down_combine(const GemmPlan& pl, const void* H, const void* Wd, int N,
                                    int K, const int32_t* row_token, const float* gates,
                                    const int32_t* route_pos, int T, void* y, hipStream_t st);

// y_packed is dtype rows (splits == 1) or fp32 partial planes (splits > 1,
// plane stride split_stride elements).
hipError_t launch_combine(bool bf16, const void* y_packed, int splits, long split_stride,
                          const int32_t* route_pos, const float* gates, const void* y_shared,
                          int T, int k, int d, void* y, hipStream_t st);
// The same with the route table and gates expert-major ([k][T]: slot j of
// token t at j*T + t), as expert choice writes them.
hipError_t launch_combine_slot_major(bool bf16, const void* y_packed, int splits,
                                     long split_stride, const int32_t* route_pos,
                                     const float* gates, const void* y_shared, int T, int k,
                                     int d, void* y, hipStream_t st);
// y[p] = sum over planes of parts[s][p] for p < offsets[E] (or M_dense rows
// when offsets is null), rounded once to dtype.
hipError_t launch_reduce_splits(bool bf16, const float* parts, int splits, long split_stride,
                                const int32_t* offsets, int E, long R_max, int N, void* y,
                                hipStream_t st);

// stats_partial_kernel + stats_final_kernel.  part holds
// stats_blocks(T) * (E + 3) floats, hpart stats_blocks(T) * n_bins ints;
// n_bins <= kMaxStatBins.
constexpr int kMaxStatBins = 256;
int stats_blocks(long T);
hipError_t launch_routing_stats(const float* logits, const float* gates, const int32_t* counts,
                                int T, int E, int k, int n_bins, float alpha, float* part,
                                int32_t* hpart, float* stats, int32_t* hist, hipStream_t st);

}  // namespace moe
