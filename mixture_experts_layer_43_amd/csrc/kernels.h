// Internal launch interface between the C-ABI layer (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// ---- router (router.hip) ----
struct RouteArgs {
  const void* x;           // [T, d] f32 or bf16
  const float* w_router;   // [N_r, d]
  const float* bias;       // [N_r] or null
  int T, d, n_routed, top_k, gate;
  bool bias_sel;           // bias enters the selection only (gates from the unbiased logits)
  bool x_bf16;
  int32_t* topk_idx;       // [T, K']
  float* topk_w;           // [T, K']
  float* partial;          // null, or scratch of router_partial_bytes(T) for split-K logits
  double* stats_part;      // null, or scratch of route_stats_bytes(T): routing statistics on
  float* lse;              // [T] or null: per-token log-sum-exp (statistics only)
  const float* w_noise;    // [N_r, d] or null: noisy top-k gating (no split, no statistics)
  const float* noise;      // [T, N_r] standard normal draws, with w_noise
  bool w_packed;           // w_router in the packed order of launch_pack_router
};
// Split-K of the matrix-core router for small batches: at most this many
// K slices, each writing a [T, 128] fp32 partial tile.
constexpr int kRouterSplit = 8;
inline size_t router_partial_bytes(int64_t T) {
  return T < 4096 ? static_cast<size_t>(kRouterSplit) * static_cast<size_t>(T) * 128 * 4 : 0;
}
hipError_t launch_route(const RouteArgs& a, hipStream_t s);

// Rows of the matrix-core router's logit tile for N_r <= 128 experts (the
// packed W_g holds this many rows of d floats).
inline int router_pad_rows(int Nr) { return Nr <= 32 ? 32 : Nr <= 64 ? 64 : 128; }
// W_g [N_r, d] -> its packed order (moe_pack_router), d % 16 == 0.
hipError_t launch_pack_router(const float* wg, float* dst, int d, int Nr, hipStream_t s);

// Routing statistics: every router workgroup (at least 32 tokens each) sums
// its tokens' softmax values, choices and squared log-sum-exps into one row
// of kStatsStride doubles; route_stats_kernel folds the rows in order.
constexpr int kStatsCount = 256;   // offset of the choice counts in a row
constexpr int kStatsZ = 512;       // offset of the sum of lse^2
constexpr int kStatsStride = 514;
inline size_t route_stats_bytes(int64_t T) {
  return static_cast<size_t>((T + 31) / 32) * kStatsStride * sizeof(double);
}
// Router (a.stats_part set, a.partial null) followed by the fold into
// stats[2 N_r + 2 D + 3] (layout in include/moe.h, moe_route_stats).
hipError_t launch_route_stats(const RouteArgs& a, int n_devices, float* stats, hipStream_t s);

// ---- dispatch (dispatch.hip) ----
constexpr int kCountBlock = 256;  // tokens per counting block
struct PermuteArgs {
  const int32_t* topk_idx;  // [T, K']
  const void* x;            // [T, d] (only when x_perm != null)
  int T, d, n_routed, top_k, elt_bytes;
  int32_t* counts;          // [N_r]
  int32_t* offsets;         // [N_r + 1]
  int32_t* row_token;       // [P]
  int32_t* slot_row;        // [P]
  void* x_perm;             // [P, d] or null
  int32_t* block_counts;    // ws: [NB, N_r]
  int32_t* block_base;      // ws: [NB, N_r]
  int32_t* local_rank;      // ws: [P]
  // Expert capacity (capacity > 0): at most `capacity` assignments per expert
  // in every group of `group_len` consecutive tokens (n_groups groups).  The
  // dropless dispatch goes to the full_* buffers first.
  int capacity, group_len, n_groups;
  int32_t* full_counts;     // ws: [N_r]
  int32_t* full_offsets;    // ws: [N_r + 1]
  int32_t* full_row_token;  // ws: [P]
  int32_t* full_slot_row;   // ws: [P]
  int32_t* group_start;     // ws: [n_groups + 1, N_r]
  int32_t* group_base;      // ws: [N_r, n_groups]
};
hipError_t launch_permute(const PermuteArgs& a, hipStream_t s);
// *bad = 0, then 1 if any token's K' <= 16 ids leave [0, Nr) or repeat
// (the checked build's moe_permute).
hipError_t launch_check_topk(const int32_t* topk_idx, int T, int K, int Nr, int32_t* bad,
                             hipStream_t s);


// ---- grouped GEMMs (gemm_bf16.hip, gemm_f32.hip) ----
enum GemmMode { kGateUp = 0, kDown = 1 };

// Packed weight layout (bf16): a [N, K] matrix is cut into tiles of
// kPackRows rows (N % kPackRows == 0); a tile holds its K/64 steps one after
// the other, each step kPackRows rows x 64 values, row-major.  Element (n, k)
// sits at (n / kPackRows) * kPackRows * K + (k / 64) * kPackRows * 64 +
// (n % kPackRows) * 64 + k % 64, so one K step of a tile is 16 KB of
// contiguous memory.
constexpr int kPackRows = 128;
// dst = the packed form of `count` row-major [rows, cols] bf16 matrices.
hipError_t launch_pack(const void* src, void* dst, int64_t count, int rows, int cols, hipStream_t s);

// Rows of group g are [offsets[g], offsets[g+1]) of a row-concatenated
// matrix (offsets null: one group of M rows).  A row r lives at
// A + (gather ? gather[r] : r) * lda.  B element (n, k) of group g is
// B + g*b_group_stride + (k / k_sub)*b_sub_stride + n*ldb + (k % k_sub).
// kGateUp: C[r, n] = silu(A_r . B0_n) * (A_r . B1_n), n < N.
// kDown:   C[r, n] = A_r . B0_n.
//
// Extra groups (grouped calls only; the shared experts folded into the
// routed launch): group n_groups + s, s < n_extra, holds rows
// [extra_base + s*extra_rows, extra_base + (s+1)*extra_rows), takes B from
// Bx0/Bx1 + s*bx_group_stride (bx_bytes per matrix), and with a gather its
// row r reads A row (r - extra_base) % extra_rows (every token once).
struct GemmArgs {
  bool relu;               // kDown only: C[r, n] = max(A_r . B0_n, 0) (ReLU expert FFN)
  bool packed;             // B (and Bx) in the packed layout (bf16 only; k_sub is the K of one matrix)
  int64_t a_bytes;         // bytes of A readable through row indices (< 4 GB)
  int64_t b_bytes;         // bytes of one group's B0 (and of its B1) (< 4 GB)
  const int32_t* offsets;
  int n_groups;
  int64_t rows_total;      // upper bound of the row space (host known: P or T, plus the
                           // extra groups); with an expert capacity the groups end at
                           // offsets[n_groups] <= P and rows up to extra_base are unused
  const void* A;
  int64_t lda;
  const int32_t* gather;
  const void* B0;
  const void* B1;
  int64_t ldb, b_group_stride, b_sub_stride;
  int k_sub;
  int N, K;
  void* C;
  int64_t ldc;
  int mode;
  int n_extra;
  int extra_rows;
  int64_t extra_base;
  const void* Bx0;
  const void* Bx1;
  int64_t bx_group_stride, bx_bytes;
};
// Optional timing of one launch: the events take the kernel's own start and
// end (hipExtLaunchKernel), so no marker packets sit between the kernels.  A
// launch that has no work records both on the stream instead.
struct StageEvents {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
  bool any() const { return start != nullptr || stop != nullptr; }
};
hipError_t record_stage(StageEvents ev, hipStream_t s);
hipError_t launch_gemm_bf16(const GemmArgs& a, hipStream_t s, StageEvents ev = {});
hipError_t launch_gemm_f32(const GemmArgs& a, hipStream_t s);

// ---- combine (combine.hip) ----
struct CombineArgs {
  const void* y_perm;       // [P, d]
  const int32_t* slot_row;  // [P]
  const float* topk_w;      // [T, K']
  const void* y_shared;     // shared_blocks x [T, d] (shared_stride elements apart) or null
  int shared_blocks;
  int64_t shared_stride;
  const void* residual;     // [T, d] or null
  void* y;                  // [T, d]
  int T, d, top_k;
  bool bf16;
};
hipError_t launch_combine(const CombineArgs& a, hipStream_t s);
hipError_t launch_zero(void* p, size_t bytes, hipStream_t s);

}  // namespace moe
