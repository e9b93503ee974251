// Dispatch: histogram, exclusive scan and stable scatter of the T*K'
// (token, expert) assignments, so that only the chosen experts run (MoE-survey
// blog page, section 2: E_i(x) is not computed where G(x)_i = 0; the
// per-expert count is GShard's running counter c_e, ibid. section 3).
//
// Three launches (one for small batches without the row copy), no host
// synchronisation:
//   count   one thread per token, 256 tokens per block.  Per wave, one ballot
//           per expert gives the set of lanes that chose it; its popcount is
//           the wave's count, and popcount(mask & lanes-below) is the stable
//           rank of a token inside the wave.  Block totals go to block_counts.
//   scan    one block: per-expert totals over blocks, exclusive scan over
//           experts (offsets), and the first row of every (block, expert).
//   scatter row = block_base[block, e] + local rank: writes row_token,
//           slot_row and, when asked, copies x rows into x_perm (one wave per
//           token reads the row once and writes it K' times, 16 B per lane).
#include "common.h"
#include "dispatch_small.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kMaxK = 16;
constexpr int kMaxExperts = 256;

__global__ __launch_bounds__(kCountBlock) void count_kernel(
    const int32_t* __restrict__ idx, int T, int K, int Nr, int32_t* __restrict__ block_counts,
    int32_t* __restrict__ local_rank) {
  __shared__ uint64_t masks[kCountBlock / kWave][kMaxExperts];
  __shared__ int cnt[kCountBlock / kWave][kMaxExperts];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kCountBlock + threadIdx.x;
  const bool valid = t < T;

  int ids[kMaxK];
  uint64_t bits0 = 0, bits1 = 0, bits2 = 0, bits3 = 0;
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    ids[j] = -1;
    if (j < K && valid) {
      const int e = idx[t * K + j];
      ids[j] = e;
      const uint64_t b = 1ull << (e & 63);
      const int w = e >> 6;
      bits0 |= (w == 0) ? b : 0ull;
      bits1 |= (w == 1) ? b : 0ull;
      bits2 |= (w == 2) ? b : 0ull;
      bits3 |= (w == 3) ? b : 0ull;
    }
  }
  for (int e = 0; e < Nr; ++e) {
    const int w = e >> 6;
    const uint64_t bits = (w == 0) ? bits0 : (w == 1) ? bits1 : (w == 2) ? bits2 : bits3;
    const uint64_t m = __ballot((bits >> (e & 63)) & 1ull);
    if (lane == 0) {
      masks[wave][e] = m;
      cnt[wave][e] = __popcll(m);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < Nr; e += kCountBlock) {
    int s = 0;
#pragma unroll
    for (int w = 0; w < kCountBlock / kWave; ++w) s += cnt[w][e];
    block_counts[static_cast<int64_t>(blockIdx.x) * Nr + e] = s;
  }
  if (!valid) return;
  const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    if (j < K) {
      const int e = ids[j];
      int r = __popcll(masks[wave][e] & below);
      for (int w = 0; w < wave; ++w) r += cnt[w][e];
      local_rank[t * K + j] = r;
    }
  }
}

constexpr int kScanThreads = 1024;

__global__ __launch_bounds__(kScanThreads) void scan_kernel(
    const int32_t* __restrict__ block_counts, int NB, int Nr, int32_t* __restrict__ block_base,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets) {
  __shared__ int part[kScanThreads];
  __shared__ int tot[kMaxExperts];
  __shared__ int offs[kMaxExperts + 1];
  int L = 1;
  while (L * 2 * Nr <= kScanThreads) L *= 2;  // lanes per expert
  const int e = threadIdx.x / L;
  const int sub = threadIdx.x % L;
  const bool active = e < Nr;
  const int C = (NB + L - 1) / L;
  const int b0 = min(NB, sub * C), b1 = min(NB, b0 + C);
  int s = 0;
  if (active)
    for (int b = b0; b < b1; ++b) s += block_counts[static_cast<int64_t>(b) * Nr + e];
  part[threadIdx.x] = s;
  __syncthreads();
  if (active && sub == 0) {
    int run = 0;
    for (int i = 0; i < L; ++i) {
      const int v = part[e * L + i];
      part[e * L + i] = run;
      run += v;
    }
    tot[e] = run;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int i = 0; i < Nr; ++i) {
      offs[i] = run;
      run += tot[i];
    }
    offs[Nr] = run;
  }
  __syncthreads();
  if (threadIdx.x < Nr) {
    counts[threadIdx.x] = tot[threadIdx.x];
    offsets[threadIdx.x] = offs[threadIdx.x];
  }
  if (threadIdx.x == 0) offsets[Nr] = offs[Nr];
  if (active) {
    int run = offs[e] + part[threadIdx.x];
    for (int b = b0; b < b1; ++b) {
      const int64_t i = static_cast<int64_t>(b) * Nr + e;
      block_base[i] = run;
      run += block_counts[i];
    }
  }
}

// Index-only scatter: one thread per assignment.
__global__ __launch_bounds__(256) void scatter_index_kernel(
    const int32_t* __restrict__ idx, const int32_t* __restrict__ local_rank,
    const int32_t* __restrict__ block_base, int64_t P, int K, int Nr,
    int32_t* __restrict__ row_token, int32_t* __restrict__ slot_row) {
  const int64_t a = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (a >= P) return;
  const int e = idx[a];
  const int64_t t = a / K;
  const int64_t blk = t / kCountBlock;
  const int row = block_base[blk * Nr + e] + local_rank[a];
  slot_row[a] = row;
  row_token[row] = static_cast<int32_t>(t);
}

// Scatter with row copy: one wave per token, 16-byte chunks.
__global__ __launch_bounds__(256) void scatter_copy_kernel(
    const int32_t* __restrict__ idx, const int32_t* __restrict__ local_rank,
    const int32_t* __restrict__ block_base, int T, int K, int Nr, const uint4* __restrict__ x,
    int chunks_per_row, int32_t* __restrict__ row_token, int32_t* __restrict__ slot_row,
    uint4* __restrict__ x_perm) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t t = static_cast<int64_t>(blockIdx.x) * (256 / kWave) + threadIdx.x / kWave;
  if (t >= T) return;
  int row = 0;
  if (lane < K) {
    const int64_t a = t * K + lane;
    const int e = idx[a];
    row = block_base[(t / kCountBlock) * Nr + e] + local_rank[a];
    slot_row[a] = row;
    row_token[row] = static_cast<int32_t>(t);
  }
  // Broadcast the K' destination rows while every lane is active.
  int rows[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) rows[j] = __shfl(row, j, kWave);
  const uint4* src = x + t * chunks_per_row;
  for (int c = lane; c < chunks_per_row; c += kWave) {
    const uint4 v = src[c];
#pragma unroll
    for (int j = 0; j < kMaxK; ++j)
      if (j < K) x_perm[static_cast<int64_t>(rows[j]) * chunks_per_row + c] = v;
  }
}

// Small batches (T <= kSmallTokens, no row copy): the three steps above in
// one workgroup, one thread per token (small_dispatch, dispatch_small.h).
__global__ __launch_bounds__(kSmallTokens) void dispatch_small_kernel(
    const int32_t* __restrict__ idx, int T, int K, int Nr, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ row_token, int32_t* __restrict__ slot_row) {
  __shared__ SmallDispatchLds sh;
  small_dispatch(idx, T, K, Nr, counts, offsets, row_token, slot_row, sh);
}

}  // namespace

hipError_t launch_permute(const PermuteArgs& a, hipStream_t s) {
  if (a.T == 0) {
    // Empty batch: all counts and offsets are zero.
    hipError_t err = launch_zero(a.counts, sizeof(int32_t) * a.n_routed, s);
    if (err != hipSuccess) return err;
    return launch_zero(a.offsets, sizeof(int32_t) * (a.n_routed + 1), s);
  }
  if (a.T <= kSmallTokens && a.x_perm == nullptr) {
    hipLaunchKernelGGL(dispatch_small_kernel, dim3(1), dim3(kSmallTokens), 0, s, a.topk_idx, a.T,
                       a.top_k, a.n_routed, a.counts, a.offsets, a.row_token, a.slot_row);
    return hipGetLastError();
  }
  const int NB = (a.T + kCountBlock - 1) / kCountBlock;
  hipLaunchKernelGGL(count_kernel, dim3(NB), dim3(kCountBlock), 0, s, a.topk_idx, a.T, a.top_k,
                     a.n_routed, a.block_counts, a.local_rank);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(kScanThreads), 0, s, a.block_counts, NB,
                     a.n_routed, a.block_base, a.counts, a.offsets);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int64_t P = static_cast<int64_t>(a.T) * a.top_k;
  if (a.x_perm == nullptr) {
    const int grid = static_cast<int>((P + 255) / 256);
    hipLaunchKernelGGL(scatter_index_kernel, dim3(grid), dim3(256), 0, s, a.topk_idx,
                       a.local_rank, a.block_base, P, a.top_k, a.n_routed, a.row_token,
                       a.slot_row);
  } else {
    const int grid = (a.T + 3) / 4;
    const int chunks = static_cast<int>((static_cast<int64_t>(a.d) * a.elt_bytes) / 16);
    hipLaunchKernelGGL(scatter_copy_kernel, dim3(grid), dim3(256), 0, s, a.topk_idx,
                       a.local_rank, a.block_base, a.T, a.top_k, a.n_routed,
                       static_cast<const uint4*>(a.x), chunks, a.row_token, a.slot_row,
                       static_cast<uint4*>(a.x_perm));
  }
  return hipGetLastError();
}

}  // namespace moe
