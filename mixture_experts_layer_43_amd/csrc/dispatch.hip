// Dispatch: histogram, exclusive scan and stable scatter of the T*K'
// (token, expert) assignments, so that only the chosen experts run (MoE-survey
// blog page, section 2: E_i(x) is not computed where G(x)_i = 0; the
// per-expert count is GShard's running counter c_e, ibid. section 3).
//
// Three launches (one for small batches without the row copy), no host
// synchronisation:
//   count   one thread per token, 256 tokens per block.  Per wave, a 64-bit
//           mask per expert of the lanes that chose it (built with LDS
//           atomic ORs); its popcount is the wave's count, and
//           popcount(mask & lanes-below) is the stable rank of a token inside
//           the wave.  Block totals go to block_counts.
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
static_assert(kMaxExperts <= 4 * kWave, "the expert scans take four experts per lane");

__global__ __launch_bounds__(kCountBlock) void count_kernel(
    const int32_t* __restrict__ idx, int T, int K, int Nr, int32_t* __restrict__ block_counts,
    int32_t* __restrict__ local_rank) {
  __shared__ uint64_t masks[kCountBlock / kWave][kMaxExperts];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kCountBlock + threadIdx.x;
  const bool valid = t < T;

  // Each wavefront clears its 64-bit mask per expert, then every lane ORs
  // its bit into the masks of its K experts (a wavefront's LDS operations
  // run in order, so no barrier in between).
  int ids[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    ids[j] = -1;
    if (j < K && valid) ids[j] = idx[t * K + j];
  }
  for (int e = lane; e < Nr; e += kWave) masks[wave][e] = 0ull;
#pragma unroll
  for (int j = 0; j < kMaxK; ++j)
    if (j < K && valid) atomicOr(&masks[wave][ids[j]], 1ull << lane);
  __syncthreads();
  for (int e = threadIdx.x; e < Nr; e += kCountBlock) {
    int s = 0;
#pragma unroll
    for (int w = 0; w < kCountBlock / kWave; ++w) s += __popcll(masks[w][e]);
    block_counts[static_cast<int64_t>(blockIdx.x) * Nr + e] = s;
  }
  if (!valid) return;
  const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    if (j < K) {
      const int e = ids[j];
      int r = __popcll(masks[wave][e] & below);
      for (int w = 0; w < wave; ++w) r += __popcll(masks[w][e]);
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
  // Exclusive scan over the experts in wavefront 0: four experts per lane,
  // shuffle prefix sums.
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    int v[4], sum = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int ei = lane * 4 + q;
      v[q] = ei < Nr ? tot[ei] : 0;
      sum += v[q];
    }
    int incl = sum;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int u = __shfl_up(incl, o, kWave);
      if (lane >= o) incl += u;
    }
    int run = incl - sum;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int ei = lane * 4 + q;
      if (ei < Nr) offs[ei] = run;
      run += v[q];
    }
    if (lane == kWave - 1) offs[Nr] = incl;
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

// ---- expert capacity ---------------------------------------------------------
// GShard's expert capacity with local group dispatching (MoE-survey blog page,
// section 3; Switch, section 4): in every group of S consecutive tokens an
// expert keeps its first C assignments in token order, the rest are dropped.
// Built on the dropless dispatch, whose rows of expert e already hold its
// tokens in ascending order:
//   bounds   start[g][e] = number of e's rows whose token is below g*S (binary
//            search in e's sorted rows), g = 0..G
//   scan     kept(e, g) = min(start[g+1][e] - start[g][e], C); one exclusive
//            scan in (e, g) order gives every (expert, group) its first row,
//            and the counts and offsets of the kept rows
//   scatter  the slot of token t with dropless row r of expert e has rank
//            q = r - full_offsets[e] - start[t/S][e] inside its group; it
//            keeps row base[e][t/S] + q when q < C, else slot_row = -1.
__global__ __launch_bounds__(256) void cap_bounds_kernel(
    const int32_t* __restrict__ full_row_token, const int32_t* __restrict__ full_offsets, int S,
    int G, int Nr, int32_t* __restrict__ start) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= static_cast<int64_t>(G + 1) * Nr) return;
  const int g = static_cast<int>(i / Nr), e = static_cast<int>(i % Nr);
  const int first = full_offsets[e], n = full_offsets[e + 1] - first;
  int lo = 0;
  if (g == G) {
    lo = n;
  } else {
    const int64_t key = static_cast<int64_t>(g) * S;   // first token of group g
    int hi = n;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (full_row_token[first + mid] < key) lo = mid + 1; else hi = mid;
    }
  }
  start[i] = lo;
}

constexpr int kCapScanThreads = 1024;

// One workgroup: exclusive scan of kept(e, g) over the N_r*G entries in
// (e, g) order, each thread a contiguous run of entries; wavefront prefix
// sums by shuffles, then the 16 wavefront totals.
__global__ __launch_bounds__(kCapScanThreads) void cap_scan_kernel(
    const int32_t* __restrict__ start, int G, int Nr, int C, int32_t* __restrict__ base,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets) {
  constexpr int W = kCapScanThreads / kWave;
  __shared__ int wsum[W], wpre[W];
  __shared__ int offs[kMaxExperts + 1];
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int64_t M = static_cast<int64_t>(Nr) * G;
  const int64_t per = (M + kCapScanThreads - 1) / kCapScanThreads;
  const int64_t i0 = min(M, per * threadIdx.x), i1 = min(M, i0 + per);
  auto kept = [&](int64_t i) {
    const int e = static_cast<int>(i / G), g = static_cast<int>(i % G);
    return min(start[static_cast<int64_t>(g + 1) * Nr + e] - start[static_cast<int64_t>(g) * Nr + e], C);
  };
  int s = 0;
  for (int64_t i = i0; i < i1; ++i) s += kept(i);
  int incl = s;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int y = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += y;
  }
  if (lane == kWave - 1) wsum[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    const int w = lane < W ? wsum[lane] : 0;
    int wi = w;
#pragma unroll
    for (int o = 1; o < W; o <<= 1) {
      const int y = __shfl_up(wi, o, kWave);
      if (lane >= o) wi += y;
    }
    if (lane < W) wpre[lane] = wi - w;
    if (lane == W - 1) offs[Nr] = wi;
  }
  __syncthreads();
  int run = wpre[wave] + incl - s;
  for (int64_t i = i0; i < i1; ++i) {
    if (i % G == 0) offs[i / G] = run;
    base[i] = run;
    run += kept(i);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < Nr; e += kCapScanThreads) {
    offsets[e] = offs[e];
    counts[e] = offs[e + 1] - offs[e];
  }
  if (threadIdx.x == 0) offsets[Nr] = offs[Nr];
}

__global__ __launch_bounds__(256) void cap_scatter_kernel(
    const int32_t* __restrict__ idx, const int32_t* __restrict__ full_slot_row,
    const int32_t* __restrict__ full_offsets, const int32_t* __restrict__ start,
    const int32_t* __restrict__ base, int64_t P, int K, int Nr, int S, int G, int C,
    int32_t* __restrict__ row_token, int32_t* __restrict__ slot_row) {
  const int64_t a = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (a >= P) return;
  const int e = idx[a];
  const int64_t t = a / K;
  const int g = static_cast<int>(t / S);
  const int q = full_slot_row[a] - full_offsets[e] - start[static_cast<int64_t>(g) * Nr + e];
  if (q < C) {
    const int row = base[static_cast<int64_t>(e) * G + g] + q;
    slot_row[a] = row;
    row_token[row] = static_cast<int32_t>(t);
  } else {
    slot_row[a] = -1;
  }
}

// x_perm[r] = x[row_token[r]] for the rows below offsets[N_r] (read on the
// device): one wavefront per row, 16 bytes per lane.
__global__ __launch_bounds__(256) void gather_rows_kernel(
    const int32_t* __restrict__ row_token, const int32_t* __restrict__ total, int64_t P,
    const uint4* __restrict__ x, int chunks_per_row, uint4* __restrict__ x_perm) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t r = static_cast<int64_t>(blockIdx.x) * (256 / kWave) + threadIdx.x / kWave;
  if (r >= P || r >= *total) return;
  const uint4* src = x + static_cast<int64_t>(row_token[r]) * chunks_per_row;
  uint4* dst = x_perm + r * chunks_per_row;
  for (int c = lane; c < chunks_per_row; c += kWave) dst[c] = src[c];
}

hipError_t launch_dropless(const PermuteArgs& a, hipStream_t s) {
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

}  // namespace

// Caller-supplied routing checked before a dispatch uses it: one thread per
// token sets *bad when an id lies outside [0, N_r) or repeats within the
// token's K' ids.  Reads topk_idx only.
__global__ __launch_bounds__(256) void check_topk_kernel(const int32_t* __restrict__ topk_idx, int T,
                                                         int K, int Nr, int32_t* __restrict__ bad) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= T) return;
  int32_t id[16];
  bool ok = true;
  for (int j = 0; j < K; ++j) {
    id[j] = topk_idx[static_cast<int64_t>(t) * K + j];
    ok = ok && id[j] >= 0 && id[j] < Nr;
    for (int i = 0; i < j; ++i) ok = ok && id[i] != id[j];
  }
  if (!ok) *bad = 1;
}

hipError_t launch_check_topk(const int32_t* topk_idx, int T, int K, int Nr, int32_t* bad,
                             hipStream_t s) {
  hipError_t err = launch_zero(bad, sizeof(int32_t), s);
  if (err != hipSuccess || T == 0) return err;
  hipLaunchKernelGGL(check_topk_kernel, dim3(static_cast<unsigned>((T + 255) / 256)), dim3(256), 0, s,
                     topk_idx, T, K, Nr, bad);
  return hipGetLastError();
}

hipError_t launch_permute(const PermuteArgs& a, hipStream_t s) {
  if (a.T == 0) {
    // Empty batch: all counts and offsets are zero.
    hipError_t err = launch_zero(a.counts, sizeof(int32_t) * a.n_routed, s);
    if (err != hipSuccess) return err;
    return launch_zero(a.offsets, sizeof(int32_t) * (a.n_routed + 1), s);
  }
  if (a.capacity <= 0) return launch_dropless(a, s);

  PermuteArgs f = a;
  f.counts = a.full_counts;
  f.offsets = a.full_offsets;
  f.row_token = a.full_row_token;
  f.slot_row = a.full_slot_row;
  f.x_perm = nullptr;
  hipError_t err = launch_dropless(f, s);
  if (err != hipSuccess) return err;
  const int G = a.n_groups, Nr = a.n_routed;
  const int64_t nb = (static_cast<int64_t>(G + 1) * Nr + 255) / 256;
  hipLaunchKernelGGL(cap_bounds_kernel, dim3(static_cast<unsigned>(nb)), dim3(256), 0, s,
                     a.full_row_token, a.full_offsets, a.group_len, G, Nr, a.group_start);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  hipLaunchKernelGGL(cap_scan_kernel, dim3(1), dim3(kCapScanThreads), 0, s, a.group_start, G, Nr,
                     a.capacity, a.group_base, a.counts, a.offsets);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  const int64_t P = static_cast<int64_t>(a.T) * a.top_k;
  hipLaunchKernelGGL(cap_scatter_kernel, dim3(static_cast<unsigned>((P + 255) / 256)), dim3(256), 0,
                     s, a.topk_idx, a.full_slot_row, a.full_offsets, a.group_start, a.group_base, P,
                     a.top_k, Nr, a.group_len, G, a.capacity, a.row_token, a.slot_row);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (a.x_perm != nullptr) {
    const int chunks = static_cast<int>((static_cast<int64_t>(a.d) * a.elt_bytes) / 16);
    hipLaunchKernelGGL(gather_rows_kernel, dim3(static_cast<unsigned>((P + 3) / 4)), dim3(256), 0, s,
                       a.row_token, a.offsets + Nr, P, static_cast<const uint4*>(a.x), chunks,
                       static_cast<uint4*>(a.x_perm));
    err = hipGetLastError();
  }
  return err;
}

}  // namespace moe
