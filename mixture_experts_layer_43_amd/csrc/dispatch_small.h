// Dispatch of a small batch inside one workgroup of kSmallTokens threads
// (the single-workgroup path of dispatch.hip).
#pragma once

#include "common.h"

namespace moe {

constexpr int kSmallTokens = 1024;
constexpr int kDispatchMaxK = 16;
constexpr int kDispatchMaxExperts = 256;

// Stable counting sort of the T*K assignments of topk_idx (T <= kSmallTokens)
// by expert, one thread per token.  Each wavefront that holds tokens keeps a
// 64-bit mask per expert of its lanes (tokens) that chose it: it clears its
// own masks, then every lane ORs its bit into the masks of its K experts
// (LDS operations of one wavefront run in order, so no barrier is needed in
// between).  Popcounts of the masks give per-wave counts and in-wave ranks;
// the scan runs over experts in LDS; a row is the first row of (wave,
// expert) - offsets[e] plus the rows of e in earlier waves - plus the rank
// in the wave, i.e. ascending token order.  Every thread of the workgroup
// must call it.
struct SmallDispatchLds {
  uint64_t masks[kSmallTokens / kWave][kDispatchMaxExperts];
  int cnt[kSmallTokens / kWave][kDispatchMaxExperts];   // first row of (wave, expert)
  int offs[kDispatchMaxExperts + 1];
};

__device__ __forceinline__ void small_dispatch(const int32_t* __restrict__ idx, int T, int K, int Nr,
                                               int32_t* __restrict__ counts,
                                               int32_t* __restrict__ offsets,
                                               int32_t* __restrict__ row_token,
                                               int32_t* __restrict__ slot_row, SmallDispatchLds& sh) {
  const int NWV = (T + kWave - 1) / kWave;   // wavefronts that hold tokens
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int t = threadIdx.x;
  const bool valid = t < T;
  int ids[kDispatchMaxK];
#pragma unroll
  for (int j = 0; j < kDispatchMaxK; ++j) {
    ids[j] = -1;
    if (j < K && valid) ids[j] = idx[static_cast<int64_t>(t) * K + j];
  }
  if (wave < NWV) {
    for (int e = lane; e < Nr; e += kWave) sh.masks[wave][e] = 0ull;
#pragma unroll
    for (int j = 0; j < kDispatchMaxK; ++j)
      if (j < K && valid) atomicOr(&sh.masks[wave][ids[j]], 1ull << lane);
  }
  __syncthreads();
  // Per-expert totals in parallel, then an exclusive scan over the experts
  // in wavefront 0 (four experts per lane, shuffle prefix sums).
  if (threadIdx.x < Nr) {
    int c = 0;
    for (int w = 0; w < NWV; ++w) c += __popcll(sh.masks[w][threadIdx.x]);
    sh.offs[threadIdx.x + 1] = c;
  }
  __syncthreads();
  if (wave == 0) {
    int v[4], sum = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = lane * 4 + q;
      v[q] = e < Nr ? sh.offs[e + 1] : 0;
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
      const int e = lane * 4 + q;
      if (e < Nr) sh.offs[e] = run;
      run += v[q];
    }
    if (lane == kWave - 1) sh.offs[Nr] = incl;
  }
  __syncthreads();
  for (int e = threadIdx.x; e <= Nr; e += kSmallTokens) {
    offsets[e] = sh.offs[e];
    if (e < Nr) counts[e] = sh.offs[e + 1] - sh.offs[e];
  }
  // First row of each (wavefront, expert): the expert's offset plus the
  // rows of the wavefronts before.
  if (threadIdx.x < Nr) {
    int run = sh.offs[threadIdx.x];
    for (int w = 0; w < NWV; ++w) {
      sh.cnt[w][threadIdx.x] = run;
      run += __popcll(sh.masks[w][threadIdx.x]);
    }
  }
  __syncthreads();
  if (!valid) return;
  const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
  for (int j = 0; j < kDispatchMaxK; ++j) {
    if (j < K) {
      const int e = ids[j];
      const int r = sh.cnt[wave][e] + __popcll(sh.masks[wave][e] & below);
      slot_row[static_cast<int64_t>(t) * K + j] = r;
      row_token[r] = t;
    }
  }
}

}  // namespace moe
