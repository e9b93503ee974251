// Router: fp32 logits, softmax and per-token top-K' on one wavefront.
//
// DeepSeekMoE page, section 3.2, eq. 10-11: s = Softmax_i(u^T e_i) over the
// routed experts, keep the top K' values as gates.  MoE-survey blog page,
// section 2: Softmax(KeepTopK(H, k)) (noise off) for the second gate kind;
// section 5: router probabilities are computed in float32.
//
// Layout: a wavefront is split into groups of NP lanes; each group owns
// TPL tokens and lane j of a group owns experts j, j+NP, ... (EPL of them),
// so the softmax and arg-max over experts are cross-lane reductions inside
// the group (xor shuffles), and the chosen set is ranked with a ballot.
// Logits accumulate over d in fp32 with one FMA chain per (token, expert).
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kRouterThreads = 256;
constexpr int kTPL = 8;

template <typename XT>
__device__ __forceinline__ void load4(const XT* p, float (&v)[4]);
template <>
__device__ __forceinline__ void load4<float>(const float* p, float (&v)[4]) {
  float4 q = *reinterpret_cast<const float4*>(p);
  v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
}
template <>
__device__ __forceinline__ void load4<bf16_t>(const bf16_t* p, float (&v)[4]) {
  uint2 q = *reinterpret_cast<const uint2*>(p);
  v[0] = __uint_as_float(q.x << 16);
  v[1] = __uint_as_float(q.x & 0xFFFF0000u);
  v[2] = __uint_as_float(q.y << 16);
  v[3] = __uint_as_float(q.y & 0xFFFF0000u);
}

template <typename XT, int NP, int EPL>
__global__ __launch_bounds__(kRouterThreads) void router_kernel(
    const XT* __restrict__ x, const float* __restrict__ wg, const float* __restrict__ bias,
    int T, int d, int Nr, int K, int gate, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_w) {
  constexpr int G = kWave / NP;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int grp = lane / NP;
  const int gl = lane % NP;
  const int64_t tok0 =
      (static_cast<int64_t>(blockIdx.x) * (kRouterThreads / kWave) + wave) * (G * kTPL) +
      grp * kTPL;
  if (tok0 >= T) return;

  int e[EPL];
  bool ev[EPL];
  const float* wrow[EPL];
#pragma unroll
  for (int q = 0; q < EPL; ++q) {
    e[q] = gl + NP * q;
    ev[q] = e[q] < Nr;
    wrow[q] = wg + static_cast<int64_t>(ev[q] ? e[q] : Nr - 1) * d;
  }
  const XT* xrow[kTPL];
#pragma unroll
  for (int i = 0; i < kTPL; ++i) {
    int64_t t = tok0 + i;
    xrow[i] = x + (t < T ? t : T - 1) * static_cast<int64_t>(d);
  }

  float acc[kTPL][EPL];
#pragma unroll
  for (int i = 0; i < kTPL; ++i)
#pragma unroll
    for (int q = 0; q < EPL; ++q) acc[i][q] = 0.0f;

  for (int k = 0; k < d; k += 4) {
    float w[EPL][4];
#pragma unroll
    for (int q = 0; q < EPL; ++q) load4<float>(wrow[q] + k, w[q]);
#pragma unroll
    for (int i = 0; i < kTPL; ++i) {
      float xv[4];
      load4<XT>(xrow[i] + k, xv);
#pragma unroll
      for (int q = 0; q < EPL; ++q) {
        float a = acc[i][q];
        a = fmaf(xv[0], w[q][0], a);
        a = fmaf(xv[1], w[q][1], a);
        a = fmaf(xv[2], w[q][2], a);
        a = fmaf(xv[3], w[q][3], a);
        acc[i][q] = a;
      }
    }
  }

  float bq[EPL];
#pragma unroll
  for (int q = 0; q < EPL; ++q) bq[q] = (bias != nullptr && ev[q]) ? bias[e[q]] : 0.0f;

  const uint64_t gmask = (NP == 64) ? ~0ull : (((1ull << NP) - 1ull) << (grp * NP));
  const uint64_t below = (1ull << lane) - 1ull;

#pragma unroll
  for (int i = 0; i < kTPL; ++i) {
    const int64_t t = tok0 + i;
    if (t >= T) break;  // uniform within the group
    float z[EPL];
    bool sel[EPL];
#pragma unroll
    for (int q = 0; q < EPL; ++q) {
      z[q] = ev[q] ? acc[i][q] + bq[q] : -INFINITY;
      sel[q] = false;
    }
    // K' rounds of arg-max over the not-yet-chosen experts; ties -> lower id.
    float zmax = -INFINITY;
    for (int r = 0; r < K; ++r) {
      float m = -INFINITY;
#pragma unroll
      for (int q = 0; q < EPL; ++q)
        if (!sel[q]) m = fmaxf(m, z[q]);
      m = group_max<NP>(m);
      if (r == 0) zmax = m;
      int cand = 0x7FFFFFFF;
#pragma unroll
      for (int q = 0; q < EPL; ++q)
        if (!sel[q] && ev[q] && z[q] == m) cand = min(cand, e[q]);
      cand = group_min_int<NP>(cand);
#pragma unroll
      for (int q = 0; q < EPL; ++q)
        if (e[q] == cand) sel[q] = true;
    }
    float ex[EPL];
    float part = 0.0f;
#pragma unroll
    for (int q = 0; q < EPL; ++q) {
      ex[q] = ev[q] ? expf(z[q] - zmax) : 0.0f;
      if (gate == 0 || sel[q]) part += ex[q];
    }
    const float denom = group_sum<NP>(part);
    int prior = 0;
#pragma unroll
    for (int q = 0; q < EPL; ++q) {
      const uint64_t m = __ballot(sel[q]) & gmask;
      if (sel[q]) {
        const int slot = prior + __popcll(m & below);
        topk_idx[t * K + slot] = e[q];
        topk_w[t * K + slot] = ex[q] / denom;
      }
      prior += __popcll(m);
    }
  }
}

template <typename XT, int NP, int EPL>
hipError_t launch_t(const RouteArgs& a, hipStream_t s) {
  constexpr int G = kWave / NP;
  constexpr int tok_per_block = (kRouterThreads / kWave) * G * kTPL;
  const int grid = (a.T + tok_per_block - 1) / tok_per_block;
  hipLaunchKernelGGL((router_kernel<XT, NP, EPL>), dim3(grid), dim3(kRouterThreads), 0, s,
                     static_cast<const XT*>(a.x), a.w_router, a.bias, a.T, a.d, a.n_routed,
                     a.top_k, a.gate, a.topk_idx, a.topk_w);
  return hipGetLastError();
}

template <typename XT>
hipError_t launch_x(const RouteArgs& a, hipStream_t s) {
  const int n = a.n_routed;
  if (n <= 8) return launch_t<XT, 8, 1>(a, s);
  if (n <= 16) return launch_t<XT, 16, 1>(a, s);
  if (n <= 32) return launch_t<XT, 32, 1>(a, s);
  if (n <= 64) return launch_t<XT, 64, 1>(a, s);
  if (n <= 128) return launch_t<XT, 64, 2>(a, s);
  return launch_t<XT, 64, 4>(a, s);
}

}  // namespace

hipError_t launch_route(const RouteArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  return a.x_bf16 ? launch_x<bf16_t>(a, s) : launch_x<float>(a, s);
}

}  // namespace moe
