// Router: fp32 logits, softmax and per-token top-K' on one wavefront.
//
// DeepSeekMoE page, section 3.2, eq. 10-11: s = Softmax_i(u^T e_i) over the
// routed experts, keep the top K' values as gates.  MoE-survey blog page,
// section 2: Softmax(KeepTopK(H, k)) (noise off) for the second gate kind;
// section 5: router probabilities are computed in float32.
//
// Logits.  bf16 layers (N_r <= 128) compute x W_g^T on the matrix cores:
// each fp32 router weight w is split in registers into three bf16 parts
// hi + mid + lo == w exactly (24 mantissa bits = 3 x 8), every bf16 x bf16
// product is exact in fp32, and v_mfma_f32_32x32x16_bf16 accumulates the
// three partial products in fp32, so the logits keep fp32 accuracy at a
// fraction of the VALU cost.  Other layers use one fp32 FMA chain per
// (token, expert) on the vector ALUs.
//
// Selection: a wavefront is split into groups of NP lanes; lane j of a group
// owns experts j, j+NP, ... (EPL of them), so the softmax and arg-max over
// experts are cross-lane reductions inside the group (xor shuffles), and the
// chosen set is ranked with a ballot.
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

// log(1 + e^v) in fp32: the noise scale of noisy top-k gating.  Above 20
// the correction log1p(e^-v) is below fp32 resolution.
__device__ __forceinline__ float softplus_f32(float v) { return v > 20.0f ? v : log1pf(expf(v)); }

// Running sums of the routing statistics (DeepSeekMoE page, section 3.3,
// eq. 13-14; MoE-survey blog page, section 5, z-loss) over the tokens one
// lane's group has selected for: s_i and times chosen for each expert the
// lane owns, and the squared log-sum-exp (the same on every lane of a group).
template <int EPL>
struct StatAcc {
  double p[EPL];
  int c[EPL];
  double z2;
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int q = 0; q < EPL; ++q) { p[q] = 0.0; c[q] = 0; }
    z2 = 0.0;
  }
};

// Top-K' of one token (lane-per-expert inside a group of NP lanes, EPL
// experts per lane: expert e[q] = lane-in-group + NP*q), gate values, and
// the ascending-id store.  K' rounds of group arg-max on the selection
// logits z, ties to the lower id; gate values from the gate logits zg:
// softmax over all routed experts (gate 0) or over the chosen ones (gate 1),
// relative to the largest logit of that set.  zg is z itself unless the bias
// is for selection only (bias_sel).  STATS: also adds the token's full
// softmax of zg (both gates), its choices and lse(zg)^2 to sa, and writes
// lse[t] when lse is set.
template <int NP, int EPL, bool STATS = false>
__device__ __forceinline__ void select_and_store(const float (&z)[EPL], const float (&zg)[EPL],
                                                 bool bias_sel, const int (&e)[EPL],
                                                 const bool (&ev)[EPL], int64_t t, int K,
                                                 int gate, int grp, int lane,
                                                 int32_t* __restrict__ topk_idx,
                                                 float* __restrict__ topk_w,
                                                 StatAcc<EPL>* sa = nullptr,
                                                 float* __restrict__ lse = nullptr) {
  // zs: the logits still in the running, NaN for experts past N_r and for
  // the chosen ones (fmaxf skips NaN and NaN equals nothing).  A lane's
  // experts ascend with q, so its first q whose logit equals the group
  // maximum is its lowest candidate id.  The chosen id c lives on lane
  // c % NP as q = c / NP.
  bool sel[EPL];
  float zs[EPL];
#pragma unroll
  for (int q = 0; q < EPL; ++q) {
    sel[q] = false;
    zs[q] = ev[q] ? z[q] : __builtin_nanf("");
  }
  const int gl = lane % NP;
  float zmax = -INFINITY;
  for (int r = 0; r < K; ++r) {
    float m = -INFINITY;
#pragma unroll
    for (int q = 0; q < EPL; ++q) m = fmaxf(m, zs[q]);
    m = group_max<NP>(m);
    if (r == 0) zmax = m;
    int cand = 0x7FFFFFFF;
#pragma unroll
    for (int q = EPL - 1; q >= 0; --q) cand = zs[q] == m ? e[q] : cand;
    cand = group_min_int<NP>(cand);
    const int qc = (cand & (NP - 1)) == gl ? static_cast<int>(static_cast<unsigned>(cand) / NP) : -1;
#pragma unroll
    for (int q = 0; q < EPL; ++q) {
      if (q == qc) {
        sel[q] = true;
        zs[q] = __builtin_nanf("");
      }
    }
  }
  if (bias_sel) {
    // Gates from the unbiased logits: the largest over all experts (gate 0)
    // or over the chosen ones (gate 1).
    float m = -INFINITY;
#pragma unroll
    for (int q = 0; q < EPL; ++q)
      if (gate == 0 || sel[q]) m = fmaxf(m, zg[q]);
    zmax = group_max<NP>(m);
  }
  float ex[EPL];
  float part = 0.0f;
#pragma unroll
  for (int q = 0; q < EPL; ++q) {
    ex[q] = ev[q] ? expf(zg[q] - zmax) : 0.0f;
    if (gate == 0 || sel[q]) part += ex[q];
  }
  const float denom = group_sum<NP>(part);
  const uint64_t gmask = (NP == 64) ? ~0ull : (((1ull << NP) - 1ull) << (grp * NP));
  const uint64_t below = (1ull << lane) - 1ull;
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
  if constexpr (STATS) {
    // Full softmax of zg relative to its largest value.  ex already is,
    // except for gate 1 with a selection-only bias (its zmax is the chosen
    // set's).
    float zall = zmax;
    float exs[EPL];
#pragma unroll
    for (int q = 0; q < EPL; ++q) exs[q] = ex[q];
    if (bias_sel && gate != 0) {
      float m = -INFINITY;
#pragma unroll
      for (int q = 0; q < EPL; ++q) m = fmaxf(m, zg[q]);
      zall = group_max<NP>(m);
#pragma unroll
      for (int q = 0; q < EPL; ++q) exs[q] = ev[q] ? expf(zg[q] - zall) : 0.0f;
    }
    float full = denom;
    if (gate != 0) {
      float pf = 0.0f;
#pragma unroll
      for (int q = 0; q < EPL; ++q) pf += exs[q];
      full = group_sum<NP>(pf);
    }
#pragma unroll
    for (int q = 0; q < EPL; ++q) {
      sa->p[q] += static_cast<double>(exs[q] / full);
      sa->c[q] += sel[q] ? 1 : 0;
    }
    const double l = static_cast<double>(zall) + log(static_cast<double>(full));
    sa->z2 += l * l;
    if (lse != nullptr && (lane % NP) == 0) lse[t] = static_cast<float>(l);
  }
}

// Sum of the lanes' StatAcc over one workgroup of W wavefronts in a fixed
// order (xor shuffles across the groups of a wavefront, then the wavefronts
// in order) into row[0, NP*EPL) (sum of s per expert), row[kStatsCount + e]
// (times chosen) and row[kStatsZ] (sum of lse^2).  red: LDS scratch of
// W * (2*NP*EPL + 1) doubles, free once every wavefront reaches this call.
template <int NP, int EPL, int W>
__device__ __forceinline__ void block_stats(StatAcc<EPL>& sa, int lane, int wave,
                                            double* red, double* __restrict__ row) {
  constexpr int NPAD = NP * EPL;
  constexpr int RS = 2 * NPAD + 1;
#pragma unroll
  for (int off = NP; off < kWave; off <<= 1) {
#pragma unroll
    for (int q = 0; q < EPL; ++q) {
      sa.p[q] += __shfl_xor(sa.p[q], off, kWave);
      sa.c[q] += __shfl_xor(sa.c[q], off, kWave);
    }
    sa.z2 += __shfl_xor(sa.z2, off, kWave);
  }
  __syncthreads();
  if (lane < NP) {
#pragma unroll
    for (int q = 0; q < EPL; ++q) {
      red[wave * RS + lane + NP * q] = sa.p[q];
      red[wave * RS + NPAD + lane + NP * q] = static_cast<double>(sa.c[q]);
    }
    if (lane == 0) red[wave * RS + 2 * NPAD] = sa.z2;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < RS; i += W * kWave) {
    double v = 0.0;
    for (int w = 0; w < W; ++w) v += red[w * RS + i];
    row[i < NPAD ? i : i < 2 * NPAD ? kStatsCount + (i - NPAD) : kStatsZ] = v;
  }
}

// NOISE: noisy top-k gating (MoE-survey blog page, section 2): the logit of
// expert i is x.w_i + eps[t][i] * softplus(x.wn_i), with a second fp32 dot
// product per (token, expert) against W_noise.
template <typename XT, int NP, int EPL, bool STATS, bool NOISE>
__global__ __launch_bounds__(kRouterThreads) void router_kernel(
    const XT* __restrict__ x, const float* __restrict__ wg, const float* __restrict__ bias,
    int T, int d, int Nr, int K, int gate, bool bias_sel, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_w, double* __restrict__ stats_part, float* __restrict__ lse,
    const float* __restrict__ wn, const float* __restrict__ eps) {
  constexpr int G = kWave / NP;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int grp = lane / NP;
  const int gl = lane % NP;
  const int64_t tok0 =
      (static_cast<int64_t>(blockIdx.x) * (kRouterThreads / kWave) + wave) * (G * kTPL) +
      grp * kTPL;
  // With statistics every wavefront must reach the workgroup reduction; the
  // clamped row pointers keep an idle group's loads in bounds.
  if (!STATS && tok0 >= T) return;

  int e[EPL];
  bool ev[EPL];
  const float* wrow[EPL];
  const float* nrow[EPL];
#pragma unroll
  for (int q = 0; q < EPL; ++q) {
    e[q] = gl + NP * q;
    ev[q] = e[q] < Nr;
    wrow[q] = wg + static_cast<int64_t>(ev[q] ? e[q] : Nr - 1) * d;
    nrow[q] = NOISE ? wn + static_cast<int64_t>(ev[q] ? e[q] : Nr - 1) * d : nullptr;
  }
  const XT* xrow[kTPL];
#pragma unroll
  for (int i = 0; i < kTPL; ++i) {
    int64_t t = tok0 + i;
    xrow[i] = x + (t < T ? t : T - 1) * static_cast<int64_t>(d);
  }

  float acc[kTPL][EPL];
  float accn[NOISE ? kTPL : 1][EPL];
#pragma unroll
  for (int i = 0; i < kTPL; ++i)
#pragma unroll
    for (int q = 0; q < EPL; ++q) {
      acc[i][q] = 0.0f;
      if constexpr (NOISE) accn[i][q] = 0.0f;
    }

  for (int k = 0; k < d; k += 4) {
    float w[EPL][4];
    float wv[NOISE ? EPL : 1][4];
#pragma unroll
    for (int q = 0; q < EPL; ++q) {
      load4<float>(wrow[q] + k, w[q]);
      if constexpr (NOISE) load4<float>(nrow[q] + k, wv[q]);
    }
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
        if constexpr (NOISE) {
          float b = accn[i][q];
          b = fmaf(xv[0], wv[q][0], b);
          b = fmaf(xv[1], wv[q][1], b);
          b = fmaf(xv[2], wv[q][2], b);
          b = fmaf(xv[3], wv[q][3], b);
          accn[i][q] = b;
        }
      }
    }
  }

  float bq[EPL];
#pragma unroll
  for (int q = 0; q < EPL; ++q) bq[q] = (bias != nullptr && ev[q]) ? bias[e[q]] : 0.0f;

  StatAcc<EPL> sa;
  sa.zero();
  for (int i = 0; i < kTPL; ++i) {
    const int64_t t = tok0 + i;
    if (t >= T) break;  // uniform within the group
    float z[EPL], zg[EPL];
#pragma unroll
    for (int q = 0; q < EPL; ++q) {
      float h = acc[i][q];
      if constexpr (NOISE)
        h = fmaf(eps[t * Nr + (ev[q] ? e[q] : Nr - 1)], softplus_f32(accn[i][q]), h);
      z[q] = ev[q] ? h + bq[q] : -INFINITY;
      zg[q] = ev[q] ? (bias_sel ? h : h + bq[q]) : -INFINITY;
    }
    select_and_store<NP, EPL, STATS>(z, zg, bias_sel, e, ev, t, K, gate, grp, lane, topk_idx,
                                     topk_w, &sa, lse);
  }
  if constexpr (STATS) {
    __shared__ double red[(kRouterThreads / kWave) * (2 * NP * EPL + 1)];
    block_stats<NP, EPL, kRouterThreads / kWave>(sa, lane, wave, red,
                                                 stats_part + static_cast<int64_t>(blockIdx.x) * kStatsStride);
  }
}

// Launches the vector-ALU router; returns the number of workgroups (the
// rows of statistics written) through nblk.
template <typename XT, int NP, int EPL>
hipError_t launch_t(const RouteArgs& a, hipStream_t s, int* nblk) {
  constexpr int G = kWave / NP;
  constexpr int tok_per_block = (kRouterThreads / kWave) * G * kTPL;
  static_assert(tok_per_block >= 32, "route_stats_bytes assumes >= 32 tokens per workgroup");
  const int grid = (a.T + tok_per_block - 1) / tok_per_block;
  *nblk = grid;
  if (a.w_noise != nullptr)
    hipLaunchKernelGGL((router_kernel<XT, NP, EPL, false, true>), dim3(grid), dim3(kRouterThreads), 0,
                       s, static_cast<const XT*>(a.x), a.w_router, a.bias, a.T, a.d, a.n_routed,
                       a.top_k, a.gate, a.bias_sel, a.topk_idx, a.topk_w, nullptr, nullptr,
                       a.w_noise, a.noise);
  else if (a.stats_part != nullptr)
    hipLaunchKernelGGL((router_kernel<XT, NP, EPL, true, false>), dim3(grid), dim3(kRouterThreads), 0,
                       s, static_cast<const XT*>(a.x), a.w_router, a.bias, a.T, a.d, a.n_routed,
                       a.top_k, a.gate, a.bias_sel, a.topk_idx, a.topk_w, a.stats_part, a.lse,
                       nullptr, nullptr);
  else
    hipLaunchKernelGGL((router_kernel<XT, NP, EPL, false, false>), dim3(grid), dim3(kRouterThreads), 0,
                       s, static_cast<const XT*>(a.x), a.w_router, a.bias, a.T, a.d, a.n_routed,
                       a.top_k, a.gate, a.bias_sel, a.topk_idx, a.topk_w, nullptr, nullptr,
                       nullptr, nullptr);
  return hipGetLastError();
}


// ---- matrix-core logits (bf16 x) --------------------------------------------

// v == hi + mid + lo exactly, each part a bf16 value held as an fp32 pattern
// with a zero low half: truncation keeps the top 8 significant bits and the
// remainders are exact fp32 differences (same sign and binade).
__device__ __forceinline__ void split3(float v, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
  hi = __float_as_uint(v) & 0xFFFF0000u;
  const float r1 = v - __uint_as_float(hi);
  mid = __float_as_uint(r1) & 0xFFFF0000u;
  const float r2 = r1 - __uint_as_float(mid);
  lo = __float_as_uint(r2);  // the pack below keeps the high half, as for hi and mid
}

// High halves of two fp32 patterns -> one packed bf16 pair (lo element first).
__device__ __forceinline__ uint32_t pack_hi(uint32_t first, uint32_t second) {
  return __builtin_amdgcn_perm(second, first, 0x07060302u);
}

constexpr int kRW = 8;   // wavefronts per matrix-core router workgroup

// W_g values for K slice s (k = 16s .. 16s+15): lane l holds the 8
// consecutive k of expert row nb*32 + l%32 starting at 16s + 8*(l/32), as
// two float4.  Row-major W_g: wp[nb] points at that row (plus the lane's k
// half), and a load instruction touches 32 rows, 32 bytes of each.  Packed
// W_g (moe_pack_router): the float4 of (s, nb, half j, lane l) is number
// ((s*NBLK + nb)*2 + j)*64 + l, so each load instruction reads 1 KB of
// contiguous memory; wp[nb] points at (nb, lane) of slice 0.
constexpr int kPackSliceFloats = 512;   // packed floats per (slice, 32-row block)

template <int NBLK, bool PK>
__device__ __forceinline__ void load_w_slice(float4 (&w)[NBLK][2], const float* const (&wp)[NBLK],
                                             int s) {
#pragma unroll
  for (int nb = 0; nb < NBLK; ++nb) {
    if constexpr (PK) {
      const float* q = wp[nb] + s * NBLK * kPackSliceFloats;
      w[nb][0] = *reinterpret_cast<const float4*>(q);
      w[nb][1] = *reinterpret_cast<const float4*>(q + kPackSliceFloats / 2);
    } else {
      w[nb][0] = *reinterpret_cast<const float4*>(wp[nb] + s * 16);
      w[nb][1] = *reinterpret_cast<const float4*>(wp[nb] + s * 16 + 4);
    }
  }
}

// acc[mb][nb] += x_slice[mb] . (hi + mid + lo)(W_g slice nb)^T, smallest
// part first.  One split of W_g serves all MBLK token blocks, and
// consecutive MFMAs go to different accumulators.
template <int MBLK, int NBLK>
__device__ __forceinline__ void router_mma(f32x16 (&acc)[MBLK][NBLK], const bf16x8 (&a)[MBLK],
                                           const float4 (&w)[NBLK][2]) {
  bf16x8 bp[NBLK][3];
#pragma unroll
  for (int nb = 0; nb < NBLK; ++nb) {
    const float v[8] = {w[nb][0].x, w[nb][0].y, w[nb][0].z, w[nb][0].w,
                        w[nb][1].x, w[nb][1].y, w[nb][1].z, w[nb][1].w};
    uint32_t h[8], m[8], l[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) split3(v[i], h[i], m[i], l[i]);
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    u32x4 ph, pm, pl;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ph[i] = pack_hi(h[2 * i], h[2 * i + 1]);
      pm[i] = pack_hi(m[2 * i], m[2 * i + 1]);
      pl[i] = pack_hi(l[2 * i], l[2 * i + 1]);
    }
    bp[nb][0] = __builtin_bit_cast(bf16x8, pl);
    bp[nb][1] = __builtin_bit_cast(bf16x8, pm);
    bp[nb][2] = __builtin_bit_cast(bf16x8, ph);
  }
#pragma unroll
  for (int q = 0; q < 3; ++q)
#pragma unroll
    for (int mb = 0; mb < MBLK; ++mb)
#pragma unroll
      for (int nb = 0; nb < NBLK; ++nb)
        acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mb], bp[nb][q], acc[mb][nb], 0, 0, 0);
}

// R consecutive K slices starting at slice rs: every x fragment is loaded
// up front (one trip to HBM), W_g streams through a ring of min(RD, R)
// slices.  No branches, so every wait on a load is an exact count.
template <int R, int RD, int MBLK, int NBLK, bool PK>
__device__ __forceinline__ void router_round(f32x16 (&acc)[MBLK][NBLK],
                                             const bf16_t* const (&xp)[MBLK],
                                             const float* const (&wp)[NBLK], int rs) {
  constexpr int D = RD < R ? RD : R;
  bf16x8 xa[R][MBLK];
#pragma unroll
  for (int i = 0; i < R; ++i)
#pragma unroll
    for (int mb = 0; mb < MBLK; ++mb) xa[i][mb] = *reinterpret_cast<const bf16x8*>(xp[mb] + (rs + i) * 16);
  float4 wr[D][NBLK][2];
#pragma unroll
  for (int i = 0; i < D; ++i) load_w_slice<NBLK, PK>(wr[i], wp, rs + i);
  // Keep every load above at the top: the scheduler would otherwise sink
  // them next to their first use and serialise the round trips.
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < R; ++i) {
    router_mma<MBLK, NBLK>(acc, xa[i], wr[i % D]);
    if (i + D < R) load_w_slice<NBLK, PK>(wr[i % D], wp, rs + i + D);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Streamed K ranges: blocks of four slices (64 k, one 128-byte line of
// every token row).  A block's x rows go global -> LDS by DMA
// (buffer_load ... lds, 16 bytes per lane, eight lanes per 128-byte row
// segment, so each load instruction moves 8 whole lines) into a two-block
// ring private to the wavefront; the MFMA fragments are then read from LDS.
// Loaded straight into registers, a fragment load touches 32 token rows,
// 32 bytes of each, and every line of x is requested four times.  Chunk c
// of ring row r sits at position c ^ xswz(r), which keeps the 16-byte
// fragment reads of 16 consecutive rows on distinct banks.
__device__ __forceinline__ int xswz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

typedef __attribute__((address_space(3))) void* lds_void_ptr;

// s_waitcnt with vmcnt <= N (gfx9 encoding: vmcnt in bits 3:0 and 15:14;
// expcnt and lgkmcnt at their maxima, i.e. not waited for).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// The four slices of one ring block.  In flight on entry, in issue order:
// the block's x DMA, its four slices of W_g, and (MORE) the next block's x
// DMA.  After slice i the W_g loads of slice i of the next block are issued
// into the registers slice i frees, so before slice i exactly 3*NW + ND
// later loads may still be in flight (MORE), or (3 - i)*NW in the last
// block.  Loads retire in issue order for the counter, so the wait for
// slice i's W_g also covers this block's x DMA, issued before it.
template <int MBLK, int NBLK, bool PK, bool MORE>
__device__ __forceinline__ void stream_block(f32x16 (&acc)[MBLK][NBLK], float4 (&wr)[4][NBLK][2],
                                             const float* const (&wp)[NBLK], int snext,
                                             const bf16_t* cur, int lane) {
  constexpr int ND = MBLK * 4;   // x DMA loads per block (8 rows each)
  constexpr int NW = NBLK * 2;   // W_g loads per slice
  const int r = lane & 31, h = lane >> 5;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (MORE) {
      wait_vmcnt<3 * NW + ND>();
    } else {
      if (i == 0) wait_vmcnt<3 * NW>();
      else if (i == 1) wait_vmcnt<2 * NW>();
      else if (i == 2) wait_vmcnt<NW>();
      else wait_vmcnt<0>();
    }
    // The DMA's LDS writes are not visible to the compiler: keep the
    // fragment reads below the wait.
    asm volatile("" ::: "memory");
    bf16x8 xa[MBLK];
#pragma unroll
    for (int mb = 0; mb < MBLK; ++mb) {
      const int row = mb * 32 + r;
      xa[mb] = *reinterpret_cast<const bf16x8*>(cur + row * 64 + ((2 * i + h) ^ xswz(row)) * 8);
    }
    router_mma<MBLK, NBLK>(acc, xa, wr[i]);
    if constexpr (MORE) load_w_slice<NBLK, PK>(wr[i], wp, snext + i);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Slices [s0, s0 + n), n a multiple of 4 and at least 8.  ring: this
// wavefront's 2 * 32*MBLK * 64 bf16 of LDS; xoff: per-lane byte offsets of
// its DMA chunks at k = 0 (the block's k goes in the scalar offset).
template <int MBLK, int NBLK, bool PK>
__device__ __forceinline__ void router_stream(f32x16 (&acc)[MBLK][NBLK], __amdgpu_buffer_rsrc_t rx,
                                              const uint32_t (&xoff)[4 * MBLK],
                                              const float* const (&wp)[NBLK], int s0, int n,
                                              bf16_t* ring, int lane) {
  constexpr int ND = MBLK * 4;
  constexpr int BLK = 32 * MBLK * 64;   // bf16 per ring block
  auto dma = [&](int b) {
    const uint32_t so = static_cast<uint32_t>((s0 + 4 * b) * 16) * 2u;
    bf16_t* dst = ring + (b & 1) * BLK;
#pragma unroll
    for (int q = 0; q < ND; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void_ptr)(dst + q * 512), 16, xoff[q], so, 0, 0);
  };
  float4 wr[4][NBLK][2];
  dma(0);
#pragma unroll
  for (int i = 0; i < 4; ++i) load_w_slice<NBLK, PK>(wr[i], wp, s0 + i);
  __builtin_amdgcn_sched_barrier(0);
  const int nblocks = n / 4;
  int b = 0;
  for (; b + 1 < nblocks; ++b) {
    dma(b + 1);
    __builtin_amdgcn_sched_barrier(0);
    stream_block<MBLK, NBLK, PK, true>(acc, wr, wp, s0 + 4 * (b + 1), ring + (b & 1) * BLK, lane);
  }
  stream_block<MBLK, NBLK, PK, false>(acc, wr, wp, 0, ring + (b & 1) * BLK, lane);
}

// One workgroup: 32*MBLK tokens x 32*NBLK experts, kRW wavefronts.  The
// d/16 K slices are cut into contiguous ranges, one per wavefront (kRW per
// workgroup, KS*kRW with split K), at block boundaries of four slices
// where each range gets two blocks or more.  A range of at least two whole
// blocks streams (router_stream:
// x through an LDS ring, W_g - which every workgroup reads, so it stays in
// L2 - into registers four slices ahead); other ranges load the x
// fragments of up to RS slices at once (one trip to HBM per round) and
// stream W_g through a ring of RD slices.  Each W_g value is split once for
// all MBLK token blocks.  The partial logit tiles are summed in
// LDS in wavefront order (deterministic), then each wavefront selects for
// its TB / kRW tokens in one pass.  PK: W_g in the packed order of
// moe_pack_router.
//
// Small batches split K over KS workgroups per token block as well
// (blockIdx.y); each then writes its summed tile to partial[ks][t][e] and
// router_select_kernel finishes the sum in ks order and selects.
template <int MBLK, int NBLK, bool STATS, bool PK>
__global__ __launch_bounds__(kRW * kWave) void router_mfma_kernel(
    const bf16_t* __restrict__ x, const float* __restrict__ wg, const float* __restrict__ bias,
    int T, int d, int Nr, int K, int gate, bool bias_sel, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_w, int KS, float* __restrict__ partial,
    double* __restrict__ stats_part, float* __restrict__ lse, const float* __restrict__ wn,
    const float* __restrict__ eps) {
  constexpr int TB = 32 * MBLK;
  constexpr int NPAD = 32 * NBLK;
  // Selection: one token per group of NP lanes, so that the workgroup's
  // kRW * 64 lanes take all TB tokens in one pass (16 lanes for 32 tokens,
  // 8 for 64; DPP reductions of 4 or 3 steps).
  constexpr int NP = kRW * kWave / TB;
  constexpr int EPL = NPAD / NP;
  constexpr int G = kWave / NP;
  static_assert(NP == 8 || NP == 16, "selection groups");
  constexpr int RS = 16 / MBLK;               // x slices per round
  constexpr int RD = (MBLK * NBLK <= 2) ? 4 : 2;  // W_g slices in flight
  static_assert((TB / kRW) % G == 0, "token split");

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int64_t tok0 = static_cast<int64_t>(blockIdx.x) * TB;
  const int lr = lane & 31;
  const int kh = (lane >> 5) * 8;

  const bf16_t* xp[MBLK];
#pragma unroll
  for (int mb = 0; mb < MBLK; ++mb) {
    const int64_t t = tok0 + mb * 32 + lr;
    xp[mb] = x + (t < T ? t : static_cast<int64_t>(T) - 1) * d + kh;
  }
  // Rows of the logit tile: the N_r experts of W_g, then, for noisy gating
  // (wn set; row-major W_g only), the N_r rows of W_noise (2 N_r <=
  // 32*NBLK).  Tile rows past them read the last real row again (the packed
  // order repeats it); their logit columns are never read.
  const int NE = wn != nullptr ? 2 * Nr : Nr;
  const float* wp[NBLK];
#pragma unroll
  for (int nb = 0; nb < NBLK; ++nb) {
    if constexpr (PK) {
      wp[nb] = wg + nb * kPackSliceFloats + lane * 4;
    } else {
      const int e = min(nb * 32 + lr, NE - 1);
      wp[nb] = (e < Nr ? wg + static_cast<int64_t>(e) * d : wn + static_cast<int64_t>(e - Nr) * d) + kh;
    }
  }

  f32x16 acc[MBLK][NBLK];
#pragma unroll
  for (int mb = 0; mb < MBLK; ++mb)
#pragma unroll
    for (int nb = 0; nb < NBLK; ++nb)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mb][nb][v] = 0.0f;

  // One LDS slot per wavefront: its x ring while it streams, then its
  // partial logit tile (the ring is idle by then and private to the
  // wavefront, so no barrier separates the two uses).  The tile is stored
  // column-major, logit (t, e) at e*LDT + t: a lane's accumulator holds four
  // consecutive tokens of one expert, one 16-byte write, and the padding of
  // LDT keeps 16 consecutive experts on distinct banks.
  constexpr int LDT = TB + 4;
  constexpr int SLOTF = NPAD * LDT > 64 * TB ? NPAD * LDT : 64 * TB;
  static_assert(SLOTF * 4 >= 2 * TB * 128, "x ring");
  static_assert(!STATS || (kRW - 1) * SLOTF * 4 >= kRW * (2 * NPAD + 1) * 8,
                "statistics reduction reuses slots 1..");
  __shared__ __align__(16) float slot[kRW][SLOTF];

  const int S = d / 16;
  const int range = blockIdx.y * kRW + wave, nranges = KS * kRW;
  // Ranges of whole blocks of four slices where every range gets at least
  // two of them (all stream; e.g. d = 1280: 8 or 12 slices per wavefront
  // instead of 10), else equal shares of slices.
  const int NBK = S / 4;
  const bool by_block = NBK >= 2 * nranges;
  const int s0 = by_block ? 4 * (range * NBK / nranges) : range * S / nranges;
  const int s1 = by_block ? 4 * ((range + 1) * NBK / nranges) : (range + 1) * S / nranges;
  // Full rounds of RS slices, then the remainder in rounds of 8, 4, 2, 1.
  int rs = s0;
  // Ranges of two or more whole blocks of four slices stream; the rest (and
  // short ranges) go round by round.
#if defined(__HIP_DEVICE_COMPILE__)  // buffer resources exist only in the device pass
  if (s1 - s0 >= 8 && (s1 - s0) % 4 == 0) {
    // x is below 4 GB (a layer requirement), so byte offsets fit 32 bits.
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<bf16_t*>(x), 0, static_cast<uint32_t>(static_cast<int64_t>(T) * d * 2), 0x00020000);
    // DMA chunk q of a block: ring row 8q + lane/8, position lane%8, which
    // holds logical chunk (lane%8) ^ xswz(row) of that token's 64 k.
    uint32_t xoff[4 * MBLK];
#pragma unroll
    for (int q = 0; q < 4 * MBLK; ++q) {
      const int row = q * 8 + lane / 8;
      const int64_t t = min(tok0 + row, static_cast<int64_t>(T) - 1);
      xoff[q] = static_cast<uint32_t>(t * d * 2 + ((lane % 8) ^ xswz(row)) * 16);
    }
    router_stream<MBLK, NBLK, PK>(acc, rx, xoff, wp, s0, s1 - s0,
                                  reinterpret_cast<bf16_t*>(&slot[wave][0]), lane);
    rs = s1;
  }
#endif
  for (; rs + RS <= s1; rs += RS) router_round<RS, RD, MBLK, NBLK, PK>(acc, xp, wp, rs);
  if constexpr (RS > 8) {
    if (rs + 8 <= s1) { router_round<8, RD, MBLK, NBLK, PK>(acc, xp, wp, rs); rs += 8; }
  }
  if (rs + 4 <= s1) { router_round<4, RD, MBLK, NBLK, PK>(acc, xp, wp, rs); rs += 4; }
  if (rs + 2 <= s1) { router_round<2, RD, MBLK, NBLK, PK>(acc, xp, wp, rs); rs += 2; }
  if (rs + 1 <= s1) router_round<1, RD, MBLK, NBLK, PK>(acc, xp, wp, rs);

  // Sum of the wavefronts' partial tiles in wavefront order: each writes its
  // tile to its own LDS slot, then every thread adds the kRW values of its
  // elements in order (the same additions as accumulating wave by wave),
  // up to four tokens of one expert at a time, into slot 0 in place (no
  // other thread reads those elements).
  // D[row][col] of a 32x32 block: lane (col + 32*h), register v, row 8*(v/4) + 4*h + v%4.
#pragma unroll
  for (int mb = 0; mb < MBLK; ++mb)
#pragma unroll
    for (int nb = 0; nb < NBLK; ++nb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r0 = mb * 32 + 8 * j + 4 * (lane >> 5);
        const f32x4 v = {acc[mb][nb][4 * j], acc[mb][nb][4 * j + 1], acc[mb][nb][4 * j + 2],
                         acc[mb][nb][4 * j + 3]};
        *reinterpret_cast<f32x4*>(&slot[wave][(nb * 32 + lr) * LDT + r0]) = v;
      }
  __syncthreads();
  // VW consecutive tokens per thread and step: 4 where the tile gives every
  // thread at least that many elements, else fewer, so all threads work.
  constexpr int VW = TB * NPAD >= 4 * kRW * kWave ? 4 : TB * NPAD >= 2 * kRW * kWave ? 2 : 1;
  typedef float fvw __attribute__((ext_vector_type(VW)));
  for (int g = threadIdx.x; g < NPAD * (TB / VW); g += kRW * kWave) {
    const int off = (g / (TB / VW)) * LDT + (g % (TB / VW)) * VW;
    fvw v[kRW];
#pragma unroll
    for (int w = 0; w < kRW; ++w) v[w] = *reinterpret_cast<const fvw*>(&slot[w][off]);
    fvw sum = v[0];
#pragma unroll
    for (int w = 1; w < kRW; ++w) sum += v[w];
    *reinterpret_cast<fvw*>(&slot[0][off]) = sum;
  }
  __syncthreads();
  const float* lgt = &slot[0][0];   // logit (t, e) at e*LDT + t

  if (KS > 1) {
    for (int i = threadIdx.x; i < TB * NPAD; i += kRW * kWave) {
      const int tl = i / NPAD, c = i % NPAD;
      const int64_t t = tok0 + tl;
      if (t < T) partial[(static_cast<int64_t>(blockIdx.y) * T + t) * NPAD + c] = lgt[c * LDT + tl];
    }
    return;
  }

  const int grp = lane / NP;
  const int gl = lane % NP;
  int e[EPL];
  bool evq[EPL];
  float bq[EPL];
#pragma unroll
  for (int q = 0; q < EPL; ++q) {
    e[q] = gl + NP * q;
    evq[q] = e[q] < Nr;
    bq[q] = (bias != nullptr && evq[q]) ? bias[e[q]] : 0.0f;
  }
  StatAcc<EPL> sa;
  sa.zero();
  for (int tl = wave * (TB / kRW) + grp; tl < (wave + 1) * (TB / kRW); tl += G) {
    const int64_t t = tok0 + tl;
    if (t >= T) break;  // uniform within the group
    float z[EPL], zg[EPL];
#pragma unroll
    for (int q = 0; q < EPL; ++q) {
      // Read first, then select values (e[q] < NPAD, inside the tile): a
      // select between two loads would become a load through a selected
      // pointer and push z to scratch.
      float v = lgt[e[q] * LDT + tl];
      if (wn != nullptr) {   // noisy gating: + eps * softplus(x . wn_e), row N_r + e
        const float nv = lgt[min(Nr + e[q], NPAD - 1) * LDT + tl];
        v = fmaf(eps[t * Nr + min(e[q], Nr - 1)], softplus_f32(nv), v);
      }
      z[q] = evq[q] ? v + bq[q] : -INFINITY;
      zg[q] = evq[q] ? (bias_sel ? v : v + bq[q]) : -INFINITY;
    }
    select_and_store<NP, EPL, STATS>(z, zg, bias_sel, e, evq, t, K, gate, grp, lane, topk_idx,
                                     topk_w, &sa, lse);
  }
  if constexpr (STATS)
    block_stats<NP, EPL, kRW>(sa, lane, wave, reinterpret_cast<double*>(&slot[1][0]),
                              stats_part + static_cast<int64_t>(blockIdx.x) * kStatsStride);
}

// Logit (t, e) as the sum of the KS <= kRouterSplit partial tiles, in ks
// order; all loads are issued before the first add.
template <int NPAD>
__device__ __forceinline__ float sum_partials(const float* __restrict__ partial, int KS, int T,
                                              int64_t t, int e) {
  float v[kRouterSplit];
#pragma unroll
  for (int ks = 0; ks < kRouterSplit; ++ks)
    v[ks] = partial[(static_cast<int64_t>(min(ks, KS - 1)) * T + t) * NPAD + e];
  float acc = 0.0f;
#pragma unroll
  for (int ks = 0; ks < kRouterSplit; ++ks)
    if (ks < KS) acc += v[ks];
  return acc;
}

// Sum of the KS partial logit tiles (in ks order) and selection: one
// wavefront per four tokens, 16 lanes per token.
template <int NBLK>
__global__ __launch_bounds__(kWave) void router_select_kernel(
    const float* __restrict__ partial, const float* __restrict__ bias, int T, int Nr, int K,
    int gate, bool bias_sel, int KS, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w) {
  constexpr int NPAD = 32 * NBLK;
  constexpr int NP = 16;
  constexpr int EPL = NPAD / NP;
  const int lane = threadIdx.x;
  const int grp = lane / NP;
  const int gl = lane % NP;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * (kWave / NP) + grp;
  if (t >= T) return;  // uniform within the group
  int e[EPL];
  bool evq[EPL];
  float z[EPL], zg[EPL];
#pragma unroll
  for (int q = 0; q < EPL; ++q) {
    e[q] = gl + NP * q;
    evq[q] = e[q] < Nr;
    const float v = sum_partials<NPAD>(partial, KS, T, t, e[q]);
    const float b = bias != nullptr && evq[q] ? bias[e[q]] : 0.0f;
    z[q] = evq[q] ? v + b : -INFINITY;
    zg[q] = evq[q] ? (bias_sel ? v : v + b) : -INFINITY;
  }
  select_and_store<NP, EPL>(z, zg, bias_sel, e, evq, t, K, gate, grp, lane, topk_idx, topk_w);
}

template <int MBLK, int NBLK, bool PK>
hipError_t launch_mfma_w(const RouteArgs& a, hipStream_t s, int* nblk) {
  constexpr int TB = 32 * MBLK;
  const int blocks = (a.T + TB - 1) / TB;
  *nblk = blocks;
  if (a.stats_part != nullptr) {
    hipLaunchKernelGGL((router_mfma_kernel<MBLK, NBLK, true, PK>), dim3(blocks, 1), dim3(kRW * kWave), 0,
                       s, static_cast<const bf16_t*>(a.x), a.w_router, a.bias, a.T, a.d,
                       a.n_routed, a.top_k, a.gate, a.bias_sel, a.topk_idx, a.topk_w, 1, nullptr,
                       a.stats_part, a.lse, nullptr, nullptr);
    return hipGetLastError();
  }
  if (a.w_noise != nullptr) {
    hipLaunchKernelGGL((router_mfma_kernel<MBLK, NBLK, false, PK>), dim3(blocks, 1), dim3(kRW * kWave), 0,
                       s, static_cast<const bf16_t*>(a.x), a.w_router, a.bias, a.T, a.d,
                       a.n_routed, a.top_k, a.gate, a.bias_sel, a.topk_idx, a.topk_w, 1, nullptr,
                       nullptr, nullptr, a.w_noise, a.noise);
    return hipGetLastError();
  }
  // Split K when the token blocks alone would leave most CUs idle.
  const int KS = (a.partial != nullptr && MBLK == 1) ? max(1, min(kRouterSplit, 128 / blocks)) : 1;
  hipLaunchKernelGGL((router_mfma_kernel<MBLK, NBLK, false, PK>), dim3(blocks, KS), dim3(kRW * kWave), 0, s,
                     static_cast<const bf16_t*>(a.x), a.w_router, a.bias, a.T, a.d, a.n_routed,
                     a.top_k, a.gate, a.bias_sel, a.topk_idx, a.topk_w, KS, a.partial, nullptr,
                     nullptr, nullptr, nullptr);
  if (KS == 1) return hipGetLastError();
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL((router_select_kernel<NBLK>), dim3((a.T + 3) / 4), dim3(kWave), 0, s,
                     a.partial, a.bias, a.T, a.n_routed, a.top_k, a.gate, a.bias_sel, KS, a.topk_idx,
                     a.topk_w);
  return hipGetLastError();
}

template <int MBLK, int NBLK>
hipError_t launch_mfma(const RouteArgs& a, hipStream_t s, int* nblk) {
  return a.w_packed ? launch_mfma_w<MBLK, NBLK, true>(a, s, nblk)
                    : launch_mfma_w<MBLK, NBLK, false>(a, s, nblk);
}

template <typename XT>
hipError_t launch_x(const RouteArgs& a, hipStream_t s, int* nblk) {
  const int n = a.n_routed;
  if (n <= 8) return launch_t<XT, 8, 1>(a, s, nblk);
  if (n <= 16) return launch_t<XT, 16, 1>(a, s, nblk);
  if (n <= 32) return launch_t<XT, 32, 1>(a, s, nblk);
  if (n <= 64) return launch_t<XT, 64, 1>(a, s, nblk);
  if (n <= 128) return launch_t<XT, 64, 2>(a, s, nblk);
  return launch_t<XT, 64, 4>(a, s, nblk);
}

hipError_t launch_router(const RouteArgs& a, hipStream_t s, int* nblk) {
  // Packed W_g is only read by the matrix-core kernel; the host accepts it
  // only where that kernel runs (bf16 x, d % 64 == 0, N_r <= 128, no noise).
  if (a.x_bf16 && a.d % 64 == 0) {
    // Two token blocks per wavefront once there are enough tokens to fill
    // the chip with 64-token workgroups.  Noisy gating needs 2 N_r rows.
    const bool wide = a.T >= 64 * 256;
    const int rows = a.w_noise != nullptr ? 2 * a.n_routed : a.n_routed;
    if (rows <= 32) return wide ? launch_mfma<2, 1>(a, s, nblk) : launch_mfma<1, 1>(a, s, nblk);
    if (rows <= 64) return wide ? launch_mfma<2, 2>(a, s, nblk) : launch_mfma<1, 2>(a, s, nblk);
    if (rows <= 128) return launch_mfma<1, 4>(a, s, nblk);
  }
  return a.x_bf16 ? launch_x<bf16_t>(a, s, nblk) : launch_x<float>(a, s, nblk);
}

constexpr int kFoldThreads = 1024;

// Routing statistics from the router's per-workgroup rows (DeepSeekMoE page,
// section 3.3, eq. 12-17; MoE-survey blog page, section 5, z-loss), one
// workgroup.  The 2 N_r + 1 used columns are taken in NCH chunks of 64, one
// per lane; wavefront w sums rows w, w + 16, ... (every chunk's load for a
// row issued together, no branches), then the 16 partial sums are added in
// wavefront order, so the result does not depend on timing.  Then
//   P_i = sum_s / T, f_i = count_i * N_r / (K' T),
//   f'_g = mean of f over [g N_r/D, (g+1) N_r/D), P'_g = sum of P there,
//   L_ExpBal = sum f_i P_i, L_DevBal = sum f'_g P'_g, z = sum lse^2 / T,
// all in fp64, stored as fp32.  An empty batch gives zeros.
template <int NCH>
__global__ __launch_bounds__(kFoldThreads) void route_stats_kernel(
    const double* __restrict__ rows, int nblk, int T, int Nr, int K, int D,
    float* __restrict__ stats) {
  constexpr int W = kFoldThreads / kWave;
  __shared__ double tot[kStatsStride];
  __shared__ double red[W][kWave];
  __shared__ double fv[256], pv[256], fd[256], pd[256];
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int ncol = 2 * Nr + 1;
  int col[NCH];
  bool used[NCH];
  double v[NCH];
#pragma unroll
  for (int ch = 0; ch < NCH; ++ch) {
    const int ci = ch * kWave + lane;
    used[ch] = ci < ncol;
    col[ch] = ci < Nr ? ci : ci < 2 * Nr ? kStatsCount + (ci - Nr) : kStatsZ;
    v[ch] = 0.0;
  }
#pragma unroll 2
  for (int b = wave; b < nblk; b += W) {
    const double* r = rows + static_cast<int64_t>(b) * kStatsStride;
    double x[NCH];
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) x[ch] = r[col[ch]];
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) v[ch] += used[ch] ? x[ch] : 0.0;
  }
#pragma unroll
  for (int ch = 0; ch < NCH; ++ch) {
    red[wave][lane] = v[ch];
    __syncthreads();
    if (wave == 0 && used[ch]) {
      double sum = 0.0;
      for (int w = 0; w < W; ++w) sum += red[w][lane];
      tot[col[ch]] = sum;
    }
    __syncthreads();
  }
  const double invT = T > 0 ? 1.0 / T : 0.0;
  const double fscale = T > 0 ? static_cast<double>(Nr) / (static_cast<double>(K) * T) : 0.0;
  for (int i = threadIdx.x; i < Nr; i += kFoldThreads) {
    pv[i] = tot[i] * invT;
    fv[i] = tot[kStatsCount + i] * fscale;
    stats[i] = static_cast<float>(pv[i]);
    stats[Nr + i] = static_cast<float>(fv[i]);
  }
  __syncthreads();
  const int gs = Nr / D;
  for (int g = threadIdx.x; g < D; g += kFoldThreads) {
    double fs = 0.0, ps = 0.0;
    for (int j = g * gs; j < (g + 1) * gs; ++j) {
      fs += fv[j];
      ps += pv[j];
    }
    fd[g] = fs / gs;
    pd[g] = ps;
    stats[2 * Nr + g] = static_cast<float>(fd[g]);
    stats[2 * Nr + D + g] = static_cast<float>(pd[g]);
  }
  __syncthreads();
  if (wave == 0) {
    double le = 0.0, ld = 0.0;
    for (int i = lane; i < Nr; i += kWave) le += fv[i] * pv[i];
    for (int g = lane; g < D; g += kWave) ld += fd[g] * pd[g];
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) {
      le += __shfl_xor(le, o, kWave);
      ld += __shfl_xor(ld, o, kWave);
    }
    if (lane == 0) {
      stats[2 * Nr + 2 * D] = static_cast<float>(le);
      stats[2 * Nr + 2 * D + 1] = static_cast<float>(ld);
      stats[2 * Nr + 2 * D + 2] = static_cast<float>(tot[kStatsZ] * invT);
    }
  }
}

// moe_pack_router: W_g [N_r, d] row-major -> the packed order (see
// load_w_slice), one float4 per thread.  Rows past N_r up to router_pad_rows
// repeat row N_r - 1, as the row-major kernel reads them.
__global__ __launch_bounds__(256) void pack_router_kernel(const float* __restrict__ wg,
                                                          float* __restrict__ dst, int d, int Nr,
                                                          int nblk) {
  const int64_t n4 = static_cast<int64_t>(d / 16) * nblk * 128;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= n4) return;
  const int l = static_cast<int>(idx & 63);
  const int j = static_cast<int>((idx >> 6) & 1);
  const int nb = static_cast<int>((idx >> 7) % nblk);
  const int64_t sl = idx / (static_cast<int64_t>(nblk) * 128);
  const int e = min(nb * 32 + (l & 31), Nr - 1);
  const int64_t k = 16 * sl + 8 * (l >> 5) + 4 * j;
  reinterpret_cast<float4*>(dst)[idx] = *reinterpret_cast<const float4*>(wg + static_cast<int64_t>(e) * d + k);
}

}  // namespace

hipError_t launch_pack_router(const float* wg, float* dst, int d, int Nr, hipStream_t s) {
  const int nblk = router_pad_rows(Nr) / 32;
  const int64_t n4 = static_cast<int64_t>(d / 16) * nblk * 128;
  hipLaunchKernelGGL(pack_router_kernel, dim3(static_cast<unsigned>((n4 + 255) / 256)), dim3(256), 0, s,
                     wg, dst, d, Nr, nblk);
  return hipGetLastError();
}

hipError_t launch_route(const RouteArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  int nblk = 0;
  return launch_router(a, s, &nblk);
}

hipError_t launch_route_stats(const RouteArgs& a, int n_devices, float* stats, hipStream_t s) {
  int nblk = 0;
  if (a.T > 0) {
    const hipError_t err = launch_router(a, s, &nblk);
    if (err != hipSuccess) return err;
  }
  const int nch = (2 * a.n_routed + 1 + kWave - 1) / kWave;
  const double* rows = a.stats_part;
#define MOE_FOLD(N)                                                                              \
  case N:                                                                                        \
    hipLaunchKernelGGL(route_stats_kernel<N>, dim3(1), dim3(kFoldThreads), 0, s, rows, nblk, a.T, \
                       a.n_routed, a.top_k, n_devices, stats);                                   \
    break;
  switch (nch) {
    MOE_FOLD(1) MOE_FOLD(2) MOE_FOLD(3) MOE_FOLD(4) MOE_FOLD(5) MOE_FOLD(6) MOE_FOLD(7)
    MOE_FOLD(8) MOE_FOLD(9)
    default: return hipErrorInvalidValue;
  }
#undef MOE_FOLD
  return hipGetLastError();
}

}  // namespace moe
