// Gate-weighted combine (DeepSeekMoE page, section 3.2, eq. 9):
//   y_t = sum_j g_{t,j} FFN_{e_j}(u_t) + sum_s FFN^sh_s(u_t) (+ u_t)
// Each token's K' expert rows are gathered through slot_row and accumulated
// in fp32 in ascending j, then the shared-expert rows (one sum, or one row
// per shared expert in order) and the residual are added, and the sum is
// rounded once.  A slot dropped by the expert capacity (slot_row -1) adds
// nothing.
// Pure streaming: bound by HBM bandwidth.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

// Up to this many tokens the combine spreads a token over several wavefronts.
constexpr int kCombineSplitTokens = 1024;

// 16 bytes of T as fp32 lanes.  Every row is read once, so the loads carry
// the non-temporal hint: the 16B-shaped layer's combine (604 MB) takes 97
// instead of 123 us with it, bit for bit the same.
template <typename T>
struct Vec16;
template <>
struct Vec16<bf16_t> {
  static constexpr int N = 8;
  static __device__ __forceinline__ void load(const void* p, float (&v)[8]) {
    const u32x4 q = __builtin_nontemporal_load(static_cast<const u32x4*>(p));
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
  static __device__ __forceinline__ void store(void* p, const float (&v)[8]) {
    uint4 q;
    q.x = pack_bf16x2(v[0], v[1]);
    q.y = pack_bf16x2(v[2], v[3]);
    q.z = pack_bf16x2(v[4], v[5]);
    q.w = pack_bf16x2(v[6], v[7]);
    *static_cast<uint4*>(p) = q;
  }
};
template <>
struct Vec16<float> {
  static constexpr int N = 4;
  static __device__ __forceinline__ void load(const void* p, float (&v)[4]) {
    const f32x4 q = __builtin_nontemporal_load(static_cast<const f32x4*>(p));
    v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
  }
  static __device__ __forceinline__ void store(void* p, const float (&v)[4]) {
    *static_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  }
};

// SPLIT wavefronts per token (1, or up to 4 for small batches so that more
// loads are in flight); wavefront p of a token owns the column chunks
// 64 p + l, 64 (p + SPLIT) + l, ... (CPL of them per pass), lane l.  The
// token's K' row indices and gate values are loaded once, by lanes 0..K'-1,
// and broadcast.  The rows to sum are the K' routed rows (weight topk_w),
// then the shared-expert rows and the residual (weight 1), taken JG at a time
// with all their loads in flight before any is used.
template <typename E, int CPL, int SPLIT>
__global__ __launch_bounds__(256) void combine_kernel(
    const char* __restrict__ y_perm, const int32_t* __restrict__ slot_row,
    const float* __restrict__ topk_w, const char* __restrict__ y_shared,
    int shared_blocks, int64_t shared_stride_bytes, const char* __restrict__ residual,
    char* __restrict__ y, int T, int chunks, int K) {
  using V = Vec16<E>;
  constexpr int N = V::N;
  constexpr int JG = CPL == 1 ? 8 : CPL <= 4 ? 4 : 2;
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t gw = static_cast<int64_t>(blockIdx.x) * (256 / kWave) + threadIdx.x / kWave;
  const int64_t t = gw / SPLIT;
  const int part = static_cast<int>(gw % SPLIT);
  if (t >= T) return;
  const int64_t row_bytes = static_cast<int64_t>(chunks) * 16;
  const int nrows = K + shared_blocks + (residual != nullptr ? 1 : 0);
  int my_sr = 0;
  float my_w = 0.0f;
  if (lane < K) {
    my_sr = slot_row[t * K + lane];
    my_w = topk_w[t * K + lane];
  }
  for (int cb = part * kWave * CPL; cb < chunks; cb += SPLIT * kWave * CPL) {
    float acc[CPL][N];
#pragma unroll
    for (int i = 0; i < CPL; ++i)
#pragma unroll
      for (int n = 0; n < N; ++n) acc[i][n] = 0.0f;
    for (int j0 = 0; j0 < nrows; j0 += JG) {
      // Branch-free issue (so all loads of the group are in flight together):
      // rows past the end re-read the last row, columns past the end re-read
      // the last chunk; neither is used.
      float v[JG][CPL][N];
      bool dropped[JG];
#pragma unroll
      for (int jj = 0; jj < JG; ++jj) {
        const int j = min(j0 + jj, nrows - 1);
        // slot_row -1: an assignment dropped by the expert capacity (gate 0);
        // row 0 is read in its place and not used.
        const int sr = __shfl(my_sr, min(j, K - 1), kWave);
        dropped[jj] = j < K && sr < 0;
        const char* routed = y_perm + static_cast<int64_t>(max(sr, 0)) * row_bytes;
        const char* shared = (shared_blocks > 0 ? y_shared : y_perm) +
                             max(j - K, 0) * shared_stride_bytes + t * row_bytes;
        const char* res = (residual != nullptr ? residual : y_perm) + t * row_bytes;
        const char* row = j < K ? routed : (j < K + shared_blocks ? shared : res);
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
          const int c = min(cb + lane + kWave * i, chunks - 1);
          V::load(row + static_cast<int64_t>(c) * 16, v[jj][i]);
        }
      }
#pragma unroll
      for (int jj = 0; jj < JG; ++jj) {
        const int j = j0 + jj;
        if (j >= nrows) break;
        if (dropped[jj]) continue;  // uniform: one token per wavefront
        const float w = j < K ? __shfl(my_w, j, kWave) : 1.0f;
#pragma unroll
        for (int i = 0; i < CPL; ++i)
#pragma unroll
          for (int n = 0; n < N; ++n) acc[i][n] = fmaf(w, v[jj][i][n], acc[i][n]);
      }
    }
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int c = cb + lane + kWave * i;
      if (c < chunks) V::store(y + t * row_bytes + static_cast<int64_t>(c) * 16, acc[i]);
    }
  }
}

template <typename E>
hipError_t launch_combine_t(const CombineArgs& a, int chunks, hipStream_t s) {
  const int blocks = a.y_shared ? a.shared_blocks : 0;
  const int64_t stride = a.shared_stride * static_cast<int64_t>(sizeof(E));
  const char* yp = static_cast<const char*>(a.y_perm);
  const char* ys = static_cast<const char*>(a.y_shared);
  const char* res = static_cast<const char*>(a.residual);
  char* y = static_cast<char*>(a.y);
#define MOE_COMBINE(CPL, SPLIT)                                                                    \
  hipLaunchKernelGGL((combine_kernel<E, CPL, SPLIT>),                                            \
                     dim3(static_cast<unsigned>((static_cast<int64_t>(a.T) * SPLIT + 3) / 4)),    \
                     dim3(256), 0, s, yp, a.slot_row, a.topk_w, ys, blocks, stride, res, y, a.T, \
                     chunks, a.top_k)
  // Small batches: a token's rows over several wavefronts, one chunk per
  // lane per row, all rows of the token in flight at once.
  const int split = a.T <= kCombineSplitTokens ? min(4, max(1, chunks / kWave)) : 1;
  const int cpl = (chunks + kWave - 1) / kWave;
  if (split == 4) MOE_COMBINE(1, 4);
  else if (split == 3) MOE_COMBINE(1, 3);
  else if (split == 2) MOE_COMBINE(1, 2);
  else if (cpl <= 1) MOE_COMBINE(1, 1);
  else if (cpl <= 2) MOE_COMBINE(2, 1);
  else if (cpl <= 4) MOE_COMBINE(4, 1);
  else MOE_COMBINE(8, 1);  // rows longer than 8 KB take several passes of 512 chunks
#undef MOE_COMBINE
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void zero_kernel(uint32_t* p, int64_t words) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < words;
       i += static_cast<int64_t>(gridDim.x) * 256)
    p[i] = 0u;
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  const int elt = a.bf16 ? 2 : 4;
  const int chunks = static_cast<int>(static_cast<int64_t>(a.d) * elt / 16);
  return a.bf16 ? launch_combine_t<bf16_t>(a, chunks, s) : launch_combine_t<float>(a, chunks, s);
}

// Fill kernel instead of hipMemsetAsync so a caller may capture it in a graph.
hipError_t launch_zero(void* p, size_t bytes, hipStream_t s) {
  if (bytes == 0) return hipSuccess;
  const int64_t words = static_cast<int64_t>((bytes + 3) / 4);
  const int64_t want = (words + 255) / 256;
  const int grid = static_cast<int>(want < 4096 ? want : 4096);
  hipLaunchKernelGGL(zero_kernel, dim3(grid), dim3(256), 0, s, static_cast<uint32_t*>(p), words);
  return hipGetLastError();
}

}  // namespace moe
