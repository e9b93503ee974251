// Grouped fp32 expert GEMMs (layers stored in float32).
//
// Same contract as the bf16 path (see GemmArgs): one thread per output
// element over rows_total rows, its group found by binary search in offsets
// (rows between offsets[n_groups] and extra_base are skipped), dot products
// accumulated in fp32 in ascending k.  fp32 layers here are the small
// parity-sized ones, so this path favours plainness over speed.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

__device__ __forceinline__ int find_group(const int32_t* off, int G, int64_t r) {
  int lo = 0, hi = G - 1;  // largest g with off[g] <= r
  while (lo < hi) {
    const int mid = (lo + hi + 1) / 2;
    if (off[mid] <= r) lo = mid; else hi = mid - 1;
  }
  return lo;
}

template <int MODE>
__global__ __launch_bounds__(256) void grouped_gemm_f32(GemmArgs p) {
  const int64_t total = p.rows_total * p.N;
  const float* A = static_cast<const float*>(p.A);
  float* C = static_cast<float*>(p.C);
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < total;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t r = i / p.N;
    const int n = static_cast<int>(i % p.N);
    const bool extra = p.n_extra > 0 && r >= p.extra_base;
    const float* b0;
    const float* b1 = nullptr;
    int64_t arow;
    if (extra) {
      const int64_t s = (r - p.extra_base) / p.extra_rows;
      b0 = static_cast<const float*>(p.Bx0) + s * p.bx_group_stride + n * p.ldb;
      if (MODE == kGateUp) b1 = static_cast<const float*>(p.Bx1) + s * p.bx_group_stride + n * p.ldb;
      arow = p.gather ? (r - p.extra_base) % p.extra_rows : r;
    } else {
      // Rows past the last group's end (the rows an expert capacity dropped,
      // below extra_base) hold no assignment and no valid gather index.
      if (p.offsets != nullptr && r >= p.offsets[p.n_groups]) continue;
      const int g = p.offsets ? find_group(p.offsets, p.n_groups, r) : 0;
      b0 = static_cast<const float*>(p.B0) + g * p.b_group_stride + n * p.ldb;
      if (MODE == kGateUp) b1 = static_cast<const float*>(p.B1) + g * p.b_group_stride + n * p.ldb;
      arow = p.gather ? p.gather[r] : r;
    }
    const float* a = A + arow * p.lda;
    if (MODE == kGateUp) {
      float s0 = 0.0f, s1 = 0.0f;
      for (int k = 0; k < p.K; ++k) {
        const int64_t bo = static_cast<int64_t>(k / p.k_sub) * p.b_sub_stride + (k % p.k_sub);
        s0 = fmaf(a[k], b0[bo], s0);
        s1 = fmaf(a[k], b1[bo], s1);
      }
      C[r * p.ldc + n] = (s0 / (1.0f + expf(-s0))) * s1;
    } else {
      float s0 = 0.0f;
      for (int k = 0; k < p.K; ++k) {
        const int64_t bo = static_cast<int64_t>(k / p.k_sub) * p.b_sub_stride + (k % p.k_sub);
        s0 = fmaf(a[k], b0[bo], s0);
      }
      C[r * p.ldc + n] = p.relu ? fmaxf(s0, 0.0f) : s0;
    }
  }
}

}  // namespace

hipError_t launch_gemm_f32(const GemmArgs& a, hipStream_t s) {
  const int64_t total = a.rows_total * a.N;
  if (total == 0) return hipSuccess;
  const int64_t want = (total + 255) / 256;
  const int grid = static_cast<int>(want < 65536 ? want : 65536);
  if (a.mode == kGateUp)
    hipLaunchKernelGGL(grouped_gemm_f32<kGateUp>, dim3(grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(grouped_gemm_f32<kDown>, dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
