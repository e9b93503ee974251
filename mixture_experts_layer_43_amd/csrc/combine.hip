// Gate-weighted combine (DeepSeekMoE page, section 3.2, eq. 9):
//   y_t = sum_j g_{t,j} FFN_{e_j}(u_t) + sum_s FFN^sh_s(u_t) (+ u_t)
// One wavefront per token; each lane owns 16-byte column chunks, gathers the
// K' expert rows of the token through slot_row, accumulates in fp32 in
// ascending j, adds the shared-expert sum and the residual, and rounds once.
// Pure streaming: bound by HBM bandwidth.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kMaxK = 16;

template <typename T>
struct Vec16;  // 16 bytes of T as fp32 lanes
template <>
struct Vec16<bf16_t> {
  static constexpr int N = 8;
  static __device__ __forceinline__ void load(const void* p, float (&v)[8]) {
    const uint4 q = *static_cast<const uint4*>(p);
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
    const float4 q = *static_cast<const float4*>(p);
    v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
  }
  static __device__ __forceinline__ void store(void* p, const float (&v)[4]) {
    *static_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  }
};

template <typename E>
__global__ __launch_bounds__(256) void combine_kernel(
    const char* __restrict__ y_perm, const int32_t* __restrict__ slot_row,
    const float* __restrict__ topk_w, const char* __restrict__ y_shared,
    const char* __restrict__ residual, char* __restrict__ y, int T, int chunks, int K) {
  using V = Vec16<E>;
  constexpr int N = V::N;
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t t = static_cast<int64_t>(blockIdx.x) * (256 / kWave) + threadIdx.x / kWave;
  if (t >= T) return;
  const int64_t row_bytes = static_cast<int64_t>(chunks) * 16;
  int64_t src[kMaxK];
  float w[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    if (j < K) {
      src[j] = static_cast<int64_t>(slot_row[t * K + j]) * row_bytes;
      w[j] = topk_w[t * K + j];
    }
  }
  for (int c = lane; c < chunks; c += kWave) {
    const int64_t cb = static_cast<int64_t>(c) * 16;
    float acc[N];
#pragma unroll
    for (int i = 0; i < N; ++i) acc[i] = 0.0f;
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
      if (j < K) {
        float v[N];
        V::load(y_perm + src[j] + cb, v);
#pragma unroll
        for (int i = 0; i < N; ++i) acc[i] = fmaf(w[j], v[i], acc[i]);
      }
    }
    if (y_shared) {
      float v[N];
      V::load(y_shared + t * row_bytes + cb, v);
#pragma unroll
      for (int i = 0; i < N; ++i) acc[i] += v[i];
    }
    if (residual) {
      float v[N];
      V::load(residual + t * row_bytes + cb, v);
#pragma unroll
      for (int i = 0; i < N; ++i) acc[i] += v[i];
    }
    V::store(y + t * row_bytes + cb, acc);
  }
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
  const int grid = (a.T + 3) / 4;
  if (a.bf16)
    hipLaunchKernelGGL(combine_kernel<bf16_t>, dim3(grid), dim3(256), 0, s,
                       static_cast<const char*>(a.y_perm), a.slot_row, a.topk_w,
                       static_cast<const char*>(a.y_shared), static_cast<const char*>(a.residual),
                       static_cast<char*>(a.y), a.T, chunks, a.top_k);
  else
    hipLaunchKernelGGL(combine_kernel<float>, dim3(grid), dim3(256), 0, s,
                       static_cast<const char*>(a.y_perm), a.slot_row, a.topk_w,
                       static_cast<const char*>(a.y_shared), static_cast<const char*>(a.residual),
                       static_cast<char*>(a.y), a.T, chunks, a.top_k);
  return hipGetLastError();
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
