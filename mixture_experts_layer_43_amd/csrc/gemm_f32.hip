// Grouped fp32 expert GEMMs (layers stored in float32) on the matrix cores.
//
// Same contract as the bf16 path (GemmArgs): gate/up C = silu(A.W1^T) *
// (A.W3^T), down C = A.W2^T (ReLU-clamped for the ReLU FFN), rows grouped
// per expert by offsets, extra groups for the folded shared experts, A rows
// optionally gathered, B addressed through k_sub / b_sub_stride.  A
// workgroup of four wavefronts computes a 64 x 64 output tile with
// v_mfma_f32_32x32x2_f32 (fp32 products, fp32 accumulation); the tile's A
// rows and B rows pass through LDS 32 values of K at a time, zero-filled past
// K, so any K that is a multiple of 4 works.  Workgroups find their (group,
// row tile, column tile) from offsets on the device; surplus ones exit.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

typedef float f32x16v __attribute__((ext_vector_type(16)));

constexpr int kTM = 64;   // output rows per tile
constexpr int kTN = 64;   // output columns per tile
constexpr int kBK = 32;   // K values per LDS step
constexpr int kThreads = 256;

template <int MODE>
__global__ __launch_bounds__(kThreads) void grouped_gemm_f32(GemmArgs p) {
  constexpr int BROWS = (MODE == kGateUp) ? 2 * kTN : kTN;   // B rows of a tile (W1 then W3)
  __shared__ float As[kTM][kBK + 1];
  __shared__ float Bs[BROWS][kBK + 1];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int wm = wave / 2, wn = wave % 2;
  const int n_ntiles = (p.N + kTN - 1) / kTN;

  // ---- this workgroup's tile: groups in order, row tiles, then column tiles
  const int G = p.offsets ? p.n_groups + p.n_extra : 1;
  int64_t t = blockIdx.x;
  int g = -1;
  int64_t row0 = 0;
  int rows = 0;
  for (int gi = 0; gi < G; ++gi) {
    int64_t start, m;
    if (!p.offsets) {
      start = 0;
      m = p.rows_total;
    } else if (gi < p.n_groups) {
      start = p.offsets[gi];
      m = p.offsets[gi + 1] - p.offsets[gi];
    } else {
      start = p.extra_base + static_cast<int64_t>(gi - p.n_groups) * p.extra_rows;
      m = p.extra_rows;
    }
    const int64_t tiles = (m + kTM - 1) / kTM * n_ntiles;
    if (t < tiles) {
      g = gi;
      row0 = start + (t / n_ntiles) * kTM;
      rows = static_cast<int>(min<int64_t>(kTM, start + m - row0));
      break;
    }
    t -= tiles;
  }
  if (g < 0) return;
  const int nt = static_cast<int>(t % n_ntiles);
  const bool extra = p.offsets && g >= p.n_groups;
  const int64_t gx = extra ? g - p.n_groups : g;
  const float* B0 = static_cast<const float*>(extra ? p.Bx0 : p.B0) +
                    gx * (extra ? p.bx_group_stride : p.b_group_stride);
  const float* B1 = (MODE == kGateUp) ? static_cast<const float*>(extra ? p.Bx1 : p.B1) +
                                            gx * (extra ? p.bx_group_stride : p.b_group_stride)
                                      : nullptr;
  const float* A = static_cast<const float*>(p.A);

  // Staging assignment: thread tid copies column c = tid % 32 of rows
  // tid / 32, + 8, + 16, ... of the A tile and of the B tile.
  const int cc = tid % kBK;
  const int r8 = tid / kBK;   // 0..7
  const float* arow[kTM / 8];
#pragma unroll
  for (int i = 0; i < kTM / 8; ++i) {
    const int64_t grow = row0 + min(r8 + 8 * i, rows - 1);
    const int64_t ar = !p.gather ? grow : extra ? (grow - p.extra_base) % p.extra_rows : p.gather[grow];
    arow[i] = A + ar * p.lda;
  }
  const float* brow[BROWS / 8];
#pragma unroll
  for (int i = 0; i < BROWS / 8; ++i) {
    const int r = r8 + 8 * i;
    const bool up = (MODE == kGateUp) && r >= kTN;
    const int n = min(nt * kTN + (up ? r - kTN : r), p.N - 1);
    brow[i] = (up ? B1 : B0) + static_cast<int64_t>(n) * p.ldb;
  }

  f32x16v acc0, acc1;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    acc0[v] = 0.0f;
    acc1[v] = 0.0f;
  }
  const int lr = lane & 31;     // row (A) / column (B) inside the 32-block
  const int kh = lane >> 5;     // which of the MFMA's two K values
  for (int k0 = 0; k0 < p.K; k0 += kBK) {
    const int k = k0 + cc;
    const bool kin = k < p.K;
    const int64_t bk = kin ? static_cast<int64_t>(k / p.k_sub) * p.b_sub_stride + k % p.k_sub : 0;
#pragma unroll
    for (int i = 0; i < kTM / 8; ++i) As[r8 + 8 * i][cc] = kin ? arow[i][k] : 0.0f;
#pragma unroll
    for (int i = 0; i < BROWS / 8; ++i) Bs[r8 + 8 * i][cc] = kin ? brow[i][bk] : 0.0f;
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kBK; kk += 2) {
      const float a = As[wm * 32 + lr][kk + kh];
      const float b0 = Bs[wn * 32 + lr][kk + kh];
      acc0 = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b0, acc0, 0, 0, 0);
      if constexpr (MODE == kGateUp) {
        const float b1 = Bs[kTN + wn * 32 + lr][kk + kh];
        acc1 = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b1, acc1, 0, 0, 0);
      }
    }
    __syncthreads();
  }

  // D[row][col] of a 32x32 block: lane (col + 32*h), register v,
  // row = 8*(v/4) + 4*h + v%4.
  float* C = static_cast<float*>(p.C);
  const int col = nt * kTN + wn * 32 + lr;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int r = wm * 32 + 8 * (v >> 2) + 4 * kh + (v & 3);
    if (r < rows && col < p.N) {
      float o;
      if constexpr (MODE == kGateUp) o = (acc0[v] / (1.0f + expf(-acc0[v]))) * acc1[v];
      else o = p.relu ? fmaxf(acc0[v], 0.0f) : acc0[v];
      C[(row0 + r) * p.ldc + col] = o;
    }
  }
}

}  // namespace

hipError_t launch_gemm_f32(const GemmArgs& a, hipStream_t s) {
  if (a.rows_total == 0 || a.N == 0) return hipSuccess;
  if (a.k_sub <= 0 || a.K % a.k_sub != 0) return hipErrorInvalidValue;
  const int64_t n_ntiles = (a.N + kTN - 1) / kTN;
  // sum_g ceil(M_g / kTM) <= (sum_g M_g + G (kTM - 1)) / kTM
  const int64_t G = a.offsets ? a.n_groups + a.n_extra : 1;
  const int64_t max_mtiles = (a.rows_total + G * (kTM - 1)) / kTM;
  const int64_t grid = max_mtiles * n_ntiles;
  if (grid == 0) return hipSuccess;
  if (a.mode == kGateUp)
    hipLaunchKernelGGL(grouped_gemm_f32<kGateUp>, dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(grouped_gemm_f32<kDown>, dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
