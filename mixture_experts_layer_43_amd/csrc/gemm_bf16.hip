// Grouped bf16 GEMMs for the expert FFNs on gfx950 matrix cores.
//
// FFN_i(u) = W2 (silu(W1 u) * (W3 u)) for every chosen (token, expert) pair
// (DeepSeekMoE page, section 3.1-3.2: fine-grained experts are narrow FFNs of
// width I = I_base / m, and only the chosen ones run).  Each group is one
// expert: its rows are [offsets[g], offsets[g+1]) of the dispatched matrix,
// a count known only on the device, so each workgroup derives its
// (group, row tile) from offsets itself and workgroups past the last tile
// exit at once.  No host synchronisation is needed between dispatch and here.
//
// Tiles: BM rows x BN B-rows x BK=64, WM x WN wavefronts.  Gate/up mode
// packs BN/2 rows of W1 and the same BN/2 rows of W3 into one B tile, so a
// wavefront holds matching gate and up accumulators and applies
// silu(gate) * up in registers before the single bf16 store of H.  Down mode
// is a plain A . B^T.  Operands go global -> LDS directly
// (global_load_lds_dwordx4, no staging registers; two stages; 16-byte chunks
// in XOR-swizzled rows so the 16-byte fragment reads of a quarter-wave hit
// distinct banks) -> v_mfma_f32_32x32x16_bf16 with fp32 accumulation.  Workgroup ids are remapped so that consecutive tiles run on
// the same XCD and share its L2.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int BK = 64;          // bf16 elements per K step (128 B per row)
constexpr int kChunks = BK / 8; // 16-byte chunks per row
constexpr int kXcds = 8;
constexpr int kMaxGroups = 256;

// 16 bytes per lane from global memory straight into LDS (the 64 lanes of the
// wavefront fill 1 KB starting at the wave-uniform address lds).
__device__ __forceinline__ void copy_to_lds16(const bf16_t* src, bf16_t* lds) {
  __builtin_amdgcn_global_load_lds(src, lds, 16, 0, 0);
}

// silu(a) = a * sigmoid(a) with the hardware reciprocal (epilogue only).
__device__ __forceinline__ float silu_fast(float a) {
  return a * __builtin_amdgcn_rcpf(1.0f + __expf(-a));
}

// 16-byte chunk c of tile row r is stored at chunk position c ^ swz(r).
__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  const int xcd = bid % kXcds;
  const int local = bid / kXcds;
  const int base = nblocks / kXcds;
  const int rem = nblocks % kXcds;
  return xcd * base + min(xcd, rem) + local;
}

// GROUPED: rows come in per-expert groups described by offsets (routed
// experts); otherwise one dense group (shared experts).
template <int BM, int BN, int WM, int WN, int MODE, bool GROUPED>
__global__ __launch_bounds__(WM * WN * kWave) void grouped_gemm_bf16(GemmArgs p) {
  constexpr int NT = WM * WN * kWave;
  constexpr int TM = BM / WM;               // rows per wavefront
  constexpr int TN = BN / WN;               // B rows per wavefront
  constexpr int MB = TM / 32;
  constexpr int NB = TN / 32;
  constexpr int OUT_N = (MODE == kGateUp) ? BN / 2 : BN;
  constexpr int NW = WM * WN;
  constexpr int A_LD = BM / 8 / NW;         // 8-row LDS loads per wavefront per K step
  constexpr int B_LD = BN / 8 / NW;
  static_assert(A_LD * 8 * NW == BM && B_LD * 8 * NW == BN, "tile/wave mismatch");
  static_assert(MODE == kDown || NB % 2 == 0, "gate/up needs paired blocks");

  __shared__ __attribute__((aligned(16))) bf16_t smem[2][(BM + BN) * BK];
  __shared__ int s_tiles[kMaxGroups + 1];
  __shared__ int s_group, s_row0, s_rows;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int wm = wave / WN, wn = wave % WN;

  const int n_ntiles = (p.N + OUT_N - 1) / OUT_N;
  const int bid = xcd_remap(blockIdx.x, gridDim.x);
  const int mt = bid / n_ntiles;
  const int nt = bid % n_ntiles;

  // ---- locate (group, first row, rows) of row tile mt ------------------
  int g, row0, rows;
  if (!GROUPED) {
    g = 0;
    row0 = mt * BM;
    rows = static_cast<int>(min<int64_t>(BM, p.rows_total - row0));
    if (rows <= 0) return;
  } else {
    const int G = p.n_groups;
    // inclusive scan of per-group tile counts (G <= 256, NT >= 64)
    for (int i = tid; i < G; i += NT) {
      const int m = p.offsets[i + 1] - p.offsets[i];
      s_tiles[i + 1] = (m + BM - 1) / BM;
    }
    if (tid == 0) s_tiles[0] = 0;
    __syncthreads();
    if (tid == 0) {
      int run = 0;
      int found = -1;
      for (int i = 0; i < G; ++i) {
        const int c = s_tiles[i + 1];
        if (found < 0 && mt < run + c) {
          found = i;
          s_row0 = p.offsets[i] + (mt - run) * BM;
          s_rows = min(BM, p.offsets[i + 1] - s_row0);
        }
        run += c;
      }
      s_group = found;
    }
    __syncthreads();
    g = s_group;
    if (g < 0) return;
    row0 = s_row0;
    rows = s_rows;
  }

  const bf16_t* A = static_cast<const bf16_t*>(p.A);
  const bf16_t* B0 = static_cast<const bf16_t*>(p.B0) + static_cast<int64_t>(g) * p.b_group_stride;
  const bf16_t* B1 = (MODE == kGateUp)
                         ? static_cast<const bf16_t*>(p.B1) + static_cast<int64_t>(g) * p.b_group_stride
                         : nullptr;

  // ---- per-lane source chunks (fixed over K) -----------------------------
  // One global_load_lds_dwordx4 moves 64 lanes x 16 B into a contiguous 1 KB
  // of LDS: 8 tile rows of one K step.  Lane L lands on row L/8, chunk
  // position L%8, so it fetches logical chunk (L%8) ^ swz(row): the load
  // itself writes the swizzled layout.
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int lr = lane >> 3;
  const int lp = lane & 7;
  const bf16_t* a_src[A_LD];
#pragma unroll
  for (int i = 0; i < A_LD; ++i) {
    const int r = (wv * A_LD + i) * 8 + lr;
    const int c = lp ^ swz(r);
    const int64_t grow = row0 + min(r, rows - 1);
    const int64_t arow = p.gather ? p.gather[grow] : grow;
    a_src[i] = A + arow * p.lda + c * 8;
  }
  const bf16_t* b_src[B_LD];
#pragma unroll
  for (int i = 0; i < B_LD; ++i) {
    const int r = (wv * B_LD + i) * 8 + lr;
    const int c = lp ^ swz(r);
    const bf16_t* base;
    int n;
    if (MODE == kGateUp) {
      const bool up = r >= BN / 2;
      n = nt * OUT_N + (up ? r - BN / 2 : r);
      base = up ? B1 : B0;
    } else {
      n = nt * OUT_N + r;
      base = B0;
    }
    n = min(n, p.N - 1);
    b_src[i] = base + static_cast<int64_t>(n) * p.ldb + c * 8;
  }

  // Asynchronous global -> LDS copy of K step kt into stage buffer s.
  auto issue = [&](int kt, bf16_t* s) {
    const int k = kt * BK;
    const int64_t boff = static_cast<int64_t>(k / p.k_sub) * p.b_sub_stride + (k % p.k_sub);
#pragma unroll
    for (int i = 0; i < A_LD; ++i)
      copy_to_lds16(a_src[i] + k, s + (wv * A_LD + i) * 8 * BK);
#pragma unroll
    for (int i = 0; i < B_LD; ++i)
      copy_to_lds16(b_src[i] + boff, s + BM * BK + (wv * B_LD + i) * 8 * BK);
  };

  f32x16 acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  // Fragment rows inside the LDS tile for this lane.
  const int lrow = lane & 31;
  const int khalf = lane >> 5;  // which 8-element half of a 16-wide K slice
  int a_row[MB], b_row[NB];
#pragma unroll
  for (int i = 0; i < MB; ++i) a_row[i] = wm * TM + i * 32 + lrow;
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    if (MODE == kGateUp) {
      const int half = NB / 2;
      b_row[j] = (j < half) ? wn * (TN / 2) + j * 32 + lrow
                            : BN / 2 + wn * (TN / 2) + (j - half) * 32 + lrow;
    } else {
      b_row[j] = wn * TN + j * 32 + lrow;
    }
  }

  // Per K step: read every fragment of the current stage into registers,
  // then start the asynchronous copy of the next step into the other stage
  // (issued after the reads, so no wait on the copy is needed before them),
  // then run the step's MFMAs while the copy is in flight.
  const int nk = p.K / BK;
  issue(0, smem[0]);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int stage = kt & 1;
    const bf16_t* s = smem[stage];
    bf16x8 af[BK / 16][MB], bfr[BK / 16][NB];
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int c = kk * 2 + khalf;
#pragma unroll
      for (int i = 0; i < MB; ++i)
        af[kk][i] = *reinterpret_cast<const bf16x8*>(s + a_row[i] * BK + ((c ^ swz(a_row[i])) * 8));
#pragma unroll
      for (int j = 0; j < NB; ++j)
        bfr[kk][j] = *reinterpret_cast<const bf16x8*>(s + BM * BK + b_row[j] * BK +
                                                      ((c ^ swz(b_row[j])) * 8));
      // keep the reads in K order so each slice's MFMAs wait only for it
      __builtin_amdgcn_sched_barrier(0);
    }
    // Unconditional (the last step re-copies itself, in bounds) so no branch
    // sits between the fragment reads and the MFMAs that wait on them.
    issue(min(kt + 1, nk - 1), smem[stage ^ 1]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk)
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[kk][i], bfr[kk][j], acc[i][j], 0, 0, 0);
    // the MFMAs stay ahead of the wait for the copy
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }

  // ---- epilogue: D[row][col] of a 32x32 block sits in lane (col + 32*h),
  //      register v, row = 8*(v/4) + 4*h + v%4.
  bf16_t* C = static_cast<bf16_t*>(p.C);
  const int col_in = lane & 31;
  const int hrow = (lane >> 5) * 4;
  if (MODE == kGateUp) {
    constexpr int half = NB / 2;
#pragma unroll
    for (int i = 0; i < MB; ++i) {
#pragma unroll
      for (int j = 0; j < half; ++j) {
        const int col = nt * OUT_N + wn * (TN / 2) + j * 32 + col_in;
        if (col >= p.N) continue;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int r = wm * TM + i * 32 + 8 * (v >> 2) + hrow + (v & 3);
          if (r < rows) {
            const float gv = acc[i][j][v], uv = acc[i][j + half][v];
            C[(row0 + r) * p.ldc + col] = f32_to_bf16(silu_fast(gv) * uv);
          }
        }
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < MB; ++i) {
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int col = nt * OUT_N + wn * TN + j * 32 + col_in;
        if (col >= p.N) continue;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int r = wm * TM + i * 32 + 8 * (v >> 2) + hrow + (v & 3);
          if (r < rows) C[(row0 + r) * p.ldc + col] = f32_to_bf16(acc[i][j][v]);
        }
      }
    }
  }
}

template <int BM, int BN, int WM, int WN>
hipError_t launch_cfg(const GemmArgs& a, hipStream_t s) {
  constexpr int OUT_N = BN / 2;
  const int out_n = (a.mode == kGateUp) ? OUT_N : BN;
  const int n_ntiles = (a.N + out_n - 1) / out_n;
  int64_t max_mtiles;
  if (a.offsets == nullptr) {
    max_mtiles = (a.rows_total + BM - 1) / BM;
  } else {
    // sum_g ceil(M_g / BM) <= (sum_g M_g + G*(BM-1)) / BM
    max_mtiles = (a.rows_total + static_cast<int64_t>(a.n_groups) * (BM - 1)) / BM;
  }
  const int64_t grid = max_mtiles * n_ntiles;
  if (grid == 0) return hipSuccess;
  const dim3 block(WM * WN * kWave);
  const bool grouped = a.offsets != nullptr;
  if (a.mode == kGateUp && grouped)
    hipLaunchKernelGGL((grouped_gemm_bf16<BM, BN, WM, WN, kGateUp, true>), dim3(grid), block, 0, s, a);
  else if (a.mode == kGateUp)
    hipLaunchKernelGGL((grouped_gemm_bf16<BM, BN, WM, WN, kGateUp, false>), dim3(grid), block, 0, s, a);
  else if (grouped)
    hipLaunchKernelGGL((grouped_gemm_bf16<BM, BN, WM, WN, kDown, true>), dim3(grid), block, 0, s, a);
  else
    hipLaunchKernelGGL((grouped_gemm_bf16<BM, BN, WM, WN, kDown, false>), dim3(grid), block, 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_bf16(const GemmArgs& a, hipStream_t s) {
  if (a.rows_total == 0) return hipSuccess;
  const int64_t mean_rows = a.rows_total / (a.offsets ? a.n_groups : 1);
  if (mean_rows >= 192) return launch_cfg<256, 256, 2, 2>(a, s);
  if (mean_rows >= 64) return launch_cfg<128, 256, 2, 2>(a, s);
  return launch_cfg<32, 256, 1, 4>(a, s);
}

}  // namespace moe
