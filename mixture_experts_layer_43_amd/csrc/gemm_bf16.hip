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

// Buffer resource over `bytes` bytes at `base` (raw buffer: offsets are byte
// offsets; loads past `bytes` return zero instead of faulting).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

typedef __attribute__((address_space(3))) void* lds_void_ptr;
__device__ __forceinline__ lds_void_ptr lds_ptr(bf16_t* p) { return (lds_void_ptr)(p); }

// 16 bytes per lane straight into LDS: the 64 lanes of the wavefront fill
// the 1 KB at the wave-uniform address lds (buffer_load_dwordx4 ... lds).
__device__ __forceinline__ void copy_to_lds16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                              bf16_t* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      r, lds_ptr(lds), 16, voff, soff, 0, 0);
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

// Asynchronous global -> LDS copy of K step kt into stage buffer s: A_LD
// 8-row loads for A and B_LD for B per wavefront.  Per-lane byte offsets are
// fixed over K; the K position goes in the scalar offset.
template <int BM, int BN, int A_LD, int B_LD>
__device__ __forceinline__ void copy_step(__amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb,
                                          const uint32_t (&a_off)[A_LD], const uint32_t (&b_off)[B_LD],
                                          int kt, int k_sub, int64_t b_sub_stride, int wv, bf16_t* s) {
  const int k = kt * BK;
  const uint32_t sa = static_cast<uint32_t>(k) * 2u;
  const uint32_t sb = static_cast<uint32_t>(
      (static_cast<int64_t>(k / k_sub) * b_sub_stride + (k % k_sub)) * 2);
#pragma unroll
  for (int i = 0; i < A_LD; ++i) copy_to_lds16(ra, a_off[i], sa, s + (wv * A_LD + i) * 8 * BK);
#pragma unroll
  for (int i = 0; i < B_LD; ++i)
    copy_to_lds16(rb, b_off[i], sb, s + BM * BK + (wv * B_LD + i) * 8 * BK);
}

// One K step: start the copy of step kn into `nxt`, then read fragments of
// `cur` and run the MFMAs while the copy is in flight.  `cur` and `nxt` are
// distinct stages (restrict), so no wait on the copy is needed before the
// reads; the compiler puts it before the closing barrier.
template <int BM, int BN, int MB, int NB, int A_LD, int B_LD>
__device__ __forceinline__ void mma_step(f32x16 (&acc)[MB][NB], const bf16_t* __restrict__ cur,
                                         bf16_t* __restrict__ nxt, __amdgpu_buffer_rsrc_t ra,
                                         __amdgpu_buffer_rsrc_t rb, const uint32_t (&a_off)[A_LD],
                                         const uint32_t (&b_off)[B_LD], int kn, int k_sub,
                                         int64_t b_sub_stride, int wv, const int (&a_row)[MB],
                                         const int (&b_row)[NB], int khalf) {
  {
    const int k = kn * BK;
    const uint32_t sa = static_cast<uint32_t>(k) * 2u;
    const uint32_t sb = static_cast<uint32_t>(
        (static_cast<int64_t>(k / k_sub) * b_sub_stride + (k % k_sub)) * 2);
#pragma unroll
    for (int i = 0; i < A_LD; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          ra, lds_ptr(nxt + (wv * A_LD + i) * 8 * BK),
          16, a_off[i], sa, 0, 0);
#pragma unroll
    for (int i = 0; i < B_LD; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rb,
          lds_ptr(nxt + BM * BK + (wv * B_LD + i) * 8 * BK),
          16, b_off[i], sb, 0, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
  // Fragments of K slice kk+1 are read while the MFMAs of slice kk run.
  bf16x8 af[2][MB], bfr[2][NB];
  auto read = [&](int kk, int buf) {
    const int c = kk * 2 + khalf;
#pragma unroll
    for (int i = 0; i < MB; ++i)
      af[buf][i] = *reinterpret_cast<const bf16x8*>(cur + a_row[i] * BK + ((c ^ swz(a_row[i])) * 8));
#pragma unroll
    for (int j = 0; j < NB; ++j)
      bfr[buf][j] = *reinterpret_cast<const bf16x8*>(cur + BM * BK + b_row[j] * BK +
                                                     ((c ^ swz(b_row[j])) * 8));
  };
  read(0, 0);
#pragma unroll
  for (int kk = 0; kk < BK / 16; ++kk) {
    if (kk + 1 < BK / 16) read(kk + 1, (kk + 1) & 1);
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[kk & 1][i], bfr[kk & 1][j], acc[i][j],
                                                            0, 0, 0);
    // Interleave: the MB+NB fragment reads of the next slice between this
    // slice's MB*NB MFMAs, so their latency hides behind the matrix cores.
    if (kk + 1 < BK / 16) {
#pragma unroll
      for (int r = 0; r < MB + NB; ++r) {
        __builtin_amdgcn_sched_group_barrier(0x008, (MB * NB) / (MB + NB), 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                      // LDS read
      }
      __builtin_amdgcn_sched_group_barrier(0x008, MB * NB - (MB * NB) / (MB + NB) * (MB + NB), 0);
    }
  }
  // The MFMAs stay ahead of the barrier; the compiler puts the wait for the
  // copy (vmcnt) right before it.
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();
}

// GROUPED: rows come in per-expert groups described by offsets (routed
// experts); otherwise one dense group (shared experts).
template <int BM, int BN, int WM, int WN, int MODE, bool GROUPED>
__global__ __launch_bounds__(WM * WN * kWave) void grouped_gemm_bf16(GemmArgs p) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the launch stub
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

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int wm = wave / WN, wn = wave % WN;

  const int n_ntiles = (p.N + OUT_N - 1) / OUT_N;

  // ---- locate (group, first row, rows) of this workgroup's tile ---------
  // Tiles are ordered row tile major (the n_ntiles column tiles of one row
  // tile are consecutive), and consecutive tiles go to the same XCD so they
  // share its L2: the remap spreads the real tiles evenly over the XCDs.
  int g, row0, rows, mt, nt;
  if (!GROUPED) {
    const int bid = xcd_remap(blockIdx.x, gridDim.x);
    mt = bid / n_ntiles;
    nt = bid % n_ntiles;
    g = 0;
    row0 = mt * BM;
    rows = static_cast<int>(min<int64_t>(BM, p.rows_total - row0));
    if (rows <= 0) return;
  } else {
    // Row tiles per group are known only on the device.  Each wavefront
    // scans the groups 64 at a time (per-lane tile counts, shuffle prefix
    // sums, ballot) - first for the total, then for the group of its tile.
    const int G = p.n_groups;
    int total = 0;
    for (int g0 = 0; g0 < G; g0 += kWave) {
      const int gi = g0 + lane;
      const int m = gi < G ? p.offsets[gi + 1] - p.offsets[gi] : 0;
      int c = (m + BM - 1) / BM;
#pragma unroll
      for (int o = kWave / 2; o > 0; o >>= 1) c += __shfl_xor(c, o, kWave);
      total += c;
    }
    total = __builtin_amdgcn_readfirstlane(total);
    const int real = total * n_ntiles;
    // XCD x owns the contiguous range of real tiles [x*real/8, (x+1)*real/8)
    const int xcd = blockIdx.x % kXcds;
    const int local = blockIdx.x / kXcds;
    const int base_n = real / kXcds, rem = real % kXcds;
    if (local >= base_n + (xcd < rem ? 1 : 0)) return;
    const int bid = xcd * base_n + min(xcd, rem) + local;
    mt = bid / n_ntiles;
    nt = bid % n_ntiles;
    g = -1;
    row0 = 0;
    rows = 0;
    int base = 0;
    for (int g0 = 0; g0 < G; g0 += kWave) {
      const int gi = g0 + lane;
      const int m = gi < G ? p.offsets[gi + 1] - p.offsets[gi] : 0;
      const int cnt = (m + BM - 1) / BM;
      int incl = cnt;
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        const int v = __shfl_up(incl, o, kWave);
        if (lane >= o) incl += v;
      }
      const int excl = incl - cnt;
      const uint64_t hit = __ballot(mt >= base + excl && mt < base + incl);
      if (hit != 0) {
        const int src = __ffsll(static_cast<unsigned long long>(hit)) - 1;
        g = g0 + src;
        const int first = base + __shfl(excl, src, kWave);
        row0 = p.offsets[g] + (mt - first) * BM;
        rows = min(BM, p.offsets[g + 1] - row0);
        break;
      }
      base += __shfl(incl, kWave - 1, kWave);
    }
    g = __builtin_amdgcn_readfirstlane(g);
    if (g < 0) return;
    row0 = __builtin_amdgcn_readfirstlane(row0);
    rows = __builtin_amdgcn_readfirstlane(rows);
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
  // Byte offsets (32-bit: every operand matrix is below 4 GB, checked by the
  // host) into buffer resources over A and over this wavefront's B matrix.
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(A, static_cast<uint32_t>(p.a_bytes));
  uint32_t a_off[A_LD];
#pragma unroll
  for (int i = 0; i < A_LD; ++i) {
    const int r = (wv * A_LD + i) * 8 + lr;
    const int c = lp ^ swz(r);
    const int64_t grow = row0 + min(r, rows - 1);
    const int64_t arow = p.gather ? p.gather[grow] : grow;
    a_off[i] = static_cast<uint32_t>((arow * p.lda + c * 8) * 2);
  }
  // All B rows one wavefront copies come from the same matrix (W1 or W3 in
  // gate/up mode: the wavefront's 8*B_LD rows never straddle the boundary).
  const bool up = (MODE == kGateUp) && (wv * B_LD * 8 >= BN / 2);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(up ? B1 : B0, static_cast<uint32_t>(p.b_bytes));
  uint32_t b_off[B_LD];
#pragma unroll
  for (int i = 0; i < B_LD; ++i) {
    const int r = (wv * B_LD + i) * 8 + lr;
    const int c = lp ^ swz(r);
    int n = nt * OUT_N + ((MODE == kGateUp && up) ? r - BN / 2 : r);
    n = min(n, p.N - 1);
    b_off[i] = static_cast<uint32_t>((static_cast<int64_t>(n) * p.ldb + c * 8) * 2);
  }
  static_assert(MODE == kDown || (BN / 2) % (8 * B_LD) == 0, "B rows of a wavefront straddle W1/W3");

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

  // Two-stage pipeline: each step first starts the asynchronous copy of the
  // next K step into the other stage, then runs this step's MFMAs on the
  // current stage, then waits for the copy.  The copy of the last step is
  // repeated in bounds so the step body has no branch.
  const int nk = p.K / BK;
  const int64_t kstride_b = p.b_sub_stride;
  copy_step<BM, BN, A_LD, B_LD>(ra, rb, a_off, b_off, 0, p.k_sub, kstride_b, wv, smem[0]);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int stage = kt & 1;
    mma_step<BM, BN, MB, NB, A_LD, B_LD>(acc, smem[stage], smem[stage ^ 1], ra, rb, a_off, b_off,
                                         min(kt + 1, nk - 1), p.k_sub, kstride_b, wv, a_row, b_row,
                                         khalf);
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
#endif
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
  if (mean_rows >= 192) return launch_cfg<256, 256, 2, 4>(a, s);
  if (mean_rows >= 64) return launch_cfg<128, 256, 2, 2>(a, s);
  return launch_cfg<32, 256, 1, 4>(a, s);
}

}  // namespace moe
