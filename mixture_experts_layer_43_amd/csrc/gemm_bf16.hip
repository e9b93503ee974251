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
// (global_load_lds_dwordx4, no staging registers; two to four stages;
// 16-byte chunks in XOR-swizzled rows so the 16-byte fragment reads of a
// quarter-wave hit distinct banks) -> v_mfma_f32_32x32x16_bf16 with fp32
// accumulation.  Workgroup ids are remapped so that consecutive tiles run on
// the same XCD and share its L2.  A K that is a multiple of 8 but not of BK
// takes a separate instantiation (RAGGED) whose last step per weight matrix
// is partial; the aligned instantiation does not carry its checks.  The
// tile configuration and the weight copies' cache policy follow the mean
// rows per group (launch_gemm_bf16); every configuration sums each output
// over K in the same order, so the choice changes no result.
#include "common.h"
#include <hip/hip_ext.h>

#include <cmath>

#include "kernels.h"

namespace moe {

namespace {

constexpr int kXcds = 8;
constexpr int kPanel = 8;   // row tiles per panel in the grouped tile order
// Cache policy of the weight (B) copies for tiles whose expert groups mostly
// fit in one row tile: the non-temporal hint (aux bit 1).  Each weight byte is
// then read once, and streaming it past the caches leaves them to the
// activations that are read again.
constexpr int kStreamB = 2;

// Buffer resource over `bytes` bytes at `base` (raw buffer: offsets are byte
// offsets; loads past `bytes` return zero instead of faulting).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

typedef __attribute__((address_space(3))) void* lds_void_ptr;
__device__ __forceinline__ lds_void_ptr lds_ptr(bf16_t* p) { return (lds_void_ptr)(p); }

// silu(a) = a * sigmoid(a) with the hardware reciprocal (epilogue only).
// 4x4 transpose across the lanes of each quad: lane i's m[j] becomes lane
// j's m[i].  Two exchange rounds; in round b (1, 2) lane i takes register
// j^b of lane i^b (DPP quad permutation) where bit b of i and j differ.
__device__ __forceinline__ float dpp_quad_xor1(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_quad_xor2(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
}
__device__ __forceinline__ void quad_transpose(float (&m)[4], int q4) {
  float t[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) t[j] = dpp_quad_xor1(m[j ^ 1]);
#pragma unroll
  for (int j = 0; j < 4; ++j) m[j] = ((q4 ^ j) & 1) ? t[j] : m[j];
#pragma unroll
  for (int j = 0; j < 4; ++j) t[j] = dpp_quad_xor2(m[j ^ 2]);
#pragma unroll
  for (int j = 0; j < 4; ++j) m[j] = ((q4 ^ j) & 2) ? t[j] : m[j];
}

template <bool B>
struct Flag {
  static constexpr bool value = B;
};

__device__ __forceinline__ float silu_fast(float a) {
  return a * __builtin_amdgcn_rcpf(1.0f + __expf(-a));
}

// A tile row holds BK bf16 = BK/8 16-byte chunks; chunk c of row r is stored
// at chunk position c ^ swz(r).  Both patterns keep the 16-byte fragment
// reads of any 8 (and any 16) consecutive rows on distinct LDS banks.
template <int BK>
__device__ __forceinline__ int swz(int r) {
  if constexpr (BK == 64) return (r & 7) ^ ((r >> 3) & 1);
  else return ((r >> 1) ^ (r >> 3)) & 3;
}

__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  const int xcd = bid % kXcds;
  const int local = bid / kXcds;
  const int base = nblocks / kXcds;
  const int rem = nblocks % kXcds;
  return xcd * base + min(xcd, rem) + local;
}

// s_waitcnt with vmcnt <= N (gfx9 encoding: vmcnt in bits 3:0 and 15:14;
// expcnt and lgkmcnt at their maxima, i.e. not waited for).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Wait until at most `ahead` K steps of this wavefront's copies (L loads per
// step) are still in flight; `ahead` is wave-uniform and below STAGES-1.
template <int L, int STAGES>
__device__ __forceinline__ void wait_steps(int ahead) {
  if constexpr (STAGES >= 4) {
    if (ahead >= 2) { wait_vmcnt<2 * L>(); return; }
  }
  if constexpr (STAGES >= 3) {
    if (ahead >= 1) { wait_vmcnt<L>(); return; }
  }
  wait_vmcnt<0>();
}

// Workgroup barrier with no global memory fence: the copies into LDS are
// waited for explicitly (wait_steps) so that the ones for later K steps stay
// in flight.  This wavefront's own LDS reads must have returned, though: the
// last K slice of a step is read just before the barrier and multiplied
// after it, and right after the barrier other wavefronts start copying the
// step after next into that same stage.  The empty asm keeps the compiler
// from moving LDS accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
  // lgkmcnt(0); vmcnt and expcnt at their maxima (not waited for).
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (0 << 8));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Asynchronous global -> LDS copy of the K step starting at element k into
// stage `s`: A_LD loads for A rows and B_LD for B rows per wavefront, each
// 64 lanes x 16 B = 1 KB of LDS (64/(BK/8) tile rows).  Per-lane byte
// offsets are fixed over K; the K position goes in the scalar offset.
template <int BM, int BK, int A_LD, int B_LD, int BPOL>
__device__ __forceinline__ void copy_step(__amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb,
                                          const uint32_t (&a_off)[A_LD], const uint32_t (&b_off)[B_LD],
                                          int k, int k_sub, int64_t b_sub_stride, bool packed,
                                          int wv, bf16_t* __restrict__ s) {
  constexpr int R = kWave / (BK / 8);
  const uint32_t sa = static_cast<uint32_t>(k) * 2u;
  // Row-major B: column k of the K run.  Packed B (kPackRows-row tiles, each
  // a sequence of 64-wide K steps): the step's block inside the tile, plus
  // the column inside the step when BK = 32.
  const int kin = k % k_sub;
  const int64_t kpos = packed ? static_cast<int64_t>(kin / 64) * (kPackRows * 64) + kin % 64 : kin;
  const uint32_t sb = static_cast<uint32_t>(
      (static_cast<int64_t>(k / k_sub) * b_sub_stride + kpos) * 2);
#pragma unroll
  for (int i = 0; i < A_LD; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, lds_ptr(s + (wv * A_LD + i) * R * BK), 16, a_off[i],
                                             sa, 0, 0);
#pragma unroll
  for (int i = 0; i < B_LD; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, lds_ptr(s + BM * BK + (wv * B_LD + i) * R * BK), 16,
                                             b_off[i], sb, 0, BPOL);
}

// Ragged K: the K of one sub-matrix (k_sub) is a multiple of 8 but not of
// BK (row-major B only).  A sub-matrix then takes sps = ceil(k_sub / BK)
// steps, and its last one holds kvalid = k_sub - kin < BK values.  Step kt
// covers k in [sub*k_sub + kin, +BK) of A and column kin of sub-matrix sub
// of B.  A lane whose 16-byte chunk lies past kvalid copies its row's first
// chunk of the step instead, so every address stays inside the row; the B
// fragments of those chunks are zeroed before the MFMAs (mask_b).
template <int BM, int BK, int A_LD, int B_LD, int BPOL>
__device__ __forceinline__ void copy_step_ragged(__amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb,
                                                 const uint32_t (&a_off)[A_LD],
                                                 const uint32_t (&b_off)[B_LD], int kt, int sps,
                                                 int k_sub, int64_t b_sub_stride, int wv, int lane,
                                                 bf16_t* __restrict__ s) {
  constexpr int R = kWave / (BK / 8);
  const int sub = kt / sps;
  const int kin = (kt - sub * sps) * BK;
  const int kvalid = k_sub - kin;
  const uint32_t sa = static_cast<uint32_t>(sub * k_sub + kin) * 2u;
  const uint32_t sb = static_cast<uint32_t>((static_cast<int64_t>(sub) * b_sub_stride + kin) * 2);
  const int lr = lane / (BK / 8), lp = lane % (BK / 8);
#pragma unroll
  for (int i = 0; i < A_LD; ++i) {
    const int c = lp ^ swz<BK>((wv * A_LD + i) * R + lr);
    const uint32_t o = c * 8 < kvalid ? a_off[i] : a_off[i] - static_cast<uint32_t>(c * 16);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, lds_ptr(s + (wv * A_LD + i) * R * BK), 16, o, sa, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < B_LD; ++i) {
    const int c = lp ^ swz<BK>((wv * B_LD + i) * R + lr);
    const uint32_t o = c * 8 < kvalid ? b_off[i] : b_off[i] - static_cast<uint32_t>(c * 16);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, lds_ptr(s + BM * BK + (wv * B_LD + i) * R * BK), 16, o,
                                             sb, 0, BPOL);
  }
}

// Fragments of one 16-wide K slice: lane l holds 8 consecutive k of tile row
// a_row/b_row (= l%32 within its 32-row block), K half l/32.  Only the
// first MBA of the MB row blocks are read and multiplied: row blocks past
// the last row of a partial tile are skipped.
template <int MB, int NB>
struct Frags {
  bf16x8 a[2][MB], b[2][NB];
};

template <int BM, int BK, int MB, int NB, int MBA>
__device__ __forceinline__ void read_slice(Frags<MB, NB>& f, const bf16_t* __restrict__ cur, int kk,
                                           int buf, int khalf, const int (&a_row)[MB],
                                           const int (&b_row)[NB]) {
  const int c = kk * 2 + khalf;
#pragma unroll
  for (int i = 0; i < MBA; ++i)
    f.a[buf][i] = *reinterpret_cast<const bf16x8*>(cur + a_row[i] * BK + ((c ^ swz<BK>(a_row[i])) * 8));
#pragma unroll
  for (int j = 0; j < NB; ++j)
    f.b[buf][j] =
        *reinterpret_cast<const bf16x8*>(cur + BM * BK + b_row[j] * BK + ((c ^ swz<BK>(b_row[j])) * 8));
}

template <int MB, int NB, int MBA>
__device__ __forceinline__ void mma_slice(f32x16 (&acc)[MB][NB], const Frags<MB, NB>& f, int buf) {
#pragma unroll
  for (int i = 0; i < MBA; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[buf][i], f.b[buf][j], acc[i][j], 0, 0, 0);
}

// Ragged K: B fragments of logical chunk c (k = 8c .. 8c+7 of the step) at
// or past kvalid become zero, so the chunk adds nothing to the products.
template <int MB, int NB>
__device__ __forceinline__ void mask_b(Frags<MB, NB>& f, int buf, int c, int kvalid) {
  if (c * 8 >= kvalid) {
#pragma unroll
    for (int j = 0; j < NB; ++j) f.b[buf][j] = bf16x8{};
  }
}

// Scheduling pattern for one slice's MBA*NB MFMAs with the MBA+NB fragment
// reads of the next slice spread between them.
template <int MBA, int NB>
__device__ __forceinline__ void interleave() {
  constexpr int per = (MBA * NB) / (MBA + NB);
#pragma unroll
  for (int r = 0; r < MBA + NB; ++r) {
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);    // LDS read
    __builtin_amdgcn_sched_group_barrier(0x008, per, 0);  // MFMA
  }
  __builtin_amdgcn_sched_group_barrier(0x008, MBA * NB - per * (MBA + NB), 0);
  __builtin_amdgcn_sched_barrier(0);
}

// One K step on stage `cur`, with the copy of a later step into the other
// stages already issued.  The MFMAs of the previous step's last slice
// (register buffer 1, read before the barrier) run while slice 0 of this
// step is read, so the matrix cores have work across the barrier.  The last
// slice of this step is only read here; its MFMAs run in the next step (or
// after the loop).
template <int BM, int BK, int MB, int NB, int MBA, bool RAGGED>
__device__ __forceinline__ void step_body(f32x16 (&acc)[MB][NB], Frags<MB, NB>& f,
                                          const bf16_t* __restrict__ cur, bool has_prev, int khalf,
                                          const int (&a_row)[MB], const int (&b_row)[NB], int kvalid) {
  constexpr int NS = BK / 16;
  read_slice<BM, BK, MB, NB, MBA>(f, cur, 0, 0, khalf, a_row, b_row);
  if constexpr (RAGGED) mask_b(f, 0, khalf, kvalid);
  if (has_prev) {
    mma_slice<MB, NB, MBA>(acc, f, 1);
    interleave<MBA, NB>();
  } else {
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int kk = 0; kk + 1 < NS; ++kk) {
    read_slice<BM, BK, MB, NB, MBA>(f, cur, kk + 1, (kk + 1) & 1, khalf, a_row, b_row);
    if constexpr (RAGGED) mask_b(f, (kk + 1) & 1, (kk + 1) * 2 + khalf, kvalid);
    mma_slice<MB, NB, MBA>(acc, f, kk & 1);
    interleave<MBA, NB>();
  }
}

// The STAGES-deep K loop.  The copies of the first STAGES-1 K steps were
// issued by the caller.  Step kt waits for its own copy (leaving the later
// ones in flight), meets the other wavefronts at a barrier (after which
// every copy of step kt has landed and nobody reads stage (kt-1) % STAGES
// any more), issues the copy of step kt+STAGES-1 into that stage and
// computes.  A wavefront whose rows are all past the tile's last row
// (MBA == 0) only copies and waits.
template <int BM, int BK, int STAGES, int MB, int NB, int MBA, int A_LD, int B_LD, bool RAGGED, int BPOL>
__device__ __forceinline__ void k_loop(f32x16 (&acc)[MB][NB], __amdgpu_buffer_rsrc_t ra,
                                       __amdgpu_buffer_rsrc_t rb, const uint32_t (&a_off)[A_LD],
                                       const uint32_t (&b_off)[B_LD], int nk, int k_sub,
                                       int64_t kstride_b, bool packed, int wv, int khalf,
                                       const int (&a_row)[MB],
                                       const int (&b_row)[NB], bf16_t* smem, int se, int sps,
                                       int lane) {
  constexpr int L = A_LD + B_LD;
  Frags<MB, NB> fr;
  for (int kt = 0; kt < nk; ++kt) {
    wait_steps<L, STAGES>(min(STAGES - 2, nk - 1 - kt));
    lds_barrier();
    const int kn = kt + STAGES - 1;
    if (kn < nk) {
      if constexpr (RAGGED)
        copy_step_ragged<BM, BK, A_LD, B_LD, BPOL>(ra, rb, a_off, b_off, kn, sps, k_sub, kstride_b, wv, lane,
                                             smem + (kn % STAGES) * se);
      else
        copy_step<BM, BK, A_LD, B_LD, BPOL>(ra, rb, a_off, b_off, kn * BK, k_sub, kstride_b, packed, wv,
                                      smem + (kn % STAGES) * se);
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (MBA > 0) {
      const int kvalid = RAGGED ? k_sub - (kt % sps) * BK : BK;
      step_body<BM, BK, MB, NB, MBA, RAGGED>(acc, fr, smem + (kt % STAGES) * se, kt > 0, khalf, a_row,
                                             b_row, kvalid);
    }
  }
  if constexpr (MBA > 0) mma_slice<MB, NB, MBA>(acc, fr, 1);
}

// GROUPED: rows come in per-expert groups described by offsets (routed
// experts); otherwise one dense group (shared experts).
template <int BM, int BN, int WM, int WN, int BK, int STAGES, int MODE, bool GROUPED, bool RAGGED, int BPOL>
__global__ __launch_bounds__(WM * WN * kWave) void grouped_gemm_bf16(GemmArgs p) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the launch stub
  constexpr int TM = BM / WM;               // rows per wavefront
  constexpr int TN = BN / WN;               // B rows per wavefront
  constexpr int MB = TM / 32;
  constexpr int NB = TN / 32;
  constexpr int OUT_N = (MODE == kGateUp) ? BN / 2 : BN;
  constexpr int NW = WM * WN;
  constexpr int RPL = kWave / (BK / 8);     // tile rows per 1 KB LDS load
  constexpr int A_LD = BM / RPL / NW;       // loads per wavefront per K step
  constexpr int B_LD = BN / RPL / NW;
  constexpr int SE = (BM + BN) * BK;        // elements per stage
  static_assert(BK == 32 || BK == 64, "K step");
  static_assert(STAGES >= 2 && STAGES <= 4, "stages");
  static_assert(A_LD * RPL * NW == BM && B_LD * RPL * NW == BN, "tile/wave mismatch");
  static_assert(MODE == kDown || NB % 2 == 0, "gate/up needs paired blocks");
  static_assert((BK / 16) % 2 == 0, "slices alternate register buffers");

  __shared__ __attribute__((aligned(16))) bf16_t smem[STAGES * SE];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int wm = wave / WN, wn = wave % WN;

  const int n_ntiles = (p.N + OUT_N - 1) / OUT_N;

  // ---- locate (group, first row, rows) of this workgroup's tile ---------
  // Consecutive tiles go to the same XCD so they share its L2: the remap
  // spreads the real tiles evenly over the XCDs, in contiguous ranges.  A
  // dense call orders tiles row tile major; grouped calls order them by
  // panels (below).
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
    // The extra groups follow the indexed ones.
    const int G = p.n_groups + p.n_extra;
    auto group_rows = [&](int gi) {
      return gi < p.n_groups ? p.offsets[gi + 1] - p.offsets[gi] : (gi < G ? p.extra_rows : 0);
    };
    int total = 0;
    for (int g0 = 0; g0 < G; g0 += kWave) {
      const int gi = g0 + lane;
      const int m = group_rows(gi);
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
    // Order inside a group: panels of up to kPanel row tiles; inside a
    // panel the column tile is the slow index, so the workgroups running
    // together on an XCD share a few column tiles of the weights (read from
    // HBM once per panel) and the panel's rows of A.
    g = -1;
    row0 = 0;
    rows = 0;
    mt = 0;
    nt = 0;
    int base = 0;
    for (int g0 = 0; g0 < G; g0 += kWave) {
      const int gi = g0 + lane;
      const int cnt = (group_rows(gi) + BM - 1) / BM * n_ntiles;  // tiles of group gi
      int incl = cnt;
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        const int v = __shfl_up(incl, o, kWave);
        if (lane >= o) incl += v;
      }
      const int excl = incl - cnt;
      const uint64_t hit = __ballot(bid >= base + excl && bid < base + incl);
      if (hit != 0) {
        const int src = __ffsll(static_cast<unsigned long long>(hit)) - 1;
        g = g0 + src;
        const int in_g = bid - base - __shfl(excl, src, kWave);
        const int gm = group_rows(g);
        const int mtg = (gm + BM - 1) / BM;
        const int panel = in_g / (kPanel * n_ntiles);
        const int pm = min(kPanel, mtg - panel * kPanel);
        const int r = in_g - panel * kPanel * n_ntiles;
        nt = r / pm;
        const int mloc = panel * kPanel + r % pm;
        const int64_t gstart = g < p.n_groups
                                   ? p.offsets[g]
                                   : p.extra_base + static_cast<int64_t>(g - p.n_groups) * p.extra_rows;
        row0 = static_cast<int>(gstart) + mloc * BM;
        rows = min(BM, gm - mloc * BM);
        break;
      }
      base += __shfl(incl, kWave - 1, kWave);
    }
    nt = __builtin_amdgcn_readfirstlane(nt);
    g = __builtin_amdgcn_readfirstlane(g);
    if (g < 0) return;
    row0 = __builtin_amdgcn_readfirstlane(row0);
    rows = __builtin_amdgcn_readfirstlane(rows);
  }

  const bf16_t* A = static_cast<const bf16_t*>(p.A);
  const bool extra = GROUPED && g >= p.n_groups;
  const int64_t gx = extra ? g - p.n_groups : g;
  const bf16_t* B0 = static_cast<const bf16_t*>(extra ? p.Bx0 : p.B0) +
                     gx * (extra ? p.bx_group_stride : p.b_group_stride);
  const bf16_t* B1 = (MODE == kGateUp) ? static_cast<const bf16_t*>(extra ? p.Bx1 : p.B1) +
                                             gx * (extra ? p.bx_group_stride : p.b_group_stride)
                                       : nullptr;
  const int64_t b_bytes = extra ? p.bx_bytes : p.b_bytes;

  // ---- per-lane source chunks (fixed over K) -----------------------------
  // One load moves 64 lanes x 16 B into a contiguous 1 KB of LDS: RPL tile
  // rows of one K step.  Lane L lands on row L/(BK/8), chunk position
  // L%(BK/8), so it fetches logical chunk (L%(BK/8)) ^ swz(row): the load
  // itself writes the swizzled layout.
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int lr = lane / (BK / 8);
  const int lp = lane % (BK / 8);
  // Byte offsets (32-bit: every operand matrix is below 4 GB, checked by the
  // host) into buffer resources over A and over this wavefront's B matrix.
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(A, static_cast<uint32_t>(p.a_bytes));
  uint32_t a_off[A_LD];
#pragma unroll
  for (int i = 0; i < A_LD; ++i) {
    const int r = (wv * A_LD + i) * RPL + lr;
    const int c = lp ^ swz<BK>(r);
    const int64_t grow = row0 + min(r, rows - 1);
    const int64_t arow = !p.gather ? grow : extra ? (grow - p.extra_base) % p.extra_rows : p.gather[grow];
    a_off[i] = static_cast<uint32_t>((arow * p.lda + c * 8) * 2);
  }
  // All B rows one wavefront copies come from the same matrix (W1 or W3 in
  // gate/up mode: the wavefront's RPL*B_LD rows never straddle the boundary).
  const bool up = (MODE == kGateUp) && (wv * B_LD * RPL >= BN / 2);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(up ? B1 : B0, static_cast<uint32_t>(b_bytes));
  uint32_t b_off[B_LD];
#pragma unroll
  for (int i = 0; i < B_LD; ++i) {
    const int r = (wv * B_LD + i) * RPL + lr;
    const int c = lp ^ swz<BK>(r);
    int n = nt * OUT_N + ((MODE == kGateUp && up) ? r - BN / 2 : r);
    n = min(n, p.N - 1);
    const int64_t e = p.packed ? static_cast<int64_t>(n / kPackRows) * kPackRows * p.k_sub +
                                     (n % kPackRows) * 64 + c * 8
                               : static_cast<int64_t>(n) * p.ldb + c * 8;
    b_off[i] = static_cast<uint32_t>(e * 2);
  }
  static_assert(MODE == kDown || (BN / 2) % (RPL * B_LD) == 0, "B rows of a wavefront straddle W1/W3");

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

  // ---- K loop -------------------------------------------------------------
  // K steps: BK-wide runs of K; with ragged K, ceil(k_sub / BK) per
  // sub-matrix (p.K is a whole number of sub-matrices).
  const int sps = RAGGED ? (p.k_sub + BK - 1) / BK : p.k_sub / BK;
  const int nk = RAGGED ? (p.K / p.k_sub) * sps : p.K / BK;
  const int64_t kstride_b = p.b_sub_stride;
#pragma unroll
  for (int j = 0; j < STAGES - 1; ++j) {
    if (j < nk) {
      if constexpr (RAGGED)
        copy_step_ragged<BM, BK, A_LD, B_LD, BPOL>(ra, rb, a_off, b_off, j, sps, p.k_sub, kstride_b, wv, lane,
                                             smem + j * SE);
      else
        copy_step<BM, BK, A_LD, B_LD, BPOL>(ra, rb, a_off, b_off, j * BK, p.k_sub, kstride_b, p.packed, wv,
                                      smem + j * SE);
    }
  }
  // 32-row blocks of this wavefront that hold rows of the tile.
  const int mba = __builtin_amdgcn_readfirstlane(max(0, min(MB, (rows - wm * TM + 31) / 32)));
#define MOE_K_LOOP(n)                                                                            \
  k_loop<BM, BK, STAGES, MB, NB, n, A_LD, B_LD, RAGGED, BPOL>(acc, ra, rb, a_off, b_off, nk, p.k_sub, \
                                                        kstride_b, p.packed, wv, khalf, a_row,     \
                                                        b_row, smem, SE, sps, lane)
  if (mba == MB) {
    MOE_K_LOOP(MB);
  } else if (mba == 0) {
    MOE_K_LOOP(0);
  } else {
    if constexpr (MB > 1) if (mba == 1) MOE_K_LOOP(1);
    if constexpr (MB > 2) if (mba == 2) MOE_K_LOOP(2);
    if constexpr (MB > 3) if (mba == 3) MOE_K_LOOP(3);
    static_assert(MB <= 4, "row blocks per wavefront");
  }
#undef MOE_K_LOOP

  // ---- epilogue.  D[row][col] of a 32x32 block sits in lane (col + 32*h),
  //      register v, row = 8*(v/4) + 4*h + v%4.  Rows past the tile's end
  //      and columns past N (a multiple of 8) are not stored.
  constexpr int NBO = (MODE == kGateUp) ? NB / 2 : NB;   // output blocks per wavefront row
  constexpr int TNO = (MODE == kGateUp) ? TN / 2 : TN;
  // The ReLU FFN's up projection (kDown with p.relu) clamps at 0; the two
  // cases are separate instantiations of the store loops.
  bf16_t* C = static_cast<bf16_t*>(p.C);
  const int hrow = (lane >> 5) * 4;
  if constexpr (BM <= 32) {
    // 32-row tiles (few rows per group, weight streaming): straight from
    // the accumulators, with no LDS and no barrier.  A 4x4 transpose inside
    // each quad of lanes turns the four rows of one column (registers
    // 4g..4g+3) into four columns of one row, so every lane stores 8 bytes:
    // row 8g + 4h + lane%4, columns 4 (col/4) .. +3.
    const int q4 = lane & 3;
    const int colq = (lane & 31) & ~3;
    const int col0 = nt * OUT_N + wn * TNO;
    auto store = [&](auto relu) {
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NBO; ++j)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            float m[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const int v = 4 * g4 + u;
              if constexpr (MODE == kGateUp) m[u] = silu_fast(acc[i][j][v]) * acc[i][j + NBO][v];
              else if constexpr (decltype(relu)::value) m[u] = fmaxf(acc[i][j][v], 0.0f);
              else m[u] = acc[i][j][v];
            }
            quad_transpose(m, q4);
            const int r = wm * TM + i * 32 + 8 * g4 + hrow + q4;
            const int c = col0 + j * 32 + colq;
            if (r < rows && c < p.N) {
              uint2 o;
              o.x = pack_bf16x2(m[0], m[1]);
              o.y = pack_bf16x2(m[2], m[3]);
              *reinterpret_cast<uint2*>(C + (row0 + r) * p.ldc + c) = o;
            }
          }
    };
    if (MODE == kDown && p.relu)
      store(Flag<true>{});
    else
      store(Flag<false>{});
  } else {
    // Larger tiles: the bf16 tile goes through LDS (the stage buffers are
    // free now) so that the global stores are whole 16-byte chunks of rows,
    // a row of the tile per 16..32 lanes; they are non-temporal (the tile
    // is not read again by this kernel).  In LDS, 16-byte chunk k of tile
    // row r sits at chunk k ^ csw(r), csw(r) = (r & 7) ^ 4 (r & 1).  The LDS
    // takes a dword write in two halves of 32 lanes over 32 banks; the half
    // that writes rows r and r + 1 (r even) of a wavefront's 32 columns then
    // finds them in the two different halves of the 32 banks (with
    // csw(r) = r & 7 they shared them, two ways), and the 16-byte reads of
    // eight consecutive chunks of a row still cover all banks.
    constexpr int NT = WM * WN * kWave;
    static_assert(OUT_N % 64 == 0 && BM * OUT_N <= STAGES * SE, "C tile does not fit the stages");
    __syncthreads();  // every wavefront is done reading the last stage
    bf16_t* ct = smem;
    auto csw = [](int r) { return (r & 7) ^ ((r & 1) << 2); };
    auto cpos = [&](int r, int c) { return r * OUT_N + ((((c >> 3) ^ csw(r))) << 3) + (c & 7); };
    const int col_in = lane & 31;
    // Rows r and r + 1 of a column (registers v, v + 1 for even v) are
    // converted together.  The byte address of a write is a lane part per
    // (j, v % 4) - the swizzle sees only the row's low three bits, as every
    // wavefront's rows start at a multiple of 8 - plus a row offset known
    // at compile time, which the LDS store takes as its immediate.
    static_assert(TM % 8 == 0, "wavefront rows start at multiples of 8");
    char* const cl = reinterpret_cast<char*>(smem) + (wm * TM + hrow) * (OUT_N * 2);
    // Each LDS write is a whole dword: lanes c and c ^ 1 (adjacent columns,
    // the same rows) swap halves of their converted row pairs (one DPP quad
    // exchange), so the even-column lane holds row r of columns c, c + 1
    // and the odd one row r + 1 of columns c - 1, c.  dcol: the byte offset
    // of that dword for register pair u = 0, 2 (the odd lane's row is one
    // further down).
    const int odd = col_in & 1;
    const uint32_t psel = odd ? 0x03020706u : 0x05040100u;
    int dcol[NBO][2];
#pragma unroll
    for (int j = 0; j < NBO; ++j) {
      const int c = (wn * TNO + j * 32 + col_in) & ~1;
#pragma unroll
      for (int u = 0; u < 2; ++u)
        dcol[j][u] = ((((c >> 3) ^ csw(hrow + 2 * u + odd)) << 3) + (c & 7)) * 2 + odd * (OUT_N * 2);
    }
    auto stage = [&](auto relu) {
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NBO; ++j)
#pragma unroll
          for (int v = 0; v < 16; v += 2) {
            float e0, e1;
            if constexpr (MODE == kGateUp) {
              e0 = silu_fast(acc[i][j][v]) * acc[i][j + NBO][v];
              e1 = silu_fast(acc[i][j][v + 1]) * acc[i][j + NBO][v + 1];
            } else if constexpr (decltype(relu)::value) {
              e0 = fmaxf(acc[i][j][v], 0.0f);
              e1 = fmaxf(acc[i][j][v + 1], 0.0f);
            } else {
              e0 = acc[i][j][v];
              e1 = acc[i][j][v + 1];
            }
            // pr: rows r, r + 1 of this lane's column; pq: the same of the
            // neighbour column.
            const uint32_t pr = pack_bf16x2(e0, e1);
            const uint32_t pq = static_cast<uint32_t>(
                __builtin_amdgcn_update_dpp(0, static_cast<int>(pr), 0xB1, 0xF, 0xF, false));
            const int ro = (i * 32 + 8 * (v >> 2) + (v & 3)) * (OUT_N * 2);
            *reinterpret_cast<uint32_t*>(cl + ro + dcol[j][(v & 3) >> 1]) =
                __builtin_amdgcn_perm(pq, pr, psel);
          }
    };
    if (MODE == kDown && p.relu)
      stage(Flag<true>{});
    else
      stage(Flag<false>{});
    __syncthreads();
    constexpr int CPR = OUT_N / 8;  // 16-byte chunks per tile row
    const int col0 = nt * OUT_N;
    for (int idx = tid; idx < rows * CPR; idx += NT) {
      const int r = idx / CPR, c8 = (idx % CPR) * 8;
      if (col0 + c8 < p.N)
        __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(ct + cpos(r, c8)),
                                    reinterpret_cast<u32x4*>(C + (row0 + r) * p.ldc + col0 + c8));
    }
  }
#endif
}

template <int BM, int BN, int WM, int WN, int BK, int STAGES, int MODE, int BPOL = 0>
hipError_t launch_cfg(const GemmArgs& a, hipStream_t s, StageEvents ev) {
  static_assert(BK == 32 || BK == 64, "K steps divide the packed layout's 64-wide steps");
  constexpr int OUT_N = (MODE == kGateUp) ? BN / 2 : BN;
  const int n_ntiles = (a.N + OUT_N - 1) / OUT_N;
  int64_t max_mtiles;
  if (a.offsets == nullptr) {
    max_mtiles = (a.rows_total + BM - 1) / BM;
  } else {
    // sum_g ceil(M_g / BM) <= (sum_g M_g + G*(BM-1)) / BM
    max_mtiles = (a.rows_total + static_cast<int64_t>(a.n_groups + a.n_extra) * (BM - 1)) / BM;
  }
  const int64_t grid = max_mtiles * n_ntiles;
  if (grid == 0) return record_stage(ev, s);
  const dim3 block(WM * WN * kWave);
  // K must be whole sub-matrices; ragged sub-matrices (k_sub not a multiple
  // of BK, still of 8) take the ragged instantiation, row-major B only.
  if (a.k_sub <= 0 || a.k_sub % 8 != 0 || a.K % a.k_sub != 0) return hipErrorInvalidValue;
  const bool ragged = a.k_sub % BK != 0;
  if (ragged && a.packed) return hipErrorInvalidValue;
#define MOE_GEMM_LAUNCH(G, R)                                                                        \
  hipExtLaunchKernelGGL((grouped_gemm_bf16<BM, BN, WM, WN, BK, STAGES, MODE, G, R, BPOL>), dim3(grid), block, 0, \
                        s, ev.start, ev.stop, 0, a)
  if (a.offsets != nullptr) {
    if (ragged) MOE_GEMM_LAUNCH(true, true);
    else MOE_GEMM_LAUNCH(true, false);
  } else {
    if (ragged) MOE_GEMM_LAUNCH(false, true);
    else MOE_GEMM_LAUNCH(false, false);
  }
#undef MOE_GEMM_LAUNCH
  return hipGetLastError();
}

template <int BM, int BN, int WM, int WN, int BK, int STAGES, int BPOL = 0>
hipError_t launch_both(const GemmArgs& a, hipStream_t s, StageEvents ev) {
  return a.mode == kGateUp ? launch_cfg<BM, BN, WM, WN, BK, STAGES, kGateUp, BPOL>(a, s, ev)
                           : launch_cfg<BM, BN, WM, WN, BK, STAGES, kDown, BPOL>(a, s, ev);
}

// One 16-byte chunk (8 consecutive k of one row) per thread.
__global__ __launch_bounds__(256) void pack_kernel(const uint4* __restrict__ src,
                                                   uint4* __restrict__ dst, int64_t chunks,
                                                   int rows, int cols) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= chunks) return;
  const int64_t per_row = cols / 8, per_mat = static_cast<int64_t>(rows) * per_row;
  const int64_t g = i / per_mat, rem = i % per_mat;
  const int64_t n = rem / per_row, k = (rem % per_row) * 8;
  const int64_t e = g * rows * static_cast<int64_t>(cols) + (n / kPackRows) * kPackRows * cols +
                    (k / 64) * (kPackRows * 64) + (n % kPackRows) * 64 + k % 64;
  dst[e / 8] = src[i];
}

}  // namespace

hipError_t launch_pack(const void* src, void* dst, int64_t count, int rows, int cols,
                       hipStream_t s) {
  const int64_t chunks = count * rows * static_cast<int64_t>(cols) / 8;
  if (chunks == 0) return hipSuccess;
  hipLaunchKernelGGL(pack_kernel, dim3(static_cast<unsigned>((chunks + 255) / 256)), dim3(256), 0,
                     s, static_cast<const uint4*>(src), static_cast<uint4*>(dst), chunks, rows, cols);
  return hipGetLastError();
}

hipError_t record_stage(StageEvents ev, hipStream_t s) {
  if (ev.start != nullptr) {
    const hipError_t e = hipEventRecord(ev.start, s);
    if (e != hipSuccess) return e;
  }
  return ev.stop != nullptr ? hipEventRecord(ev.stop, s) : hipSuccess;
}

// Expected number of row tiles of height h for a group whose size is
// Poisson with mean mu: the sum over j >= 0 of P(size > j h), each tail from
// the normal approximation with a continuity correction.
static double expected_row_tiles(double mu, int h) {
  if (mu <= 0.0) return 0.0;
  const double sd = std::sqrt(mu);
  double e = 0.0;
  for (int j = 0; j * static_cast<double>(h) <= mu + 8.0 * sd; ++j)
    e += 0.5 * std::erfc((j * static_cast<double>(h) + 0.5 - mu) / (sd * std::sqrt(2.0)));
  return e;
}

// Time per row of a row tile relative to the 256x256 tile.  Where all three fit
// the groups exactly (the 16B-shaped layer's GEMMs at 8k and 16k tokens)
// 192-row tiles take 1.07-1.13 and 128-row tiles 1.32-1.38.  The weights are
// fitted to the fastest tile of each GEMM, every height forced in turn, with
// the router's own spread of group sizes: the 16B-shaped layer at 1k-3k
// tokens and the 2b-shaped layer (d = 1280, I = 896, 63 + 1 experts, top-7)
// at 1k-4k tokens.  With the rounds counted below, 192-row weights from 1.10
// to 1.18 and 128-row weights from 1.38 to 1.50 pick all 26 (gate/up and
// down); without them 1.14 and 1.42 miss two of the 2b-shaped ones.
static double tile_row_cost(int h) { return h == 256 ? 1.0 : h == 192 ? 1.14 : 1.42; }

hipError_t launch_gemm_bf16(const GemmArgs& a, hipStream_t s, StageEvents ev) {
  if (a.rows_total == 0) return record_stage(ev, s);
  if (a.offsets == nullptr) {
    // One dense group (the shared experts as one FFN): the largest tile whose
    // grid still gives most CUs a tile.  A decode-sized batch would leave the
    // big tiles to a few workgroups that each stream megabytes of weights
    // alone; it takes the 32-row streaming tiles below instead.
    const int64_t nt = (a.N + (a.mode == kGateUp ? 127 : 255)) / (a.mode == kGateUp ? 128 : 256);
    if (a.rows_total >= 192 && (a.rows_total + 255) / 256 * nt >= 256)
      return launch_both<256, 256, 2, 4, 64, 2>(a, s, ev);
    if (a.rows_total >= 64 && (a.rows_total + 127) / 128 * nt >= 128)
      return launch_both<128, 256, 2, 2, 64, 3>(a, s, ev);
    if (a.mode == kDown) return launch_cfg<32, 64, 1, 2, 64, 4, kDown>(a, s, ev);
    return launch_cfg<32, 256, 1, 4, 64, 2, kGateUp>(a, s, ev);
  }
  const int64_t mean_rows = a.rows_total / (a.n_groups + a.n_extra);
  if (mean_rows >= 64) {
    // 128-, 192- or 256-row tiles, whichever finishes first.  Every tile of
    // one launch runs the same K loop, one workgroup per CU, so the launch
    // takes ceil(tiles / CUs) rounds of tiles, each as long as the tile's
    // height times its measured cost per row.  The row tiles are expected
    // counts: routed groups with their sizes as a balanced router spreads
    // them (Poisson around the mean), shared groups exactly; the column
    // tiles follow N (128 output columns per gate/up tile, 256 per down
    // tile).  Rounds matter where the grid is small: the 2b-shaped layer's
    // gate/up at 1536 tokens makes 518 tiles of 192 rows (a third round of
    // 6 tiles on 256 CUs) but 483 of 256 rows, and runs 81 against 103 us.
    const double routed = static_cast<double>(a.rows_total) -
                          static_cast<double>(a.n_extra) * static_cast<double>(a.extra_rows);
    const double mu = routed / a.n_groups;
    const int out_cols = a.mode == kGateUp ? 128 : 256;
    const double col_tiles = static_cast<double>((a.N + out_cols - 1) / out_cols);
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      cus = 256;
    double best = 0.0;
    int bm = 256;
    // Past 4096 rows per group the last row tile's padding is a few % at
    // most and 256-row tiles win.
    for (const int h : {256, 192, 128}) {
      if (h != 256 && mu > 4096.0) break;
      const double tiles = a.n_groups * expected_row_tiles(mu, h) +
                           static_cast<double>(a.n_extra) * ((a.extra_rows + h - 1) / h);
      const double rounds = std::ceil(tiles * col_tiles / cus);
      const double cost = rounds * h * tile_row_cost(h);
      if (h == 256 || cost < best) {
        best = cost;
        bm = h;
      }
    }
    // Where most groups fit in one row tile each weight byte is read once,
    // and the weight copies go non-temporal; 256-row tiles keep plain
    // copies (at 16k tokens the hint costs them 2-3 %, as a weight tile is
    // read by several row tiles there).  Three stages for 128-row tiles keep
    // two K steps of copies in flight (144 KB of LDS).
    if (bm == 128) return launch_both<128, 256, 2, 2, 64, 3, kStreamB>(a, s, ev);
    if (bm == 192) {
      if (mu <= 192.0) return launch_both<192, 256, 2, 4, 64, 2, kStreamB>(a, s, ev);
      return launch_both<192, 256, 2, 4, 64, 2>(a, s, ev);
    }
    return launch_both<256, 256, 2, 4, 64, 2>(a, s, ev);
  }
  // 17-63 rows: one 64-row tile per group, where 32-row tiles would take two
  // per group and each would stream the group's weights.  Gate/up 64x256
  // with two stages (80 KB: two workgroups per CU) beats three stages (one
  // workgroup per CU) by 8-20 % with real group sizes (e.g. 122 against 142
  // us at 31 rows, 140 against 148 us at 62 rows).
  if (mean_rows > 16) {
    if (a.mode == kDown) return launch_cfg<64, 128, 2, 2, 64, 3, kDown, kStreamB>(a, s, ev);
    return launch_cfg<64, 256, 1, 4, 64, 2, kGateUp, kStreamB>(a, s, ev);
  }
  // Few rows per group (the decode shape): the weights stream through and
  // every workgroup's time is its share of them.  Narrow down tiles (64
  // columns) split the stream finer, so the last partial round of
  // workgroups is short; four stages keep three K steps of copies in flight
  // (48 KB of LDS, three workgroups per CU).  Non-temporal weight copies:
  // gate/up 140 -> 120 us and down 72 -> 64 us at 16 rows per group.
  if (a.mode == kDown) return launch_cfg<32, 64, 1, 2, 64, 4, kDown, kStreamB>(a, s, ev);
  return launch_cfg<32, 256, 1, 4, 64, 2, kGateUp, kStreamB>(a, s, ev);
}

}  // namespace moe
