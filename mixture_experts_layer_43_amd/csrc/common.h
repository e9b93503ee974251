// Device helpers shared by the gfx950 kernels of libmoe.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;  // CDNA wavefront width

typedef uint16_t bf16_t;  // bfloat16 storage (bit pattern)
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float bf16_to_f32(bf16_t v) {
  return __uint_as_float(static_cast<uint32_t>(v) << 16);
}

// float -> bfloat16, round to nearest even (the hardware conversion,
// v_cvt_pk_bf16_f32; inputs are finite).
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v;
  v.x = static_cast<__bf16>(lo);
  v.y = static_cast<__bf16>(hi);
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(bf16_t, static_cast<__bf16>(f));
}

// Element type traits for x / weights / y.
template <typename T> struct Elt;
template <> struct Elt<float> {
  static __device__ __forceinline__ float load(const float* p) { return *p; }
  static __device__ __forceinline__ float to_f32(float v) { return v; }
  static __device__ __forceinline__ float from_f32(float v) { return v; }
};
template <> struct Elt<bf16_t> {
  static __device__ __forceinline__ float load(const bf16_t* p) { return bf16_to_f32(*p); }
  static __device__ __forceinline__ float to_f32(bf16_t v) { return bf16_to_f32(v); }
  static __device__ __forceinline__ bf16_t from_f32(float v) { return f32_to_bf16(v); }
};

// Value of the lane O places along inside this lane's row of 16 (DPP
// row_ror; no trip through LDS).
template <int O>
__device__ __forceinline__ int row_ror(int v) {
  static_assert(O >= 1 && O <= 15, "row rotation");
  return __builtin_amdgcn_update_dpp(0, v, 0x120 + O, 0xF, 0xF, false);
}
template <int O>
__device__ __forceinline__ float row_ror(float v) {
  return __int_as_float(row_ror<O>(__float_as_int(v)));
}

// DPP lane permutations inside groups of 8: the mirror of the half row
// (lane i <- lane 7 - i) and the quad swaps (i <- i ^ 2, i <- i ^ 1).
template <int CTRL>
__device__ __forceinline__ int dpp_perm(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_perm(float v) {
  return __int_as_float(dpp_perm<CTRL>(__float_as_int(v)));
}
constexpr int kDppHalfMirror = 0x141, kDppQuadXor2 = 0x4E, kDppQuadXor1 = 0xB1;

// Reductions over aligned groups of W lanes (W a power of two <= 64): a
// butterfly over the offsets W/2, ..., 2, 1, each lane combining its value
// with that of lane i ^ o.  Groups of 16 (a DPP row) take the partner by a
// row rotation by o instead: before the step with offset o every lane
// already holds the same value as the lanes i ^ 2o, i ^ 4o, ..., so lane
// i + o (mod 16), whichever way the row turns, holds the value of lane
// i ^ o.  The combined operands, and so the results, are those of the xor
// shuffles bit for bit.  Groups of 8 (half a DPP row) first combine lane i
// with lane 7 - i, then take the quad swaps i ^ 2 and i ^ 1: after the
// first step lanes i and 7 - i hold the same pair, so every lane ends with
// the same two partial results combined (in one order or the other), and
// max, min and sum come out bit-identical on all 8 lanes.
template <int W>
__device__ __forceinline__ float group_max(float v) {
  if constexpr (W == 8) {
    v = fmaxf(v, dpp_perm<kDppHalfMirror>(v));
    v = fmaxf(v, dpp_perm<kDppQuadXor2>(v));
    return fmaxf(v, dpp_perm<kDppQuadXor1>(v));
  } else if constexpr (W == 16) {
    v = fmaxf(v, row_ror<8>(v));
    v = fmaxf(v, row_ror<4>(v));
    v = fmaxf(v, row_ror<2>(v));
    return fmaxf(v, row_ror<1>(v));
  } else {
#pragma unroll
    for (int o = W / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
  }
}
template <int W>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (W == 8) {
    v += dpp_perm<kDppHalfMirror>(v);
    v += dpp_perm<kDppQuadXor2>(v);
    return v + dpp_perm<kDppQuadXor1>(v);
  } else if constexpr (W == 16) {
    v += row_ror<8>(v);
    v += row_ror<4>(v);
    v += row_ror<2>(v);
    return v + row_ror<1>(v);
  } else {
#pragma unroll
    for (int o = W / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
  }
}
template <int W>
__device__ __forceinline__ int group_min_int(int v) {
  if constexpr (W == 8) {
    v = min(v, dpp_perm<kDppHalfMirror>(v));
    v = min(v, dpp_perm<kDppQuadXor2>(v));
    return min(v, dpp_perm<kDppQuadXor1>(v));
  } else if constexpr (W == 16) {
    v = min(v, row_ror<8>(v));
    v = min(v, row_ror<4>(v));
    v = min(v, row_ror<2>(v));
    return min(v, row_ror<1>(v));
  } else {
#pragma unroll
    for (int o = W / 2; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o, kWave));
    return v;
  }
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ float silu_f32(float a) { return a / (1.0f + __expf(-a)); }

}  // namespace moe
