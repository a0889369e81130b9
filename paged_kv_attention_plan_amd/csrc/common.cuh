// Small device helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace pkv {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// bf16 halves of a packed 32-bit word, widened exactly to fp32.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 with round-to-nearest-even (finite inputs).
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return bf16_rne(lo) | (bf16_rne(hi) << 16);
}

// fp32 pair -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t cvt_bf16x2(float lo, float hi) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// acc + a.lo*b.lo + a.hi*b.hi on packed bf16 pairs (v_dot2_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), acc, false);
}

// DPP lane moves inside a row of 16 lanes.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL,
                                                            0xf, 0xf, true));
}
constexpr int kDppQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;
constexpr int kDppRowRor4 = 0x124;      // row_ror:4
constexpr int kDppRowRor8 = 0x128;      // row_ror:8 (lane i <-> lane i ^ 8 within the row)

// Lane SRC (0..15) of each row of 16 lanes, to every lane of that row
// (DPP row_newbcast).
template <int SRC>
__device__ __forceinline__ uint32_t row_bcast(uint32_t x) {
  static_assert(SRC >= 0 && SRC < 16, "row lane");
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x150 + SRC, 0xf, 0xf, true);
}
// The same with the lane given at run time: after unrolling it is a constant,
// and the switch folds to one move.
__device__ __forceinline__ uint32_t bcast16u(uint32_t x, int src) {
  switch (src) {
    case 0: return row_bcast<0>(x);    case 1: return row_bcast<1>(x);
    case 2: return row_bcast<2>(x);    case 3: return row_bcast<3>(x);
    case 4: return row_bcast<4>(x);    case 5: return row_bcast<5>(x);
    case 6: return row_bcast<6>(x);    case 7: return row_bcast<7>(x);
    case 8: return row_bcast<8>(x);    case 9: return row_bcast<9>(x);
    case 10: return row_bcast<10>(x);  case 11: return row_bcast<11>(x);
    case 12: return row_bcast<12>(x);  case 13: return row_bcast<13>(x);
    case 14: return row_bcast<14>(x);  default: return row_bcast<15>(x);
  }
}
__device__ __forceinline__ float bcast16(float x, int src) {
  return __builtin_bit_cast(float, bcast16u(__builtin_bit_cast(uint32_t, x), src));
}

// Sum over groups of N consecutive lanes (N = 4, 8 or 16); every lane of a
// group receives the group's sum.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  x += dpp<kDppQuadXor1>(x);
  x += dpp<kDppQuadXor2>(x);
  if constexpr (N >= 8) x += dpp<kDppRowHalfMirror>(x);
  if constexpr (N >= 16) x += dpp<kDppRowMirror>(x);
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// 16-byte load marked non-temporal (streamed once: keeps the caches for other data).
__device__ __forceinline__ uint4 load_nt16(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

constexpr float kLn2 = 0.69314718055994530942f;

// Read-only data viewed through the constant address space: uniform loads from
// it go through the scalar unit (s_load), whatever else the kernel does.
template <typename T>
using const_as4_ptr = const __attribute__((address_space(4))) T*;

template <typename T>
__device__ __forceinline__ const_as4_ptr<T> as_const4(const T* p) {
  return reinterpret_cast<const_as4_ptr<T>>(reinterpret_cast<uintptr_t>(p));
}

}  // namespace pkv
