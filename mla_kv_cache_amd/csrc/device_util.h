// Device helpers shared by the decode kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

constexpr float kNegInf = -__builtin_huge_valf();

// 16-byte vector load / store. Every call site guarantees 16-byte alignment.
__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

__device__ __forceinline__ uint32_t word(const uint4& u, int i) {
  return i == 0 ? u.x : (i == 1 ? u.y : (i == 2 ? u.z : u.w));
}

// bf16 halves of a packed word widened to fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Data-parallel-primitive lane moves inside a 16-lane row.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7-i inside each 8-lane half row
constexpr int kDppMirror = 0x140;     // lane i <-> 15-i inside each 16-lane row

// Sum over aligned groups of LPR consecutive lanes (LPR in {8, 16, 32}); every
// lane of a group ends with the group's total.
template <int LPR>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(LPR == 8 || LPR == 16 || LPR == 32, "unsupported group width");
  x += dpp_mov<kDppXor1>(x);
  x += dpp_mov<kDppXor2>(x);
  x += dpp_mov<kDppHalfMirror>(x);
  if constexpr (LPR >= 16) x += dpp_mov<kDppMirror>(x);
  if constexpr (LPR >= 32) x += __shfl_xor(x, 16, 64);
  return x;
}

}  // namespace attn
