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

// Word 3 of a raw buffer resource on gfx9-family parts (32-bit data format,
// no swizzle, no stride): loads at or past num_records bytes return zeros.
constexpr int kBufWord3 = 0x00020000;
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

// Value held by lane l ^ 16 (v_permlane16_swap) and by lane l ^ 32
// (v_permlane32_swap). Each swap leaves a lane with its own value and its
// partner's, in an order that depends on the lane's half; max and sum do not
// care about the order.
__device__ __forceinline__ float xor16_max(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor16_sum(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Maximum / sum over all 64 lanes; every lane ends with the result.
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp_mov<kDppXor1>(x));
  x = fmaxf(x, dpp_mov<kDppXor2>(x));
  x = fmaxf(x, dpp_mov<kDppHalfMirror>(x));
  x = fmaxf(x, dpp_mov<kDppMirror>(x));
  return xor32_max(xor16_max(x));
}
__device__ __forceinline__ float wave_sum(float x) {
  x += dpp_mov<kDppXor1>(x);
  x += dpp_mov<kDppXor2>(x);
  x += dpp_mov<kDppHalfMirror>(x);
  x += dpp_mov<kDppMirror>(x);
  return xor32_sum(xor16_sum(x));
}

// Cache policy of the cache streams (K and V rows, latent rows, projection
// weights): non-temporal. Every byte of a stream is read once per call, so
// nothing is gained by keeping it in the L2 or the last-level cache. A plain
// read of 1 GiB on MI355X streams at 6.0-6.4 TB/s with the default policy and
// at 6.7-7.1 TB/s with this one; the decode kernels run 10-13% faster with it,
// with unchanged results. In inline assembly the policy is the `nt` modifier;
// in the buffer load builtins it is this cache-policy operand.
constexpr int kLoadNonTemporal = 2;

// 16-byte vector load with the non-temporal policy.
__device__ __forceinline__ uint4 ld16_nt(const void* p) {
  typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
  const u32x4_t v = __builtin_nontemporal_load(static_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// 16-byte vector store. Every call site guarantees 16-byte alignment.
__device__ __forceinline__ void st16(void* p, const uint4& v) { *reinterpret_cast<uint4*>(p) = v; }

// Number of positions a row attends over. seq_len is the cached length
// (before the step when len_add = 1, a decode step that appends one row at
// position max(seq_len, 0) when that position is below T_max).
__device__ __forceinline__ int attended_len(int seq_len, int len_add, int T_max) {
  const int pos = max(seq_len, 0);
  return pos >= T_max ? T_max : min(pos + len_add, T_max);
}

// First attended position of a row of n positions (sliding window when window > 0).
__device__ __forceinline__ int window_lo(int n, int window) { return window > 0 ? max(0, n - window) : 0; }

// Decode step: copy one new cache row (ROW_BYTES, a multiple of 16) with the
// threads of the work-group, then make it visible to every later read of the
// same work-group (loads through the vector L1 and direct-to-LDS copies).
// Writer and readers share one CU and its L1, so the work-group-scope release
// and acquire around the barrier are enough; an agent-scope fence would write
// back and invalidate the whole L2 of the XCD. No other work-group reads the
// row in the same launch. Call from uniform control flow.
template <int ROW_BYTES>
__device__ __forceinline__ void write_row_then_sync(void* dst, const void* src) {
  static_assert(ROW_BYTES % 16 == 0, "rows are copied in 16-byte pieces");
  for (int i = threadIdx.x; i < ROW_BYTES / 16; i += blockDim.x)
    st16(static_cast<unsigned char*>(dst) + 16 * i, ld16(static_cast<const unsigned char*>(src) + 16 * i));
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const unsigned char*)p;
}

}  // namespace attn
