// Log-sum-exp merge of split-KV partials (stage 2 of the decode step).
//
// Partition p of row (b, h) holds o_p, the softmax-weighted average of V over
// its positions, and lse_p = log2 sum_t exp(s_t) over the same positions.
// The full-row softmax average is sum_p 2^(lse_p - M) o_p / sum_p 2^(lse_p - M)
// with M = max_p lse_p: the plain softmax regrouped by partition, nothing
// approximated. Only the partitions that hold positions are read: ceil(n / P),
// or ceil(min(n, window) / P) for a sliding window.
//
// One wave per row, four rows per work-group. Lane l owns VW consecutive
// output elements of each 64*VW-wide slice of the row; the partitions are
// walked eight (then four) at a time with independent loads so that several
// partials of a lane are in flight together. M and the normaliser come from a wave-wide
// pass over the log-sum-exps; each partition's weight is then recomputed
// from its (wave-uniform) log-sum-exp where it is used.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_util.h"
#include "launch.h"

namespace attn {
namespace {

constexpr int kRowsPerGroup = 4;

template <int VW>
struct Vec;
template <>
struct Vec<1> {
  typedef float type;
  static __device__ __forceinline__ float get(const type& v, int i) { (void)i; return v; }
};
template <>
struct Vec<2> {
  typedef float2 type;
  static __device__ __forceinline__ float get(const type& v, int i) { return i == 0 ? v.x : v.y; }
};
template <>
struct Vec<4> {
  typedef float4 type;
  static __device__ __forceinline__ float get(const type& v, int i) {
    return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
  }
};

template <int VW>
__device__ __forceinline__ void store_out(float* o, const float (&x)[VW]) {
#pragma unroll
  for (int i = 0; i < VW; ++i) o[i] = x[i];
}
// bf16 output: the merged rows are read by the caller's next kernel, not by
// this step's, so they are written non-temporally; cached dirty copies were
// written back while the next decode kernel streamed its cache.
template <int VW>
__device__ __forceinline__ void store_out(uint16_t* o, const float (&x)[VW]) {
  if constexpr (VW == 4) {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 v = {(uint32_t)f32_to_bf16_rne(x[0]) | ((uint32_t)f32_to_bf16_rne(x[1]) << 16),
                     (uint32_t)f32_to_bf16_rne(x[2]) | ((uint32_t)f32_to_bf16_rne(x[3]) << 16)};
    __builtin_nontemporal_store(v, reinterpret_cast<u32x2*>(o));
  } else if constexpr (VW == 2) {
    __builtin_nontemporal_store((uint32_t)f32_to_bf16_rne(x[0]) | ((uint32_t)f32_to_bf16_rne(x[1]) << 16),
                                reinterpret_cast<uint32_t*>(o));
  } else {
#pragma unroll
    for (int i = 0; i < VW; ++i) __builtin_nontemporal_store(f32_to_bf16_rne(x[i]), o + i);
  }
}

template <typename TO, int VW>
__global__ __launch_bounds__(64 * kRowsPerGroup) void lse_merge_kernel(
    const float* __restrict__ part_out, const float* __restrict__ part_lse,
    const int32_t* __restrict__ seq_lens, int len_add, int window, int rows, int H, int Dv,
    int T_max, int P, int NP, TO* __restrict__ out) {
  using V = Vec<VW>;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row = blockIdx.x * kRowsPerGroup + wave;  // b * H + h, uniform in the wave
  if (row >= rows) return;
  const int b = row / H;
  const float* lse = part_lse + (size_t)row * NP;
  const float* po = part_out + (size_t)row * NP * Dv;
  TO* o = out + (size_t)row * Dv;

  // Up to four partitions and one or two 64 VW-wide slices per row (the MLA
  // decode: four partitions of 512 values): every load of the row (its
  // sequence length, the log-sum-exps, all partials, also of partitions past
  // the row's valid ones) is issued at once, then the valid ones are combined
  // in exactly the order of the general path below, so the bits are the same.
  if (NP <= 4 && (Dv == 64 * VW || Dv == 128 * VW)) {
    const int len = seq_lens[b];
    const float lsv = lane < NP ? lse[lane] : kNegInf;
    typename V::type x[2][4];
#pragma unroll
    for (int sl = 0; sl < 2; ++sl)
#pragma unroll
      for (int p = 0; p < 4; ++p)
        if (p < NP && sl * 64 * VW < Dv)
          x[sl][p] = *reinterpret_cast<const typename V::type*>(po + (size_t)p * Dv + sl * 64 * VW + lane * VW);
    const int n = attended_len(len, len_add, T_max);
    const int span = n - window_lo(n, window);
    const int npv = span / P + (span % P != 0);
    float M = kNegInf;
    if (lane < npv) M = fmaxf(M, lsv);
    M = wave_max(M);
    float W = 0.f;
    if (lane < npv) W += fast_exp2(lsv - M);
    const float invW = 1.f / wave_sum(W);
    float wp[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) wp[p] = fast_exp2(__shfl(lsv, p, 64) - M) * invW;
#pragma unroll
    for (int sl = 0; sl < 2; ++sl) {
      if (sl * 64 * VW >= Dv) break;
      float acc[4][VW];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int i = 0; i < VW; ++i) acc[u][i] = 0.f;
      if (npv == 4) {  // the general path's four-at-a-time step
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int i = 0; i < VW; ++i) acc[u][i] = fmaf(wp[u], V::get(x[sl][u], i), acc[u][i]);
      } else {         // its one-at-a-time tail
#pragma unroll
        for (int p = 0; p < 3; ++p)
          if (p < npv)
#pragma unroll
            for (int i = 0; i < VW; ++i) acc[0][i] = fmaf(wp[p], V::get(x[sl][p], i), acc[0][i]);
      }
      float r[VW];
#pragma unroll
      for (int i = 0; i < VW; ++i) r[i] = (acc[0][i] + acc[1][i]) + (acc[2][i] + acc[3][i]);
      store_out<VW>(o + sl * 64 * VW + lane * VW, r);
    }
    return;
  }

  const int n = attended_len(seq_lens[b], len_add, T_max);
  const int span = n - window_lo(n, window);
  const int npv = span / P + (span % P != 0);

  float M = kNegInf;
  for (int p = lane; p < npv; p += 64) M = fmaxf(M, lse[p]);
  M = wave_max(M);
  float W = 0.f;
  for (int p = lane; p < npv; p += 64) W += fast_exp2(lse[p] - M);
  const float invW = 1.f / wave_sum(W);

  for (int d0 = lane * VW; d0 < Dv; d0 += 64 * VW) {
    float acc[4][VW];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int i = 0; i < VW; ++i) acc[u][i] = 0.f;
    int p = 0;
    // Eight partitions at a time: their loads are independent, so a row's
    // partials arrive in one or two memory round trips, not one per four.
    for (; p + 8 <= npv; p += 8) {
      typename V::type x[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        x[u] = *reinterpret_cast<const typename V::type*>(po + (size_t)(p + u) * Dv + d0);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float w = fast_exp2(lse[p + u] - M) * invW;
#pragma unroll
        for (int i = 0; i < VW; ++i) acc[u & 3][i] = fmaf(w, V::get(x[u], i), acc[u & 3][i]);
      }
    }
    for (; p + 4 <= npv; p += 4) {
      typename V::type x[4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        x[u] = *reinterpret_cast<const typename V::type*>(po + (size_t)(p + u) * Dv + d0);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float w = fast_exp2(lse[p + u] - M) * invW;
#pragma unroll
        for (int i = 0; i < VW; ++i) acc[u][i] = fmaf(w, V::get(x[u], i), acc[u][i]);
      }
    }
    for (; p < npv; ++p) {
      const typename V::type x = *reinterpret_cast<const typename V::type*>(po + (size_t)p * Dv + d0);
      const float w = fast_exp2(lse[p] - M) * invW;
#pragma unroll
      for (int i = 0; i < VW; ++i) acc[0][i] = fmaf(w, V::get(x, i), acc[0][i]);
    }
    float r[VW];
#pragma unroll
    for (int i = 0; i < VW; ++i) r[i] = (acc[0][i] + acc[1][i]) + (acc[2][i] + acc[3][i]);
    store_out<VW>(o + d0, r);  // npv == 0: the sums are empty and the row is zeros
  }
}

template <typename TO>
hipError_t launch_typed(const float* part_out, const float* part_lse, const int32_t* seq_lens,
                        int len_add, int window, int B, int H, int Dv, int T_max, int P, int NP,
                        TO* out, hipStream_t stream) {
  const int rows = B * H;
  const dim3 grid((unsigned)((rows + kRowsPerGroup - 1) / kRowsPerGroup));
  const dim3 block(64 * kRowsPerGroup);
  if (Dv % 256 == 0)
    hipLaunchKernelGGL((lse_merge_kernel<TO, 4>), grid, block, 0, stream, part_out, part_lse,
                       seq_lens, len_add, window, rows, H, Dv, T_max, P, NP, out);
  else if (Dv % 128 == 0)
    hipLaunchKernelGGL((lse_merge_kernel<TO, 2>), grid, block, 0, stream, part_out, part_lse,
                       seq_lens, len_add, window, rows, H, Dv, T_max, P, NP, out);
  else
    hipLaunchKernelGGL((lse_merge_kernel<TO, 1>), grid, block, 0, stream, part_out, part_lse,
                       seq_lens, len_add, window, rows, H, Dv, T_max, P, NP, out);
  return hipGetLastError();
}

__device__ __forceinline__ long long wave_sum_i64(long long x) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) x += __shfl_xor(x, off, 64);
  return x;
}

// Units (of kSplitUnit positions) of sequence b in a split decode.
__device__ __forceinline__ long long split_units(const int32_t* seq_lens, int b, int len_add, int window,
                                                 int T_max) {
  const int n = attended_len(seq_lens[b], len_add, T_max);
  return (n - window_lo(n, window) + kSplitUnit - 1) / kSplitUnit;
}

// Merge of the split partials (stage 2 of a split decode). Row (b, h) belongs
// to pair pi = b * h_kv + h / G, whose units are [base, base + units) of the
// U units of the launch (pairs in order, b-major). Work-group w of the NW
// split work-groups held units [U w / NW, U (w + 1) / NW) and wrote the
// partial of its share of each pair to slot w + pi, so the pair's partials
// are the slots of the work-groups from the one holding unit base to the one
// holding unit base + units - 1, leaving out work-groups whose run was empty
// (only when U < NW). The merge itself is the same log-sum-exp regrouping as
// for fixed partitions. One wave per row, four rows per work-group.
// Slots per row whose partial rows the merge requests up front.
constexpr int kPreSlots = 16;

template <typename TO, int VW>
__global__ __launch_bounds__(64 * kRowsPerGroup) void split_merge_kernel(
    const float* __restrict__ part_out, const float* __restrict__ part_lse,
    const int32_t* __restrict__ seq_lens, int len_add, int window, int B, int h_kv, int G, int Dv,
    int T_max, int NW, TO* __restrict__ out) {
  using V = Vec<VW>;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int H = h_kv * G;
  const int row = blockIdx.x * kRowsPerGroup + wave;  // b * H + h, uniform in the wave
  if (row >= B * H) return;
  const int b = row / H, h = row % H, j = h / G, hh = h % G;
  TO* o = out + (size_t)row * Dv;

  long long before = 0, total = 0;  // units of the sequences before b, of all sequences
  for (int b0 = 0; b0 < B; b0 += 64) {
    const int bb = b0 + lane;
    const long long u = bb < B ? split_units(seq_lens, bb, len_add, window, T_max) : 0;
    total += wave_sum_i64(u);
    before += wave_sum_i64(bb < b ? u : 0);
  }
  const long long units = split_units(seq_lens, b, len_add, window, T_max);
  if (units == 0) {  // nothing attended: the row is zeros
    float z[VW];
#pragma unroll
    for (int i = 0; i < VW; ++i) z[i] = 0.f;
    for (int d0 = lane * VW; d0 < Dv; d0 += 64 * VW) store_out<VW>(o + d0, z);
    return;
  }
  const long long U = total * h_kv;
  const long long base = before * h_kv + (long long)j * units;
  // Work-group holding unit u: the largest w with U w / NW <= u.
  auto holder = [&](long long u) { return (int)(((u + 1) * NW - 1) / U); };
  auto held = [&](int w) { return U * (w + 1) / NW > U * w / NW; };
  const int w0 = holder(base), w1 = holder(base + units - 1);
  const long long pi = (long long)b * h_kv + j;
  const int ns = w1 - w0 + 1;
  auto slot_row = [&](int s) { return ((size_t)(w0 + s + pi) * G + hh); };

  // Common case: few slots and one Dv chunk per lane. The rows are requested
  // together with the slot lse values (one lane per slot), not after the
  // maximum and the sum, which saves one round trip to memory.
  if (ns <= kPreSlots && Dv == 64 * VW) {
    const int d0 = lane * VW;
    // Slot `lane` is written when its work-group holds a unit (64-bit
    // divisions: evaluated once per slot, then shared as a mask).
    const bool hl = lane < ns && (U >= NW || held(w0 + lane));
    const uint64_t hm = __ballot(hl);
    typename V::type x[kPreSlots];
#pragma unroll
    for (int s = 0; s < kPreSlots; ++s)
      if ((hm >> s) & 1) x[s] = *reinterpret_cast<const typename V::type*>(part_out + slot_row(s) * Dv + d0);
    const float ls = hl ? part_lse[slot_row(lane)] : kNegInf;
    const float Mx = wave_max(ls);
    const float e = ls == kNegInf ? 0.f : fast_exp2(ls - Mx);
    const float inv = 1.f / wave_sum(e);
    float acc[4][VW];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int i = 0; i < VW; ++i) acc[u][i] = 0.f;
#pragma unroll
    for (int s = 0; s < kPreSlots; ++s) {
      if ((hm >> s) & 1) {
        const float w = __shfl(e, s, 64) * inv;
#pragma unroll
        for (int i = 0; i < VW; ++i) acc[s % 4][i] = fmaf(w, V::get(x[s], i), acc[s % 4][i]);
      }
    }
    float r[VW];
#pragma unroll
    for (int i = 0; i < VW; ++i) r[i] = (acc[0][i] + acc[1][i]) + (acc[2][i] + acc[3][i]);
    store_out<VW>(o + d0, r);
    return;
  }

  float M = kNegInf;
  for (int s = lane; s < ns; s += 64)
    if (held(w0 + s)) M = fmaxf(M, part_lse[slot_row(s)]);
  M = wave_max(M);
  float W = 0.f;
  for (int s = lane; s < ns; s += 64)
    if (held(w0 + s)) W += fast_exp2(part_lse[slot_row(s)] - M);
  const float invW = 1.f / wave_sum(W);

  for (int d0 = lane * VW; d0 < Dv; d0 += 64 * VW) {
    float acc[4][VW];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int i = 0; i < VW; ++i) acc[u][i] = 0.f;
    int s = 0;
    if (U >= NW) {  // every run holds at least one unit: all slots in [w0, w1] are written
      for (; s + 4 <= ns; s += 4) {
        typename V::type x[4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
          x[u] = *reinterpret_cast<const typename V::type*>(part_out + slot_row(s + u) * Dv + d0);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float w = fast_exp2(part_lse[slot_row(s + u)] - M) * invW;
#pragma unroll
          for (int i = 0; i < VW; ++i) acc[u][i] = fmaf(w, V::get(x[u], i), acc[u][i]);
        }
      }
    }
    for (; s < ns; ++s) {
      if (!held(w0 + s)) continue;
      const typename V::type x = *reinterpret_cast<const typename V::type*>(part_out + slot_row(s) * Dv + d0);
      const float w = fast_exp2(part_lse[slot_row(s)] - M) * invW;
#pragma unroll
      for (int i = 0; i < VW; ++i) acc[0][i] = fmaf(w, V::get(x, i), acc[0][i]);
    }
    float r[VW];
#pragma unroll
    for (int i = 0; i < VW; ++i) r[i] = (acc[0][i] + acc[1][i]) + (acc[2][i] + acc[3][i]);
    store_out<VW>(o + d0, r);
  }
}

template <typename TO>
hipError_t launch_split_typed(const float* part_out, const float* part_lse, const int32_t* seq_lens,
                              int len_add, int window, int B, int h_kv, int G, int Dv, int T_max,
                              int NW, TO* out, hipStream_t stream) {
  const long long rows = (long long)B * h_kv * G;
  if ((rows + kRowsPerGroup - 1) / kRowsPerGroup > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)((rows + kRowsPerGroup - 1) / kRowsPerGroup));
  const dim3 block(64 * kRowsPerGroup);
  if (Dv % 128 == 0)
    hipLaunchKernelGGL((split_merge_kernel<TO, 2>), grid, block, 0, stream, part_out, part_lse, seq_lens,
                       len_add, window, B, h_kv, G, Dv, T_max, NW, out);
  else
    hipLaunchKernelGGL((split_merge_kernel<TO, 1>), grid, block, 0, stream, part_out, part_lse, seq_lens,
                       len_add, window, B, h_kv, G, Dv, T_max, NW, out);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_split_merge(int out_dt, const float* part_out, const float* part_lse,
                              const int32_t* seq_lens, int len_add, int window, int B, int h_kv,
                              int group, int D, int T_max, int groups, void* out, hipStream_t stream) {
  if (groups < 1) return hipErrorInvalidValue;
  if (out_dt == 0)
    return launch_split_typed(part_out, part_lse, seq_lens, len_add, window, B, h_kv, group, D, T_max,
                              groups, static_cast<float*>(out), stream);
  return launch_split_typed(part_out, part_lse, seq_lens, len_add, window, B, h_kv, group, D, T_max,
                            groups, static_cast<uint16_t*>(out), stream);
}

hipError_t launch_merge(int out_dt, const float* part_out, const float* part_lse,
                        const int32_t* seq_lens, int len_add, int window, int B, int H, int Dv,
                        int T_max, int P, int NP, void* out, hipStream_t stream) {
  if (out_dt == 0)
    return launch_typed(part_out, part_lse, seq_lens, len_add, window, B, H, Dv, T_max, P, NP,
                        static_cast<float*>(out), stream);
  return launch_typed(part_out, part_lse, seq_lens, len_add, window, B, H, Dv, T_max, P, NP,
                      static_cast<uint16_t*>(out), stream);
}

}  // namespace attn
