// Split-KV decode attention for the MHA / GQA / MQA family on gfx950.
//
// One work-group (4 wave64s) owns one (sequence b, KV head j, partition p)
// triple and streams the K and V rows of positions [p*P, min(p*P+P, n)) from
// HBM exactly once. Every row it loads serves all G = h_q / h_kv query heads
// of the group (query head i reads KV head i / G, "Attention variants: MQA,
// GQA, and MLA", section "GQA: interpolating with groups"), so the bytes
// streamed per step are the cache's own size, not G times it.
//
// Data layout in registers: one K (or V) row is D * sizeof(elem) bytes =
// LPR lanes x 16 bytes, so each 16-byte vector load instruction of a wave
// covers RPI = 64 / LPR consecutive rows, i.e. one contiguous 1 KiB span.
// Lane (rr, c) holds elements [c*EPL, c*EPL + EPL) of row rr of each span.
// Scores reduce over the LPR lanes of a row with DPP moves (no LDS traffic).
//
// Softmax is computed online in the exp2 domain (scores pre-multiplied by
// scale * log2(e)). The running maximum is only moved when a new block's
// maximum exceeds it by more than kTau = 8 (a factor 256 in the weights),
// so the rescale of the accumulators is rare; the weights stay <= 2^8 and
// the result is the same softmax (the common factor cancels in acc / l).
//
// Each partition writes its normalised partial output and log2-sum-exp; the
// merge kernel in lse_merge.hip combines partitions.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_util.h"
#include "launch.h"

namespace attn {
namespace {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

struct F32Elem {
  using storage = float;
  static constexpr int EPL = 4;  // elements per 16-byte lane chunk
  static __device__ __forceinline__ float get(const uint4& u, int e) { return __uint_as_float(word(u, e)); }
  static __device__ __forceinline__ float dot(const uint4& a, const uint4& b) {
    float s = __uint_as_float(a.x) * __uint_as_float(b.x);
    s = fmaf(__uint_as_float(a.y), __uint_as_float(b.y), s);
    s = fmaf(__uint_as_float(a.z), __uint_as_float(b.z), s);
    s = fmaf(__uint_as_float(a.w), __uint_as_float(b.w), s);
    return s;
  }
};

struct BF16Elem {
  using storage = uint16_t;
  static constexpr int EPL = 8;
  static __device__ __forceinline__ float get(const uint4& u, int e) {
    const uint32_t w = word(u, e >> 1);
    return (e & 1) ? bf16_hi(w) : bf16_lo(w);
  }
  // bf16 x bf16 products are exact in fp32; v_dot2 accumulates two per lane op.
  static __device__ __forceinline__ float dot(const uint4& a, const uint4& b) {
    float s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a.x), __builtin_bit_cast(bf16x2, b.x), 0.f, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a.y), __builtin_bit_cast(bf16x2, b.y), s, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a.z), __builtin_bit_cast(bf16x2, b.z), s, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a.w), __builtin_bit_cast(bf16x2, b.w), s, false);
    return s;
  }
};

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr float kTau = 8.0f;

template <class E, int D, int G>
__global__ __launch_bounds__(kThreads) void gqa_partial_kernel(
    const typename E::storage* __restrict__ q, const typename E::storage* __restrict__ kc,
    const typename E::storage* __restrict__ vc, const int32_t* __restrict__ seq_lens, int h_kv,
    int T_max, int P, int NP, float qk_scale_log2, float* __restrict__ part_out,
    float* __restrict__ part_lse) {
  constexpr int EPL = E::EPL;
  constexpr int LPR = D / EPL;       // lanes per row
  constexpr int RPI = 64 / LPR;      // rows per wave-wide 16-byte load
  constexpr int NI = G >= 16 ? 2 : (G >= 8 ? 4 : 8);  // loads per block per tensor (bounded by registers)
  constexpr int RB = NI * RPI;       // rows per block per wave

  const int p = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
  const int n = min(max(seq_lens[b], 0), T_max);
  const int start = p * P;
  if (start >= n) return;  // no position in this partition: nothing written, the merge skips it
  const int end = min(start, n - P) + P;  // = min(start + P, n) without overflow

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rr = lane / LPR, c = lane % LPR;
  const int H = h_kv * G;

  uint4 qv[G];
  const typename E::storage* qrow = q + ((size_t)b * H + (size_t)j * G) * D + c * EPL;
#pragma unroll
  for (int h = 0; h < G; ++h) qv[h] = ld16(qrow + (size_t)h * D);

  float m[G], l[G], acc[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = kNegInf;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
  }

  const size_t head_off = ((size_t)b * h_kv + j) * (size_t)T_max * D + (size_t)c * EPL;
  const typename E::storage* kb = kc + head_off;
  const typename E::storage* vb = vc + head_off;

  for (int r0 = start + wave * RB; r0 < end; r0 += kWaves * RB) {
    uint4 kr[NI], vr[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) kr[i] = ld16(kb + (size_t)min(r0 + i * RPI + rr, end - 1) * D);
#pragma unroll
    for (int i = 0; i < NI; ++i) vr[i] = ld16(vb + (size_t)min(r0 + i * RPI + rr, end - 1) * D);

    float s[NI][G];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const bool valid = r0 + i * RPI + rr < end;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float t = group_sum<LPR>(E::dot(qv[h], kr[i])) * qk_scale_log2;
        s[i][h] = valid ? t : kNegInf;
      }
    }

    bool need = false;
    float mb[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      mb[h] = s[0][h];
#pragma unroll
      for (int i = 1; i < NI; ++i) mb[h] = fmaxf(mb[h], s[i][h]);
      need |= mb[h] > m[h] + kTau;
    }
    if (__any(need)) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const bool nh = mb[h] > m[h] + kTau;
        const float f = nh ? fast_exp2(m[h] - mb[h]) : 1.f;
        m[h] = nh ? mb[h] : m[h];
        l[h] *= f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] *= f;
      }
    }

    float pr[NI][G];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        pr[i][h] = (s[i][h] == kNegInf) ? 0.f : fast_exp2(s[i][h] - m[h]);
        l[h] += pr[i][h];
      }
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const float x = E::get(vr[i], e);
#pragma unroll
        for (int h = 0; h < G; ++h) acc[h][e] = fmaf(pr[i][h], x, acc[h][e]);
      }
    }
  }

  // Combine the RPI row groups of this wave (lanes with equal c).
#pragma unroll
  for (int off = LPR; off < 64; off <<= 1) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mo = __shfl_xor(m[h], off, 64);
      const float lo = __shfl_xor(l[h], off, 64);
      const float M = fmaxf(m[h], mo);
      const float fa = (m[h] == kNegInf) ? 0.f : fast_exp2(m[h] - M);
      const float fb = (mo == kNegInf) ? 0.f : fast_exp2(mo - M);
      l[h] = l[h] * fa + lo * fb;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const float ao = __shfl_xor(acc[h][e], off, 64);
        acc[h][e] = acc[h][e] * fa + ao * fb;
      }
      m[h] = M;
    }
  }

  // Combine the waves through LDS and write this partition's partial.
  __shared__ float sm_acc[kWaves][G][D];
  __shared__ float sm_m[kWaves][G];
  __shared__ float sm_l[kWaves][G];
  if (lane < LPR) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) sm_acc[wave][h][c * EPL + e] = acc[h][e];
      if (c == 0) {
        sm_m[wave][h] = m[h];
        sm_l[wave][h] = l[h];
      }
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < G * D; idx += kThreads) {
    const int h = idx / D, d = idx % D;
    float M = sm_m[0][h];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, sm_m[w][h]);
    float L = 0.f, A = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = sm_m[w][h];
      const float f = (mw == kNegInf) ? 0.f : fast_exp2(mw - M);
      L += sm_l[w][h] * f;
      A += sm_acc[w][h][d] * f;
    }
    const size_t row = ((size_t)b * H + (size_t)j * G + h) * NP + p;
    part_out[row * D + d] = A / L;
    if (d == 0) part_lse[row] = M + fast_log2(L);
  }
}

template <class E, int D, int G>
hipError_t launch_one(const void* q, const void* k, const void* v, const int32_t* lens, int B,
                      int h_kv, int T_max, int P, int NP, float sc, float* po, float* pl,
                      hipStream_t stream) {
  using S = typename E::storage;
  dim3 grid(NP, h_kv, B);
  hipLaunchKernelGGL((gqa_partial_kernel<E, D, G>), grid, dim3(kThreads), 0, stream,
                     static_cast<const S*>(q), static_cast<const S*>(k), static_cast<const S*>(v),
                     lens, h_kv, T_max, P, NP, sc, po, pl);
  return hipGetLastError();
}

template <class E, int D>
hipError_t launch_d(int G, const void* q, const void* k, const void* v, const int32_t* lens, int B,
                    int h_kv, int T_max, int P, int NP, float sc, float* po, float* pl,
                    hipStream_t s) {
  switch (G) {
    case 1: return launch_one<E, D, 1>(q, k, v, lens, B, h_kv, T_max, P, NP, sc, po, pl, s);
    case 2: return launch_one<E, D, 2>(q, k, v, lens, B, h_kv, T_max, P, NP, sc, po, pl, s);
    case 4: return launch_one<E, D, 4>(q, k, v, lens, B, h_kv, T_max, P, NP, sc, po, pl, s);
    case 8: return launch_one<E, D, 8>(q, k, v, lens, B, h_kv, T_max, P, NP, sc, po, pl, s);
    case 16: return launch_one<E, D, 16>(q, k, v, lens, B, h_kv, T_max, P, NP, sc, po, pl, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool gqa_supported(int dt, int D, int group) {
  const bool g_ok = group == 1 || group == 2 || group == 4 || group == 8 || group == 16;
  return (dt == 0 || dt == 1) && (D == 64 || D == 128) && g_ok;
}

hipError_t launch_gqa_partial(int dt, int D, int group, const void* q, const void* k,
                              const void* v, const int32_t* lens, int B, int h_kv, int T_max,
                              int P, int NP, float sc, float* po, float* pl, hipStream_t s) {
  if (dt == 1) {
    if (D == 128) return launch_d<BF16Elem, 128>(group, q, k, v, lens, B, h_kv, T_max, P, NP, sc, po, pl, s);
    if (D == 64) return launch_d<BF16Elem, 64>(group, q, k, v, lens, B, h_kv, T_max, P, NP, sc, po, pl, s);
  } else if (dt == 0) {
    if (D == 128) return launch_d<F32Elem, 128>(group, q, k, v, lens, B, h_kv, T_max, P, NP, sc, po, pl, s);
    if (D == 64) return launch_d<F32Elem, 64>(group, q, k, v, lens, B, h_kv, T_max, P, NP, sc, po, pl, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace attn
