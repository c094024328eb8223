// Log-sum-exp merge of split-KV partials (stage 2 of the decode step).
//
// Partition p of row (b, h) holds o_p, the softmax-weighted average of V over
// its positions, and lse_p = log2 sum_t exp(s_t) over the same positions.
// The full-row softmax average is sum_p 2^(lse_p - M) o_p / sum_p 2^(lse_p - M)
// with M = max_p lse_p: the plain softmax regrouped by partition, nothing
// approximated. Only the ceil(n / P) partitions that hold positions are read.
// One work-group per row, 4 consecutive output elements per thread.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_util.h"
#include "launch.h"

namespace attn {
namespace {

constexpr int kMergeThreads = 128;

__device__ __forceinline__ void store4(float* o, float a, float b, float c, float d) {
  *reinterpret_cast<float4*>(o) = make_float4(a, b, c, d);
}
__device__ __forceinline__ void store4(uint16_t* o, float a, float b, float c, float d) {
  uint2 u;
  u.x = (uint32_t)f32_to_bf16_rne(a) | ((uint32_t)f32_to_bf16_rne(b) << 16);
  u.y = (uint32_t)f32_to_bf16_rne(c) | ((uint32_t)f32_to_bf16_rne(d) << 16);
  *reinterpret_cast<uint2*>(o) = u;
}

template <typename TO>
__global__ __launch_bounds__(kMergeThreads) void lse_merge_kernel(
    const float* __restrict__ part_out, const float* __restrict__ part_lse,
    const int32_t* __restrict__ seq_lens, int H, int Dv, int T_max, int P, int NP,
    TO* __restrict__ out) {
  const int row = blockIdx.x;  // b * H + h
  const int b = row / H;
  const int n = min(max(seq_lens[b], 0), T_max);
  const int npv = n / P + (n % P != 0);
  const float* lse = part_lse + (size_t)row * NP;
  const float* po = part_out + (size_t)row * NP * Dv;
  TO* o = out + (size_t)row * Dv;

  float M = kNegInf;
  for (int p = 0; p < npv; ++p) M = fmaxf(M, lse[p]);
  float W = 0.f;
  for (int p = 0; p < npv; ++p) W += fast_exp2(lse[p] - M);

  for (int d = threadIdx.x * 4; d < Dv; d += kMergeThreads * 4) {
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
    for (int p = 0; p < npv; ++p) {
      const float w = fast_exp2(lse[p] - M);
      const float4 x = *reinterpret_cast<const float4*>(po + (size_t)p * Dv + d);
      a0 = fmaf(w, x.x, a0);
      a1 = fmaf(w, x.y, a1);
      a2 = fmaf(w, x.z, a2);
      a3 = fmaf(w, x.w, a3);
    }
    if (npv == 0) {
      store4(o + d, 0.f, 0.f, 0.f, 0.f);
    } else {
      store4(o + d, a0 / W, a1 / W, a2 / W, a3 / W);
    }
  }
}

}  // namespace

bool merge_supported(int out_dt, int Dv) {
  return (out_dt == 0 || out_dt == 1) && Dv >= 4 && Dv % 4 == 0 && Dv <= 1024;
}

hipError_t launch_merge(int out_dt, const float* part_out, const float* part_lse,
                        const int32_t* seq_lens, int B, int H, int Dv, int T_max, int P, int NP,
                        void* out, hipStream_t stream) {
  const dim3 grid((unsigned)B * (unsigned)H);
  if (out_dt == 0) {
    hipLaunchKernelGGL(lse_merge_kernel<float>, grid, dim3(kMergeThreads), 0, stream, part_out,
                       part_lse, seq_lens, H, Dv, T_max, P, NP, static_cast<float*>(out));
  } else {
    hipLaunchKernelGGL(lse_merge_kernel<uint16_t>, grid, dim3(kMergeThreads), 0, stream, part_out,
                       part_lse, seq_lens, H, Dv, T_max, P, NP, static_cast<uint16_t*>(out));
  }
  return hipGetLastError();
}

}  // namespace attn
