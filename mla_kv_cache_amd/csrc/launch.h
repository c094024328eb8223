// Kernel launchers behind the C ABI. Host code validates every argument before
// calling these; they only configure grids and enqueue on the given stream.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

// dt: 0 = fp32 storage, 1 = bf16 storage (values of attn_dtype).
bool gqa_supported(int dt, int D, int group);

hipError_t launch_gqa_partial(int dt, int D, int group, const void* q, const void* k,
                              const void* v, const int32_t* seq_lens, int B, int h_kv,
                              int T_max, int P, int NP, float qk_scale_log2,
                              float* part_out, float* part_lse, hipStream_t stream);

bool merge_supported(int out_dt, int Dv);

hipError_t launch_merge(int out_dt, const float* part_out, const float* part_lse,
                        const int32_t* seq_lens, int B, int H, int Dv, int T_max, int P,
                        int NP, void* out, hipStream_t stream);

bool mla_supported(int H, int d_c, int d_r);

hipError_t launch_mla_partial(const void* q_nope, const void* q_rope, const void* latent,
                              const int32_t* seq_lens, int B, int H, int T_max, int P, int NP,
                              float qk_scale_log2, float* part_out, float* part_lse,
                              hipStream_t stream);

}  // namespace attn
