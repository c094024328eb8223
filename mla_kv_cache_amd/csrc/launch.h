// Kernel launchers behind the C ABI. Host code validates every argument before
// calling these; they only configure grids and enqueue on the given stream.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "support.h"

namespace attn {

// Arguments of the GQA partial kernels (passed by value as kernel arguments).
struct GqaArgs {
  const void* q;              // [B, h_q, D]
  const void* k;              // [B, h_kv, T_max, D]; written only in a decode step
  const void* v;
  const int32_t* seq_lens;    // [B]
  const void* k_new;          // decode step: [B, h_kv, D] rows appended at seq_lens[b]
  const void* v_new;          //   before attending; nullptr: plain decode
  int window;                 // > 0: attend over [max(0, n - window), n) only; 0: all of [0, n)
  // Paged cache (block_table != nullptr): k and v are [num_pages, h_kv, page_size, D] and
  // position t of sequence b is row t % page_size of page block_table[b * max_pages + t / page_size];
  // T_max = max_pages * page_size. page_size is a power of two.
  const int32_t* block_table;
  int page_size, page_shift, max_pages, num_pages;
  int B, h_kv, T_max, P, NP;
  float qk_scale_log2;        // scale * log2(e)
  float* part_out;            // [B, h_q, NP, D]
  float* part_lse;            // [B, h_q, NP]
  // Generic kernel only (set by its launcher): the query heads of a group are
  // taken in head_chunks work-groups of group / head_chunks heads each.
  int head_chunks;
  // Generic kernel with one partition (NP == 1) only: when out is set, the
  // kernel writes the finished rows to out [B, h_q, D] (bf16 when out_bf16,
  // else fp32; empty rows as zeros) instead of partials, and no merge runs.
  void* out;
  int out_bf16;
};

hipError_t launch_gqa_partial(int dt, int D, int group, const GqaArgs& a, hipStream_t stream);

// Split decode: the persistent kernel in split mode (bf16, gqa_persistent
// shapes). The work is cut into units of kSplitUnit positions of one
// (sequence, KV head) pair; `groups` work-groups each take an equal
// contiguous run of the units, and the run's part of each pair becomes one
// partial in slot (work-group + b * h_kv + j): part_out [groups + B*h_kv, G, D],
// part_lse [groups + B*h_kv, G]. a.P must be kSplitUnit; a.NP is not used.
constexpr int kSplitUnit = 128;
// Which kernel serves a bf16 shape (page_size 0: contiguous cache).
enum class BfKernel { kGeneric, kPo, kMma16, kMatrix };
BfKernel bf16_kernel(int D, int group, int page_size);
// Work-groups of the split launch on the current device (0: no split for this
// shape), and the most any page size of the shape can use (the plan's bound).
int gqa_split_groups(int D, int group, int page_size);
int gqa_split_groups_max(int D, int group);
hipError_t launch_gqa_split(int D, int group, const GqaArgs& a, int groups, hipStream_t stream);

// The matrix-core kernel for bf16 groups of 16 to 128 heads (gqa_matrix.hip):
// work-groups of a split launch on the current device, and the launch itself
// (split: the work-balanced split with `groups` work-groups; otherwise fixed
// partitions of a.P positions, groups <= 0 picks the resident count).
int gqa_matrix_groups(int D, int group);
hipError_t launch_gqa_matrix(int D, int group, const GqaArgs& a, int groups, bool split, hipStream_t stream);

// The 16 x 16 matrix-core kernel for bf16 groups of 1 to 64 heads
// (gqa_mma16.hip): positions per tile for a group size, work-groups of a
// split launch, and the launch (same conventions as launch_gqa_matrix).
int gqa_mma16_tile(int group);
int gqa_mma16_groups(int D, int group);
hipError_t launch_gqa_mma16(int D, int group, const GqaArgs& a, int groups, bool split, hipStream_t stream);
// Merge of the split partials into out [B, h_kv * group, D].
hipError_t launch_split_merge(int out_dt, const float* part_out, const float* part_lse,
                              const int32_t* seq_lens, int len_add, int window, int B, int h_kv,
                              int group, int D, int T_max, int groups, void* out, hipStream_t stream);

// Plain copy of the new K/V rows into the caches (the decode step's write alone).
hipError_t launch_kv_append(int dt, const void* k_new, const void* v_new, void* k, void* v,
                            const int32_t* seq_lens, int B, int h_kv, int D, int T_max,
                            hipStream_t stream);

// len_add = 1 for a decode step: each row attends over min(max(seq_lens[b], 0) + 1, T_max)
// positions instead of min(max(seq_lens[b], 0), T_max). window > 0: only the last
// `window` of those positions, partitioned from the first of them.
hipError_t launch_merge(int out_dt, const float* part_out, const float* part_lse,
                        const int32_t* seq_lens, int len_add, int window, int B, int H, int Dv,
                        int T_max, int P, int NP, void* out, hipStream_t stream);

struct MlaArgs {
  const void* q_nope;         // [B, H, 512]
  const void* q_rope;         // [B, H, 64]
  const void* latent;         // [B, T_max, 576]; written only in a decode step
  const int32_t* seq_lens;    // [B]
  const void* lat_new;        // decode step: [B, 576] rows appended at seq_lens[b]; nullptr: plain decode
  // Paged cache (block_table != nullptr): latent is [num_pages, page_size, 576], page_size a
  // power of two >= 32; position t of sequence b is row t % page_size of page
  // block_table[b * max_pages + t / page_size]; T_max = max_pages * page_size.
  const int32_t* block_table;
  int page_size, page_shift, max_pages, num_pages;
  int B, H, T_max, P, NP;
  float qk_scale_log2;
  float* part_out;            // [B, H, NP, 512]
  float* part_lse;            // [B, H, NP]
};

hipError_t launch_mla_partial(const MlaArgs& a, hipStream_t stream);

hipError_t launch_latent_append(const void* lat_new, void* latent, const int32_t* seq_lens,
                                int B, int row_elems, int T_max, hipStream_t stream);

// Paged forms of the appends: the new row of sequence b goes to row pos % page_size of
// page block_table[b * max_pages + pos / page_size], pos = max(seq_lens[b], 0), unless
// pos >= max_pages * page_size or that table entry lies outside [0, num_pages).
// rows_per_page_row: h_kv for KV pages ([num_pages, h_kv, page_size, row]), 1 for latent pages.
hipError_t launch_append_paged(const void* new_a, const void* new_b, void* pages_a, void* pages_b,
                               const int32_t* block_table, const int32_t* seq_lens, int B,
                               int heads, int row_bytes, int page_size, int max_pages,
                               int num_pages, hipStream_t stream);

// MLA absorption products (bf16 in, fp32 accumulation, bf16 out).
hipError_t launch_absorb_q(const void* q, const void* w_uk, void* q_lat, int B, int H, int d_h,
                           int d_c, hipStream_t stream);
hipError_t launch_up_v(const void* o_lat, const void* w_uv, void* out, int B, int H, int d_c,
                       int d_v, hipStream_t stream);

}  // namespace attn
