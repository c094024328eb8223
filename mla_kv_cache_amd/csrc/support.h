// Which shapes the kernels are built for. Host-only predicates, shared by the
// argument checks of the C ABI and by the launchers (plain C++, no device code).
#pragma once

namespace attn {

inline bool pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

// dt: 0 = fp32 storage, 1 = bf16 storage (values of attn_dtype).
// GQA / MHA / MQA: head dim 64 or 128, group size g = h_q / h_kv any of 1 to
// 8 or a power of two up to 128 (h_kv = 1 with up to 128 query heads is MQA).
inline bool gqa_group_supported(int group) { return (group >= 1 && group <= 8) || (pow2(group) && group <= 128); }
inline bool gqa_supported(int dt, int D, int group) {
  return (dt == 0 || dt == 1) && (D == 64 || D == 128) && gqa_group_supported(group);
}

// The bf16 persistent position-per-lane kernel: groups of up to 8 heads.
inline bool gqa_persistent(int dt, int D, int group) {
  return dt == 1 && (D == 64 || D == 128) && pow2(group) && group <= 8;
}

// The bf16 matrix-core kernel: groups of 16 to 128 heads share each K/V tile.
inline bool gqa_matrix(int dt, int D, int group) {
  return dt == 1 && (D == 64 || D == 128) && pow2(group) && group >= 16 && group <= 128;
}

// Merge of split partials: any row width that is a multiple of 4 up to 1024.
inline bool merge_supported(int out_dt, int Dv) {
  return (out_dt == 0 || out_dt == 1) && Dv >= 4 && Dv % 4 == 0 && Dv <= 1024;
}

// Absorbed MLA: (d_c, d_r) = (512, 64); heads in tiles of 32, at most 128 per
// work-group (any multiple of 128 runs as several blocks).
inline bool mla_supported(int H, int d_c, int d_r) {
  return d_c == 512 && d_r == 64 && H >= 32 && H % 32 == 0 && (H <= 128 || H % 128 == 0);
}

// MLA absorption products on 32x32x16 matrix-core tiles.
inline bool absorb_supported(int d_h, int d_c) { return d_h >= 16 && d_h % 16 == 0 && d_c >= 32 && d_c % 32 == 0; }
inline bool up_supported(int d_c, int d_v) { return d_c >= 16 && d_c % 16 == 0 && d_v >= 32 && d_v % 32 == 0; }

}  // namespace attn
