// Host side of the C ABI declared in include/attn_decode.h: argument checks,
// the split-KV plan, workspace layout and kernel dispatch. Every check runs
// before anything is enqueued; nothing here allocates or synchronises.

#include "attn_decode.h"

#include <math.h>

#include <algorithm>
#include <stdint.h>
#include <string.h>

#include "launch.h"

namespace {

constexpr size_t kAlign = 256;        // start of each workspace region
constexpr int64_t kMaxElems = int64_t(1) << 40;
constexpr int kMaxTmax = 1 << 30;
constexpr int kMaxGridYZ = 65535;
constexpr double kLog2e = 1.4426950408889634074;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Whether [a, a + na) and [b, b + nb) intersect; a null pointer (an argument
// that is absent) overlaps nothing.
bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x && y && na && nb && x < y + nb && y < x + na;
}

int elem_size(attn_dtype dt) { return dt == ATTN_BF16 ? 2 : 4; }

int ceil_div(int a, int b) { return a / b + (a % b != 0); }

// Exact a*b in uint64, saturating at UINT64_MAX.
uint64_t mul_sat(uint64_t a, uint64_t b) {
  if (a == 0 || b == 0) return 0;
  if (a > UINT64_MAX / b) return UINT64_MAX;
  return a * b;
}

// ------------------------------------------------------------------ GQA plan

struct GqaShape {
  int B, h_q, h_kv, D, T_max;
  attn_dtype dt;
};

int check_gqa_shape(const GqaShape& s) {
  if (s.B < 1 || s.h_q < 1 || s.h_kv < 1 || s.D < 1 || s.T_max < 1) return ATTN_ERR_INVALID_ARG;
  if (s.h_q % s.h_kv != 0) return ATTN_ERR_INVALID_ARG;
  if (s.T_max > kMaxTmax || s.B > kMaxGridYZ || s.h_kv > kMaxGridYZ) return ATTN_ERR_INVALID_ARG;
  if (int64_t(s.B) * s.h_kv * s.T_max * s.D >= kMaxElems) return ATTN_ERR_INVALID_ARG;
  if (int64_t(s.B) * s.h_q >= (int64_t(1) << 31)) return ATTN_ERR_INVALID_ARG;
  // The generic kernel's grid has h_kv * max(1, g / 16) rows in its second dimension.
  if (int64_t(s.h_kv) * std::max(1, s.h_q / s.h_kv / 16) > kMaxGridYZ) return ATTN_ERR_INVALID_ARG;
  if (s.dt != ATTN_F32 && s.dt != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
  if (!attn::gqa_supported(int(s.dt), s.D, s.h_q / s.h_kv)) return ATTN_ERR_UNSUPPORTED;
  // The kernels address one (sequence, KV head) slab with 32-bit byte offsets.
  if (int64_t(s.T_max) * s.D * elem_size(s.dt) >= (int64_t(1) << 31)) return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

// Positions per partition: a power of two in [512, 4096]. The persistent
// kernel splits the non-empty partitions evenly over its resident
// work-groups (512 on the 256-CU part), so it aims for about 2048 partitions
// when the cache is full: few enough that each work-group's share is long
// (every partition ends with a combine of its 4 waves), enough that the
// share of a ragged batch still splits evenly. The per-partition grid
// kernel aims for about 8192 work-groups (32 per CU).
int gqa_auto_partition(const GqaShape& s) {
  const int64_t pairs = int64_t(s.B) * s.h_kv;
  const int64_t target = s.dt == ATTN_BF16 ? 2048 : 8192;
  const int64_t want = (int64_t(s.T_max) * pairs + target - 1) / target;
  int P = 512;
  while (P < want && P < 4096) P <<= 1;
  return P;
}

size_t partial_bytes(int64_t rows, int NP, int Dv) {
  return align_up(size_t(rows) * NP * Dv * sizeof(float)) + align_up(size_t(rows) * NP * sizeof(float));
}

// Split decode (bf16): work-groups of the launch for a page size (0:
// contiguous cache; 0 groups: the shape runs on fixed partitions), and the
// most any page size can use, which the plan's workspace covers. Workspace:
// one partial per slot (work-groups + B * h_kv slots of G heads).
int gqa_split_groups(const GqaShape& s, int page_size) {
  return s.dt == ATTN_BF16 ? attn::gqa_split_groups(s.D, s.h_q / s.h_kv, page_size) : 0;
}
int gqa_split_groups_max(const GqaShape& s) {
  return s.dt == ATTN_BF16 ? attn::gqa_split_groups_max(s.D, s.h_q / s.h_kv) : 0;
}
size_t split_bytes(const GqaShape& s, int groups) {
  return partial_bytes((int64_t(groups) + int64_t(s.B) * s.h_kv) * (s.h_q / s.h_kv), 1, s.D);
}

// ------------------------------------------------------------------ MLA plan

struct MlaShape {
  int B, H, d_c, d_r, T_max;
};

int check_mla_shape(const MlaShape& s) {
  if (s.B < 1 || s.H < 1 || s.d_c < 1 || s.d_r < 0 || s.T_max < 1) return ATTN_ERR_INVALID_ARG;
  if (s.T_max > kMaxTmax || s.B > kMaxGridYZ) return ATTN_ERR_INVALID_ARG;
  if (int64_t(s.B) * s.T_max * (s.d_c + s.d_r) >= kMaxElems) return ATTN_ERR_INVALID_ARG;
  // Rows (b, h) are numbered with 32-bit integers (the merge).
  if (int64_t(s.B) * s.H >= (int64_t(1) << 31)) return ATTN_ERR_INVALID_ARG;
  if (!attn::mla_supported(s.H, s.d_c, s.d_r)) return ATTN_ERR_UNSUPPORTED;
  // The kernels address one sequence's rows of a contiguous cache with 32-bit
  // byte offsets.
  if (int64_t(s.T_max) * (s.d_c + s.d_r) * 2 >= (int64_t(1) << 31)) return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

// Positions per partition for MLA: a work-group holds all heads of one
// sequence, so the grid is B x partitions; aim for about 256 work-groups
// (one per CU) with partitions of at least 256 positions.
int mla_auto_partition(const MlaShape& s) {
  const int64_t want = (int64_t(s.T_max) * s.B + 255) / 256;
  int P = 256;
  while (P < want && P < (1 << 20)) P <<= 1;
  return P;
}

// The new rows of a decode step ([B, h_kv, D] each) must not overlap the
// caches they are written into, each other, or any other argument buffer.
int check_new_rows(const GqaShape& s, const void* k_new, const void* v_new, const void* q,
                   const void* k, const void* v, const int32_t* lens, const void* out,
                   size_t out_b, const void* ws, size_t ws_b) {
  if (!k_new || !v_new) return ATTN_ERR_INVALID_ARG;
  if (!aligned16(k_new) || !aligned16(v_new)) return ATTN_ERR_UNSUPPORTED;
  const size_t es = elem_size(s.dt);
  const size_t nb = size_t(s.B) * s.h_kv * s.D * es;
  const size_t kb = size_t(s.B) * s.h_kv * size_t(s.T_max) * s.D * es;
  const size_t qb = q ? size_t(s.B) * s.h_q * s.D * es : 0;
  for (const void* x : {k_new, v_new}) {
    if (overlap(x, nb, k, kb) || overlap(x, nb, v, kb) || overlap(x, nb, lens, size_t(s.B) * 4) ||
        overlap(x, nb, out, out_b) || overlap(x, nb, ws, ws_b))
      return ATTN_ERR_INVALID_ARG;
  }
  if (overlap(k_new, nb, v_new, nb) || overlap(k, kb, v, kb) || overlap(q, qb, k, kb) ||
      overlap(q, qb, v, kb) || overlap(lens, size_t(s.B) * 4, k, kb) ||
      overlap(lens, size_t(s.B) * 4, v, kb))
    return ATTN_ERR_INVALID_ARG;
  return ATTN_OK;
}

// Same for the new latent rows of an MLA decode step ([B, d_c + d_r]).
int check_new_latent(const MlaShape& s, const void* lat_new, const void* qn, const void* qr,
                     const void* lat, const int32_t* lens, const void* out, size_t out_b,
                     const void* ws, size_t ws_b) {
  if (!lat_new) return ATTN_ERR_INVALID_ARG;
  if (!aligned16(lat_new)) return ATTN_ERR_UNSUPPORTED;
  const size_t row = size_t(s.d_c + s.d_r) * 2;
  const size_t nb = size_t(s.B) * row, lb = size_t(s.B) * size_t(s.T_max) * row;
  const size_t qnb = size_t(s.B) * s.H * s.d_c * 2, qrb = size_t(s.B) * s.H * s.d_r * 2;
  if (overlap(lat_new, nb, lat, lb) || overlap(lat_new, nb, lens, size_t(s.B) * 4) ||
      overlap(lat_new, nb, out, out_b) || overlap(lat_new, nb, ws, ws_b) ||
      overlap(qn, qnb, lat, lb) || overlap(qr, qrb, lat, lb) ||
      overlap(lens, size_t(s.B) * 4, lat, lb))
    return ATTN_ERR_INVALID_ARG;
  return ATTN_OK;
}

// A paged cache as the kernels see it (block_table == nullptr: contiguous cache).
struct Paged {
  const int32_t* block_table = nullptr;
  int page_size = 0, page_shift = 0, max_pages = 0, num_pages = 0;
};

int log2_exact(int x) {
  int s = 0;
  while ((1 << s) < x) ++s;
  return (1 << s) == x ? s : -1;
}

// Checks the page geometry; T_max of the paged cache is max_pages * page_size.
int check_paged(const Paged& pg, int min_page, int* T_max) {
  if (!pg.block_table) return ATTN_ERR_INVALID_ARG;
  if (pg.page_size < 1 || pg.max_pages < 1 || pg.num_pages < 1) return ATTN_ERR_INVALID_ARG;
  if (int64_t(pg.page_size) * pg.max_pages > kMaxTmax) return ATTN_ERR_INVALID_ARG;
  if (log2_exact(pg.page_size) < 0 || pg.page_size < min_page || pg.page_size > (1 << 20))
    return ATTN_ERR_UNSUPPORTED;
  if (reinterpret_cast<uintptr_t>(pg.block_table) % 4 != 0) return ATTN_ERR_UNSUPPORTED;
  *T_max = pg.page_size * pg.max_pages;
  return ATTN_OK;
}

int set_plan(int P, int T_max, size_t ws, int* partition_size, int* num_partitions,
             size_t* workspace_bytes) {
  if (partition_size) *partition_size = P;
  if (num_partitions) *num_partitions = ceil_div(T_max, P);
  if (workspace_bytes) *workspace_bytes = ws;
  return ATTN_OK;
}

}  // namespace

extern "C" {

const char* attn_status_str(int status) {
  switch (status) {
    case ATTN_OK: return "ATTN_OK";
    case ATTN_ERR_INVALID_ARG: return "ATTN_ERR_INVALID_ARG: invalid argument";
    case ATTN_ERR_UNSUPPORTED: return "ATTN_ERR_UNSUPPORTED: shape, dtype or alignment not supported";
    case ATTN_ERR_WORKSPACE: return "ATTN_ERR_WORKSPACE: workspace missing or too small";
    case ATTN_ERR_HIP: return "ATTN_ERR_HIP: kernel launch failed";
    default: return "unknown attn_status";
  }
}

uint64_t attn_kv_cache_bytes(uint64_t n_layers, uint64_t n_kv_heads, uint64_t head_dim,
                             uint64_t seq_len, uint64_t batch, uint64_t bytes_per_elem) {
  uint64_t x = mul_sat(2, n_layers);
  x = mul_sat(x, n_kv_heads);
  x = mul_sat(x, head_dim);
  x = mul_sat(x, seq_len);
  x = mul_sat(x, batch);
  return mul_sat(x, bytes_per_elem);
}

uint64_t attn_mla_cache_bytes(uint64_t n_layers, uint64_t d_c, uint64_t d_r, uint64_t seq_len,
                              uint64_t batch, uint64_t bytes_per_elem) {
  if (d_c > UINT64_MAX - d_r) return UINT64_MAX;
  uint64_t x = mul_sat(n_layers, d_c + d_r);
  x = mul_sat(x, seq_len);
  x = mul_sat(x, batch);
  return mul_sat(x, bytes_per_elem);
}

// ------------------------------------------------------------------ GQA

int attn_decode_gqa_plan(int B, int h_q, int h_kv, int D, int T_max, attn_dtype dt,
                         int* partition_size, int* num_partitions, size_t* workspace_bytes) {
  const GqaShape s{B, h_q, h_kv, D, T_max, dt};
  const int st = check_gqa_shape(s);
  if (st != ATTN_OK) return st;
  const int P = gqa_auto_partition(s);
  const int NP = ceil_div(T_max, P);
  const int groups = gqa_split_groups_max(s);
  size_t ws = partial_bytes(int64_t(B) * h_q, NP, D);
  if (groups > 0) ws = std::max(ws, split_bytes(s, groups));
  return set_plan(P, T_max, ws, partition_size, num_partitions, workspace_bytes);
}

size_t attn_decode_gqa_workspace_bytes(int B, int h_q, int h_kv, int D, int T_max, attn_dtype dt) {
  size_t ws = 0;
  if (attn_decode_gqa_plan(B, h_q, h_kv, D, T_max, dt, nullptr, nullptr, &ws) != ATTN_OK) return 0;
  return ws;
}

static int check_gqa_ptrs(const GqaShape& s, const void* q, const void* k, const void* v,
                          const int32_t* lens, const void* out, size_t out_bytes) {
  if (!q || !k || !v || !lens || !out) return ATTN_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return ATTN_ERR_UNSUPPORTED;
  const size_t es = elem_size(s.dt);
  const size_t qb = size_t(s.B) * s.h_q * s.D * es;
  const size_t kb = size_t(s.B) * s.h_kv * size_t(s.T_max) * s.D * es;
  if (overlap(out, out_bytes, q, qb) || overlap(out, out_bytes, k, kb) ||
      overlap(out, out_bytes, v, kb) || overlap(out, out_bytes, lens, size_t(s.B) * 4))
    return ATTN_ERR_INVALID_ARG;
  return ATTN_OK;
}

int attn_decode_gqa_partial(const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* seq_lens, int B, int h_q, int h_kv, int D, int T_max,
                            float scale, attn_dtype dt, int partition_size, float* part_out,
                            float* part_lse, hipStream_t stream) {
  const GqaShape s{B, h_q, h_kv, D, T_max, dt};
  int st = check_gqa_shape(s);
  if (st != ATTN_OK) return st;
  if (partition_size < 1 || !isfinite(scale)) return ATTN_ERR_INVALID_ARG;
  const int NP = ceil_div(T_max, partition_size);
  const size_t ob = size_t(B) * h_q * NP * D * sizeof(float);
  st = check_gqa_ptrs(s, q, k_cache, v_cache, seq_lens, part_out, ob);
  if (st != ATTN_OK) return st;
  if (!part_lse) return ATTN_ERR_INVALID_ARG;
  if (!aligned16(part_lse)) return ATTN_ERR_UNSUPPORTED;
  if (overlap(part_out, ob, part_lse, size_t(B) * h_q * NP * sizeof(float))) return ATTN_ERR_INVALID_ARG;
  const attn::GqaArgs a{q, k_cache, v_cache, seq_lens, nullptr, nullptr, 0, nullptr, 0, 0, 0, 0,
                        B, h_kv, T_max, partition_size, NP, float(double(scale) * kLog2e),
                        part_out, part_lse};
  if (attn::launch_gqa_partial(int(dt), D, h_q / h_kv, a, stream) != hipSuccess) return ATTN_ERR_HIP;
  return ATTN_OK;
}

int attn_decode_merge(const float* part_out, const float* part_lse, const int32_t* seq_lens,
                      int B, int H, int Dv, int T_max, int partition_size, attn_dtype out_dt,
                      void* out, hipStream_t stream) {
  if (B < 1 || H < 1 || Dv < 1 || T_max < 1 || partition_size < 1) return ATTN_ERR_INVALID_ARG;
  if (T_max > kMaxTmax || int64_t(B) * H >= (int64_t(1) << 31)) return ATTN_ERR_INVALID_ARG;
  if (!part_out || !part_lse || !seq_lens || !out) return ATTN_ERR_INVALID_ARG;
  if (!attn::merge_supported(int(out_dt), Dv)) return ATTN_ERR_UNSUPPORTED;
  if (!aligned16(part_out) || !aligned16(part_lse) || !aligned16(out)) return ATTN_ERR_UNSUPPORTED;
  const int NP = ceil_div(T_max, partition_size);
  const size_t rows = size_t(B) * H;
  const size_t out_b = rows * Dv * elem_size(out_dt);
  if (overlap(out, out_b, part_out, rows * NP * Dv * sizeof(float)) ||
      overlap(out, out_b, part_lse, rows * NP * sizeof(float)))
    return ATTN_ERR_INVALID_ARG;
  if (attn::launch_merge(int(out_dt), part_out, part_lse, seq_lens, 0, 0, B, H, Dv, T_max,
                         partition_size, NP, out, stream) != hipSuccess)
    return ATTN_ERR_HIP;
  return ATTN_OK;
}

}  // extern "C"

namespace {

// Whole decode (k_new == nullptr) or decode step (append the new rows, then
// attend) for the GQA family: partial kernels, then the merge.
int gqa_decode_impl(const void* q, const void* k_new, const void* v_new, const void* k_cache,
                    const void* v_cache, const int32_t* seq_lens, int B, int h_q, int h_kv, int D,
                    int T_max, int window, float scale, attn_dtype dt, void* out, void* workspace,
                    size_t workspace_bytes, hipStream_t stream, const Paged& pg = Paged(),
                    int stages = 3) {
  const GqaShape s{B, h_q, h_kv, D, T_max, dt};
  int st = check_gqa_shape(s);
  if (st != ATTN_OK) return st;
  if (!isfinite(scale) || window < 0) return ATTN_ERR_INVALID_ARG;
  const size_t out_b = size_t(B) * h_q * D * elem_size(dt);
  if (pg.block_table) {
    // The caches are page arrays [num_pages, h_kv, page_size, D]: check them as
    // one "sequence" of num_pages * page_size rows.
    // Page arrays [num_pages, h_kv, page_size, D] are addressed with 64-bit
    // offsets: only their total size is bounded.
    if (int64_t(pg.num_pages) * h_kv * pg.page_size * D >= kMaxElems) return ATTN_ERR_INVALID_ARG;
    if (!q || !k_cache || !v_cache || !seq_lens || !out) return ATTN_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
      return ATTN_ERR_UNSUPPORTED;
    const size_t kb = size_t(pg.num_pages) * h_kv * pg.page_size * D * elem_size(dt);
    if (overlap(out, out_b, k_cache, kb) || overlap(out, out_b, v_cache, kb)) return ATTN_ERR_INVALID_ARG;
    const size_t tb = size_t(B) * pg.max_pages * 4;
    if (overlap(out, out_b, q, size_t(B) * h_q * D * elem_size(dt)) ||
        overlap(out, out_b, seq_lens, size_t(B) * 4) || overlap(out, out_b, pg.block_table, tb) ||
        overlap(pg.block_table, tb, k_cache, kb) || overlap(pg.block_table, tb, v_cache, kb))
      return ATTN_ERR_INVALID_ARG;
  } else {
    st = check_gqa_ptrs(s, q, k_cache, v_cache, seq_lens, out, out_b);
    if (st != ATTN_OK) return st;
  }
  // The split decode serves the persistent kernel's shapes (and paged caches
  // whose pages hold whole 32-row tiles); the others run on fixed partitions.
  // A window attends over at most `window` positions: plan for that span.
  const int groups = gqa_split_groups(s, pg.block_table ? pg.page_size : 0);
  const int span = window > 0 && window < T_max ? window : T_max;
  const GqaShape sp{B, h_q, h_kv, D, span, dt};
  const int P = groups > 0 ? attn::kSplitUnit : gqa_auto_partition(sp);
  const int NP = groups > 0 ? 0 : ceil_div(span, P);
  const size_t need = groups > 0 ? split_bytes(s, groups) : partial_bytes(int64_t(B) * h_q, NP, D);
  if (!workspace || workspace_bytes < need) return ATTN_ERR_WORKSPACE;
  if (!aligned16(workspace)) return ATTN_ERR_UNSUPPORTED;
  const size_t kb = pg.block_table ? size_t(pg.num_pages) * h_kv * pg.page_size * D * elem_size(dt)
                                   : size_t(B) * h_kv * size_t(T_max) * D * elem_size(dt);
  if (overlap(workspace, need, out, out_b) || overlap(workspace, need, k_cache, kb) ||
      overlap(workspace, need, v_cache, kb) ||
      overlap(workspace, need, pg.block_table, size_t(B) * pg.max_pages * 4))
    return ATTN_ERR_INVALID_ARG;
  if (k_new) {
    st = check_new_rows(s, k_new, v_new, q, k_cache, v_cache, seq_lens, out, out_b, workspace, need);
    if (st != ATTN_OK) return st;
  }
  const size_t rows = groups > 0 ? (size_t(groups) + size_t(B) * h_kv) * (h_q / h_kv) : size_t(B) * h_q * NP;
  float* part_out = static_cast<float*>(workspace);
  float* part_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) + align_up(rows * D * sizeof(float)));
  const attn::GqaArgs a{q, k_cache, v_cache, seq_lens, k_new, v_new, window, pg.block_table,
                        pg.page_size, pg.page_shift, pg.max_pages, pg.num_pages, B, h_kv, T_max,
                        P, NP, float(double(scale) * kLog2e), part_out, part_lse};
  if (groups > 0) {
    if ((stages & 1) && attn::launch_gqa_split(D, h_q / h_kv, a, groups, stream) != hipSuccess)
      return ATTN_ERR_HIP;
    if ((stages & 2) && attn::launch_split_merge(int(dt), part_out, part_lse, seq_lens, k_new ? 1 : 0, window,
                                                 B, h_kv, h_q / h_kv, D, T_max, groups, out, stream) != hipSuccess)
      return ATTN_ERR_HIP;
    return ATTN_OK;
  }
  if (stages != 3) return ATTN_ERR_UNSUPPORTED;
  if (NP == 1) {  // one partition: the partial kernel writes the output itself, no merge
    attn::GqaArgs d = a;
    d.out = out;
    d.out_bf16 = dt == ATTN_BF16;
    if (attn::launch_gqa_partial(int(dt), D, h_q / h_kv, d, stream) != hipSuccess) return ATTN_ERR_HIP;
    return ATTN_OK;
  }
  if (attn::launch_gqa_partial(int(dt), D, h_q / h_kv, a, stream) != hipSuccess) return ATTN_ERR_HIP;
  if (attn::launch_merge(int(dt), part_out, part_lse, seq_lens, k_new ? 1 : 0, window, B, h_q, D,
                         T_max, P, NP, out, stream) != hipSuccess)
    return ATTN_ERR_HIP;
  return ATTN_OK;
}

}  // namespace

extern "C" {

int attn_decode_gqa(const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* seq_lens, int B, int h_q, int h_kv, int D, int T_max,
                    float scale, attn_dtype dt, void* out, void* workspace,
                    size_t workspace_bytes, hipStream_t stream) {
  return gqa_decode_impl(q, nullptr, nullptr, k_cache, v_cache, seq_lens, B, h_q, h_kv, D, T_max,
                         0, scale, dt, out, workspace, workspace_bytes, stream);
}

int attn_decode_gqa_split(const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* seq_lens, int B, int h_q, int h_kv, int D, int T_max,
                          float scale, attn_dtype dt, void* out, void* workspace,
                          size_t workspace_bytes, hipStream_t stream) {
  return gqa_decode_impl(q, nullptr, nullptr, k_cache, v_cache, seq_lens, B, h_q, h_kv, D, T_max,
                         0, scale, dt, out, workspace, workspace_bytes, stream, Paged(), 1);
}

int attn_decode_gqa_split_merge(const void* q, const void* k_cache, const void* v_cache,
                                const int32_t* seq_lens, int B, int h_q, int h_kv, int D, int T_max,
                                float scale, attn_dtype dt, void* out, void* workspace,
                                size_t workspace_bytes, hipStream_t stream) {
  return gqa_decode_impl(q, nullptr, nullptr, k_cache, v_cache, seq_lens, B, h_q, h_kv, D, T_max,
                         0, scale, dt, out, workspace, workspace_bytes, stream, Paged(), 2);
}

int attn_decode_gqa_window(const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* seq_lens, int B, int h_q, int h_kv, int D, int T_max,
                           int window, float scale, attn_dtype dt, void* out, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
  if (window < 1) return ATTN_ERR_INVALID_ARG;
  return gqa_decode_impl(q, nullptr, nullptr, k_cache, v_cache, seq_lens, B, h_q, h_kv, D, T_max,
                         window, scale, dt, out, workspace, workspace_bytes, stream);
}

int attn_decode_gqa_step(const void* q, const void* k_new, const void* v_new, void* k_cache,
                         void* v_cache, const int32_t* seq_lens, int B, int h_q, int h_kv, int D,
                         int T_max, float scale, attn_dtype dt, void* out, void* workspace,
                         size_t workspace_bytes, hipStream_t stream) {
  if (!k_new || !v_new) return ATTN_ERR_INVALID_ARG;
  return gqa_decode_impl(q, k_new, v_new, k_cache, v_cache, seq_lens, B, h_q, h_kv, D, T_max,
                         0, scale, dt, out, workspace, workspace_bytes, stream);
}

int attn_kv_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                   const int32_t* seq_lens, int B, int h_kv, int D, int T_max, attn_dtype dt,
                   hipStream_t stream) {
  const GqaShape s{B, h_kv, h_kv, D, T_max, dt};
  int st = check_gqa_shape(s);
  if (st != ATTN_OK) return st;
  if (!k_new || !v_new || !k_cache || !v_cache || !seq_lens) return ATTN_ERR_INVALID_ARG;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache))
    return ATTN_ERR_UNSUPPORTED;
  st = check_new_rows(s, k_new, v_new, nullptr, k_cache, v_cache, seq_lens, nullptr, 0, nullptr, 0);
  if (st != ATTN_OK) return st;
  if (attn::launch_kv_append(int(dt), k_new, v_new, k_cache, v_cache, seq_lens, B, h_kv, D, T_max,
                             stream) != hipSuccess)
    return ATTN_ERR_HIP;
  return ATTN_OK;
}

int attn_decode_gqa_paged(const void* q, const void* k_pages, const void* v_pages,
                          const int32_t* block_table, const int32_t* seq_lens, int B, int h_q,
                          int h_kv, int D, int num_pages, int page_size, int max_pages, float scale,
                          attn_dtype dt, void* out, void* workspace, size_t workspace_bytes,
                          hipStream_t stream) {
  Paged pg;
  pg.block_table = block_table;
  pg.page_size = page_size;
  pg.page_shift = log2_exact(page_size);
  pg.max_pages = max_pages;
  pg.num_pages = num_pages;
  int T_max = 0;
  const int st = check_paged(pg, 16, &T_max);
  if (st != ATTN_OK) return st;
  return gqa_decode_impl(q, nullptr, nullptr, k_pages, v_pages, seq_lens, B, h_q, h_kv, D, T_max, 0,
                         scale, dt, out, workspace, workspace_bytes, stream, pg);
}

int attn_kv_append_paged(const void* k_new, const void* v_new, void* k_pages, void* v_pages,
                         const int32_t* block_table, const int32_t* seq_lens, int B, int h_kv, int D,
                         int num_pages, int page_size, int max_pages, attn_dtype dt,
                         hipStream_t stream) {
  Paged pg;
  pg.block_table = block_table;
  pg.page_size = page_size;
  pg.max_pages = max_pages;
  pg.num_pages = num_pages;
  int T_max = 0;
  int st = check_paged(pg, 1, &T_max);
  if (st != ATTN_OK) return st;
  const GqaShape ps{num_pages, h_kv, h_kv, D, page_size, dt};
  st = check_gqa_shape(ps);
  if (st != ATTN_OK) return st;
  if (B < 1 || B > kMaxGridYZ || !seq_lens || !k_pages || !v_pages) return ATTN_ERR_INVALID_ARG;
  if (!aligned16(k_pages) || !aligned16(v_pages)) return ATTN_ERR_UNSUPPORTED;
  const GqaShape rows{B, h_kv, h_kv, D, 1, dt};
  st = check_new_rows(rows, k_new, v_new, nullptr, nullptr, nullptr, seq_lens, nullptr, 0, nullptr, 0);
  if (st != ATTN_OK) return st;
  const size_t es = elem_size(dt), nb = size_t(B) * h_kv * D * es;
  const size_t kb = size_t(num_pages) * h_kv * page_size * D * es, tb = size_t(B) * max_pages * 4;
  for (const void* x : {k_new, v_new, static_cast<const void*>(block_table), static_cast<const void*>(seq_lens)}) {
    const size_t xb = x == block_table ? tb : (x == seq_lens ? size_t(B) * 4 : nb);
    if (overlap(x, xb, k_pages, kb) || overlap(x, xb, v_pages, kb)) return ATTN_ERR_INVALID_ARG;
  }
  if (overlap(k_pages, kb, v_pages, kb)) return ATTN_ERR_INVALID_ARG;
  if (attn::launch_append_paged(k_new, v_new, k_pages, v_pages, block_table, seq_lens, B, h_kv,
                                int(D * es), page_size, max_pages, num_pages, stream) != hipSuccess)
    return ATTN_ERR_HIP;
  return ATTN_OK;
}

// ------------------------------------------------------------------ MLA

int attn_decode_mla_plan(int B, int H, int d_c, int d_r, int T_max, int* partition_size,
                         int* num_partitions, size_t* workspace_bytes) {
  const MlaShape s{B, H, d_c, d_r, T_max};
  const int st = check_mla_shape(s);
  if (st != ATTN_OK) return st;
  const int P = mla_auto_partition(s);
  const int NP = ceil_div(T_max, P);
  return set_plan(P, T_max, partial_bytes(int64_t(B) * H, NP, d_c), partition_size,
                  num_partitions, workspace_bytes);
}

size_t attn_decode_mla_workspace_bytes(int B, int H, int d_c, int d_r, int T_max) {
  size_t ws = 0;
  if (attn_decode_mla_plan(B, H, d_c, d_r, T_max, nullptr, nullptr, &ws) != ATTN_OK) return 0;
  return ws;
}

static int check_mla_ptrs(const MlaShape& s, const void* qn, const void* qr, const void* lat,
                          const int32_t* lens, const void* out, size_t out_bytes) {
  if (!qn || !qr || !lat || !lens || !out) return ATTN_ERR_INVALID_ARG;
  if (!aligned16(qn) || !aligned16(qr) || !aligned16(lat) || !aligned16(out))
    return ATTN_ERR_UNSUPPORTED;
  const size_t qnb = size_t(s.B) * s.H * s.d_c * 2, qrb = size_t(s.B) * s.H * s.d_r * 2;
  const size_t lb = size_t(s.B) * size_t(s.T_max) * (s.d_c + s.d_r) * 2;
  if (overlap(out, out_bytes, qn, qnb) || overlap(out, out_bytes, qr, qrb) ||
      overlap(out, out_bytes, lat, lb) || overlap(out, out_bytes, lens, size_t(s.B) * 4))
    return ATTN_ERR_INVALID_ARG;
  return ATTN_OK;
}

int attn_decode_mla_partial(const void* q_nope, const void* q_rope, const void* latent,
                            const int32_t* seq_lens, int B, int H, int d_c, int d_r, int T_max,
                            float scale, int partition_size, float* part_out, float* part_lse,
                            hipStream_t stream) {
  const MlaShape s{B, H, d_c, d_r, T_max};
  int st = check_mla_shape(s);
  if (st != ATTN_OK) return st;
  if (partition_size < 1 || !isfinite(scale)) return ATTN_ERR_INVALID_ARG;
  const int NP = ceil_div(T_max, partition_size);
  const size_t ob = size_t(B) * H * NP * d_c * sizeof(float);
  st = check_mla_ptrs(s, q_nope, q_rope, latent, seq_lens, part_out, ob);
  if (st != ATTN_OK) return st;
  if (!part_lse) return ATTN_ERR_INVALID_ARG;
  if (!aligned16(part_lse)) return ATTN_ERR_UNSUPPORTED;
  if (overlap(part_out, ob, part_lse, size_t(B) * H * NP * sizeof(float))) return ATTN_ERR_INVALID_ARG;
  const attn::MlaArgs a{q_nope, q_rope, latent, seq_lens, nullptr, nullptr, 0, 0, 0, 0, B, H, T_max,
                        partition_size, NP, float(double(scale) * kLog2e), part_out, part_lse};
  if (attn::launch_mla_partial(a, stream) != hipSuccess) return ATTN_ERR_HIP;
  return ATTN_OK;
}

}  // extern "C"

namespace {

int mla_decode_impl(const void* q_nope, const void* q_rope, const void* lat_new,
                    const void* latent, const int32_t* seq_lens, int B, int H, int d_c, int d_r,
                    int T_max, float scale, void* out, void* workspace, size_t workspace_bytes,
                    hipStream_t stream, const Paged& pg = Paged()) {
  const MlaShape s{B, H, d_c, d_r, T_max};
  int st = check_mla_shape(s);
  if (st != ATTN_OK) return st;
  if (!isfinite(scale)) return ATTN_ERR_INVALID_ARG;
  const size_t out_b = size_t(B) * H * d_c * 2;
  if (pg.block_table) {
    if (int64_t(pg.num_pages) * pg.page_size * (d_c + d_r) >= kMaxElems) return ATTN_ERR_INVALID_ARG;
    const MlaShape ps{1, H, d_c, d_r, pg.num_pages * pg.page_size};
    st = check_mla_ptrs(ps, q_nope, q_rope, latent, seq_lens, out, out_b);
    if (st != ATTN_OK) return st;
    const size_t lb = size_t(pg.num_pages) * pg.page_size * (d_c + d_r) * 2;
    const size_t tb = size_t(B) * pg.max_pages * 4;
    const size_t qnb = size_t(B) * H * d_c * 2, qrb = size_t(B) * H * d_r * 2;
    if (overlap(out, out_b, q_nope, qnb) || overlap(out, out_b, q_rope, qrb) ||
        overlap(out, out_b, seq_lens, size_t(B) * 4) || overlap(out, out_b, pg.block_table, tb) ||
        overlap(pg.block_table, tb, latent, lb))
      return ATTN_ERR_INVALID_ARG;
  } else {
    st = check_mla_ptrs(s, q_nope, q_rope, latent, seq_lens, out, out_b);
    if (st != ATTN_OK) return st;
  }
  const int P = mla_auto_partition(s);
  const int NP = ceil_div(T_max, P);
  const size_t need = partial_bytes(int64_t(B) * H, NP, d_c);
  if (!workspace || workspace_bytes < need) return ATTN_ERR_WORKSPACE;
  if (!aligned16(workspace)) return ATTN_ERR_UNSUPPORTED;
  const size_t lb = pg.block_table ? size_t(pg.num_pages) * pg.page_size * (d_c + d_r) * 2
                                   : size_t(B) * size_t(T_max) * (d_c + d_r) * 2;
  if (overlap(workspace, need, out, out_b) || overlap(workspace, need, latent, lb) ||
      overlap(workspace, need, pg.block_table, size_t(B) * pg.max_pages * 4))
    return ATTN_ERR_INVALID_ARG;
  if (lat_new) {
    st = check_new_latent(s, lat_new, q_nope, q_rope, latent, seq_lens, out, out_b, workspace, need);
    if (st != ATTN_OK) return st;
  }
  float* part_out = static_cast<float*>(workspace);
  float* part_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                             align_up(size_t(B) * H * NP * d_c * sizeof(float)));
  const attn::MlaArgs a{q_nope, q_rope, latent, seq_lens, lat_new, pg.block_table, pg.page_size,
                        pg.page_shift, pg.max_pages, pg.num_pages, B, H, T_max, P, NP,
                        float(double(scale) * kLog2e), part_out, part_lse};
  if (attn::launch_mla_partial(a, stream) != hipSuccess) return ATTN_ERR_HIP;
  if (attn::launch_merge(int(ATTN_BF16), part_out, part_lse, seq_lens, lat_new ? 1 : 0, 0, B, H,
                         d_c, T_max, P, NP, out, stream) != hipSuccess)
    return ATTN_ERR_HIP;
  return ATTN_OK;
}

}  // namespace

extern "C" {

int attn_decode_mla(const void* q_nope, const void* q_rope, const void* latent,
                    const int32_t* seq_lens, int B, int H, int d_c, int d_r, int T_max,
                    float scale, void* out, void* workspace, size_t workspace_bytes,
                    hipStream_t stream) {
  return mla_decode_impl(q_nope, q_rope, nullptr, latent, seq_lens, B, H, d_c, d_r, T_max, scale,
                         out, workspace, workspace_bytes, stream);
}

int attn_decode_mla_step(const void* q_nope, const void* q_rope, const void* latent_new,
                         void* latent_cache, const int32_t* seq_lens, int B, int H, int d_c,
                         int d_r, int T_max, float scale, void* out, void* workspace,
                         size_t workspace_bytes, hipStream_t stream) {
  if (!latent_new) return ATTN_ERR_INVALID_ARG;
  return mla_decode_impl(q_nope, q_rope, latent_new, latent_cache, seq_lens, B, H, d_c, d_r, T_max,
                         scale, out, workspace, workspace_bytes, stream);
}

int attn_decode_mla_paged(const void* q_nope, const void* q_rope, const void* latent_pages,
                          const int32_t* block_table, const int32_t* seq_lens, int B, int H, int d_c,
                          int d_r, int num_pages, int page_size, int max_pages, float scale, void* out,
                          void* workspace, size_t workspace_bytes, hipStream_t stream) {
  Paged pg;
  pg.block_table = block_table;
  pg.page_size = page_size;
  pg.page_shift = log2_exact(page_size);
  pg.max_pages = max_pages;
  pg.num_pages = num_pages;
  int T_max = 0;
  const int st = check_paged(pg, 32, &T_max);
  if (st != ATTN_OK) return st;
  return mla_decode_impl(q_nope, q_rope, nullptr, latent_pages, seq_lens, B, H, d_c, d_r, T_max,
                         scale, out, workspace, workspace_bytes, stream, pg);
}

int attn_latent_append_paged(const void* latent_new, void* latent_pages, const int32_t* block_table,
                             const int32_t* seq_lens, int B, int d_c, int d_r, int num_pages,
                             int page_size, int max_pages, hipStream_t stream) {
  Paged pg;
  pg.block_table = block_table;
  pg.page_size = page_size;
  pg.max_pages = max_pages;
  pg.num_pages = num_pages;
  int T_max = 0;
  const int st = check_paged(pg, 1, &T_max);
  if (st != ATTN_OK) return st;
  if (B < 1 || B > kMaxGridYZ || d_c < 1 || d_r < 0 || !latent_new || !latent_pages || !seq_lens)
    return ATTN_ERR_INVALID_ARG;
  if (int64_t(num_pages) * page_size * (d_c + d_r) >= kMaxElems) return ATTN_ERR_INVALID_ARG;
  if ((d_c + d_r) % 8 != 0) return ATTN_ERR_UNSUPPORTED;
  if (!aligned16(latent_new) || !aligned16(latent_pages)) return ATTN_ERR_UNSUPPORTED;
  const size_t row = size_t(d_c + d_r) * 2, nb = size_t(B) * row;
  const size_t lb = size_t(num_pages) * page_size * row, tb = size_t(B) * max_pages * 4;
  if (overlap(latent_new, nb, latent_pages, lb) || overlap(block_table, tb, latent_pages, lb) ||
      overlap(seq_lens, size_t(B) * 4, latent_pages, lb))
    return ATTN_ERR_INVALID_ARG;
  if (attn::launch_append_paged(latent_new, nullptr, latent_pages, nullptr, block_table, seq_lens, B,
                                1, int(row), page_size, max_pages, num_pages, stream) != hipSuccess)
    return ATTN_ERR_HIP;
  return ATTN_OK;
}

int attn_latent_append(const void* latent_new, void* latent_cache, const int32_t* seq_lens, int B,
                       int d_c, int d_r, int T_max, hipStream_t stream) {
  if (B < 1 || d_c < 1 || d_r < 0 || T_max < 1) return ATTN_ERR_INVALID_ARG;
  if (T_max > kMaxTmax || B > kMaxGridYZ) return ATTN_ERR_INVALID_ARG;
  if (int64_t(B) * T_max * (d_c + d_r) >= kMaxElems) return ATTN_ERR_INVALID_ARG;
  if (!latent_new || !latent_cache || !seq_lens) return ATTN_ERR_INVALID_ARG;
  if ((d_c + d_r) % 8 != 0) return ATTN_ERR_UNSUPPORTED;   // whole 16-byte pieces per row
  if (!aligned16(latent_new) || !aligned16(latent_cache)) return ATTN_ERR_UNSUPPORTED;
  const size_t nb = size_t(B) * (d_c + d_r) * 2, lb = size_t(B) * size_t(T_max) * (d_c + d_r) * 2;
  if (overlap(latent_new, nb, latent_cache, lb) || overlap(latent_new, nb, seq_lens, size_t(B) * 4) ||
      overlap(latent_cache, lb, seq_lens, size_t(B) * 4))
    return ATTN_ERR_INVALID_ARG;
  if (attn::launch_latent_append(latent_new, latent_cache, seq_lens, B, d_c + d_r, T_max, stream) !=
      hipSuccess)
    return ATTN_ERR_HIP;
  return ATTN_OK;
}

// ------------------------------------------------------------------ MLA absorption products

static int check_absorb_args(const void* x, size_t xb, const void* w, size_t wb, const void* y,
                             size_t yb) {
  if (!x || !w || !y) return ATTN_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(w) || !aligned16(y)) return ATTN_ERR_UNSUPPORTED;
  if (overlap(y, yb, x, xb) || overlap(y, yb, w, wb)) return ATTN_ERR_INVALID_ARG;
  return ATTN_OK;
}

int attn_mla_absorb_q(const void* q_nope, const void* w_uk, void* q_lat, int B, int H, int d_h,
                      int d_c, hipStream_t stream) {
  if (B < 1 || H < 1 || d_h < 1 || d_c < 1 || H > kMaxGridYZ) return ATTN_ERR_INVALID_ARG;
  if (int64_t(B) * H * (d_h > d_c ? d_h : d_c) >= kMaxElems ||
      int64_t(H) * d_c * d_h >= kMaxElems)
    return ATTN_ERR_INVALID_ARG;
  if (!attn::absorb_supported(d_h, d_c)) return ATTN_ERR_UNSUPPORTED;
  const int st = check_absorb_args(q_nope, size_t(B) * H * d_h * 2, w_uk, size_t(H) * d_c * d_h * 2,
                                   q_lat, size_t(B) * H * d_c * 2);
  if (st != ATTN_OK) return st;
  if (attn::launch_absorb_q(q_nope, w_uk, q_lat, B, H, d_h, d_c, stream) != hipSuccess) return ATTN_ERR_HIP;
  return ATTN_OK;
}

int attn_mla_up_v(const void* o_lat, const void* w_uv, void* out, int B, int H, int d_c, int d_v,
                  hipStream_t stream) {
  if (B < 1 || H < 1 || d_c < 1 || d_v < 1 || H > kMaxGridYZ) return ATTN_ERR_INVALID_ARG;
  if (int64_t(B) * H * (d_c > d_v ? d_c : d_v) >= kMaxElems ||
      int64_t(H) * d_c * d_v >= kMaxElems)
    return ATTN_ERR_INVALID_ARG;
  if (!attn::up_supported(d_c, d_v)) return ATTN_ERR_UNSUPPORTED;
  const int st = check_absorb_args(o_lat, size_t(B) * H * d_c * 2, w_uv, size_t(H) * d_c * d_v * 2,
                                   out, size_t(B) * H * d_v * 2);
  if (st != ATTN_OK) return st;
  if (attn::launch_up_v(o_lat, w_uv, out, B, H, d_c, d_v, stream) != hipSuccess) return ATTN_ERR_HIP;
  return ATTN_OK;
}

}  // extern "C"
