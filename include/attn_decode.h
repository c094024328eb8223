/*
 * attn_decode.h -- C ABI of a decode-attention library for AMD MI355X (gfx950).
 *
 * One decode step: every sequence b of a batch has ONE new query token per
 * head, and every query head attends over the n = seq_lens[b] positions
 * already in its KV cache (the new token's own key/value included: the cache
 * is appended first, then attended). There is no mask inside [0, n). The
 * *_step entry points do the append themselves: there seq_lens[b] is the
 * length before the step and the new row goes to position seq_lens[b].
 *
 *   MHA / GQA / MQA   h_q query heads share h_kv KV heads in consecutive
 *                     groups of g = h_q / h_kv: query head i reads KV head
 *                     i / g (0-indexed; "Attention variants: MQA, GQA, and
 *                     MLA", section "GQA: interpolating with groups", and
 *                     "Grouped-Query Attention: Fewer KV Heads, Same
 *                     Quality", section "Writing the formula explicitly").
 *                     h_kv == h_q is MHA, h_kv == 1 is MQA.
 *   absorbed MLA      H heads score against ONE cached row per token, the
 *                     latent c (d_c values) followed by a decoupled rotary
 *                     key (d_r values); the output of each head is the
 *                     softmax-weighted average of the latents ("Attention
 *                     variants: MQA, GQA, and MLA", section "MLA: cache a
 *                     latent, not the keys and values").
 *
 * For each row (b, i):  s_t = scale * <q[b,i,:], K[b,j,t,:]>,  t < n
 *                        out[b,i,:] = sum_t softmax(s)_t * V[b,j,t,:]
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every tensor argument is a DEVICE pointer to contiguous row-major memory
 *   with the shape written next to it. The caller owns all memory; the
 *   library never allocates, frees or keeps a pointer after returning.
 * - Work is enqueued asynchronously on `stream` (0 = the null stream). No
 *   entry point synchronises the host. Results are ready when the stream
 *   reaches the enqueued work.
 * - Return value: ATTN_OK (0) or a negative attn_status. Every argument check
 *   happens on the host BEFORE anything is enqueued; a non-zero return from
 *   a check means nothing was launched. ATTN_ERR_HIP means a launch failed
 *   (hipGetLastError); attn_status_str() names each code.
 * - Device pointers must be 16-byte aligned (ATTN_ERR_UNSUPPORTED otherwise).
 *   `out` must not overlap any input (ATTN_ERR_INVALID_ARG).
 * - seq_lens: int32[B] on the device. A value is clamped to [0, T_max] in the
 *   kernels; n == 0 yields an all-zero output row. Positions t >= n are
 *   never read, so padding may hold any bits, NaN included.
 * - Accumulation is fp32 whatever the storage type; out has q's dtype and is
 *   rounded to nearest-even. Results are deterministic: same inputs and plan,
 *   bit-identical output (no atomics, fixed reduction order).
 * - Split-KV: positions are cut into partitions of `partition_size`; each
 *   partition produces its softmax-normalised partial output and its log-sum-
 *   exp, and a second kernel merges the partials. The *_partial / merge entry
 *   points expose the two stages (for a caller that merges partials itself,
 *   e.g. across devices); the one-call entry points run both with the
 *   library's own partition size and a caller-provided workspace.
 * - bf16 GQA (every supported g; contiguous caches, and paged caches whose
 *   pages hold at least 32 positions, 16 at g = 64, 64 at g in {3, 5, 6, 7})
 *   is split differently
 *   by the one-call entry points: every resident work-group takes an equal
 *   share of all (sequence, KV head, 128-position unit) work, and each
 *   work-group's share of a (sequence, KV head) row is one partial. The cut
 *   points then depend on the sequence lengths and on the device's compute-
 *   unit count; on one device the output is still bit-identical from run to
 *   run. Which kernel runs is a function of (D, g, page size): g in {1, 2, 4}
 *   streams one position per lane on the vector ALUs; g = 8 to 64, and g in
 *   {3, 5, 6, 7}, scores and sums on 16x16 matrix-core tiles (the groups below
 *   16 in masked head columns); g = 128 on 32x32 tiles (a paged cache picks
 *   among them by which tile its pages hold whole). fp32 caches, and bf16
 *   pages too small for any of those tiles, run on fixed partitions through
 *   a generic kernel.
 * - Host state: the library keeps, per device index, the device's compute-
 *   unit count, and per process the resident work-groups per compute unit of
 *   each persistent kernel (a property of the kernel on gfx950), both read
 *   once from the HIP runtime on first use (thread-safe, written once).
 *   Nothing else persists between calls, and no call depends on a previous
 *   one.
 */
#ifndef ATTN_DECODE_H
#define ATTN_DECODE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_INVALID_ARG = -1,  /* null pointer, non-positive size, h_q % h_kv != 0, overlap, overflow */
  ATTN_ERR_UNSUPPORTED = -2,  /* valid but not built: head dim, group size, dtype, alignment */
  ATTN_ERR_WORKSPACE = -3,    /* workspace pointer null or workspace_bytes too small */
  ATTN_ERR_HIP = -4           /* a kernel launch reported an error */
} attn_status;

/* Storage type of q, the caches and out. C callers may pass any int: values
 * other than these two are rejected (ATTN_ERR_UNSUPPORTED). The C++ view gives
 * the enumeration a fixed underlying int, so that such a value is a valid
 * object to check rather than undefined behaviour (same ABI as the C view). */
#ifdef __cplusplus
typedef enum attn_dtype_e : int { ATTN_F32 = 0, ATTN_BF16 = 1 } attn_dtype;
#else
typedef enum { ATTN_F32 = 0, ATTN_BF16 = 1 } attn_dtype;
#endif

/* Human-readable name of a status code (static string, never NULL). */
const char* attn_status_str(int status);

/* ---------------------------------------------------------------- cache-size helpers
 * Exact host-only integer arithmetic; no device is touched.
 *
 * attn_kv_cache_bytes: bytes of K plus V, each [batch, n_kv_heads, seq_len,
 * head_dim] per layer, i.e. 2 * n_layers * n_kv_heads * head_dim * seq_len *
 * batch * bytes_per_elem ("Attention variants: MQA, GQA, and MLA", section
 * "The KV cache bill, worked numerically"; same argument order as the page's
 * helper, whose defaults are batch = 1 and bytes_per_elem = 2).
 *
 * attn_mla_cache_bytes: bytes of an MLA cache, one (d_c + d_r)-wide row per
 * token per layer per sequence (same page, section "MLA: cache a latent, not
 * the keys and values").
 *
 * Both return UINT64_MAX if the exact product does not fit in 64 bits.
 */
uint64_t attn_kv_cache_bytes(uint64_t n_layers, uint64_t n_kv_heads, uint64_t head_dim,
                             uint64_t seq_len, uint64_t batch, uint64_t bytes_per_elem);
uint64_t attn_mla_cache_bytes(uint64_t n_layers, uint64_t d_c, uint64_t d_r,
                              uint64_t seq_len, uint64_t batch, uint64_t bytes_per_elem);

/* ---------------------------------------------------------------- GQA / MHA / MQA
 * q        [B, h_q, D]           dtype dt
 * k_cache  [B, h_kv, T_max, D]   dtype dt
 * v_cache  [B, h_kv, T_max, D]   dtype dt
 * seq_lens int32 [B]
 * out      [B, h_q, D]           dtype dt
 * Supported: D in {64, 128}; g = h_q / h_kv any of 1 to 8, or a power of two
 * up to 128 (MHA g = 1; MQA h_kv = 1 with h_q up to 128; other g:
 * ATTN_ERR_UNSUPPORTED); dt
 * in {ATTN_F32, ATTN_BF16}. B, h_kv and h_kv * max(1, g / 16) at most 65535
 * (ATTN_ERR_INVALID_ARG otherwise). Any B >= 1, T_max >= 1 with
 * B*h_kv*T_max*D < 2^40; one (sequence, KV head) slab, T_max*D*sizeof(elem),
 * must stay below 2 GiB (ATTN_ERR_UNSUPPORTED otherwise).
 */

/* The library's plan for a shape: partition size (positions per split, as
 * attn_decode_gqa_partial would use it), number of partitions
 * ceil(T_max / partition_size), and the workspace bytes attn_decode_gqa needs
 * on the current device (the work-balanced split's partials scale with its
 * compute-unit count). Outputs may be NULL. Returns a status. */
int attn_decode_gqa_plan(int B, int h_q, int h_kv, int D, int T_max, attn_dtype dt,
                         int* partition_size, int* num_partitions, size_t* workspace_bytes);

/* Workspace bytes attn_decode_gqa needs for this shape; 0 if the shape is invalid
 * or unsupported (every valid shape needs more than 0 bytes). */
size_t attn_decode_gqa_workspace_bytes(int B, int h_q, int h_kv, int D, int T_max, attn_dtype dt);

/* One decode step: split-KV partial kernel then log-sum-exp merge, both on
 * `stream`. workspace: device memory of at least attn_decode_gqa_workspace_bytes
 * bytes, 16-byte aligned, contents ignored on entry and clobbered. */
int attn_decode_gqa(const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* seq_lens, int B, int h_q, int h_kv, int D, int T_max,
                    float scale, attn_dtype dt, void* out,
                    void* workspace, size_t workspace_bytes, hipStream_t stream);

/* The two stages of attn_decode_gqa where it runs the work-balanced split
 * (bf16 storage, every supported D and g; ATTN_ERR_UNSUPPORTED for fp32). They take exactly attn_decode_gqa's arguments and checks.
 * attn_decode_gqa_split runs stage 1 only: it writes the partials into the
 * workspace and does not touch `out`. attn_decode_gqa_split_merge runs stage 2
 * only: it reads those partials and seq_lens (which must not have changed)
 * and writes `out`; q, k_cache and v_cache are checked but not read. Both
 * must run on the same device, in stream order, with the same shape and
 * workspace; together they produce the same bits as attn_decode_gqa. They
 * exist so that each stage can be timed on its own. */
int attn_decode_gqa_split(const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* seq_lens, int B, int h_q, int h_kv, int D, int T_max,
                          float scale, attn_dtype dt, void* out,
                          void* workspace, size_t workspace_bytes, hipStream_t stream);
int attn_decode_gqa_split_merge(const void* q, const void* k_cache, const void* v_cache,
                                const int32_t* seq_lens, int B, int h_q, int h_kv, int D, int T_max,
                                float scale, attn_dtype dt, void* out,
                                void* workspace, size_t workspace_bytes, hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * attn_decode_gqa without a workspace argument. The library supplies the
 * workspace from one static device array of ATTN_NOALLOC_SCRATCH_BYTES per
 * device (allocated with the library's code, held until the process ends);
 * the call itself allocates nothing. Same arguments, checks, kernels and bits
 * as attn_decode_gqa. Shapes whose workspace
 * (attn_decode_gqa_workspace_bytes) exceeds ATTN_NOALLOC_SCRATCH_BYTES return
 * ATTN_ERR_WORKSPACE before anything is launched. Every call on one device
 * uses the same array: calls that may overlap in time on one device
 * (different streams, or host threads without ordering) race and give
 * undefined results; calls ordered on one stream are safe. Nothing in the
 * array needs to be zero on entry. ATTN_ERR_HIP if the array's device address
 * cannot be obtained. */
#define ATTN_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int attn_decode_gqa_noalloc(const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* seq_lens, int B, int h_q, int h_kv, int D, int T_max,
                            float scale, attn_dtype dt, void* out, hipStream_t stream);

/* Sliding-window decode ("Grouped-Query Attention: Fewer KV Heads, Same
 * Quality", section "GQA and Related KV-Head Choices in Modern Architectures":
 * Mistral 7B pairs grouped KV heads with a window of w = 4096 positions). Each
 * row attends over the last `window` of its n positions, t in
 * [max(0, n - window), n); window >= n is the full decode. window >= 1.
 * Positions before the window are never read. Workspace: at least
 * attn_decode_gqa_workspace_bytes(B, h_q, h_kv, D, min(window, T_max), dt)
 * bytes (the plan covers the window's span only). */
int attn_decode_gqa_window(const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* seq_lens, int B, int h_q, int h_kv, int D, int T_max,
                           int window, float scale, attn_dtype dt, void* out,
                           void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Decode step that first appends the new token ("Attention Variants: MHA,
 * MQA, GQA — Speed vs Quality at Scale", section "The KV Cache Problem": each
 * new token's K and V are stored in the cache, then the token attends over
 * every cached pair, its own included).
 * k_new, v_new [B, h_kv, D] dtype dt: the new token's key and value per KV head.
 * Here seq_lens[b] is the cached length BEFORE the step. Row pos =
 * max(seq_lens[b], 0) of KV head j of k_cache / v_cache receives k_new[b, j] /
 * v_new[b, j] (bit-exact copies), then every query head attends over pos + 1
 * positions, exactly as attn_decode_gqa would with seq_lens[b] + 1. A
 * sequence whose cache is full (pos >= T_max) is not written and attends over
 * its T_max cached positions. Only row pos of each head is written; seq_lens
 * is not modified (advancing it is the caller's job). k_new and v_new must not
 * overlap each other, the caches or any other argument (ATTN_ERR_INVALID_ARG).
 * Same plan and workspace as attn_decode_gqa. */
int attn_decode_gqa_step(const void* q, const void* k_new, const void* v_new,
                         void* k_cache, void* v_cache, const int32_t* seq_lens,
                         int B, int h_q, int h_kv, int D, int T_max, float scale, attn_dtype dt,
                         void* out, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* The write of attn_decode_gqa_step alone, same rules (h_q = h_kv for the
 * shape checks): k_new / v_new [B, h_kv, D] copied bit for bit into row
 * max(seq_lens[b], 0) of each KV head unless the cache is full. */
int attn_kv_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                   const int32_t* seq_lens, int B, int h_kv, int D, int T_max, attn_dtype dt,
                   hipStream_t stream);

/* Decode over a paged KV cache ("Attention variants: MQA, GQA, and MLA",
 * section "Against the real libraries": serving engines keep the cache in
 * fixed-size pages allocated like virtual memory and shared by sequences with
 * a common prefix).
 * k_pages, v_pages [num_pages, h_kv, page_size, D] dtype dt: page p holds
 *                  page_size consecutive positions of every KV head;
 * block_table      int32 [B, max_pages]: position t of sequence b lives in
 *                  row t % page_size of page block_table[b, t / page_size].
 * A sequence holds at most T_max = max_pages * page_size positions (seq_lens
 * clamped to it); entries past a sequence's last used page are never read,
 * and pages may be shared between sequences (read-only here). page_size: a
 * power of two >= 16; the bf16 split kernels need pages of at least 32 rows
 * (16 at g = 64, 64 at g in {3, 5, 6, 7}); smaller pages go through the
 * generic kernel's per-row gather (slower). A used table entry outside
 * [0, num_pages) never faults: its rows read as zeros (or as a clamped page on
 * the per-row path) and the result for that sequence is unspecified.
 * Workspace: attn_decode_gqa_workspace_bytes(B, h_q, h_kv, D, T_max, dt). */
int attn_decode_gqa_paged(const void* q, const void* k_pages, const void* v_pages,
                          const int32_t* block_table, const int32_t* seq_lens,
                          int B, int h_q, int h_kv, int D, int num_pages, int page_size,
                          int max_pages, float scale, attn_dtype dt, void* out,
                          void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Append into a paged cache: k_new / v_new [B, h_kv, D] go to logical
 * position pos = max(seq_lens[b], 0) (row pos % page_size of page
 * block_table[b, pos / page_size]) unless pos >= T_max or that table entry is
 * outside [0, num_pages); bit-exact copies. page_size: any power of two. */
int attn_kv_append_paged(const void* k_new, const void* v_new, void* k_pages, void* v_pages,
                         const int32_t* block_table, const int32_t* seq_lens, int B, int h_kv,
                         int D, int num_pages, int page_size, int max_pages, attn_dtype dt,
                         hipStream_t stream);

/* Stage 1 alone, with an explicit partition_size P >= 1 and NP = ceil(T_max / P):
 * part_out [B, h_q, NP, D] fp32: softmax-weighted average of V over the valid
 *          positions of partition p, i.e. t in [p*P, min((p+1)*P, n));
 * part_lse [B, h_q, NP]    fp32: log2 of sum_t exp(s_t) over the same positions
 *          (natural-exp scores, base-2 logarithm).
 * Partitions with p*P >= n are not written (they hold no position). */
int attn_decode_gqa_partial(const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* seq_lens, int B, int h_q, int h_kv, int D, int T_max,
                            float scale, attn_dtype dt, int partition_size,
                            float* part_out, float* part_lse, hipStream_t stream);

/* Stage 2: merge NP = ceil(T_max / partition_size) partials per row into
 * out [B, H, Dv] (dtype out_dt), reading only the ceil(n / partition_size)
 * partitions that hold positions: out = sum_p 2^(lse_p - M) part_out_p /
 * sum_p 2^(lse_p - M) with M = max_p lse_p. Dv in {64, 128, 512} (a multiple of 4, at most 1024). */
int attn_decode_merge(const float* part_out, const float* part_lse, const int32_t* seq_lens,
                      int B, int H, int Dv, int T_max, int partition_size,
                      attn_dtype out_dt, void* out, hipStream_t stream);

/* ---------------------------------------------------------------- absorbed MLA (bf16)
 * q_nope_absorbed [B, H, d_c]          bf16: query times the key up-projection
 * q_rope          [B, H, d_r]          bf16: query part for the rotary key
 * latent_cache    [B, T_max, d_c+d_r]  bf16: [latent | rotary key] per token
 * seq_lens        int32 [B]
 * out             [B, H, d_c]          bf16: weighted average of latents
 * s_t = scale * (<q_nope, latent[t, :d_c]> + <q_rope, latent[t, d_c:]>).
 * Supported: (d_c, d_r) = (512, 64); H in {32, 64, 96, 128} or any multiple of
 * 128 (MFMA tiles of 32 heads, one work-group per block of up to 128 heads);
 * bf16 only; one sequence's rows, T_max * (d_c + d_r) * 2 bytes, below 2 GiB
 * (ATTN_ERR_UNSUPPORTED otherwise: the kernels address them with 32-bit
 * offsets); B * H below 2^31 rows (ATTN_ERR_INVALID_ARG otherwise). The
 * rotary key is used as stored: rotating it and q_rope by position is the
 * caller's job.
 */
int attn_decode_mla_plan(int B, int H, int d_c, int d_r, int T_max,
                         int* partition_size, int* num_partitions, size_t* workspace_bytes);
size_t attn_decode_mla_workspace_bytes(int B, int H, int d_c, int d_r, int T_max);

int attn_decode_mla(const void* q_nope_absorbed, const void* q_rope, const void* latent_cache,
                    const int32_t* seq_lens, int B, int H, int d_c, int d_r, int T_max,
                    float scale, void* out, void* workspace, size_t workspace_bytes,
                    hipStream_t stream);

/* Decode step that first appends the new token's cache row ("Attention
 * variants: MQA, GQA, and MLA", section "MLA: cache a latent, not the keys
 * and values": the new latent is concatenated to the cache, then the scores
 * and the average run over the extended cache).
 * latent_new [B, d_c+d_r] bf16: [latent | rotary key] of the new token.
 * seq_lens[b] is the cached length BEFORE the step; row pos = max(seq_lens[b], 0)
 * of latent_cache receives latent_new[b] (bit-exact copy), then every head
 * attends over pos + 1 positions; a full cache (pos >= T_max) is not written
 * and is attended over its T_max positions. seq_lens is not modified.
 * latent_new must not overlap any other argument. Same workspace as
 * attn_decode_mla. */
int attn_decode_mla_step(const void* q_nope_absorbed, const void* q_rope, const void* latent_new,
                         void* latent_cache, const int32_t* seq_lens, int B, int H, int d_c,
                         int d_r, int T_max, float scale, void* out, void* workspace,
                         size_t workspace_bytes, hipStream_t stream);

/* The write of attn_decode_mla_step alone: latent_new [B, d_c+d_r] bf16 copied
 * bit for bit into row max(seq_lens[b], 0) of latent_cache unless it is full.
 * Any d_c + d_r that is a multiple of 8. */
int attn_latent_append(const void* latent_new, void* latent_cache, const int32_t* seq_lens,
                       int B, int d_c, int d_r, int T_max, hipStream_t stream);

/* Absorbed MLA over a paged latent cache (same page rules as
 * attn_decode_gqa_paged): latent_pages [num_pages, page_size, d_c+d_r] bf16,
 * block_table int32 [B, max_pages]; page_size a power of two >= 32 (one
 * 32-position tile never spans two pages). Workspace:
 * attn_decode_mla_workspace_bytes(B, H, d_c, d_r, max_pages * page_size). */
int attn_decode_mla_paged(const void* q_nope_absorbed, const void* q_rope, const void* latent_pages,
                          const int32_t* block_table, const int32_t* seq_lens, int B, int H,
                          int d_c, int d_r, int num_pages, int page_size, int max_pages,
                          float scale, void* out, void* workspace, size_t workspace_bytes,
                          hipStream_t stream);

/* Append into a paged latent cache: latent_new [B, d_c+d_r] bf16 goes to
 * logical position max(seq_lens[b], 0), same rules as attn_kv_append_paged. */
int attn_latent_append_paged(const void* latent_new, void* latent_pages, const int32_t* block_table,
                             const int32_t* seq_lens, int B, int d_c, int d_r, int num_pages,
                             int page_size, int max_pages, hipStream_t stream);

/* Stage 1 alone; same partial layout as attn_decode_gqa_partial with h_q = H
 * and D = d_c. Merge with attn_decode_merge(..., Dv = d_c, out_dt = ATTN_BF16). */
int attn_decode_mla_partial(const void* q_nope_absorbed, const void* q_rope,
                            const void* latent_cache, const int32_t* seq_lens,
                            int B, int H, int d_c, int d_r, int T_max, float scale,
                            int partition_size, float* part_out, float* part_lse,
                            hipStream_t stream);

/* ---------------------------------------------------------------- MLA absorption products
 * The per-head matrix products on either side of the absorbed MLA decode
 * ("Attention variants: MQA, GQA, and MLA", section "MLA: cache a latent, not
 * the keys and values": the key up-projection is absorbed into the query,
 * the value up-projection is applied to the averaged latent). Weights use
 * the page's layout [H, d_c, d_head]. bf16 in, fp32 accumulation on the
 * matrix cores, bf16 out (round to nearest even).
 *
 * attn_mla_absorb_q:  q_lat[b, h, c] = sum_d q_nope[b, h, d] * w_uk[h, c, d]
 *   q_nope [B, H, d_h], w_uk [H, d_c, d_h], q_lat [B, H, d_c] (the decode's
 *   q_nope_absorbed). d_h a multiple of 16, d_c a multiple of 32.
 * attn_mla_up_v:  out[b, h, d] = sum_c o_lat[b, h, c] * w_uv[h, c, d]
 *   o_lat [B, H, d_c] (the decode's output), w_uv [H, d_c, d_v], out
 *   [B, H, d_v]. d_c a multiple of 16, d_v a multiple of 32.
 * The output must not overlap the inputs. */
int attn_mla_absorb_q(const void* q_nope, const void* w_uk, void* q_lat, int B, int H, int d_h,
                      int d_c, hipStream_t stream);
int attn_mla_up_v(const void* o_lat, const void* w_uv, void* out, int B, int H, int d_c, int d_v,
                  hipStream_t stream);

#ifdef __cplusplus
}  /* extern "C" */
#endif

#endif /* ATTN_DECODE_H */
