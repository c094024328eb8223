// Split-KV decode attention for the MHA / GQA / MQA family on gfx950.
//
// A work-group (4 wave64s) streams the K and V rows of one (sequence b, KV
// head j, partition p) triple, positions [p*P, min(p*P+P, n)), from HBM
// exactly once. Every row it loads serves all G = h_q / h_kv query heads of
// the group (query head i reads KV head i / G, "Attention variants: MQA,
// GQA, and MLA", section "GQA: interpolating with groups"), so the bytes
// streamed per step are the cache's own size, not G times it. The bf16
// kernel (gqa_partial_po_kernel, the second half of this file) is persistent
// and takes such triples in turn; the general kernel (fp32 caches, groups of
// 16, pages shorter than its tile) gets one work-group per triple.
//
// Data layout in registers of the general kernel: one K (or V) row is
// D * sizeof(elem) bytes = LPR lanes x 16 bytes, so each 16-byte vector load
// instruction of a wave covers RPI = 64 / LPR consecutive rows, i.e. one
// contiguous 1 KiB span. Lane (rr, c) holds elements [c*EPL, c*EPL + EPL) of
// row rr of each span. Scores reduce over the LPR lanes of a row with DPP
// moves (no LDS traffic).
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

#include <algorithm>
#include <atomic>
#include <type_traits>

#include "device_util.h"
#include "launch.h"
#include "split_items.h"

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
__global__ __launch_bounds__(kThreads) void gqa_partial_kernel(const GqaArgs a) {
  using S = typename E::storage;
  constexpr int EPL = E::EPL;
  constexpr int LPR = D / EPL;       // lanes per row
  constexpr int RPI = 64 / LPR;      // rows per wave-wide 16-byte load
  constexpr int NI = G >= 16 ? 2 : (G >= 8 ? 4 : 8);  // loads per block per tensor (bounded by registers)
  constexpr int RB = NI * RPI;       // rows per block per wave
  const S* __restrict__ q = static_cast<const S*>(a.q);
  // Not restrict: a decode step writes one row of each cache before reading.
  const S* kc = static_cast<const S*>(a.k);
  const S* vc = static_cast<const S*>(a.v);
  float* __restrict__ part_out = a.part_out;
  float* __restrict__ part_lse = a.part_lse;
  const int h_kv = a.h_kv, T_max = a.T_max, P = a.P, NP = a.NP;
  const float qk_scale_log2 = a.qk_scale_log2;

  // Groups above G heads are taken in head_chunks work-groups of G heads each
  // (blockIdx.y = KV head * head_chunks + chunk); each reads the group's K/V rows.
  const int chunks = a.head_chunks;
  const int p = blockIdx.x, j = blockIdx.y / chunks, hc = blockIdx.y % chunks, b = blockIdx.z;
  const int GG = G * chunks;  // query heads per KV head
  const int len0 = a.seq_lens[b];
  const int n = attended_len(len0, a.k_new ? 1 : 0, T_max);
  const int start = window_lo(n, a.window) + p * P;
  if (start >= n) {  // no position in this partition: nothing written, the merge skips it
    if (a.out) {     // single partition written as the output: an empty row is zeros
      const size_t orow = ((size_t)b * h_kv * GG + (size_t)j * GG + (size_t)hc * G) * D;
      for (int idx = threadIdx.x; idx < G * D; idx += kThreads) {
        if (a.out_bf16) static_cast<uint16_t*>(a.out)[orow + idx] = 0;
        else static_cast<float*>(a.out)[orow + idx] = 0.f;
      }
    }
    return;
  }
  const int end = min(start, n - P) + P;  // = min(start + P, n) without overflow
  if (a.k_new) {  // decode step: the work-group that reads the new row writes it first
    const int pos = max(len0, 0);
    if (pos < T_max && pos >= start && pos < end) {
      const size_t row = (((size_t)b * h_kv + j) * (size_t)T_max + pos) * D;
      const size_t src = ((size_t)b * h_kv + j) * D;
      write_row_then_sync<D * sizeof(S)>(const_cast<S*>(kc) + row, static_cast<const S*>(a.k_new) + src);
      write_row_then_sync<D * sizeof(S)>(const_cast<S*>(vc) + row, static_cast<const S*>(a.v_new) + src);
    }
  }

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rr = lane / LPR, c = lane % LPR;
  const int H = h_kv * GG;

  uint4 qv[G];
  const typename E::storage* qrow = q + ((size_t)b * H + (size_t)j * GG + (size_t)hc * G) * D + c * EPL;
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

  const bool paged = a.block_table != nullptr;
  const size_t head_off = paged ? (size_t)j * a.page_size * D + (size_t)c * EPL
                                : ((size_t)b * h_kv + j) * (size_t)T_max * D + (size_t)c * EPL;
  const typename E::storage* kb = kc + head_off;
  const typename E::storage* vb = vc + head_off;
  // Element offset of row r (clamped to the partition) from kb / vb. Paged:
  // page lookup per row; a table entry outside [0, num_pages) is clamped
  // into range (the row's values are then unspecified, never a fault).
  const int32_t* bt = paged ? a.block_table + (size_t)b * a.max_pages : nullptr;
  auto row_off = [&](int r) -> size_t {
    r = min(r, end - 1);
    if (!paged) return (size_t)r * D;
    const int phys = min(max(bt[r >> a.page_shift], 0), a.num_pages - 1);
    return (((size_t)phys * h_kv) * a.page_size + (r & (a.page_size - 1))) * D;
  };

  for (int r0 = start + wave * RB; r0 < end; r0 += kWaves * RB) {
    uint4 kr[NI], vr[NI];
    size_t ro[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) ro[i] = row_off(r0 + i * RPI + rr);
#pragma unroll
    for (int i = 0; i < NI; ++i) kr[i] = ld16_nt(kb + ro[i]);
#pragma unroll
    for (int i = 0; i < NI; ++i) vr[i] = ld16_nt(vb + ro[i]);

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
    if (a.out) {  // the only partition: finished output row
      const size_t orow = (size_t)b * H + (size_t)j * GG + (size_t)hc * G + h;
      if (a.out_bf16) static_cast<uint16_t*>(a.out)[orow * D + d] = f32_to_bf16_rne(A / L);
      else static_cast<float*>(a.out)[orow * D + d] = A / L;
      continue;
    }
    const size_t row = ((size_t)b * H + (size_t)j * GG + (size_t)hc * G + h) * NP + p;
    part_out[row * D + d] = A / L;
    if (d == 0) part_lse[row] = M + fast_log2(L);
  }
}

// ---------------------------------------------------------------------------
// bf16 kernel, one cached position per pair of lanes for the scores.
//
// The kernel is persistent: as many work-groups as the device holds at once
// take equal runs of the non-empty (sequence, KV head, partition) items
// (items::ItemRun in split_items.h), so a ragged batch leaves no CU idle. Within an item the 4
// waves take 32-position tiles in turn. For a tile:
//  * K rows go straight from HBM into the wave's own LDS area (direct copy,
//    16 bytes per lane per instruction). Within each row the 16-byte chunks
//    are stored XOR-permuted by the row index, so that 16 lanes reading the
//    same logical chunk of 16 different rows hit 16 different bank groups.
//  * Lane l scores position t0 + l % 32 over the dimensions of half l / 32 of
//    the head, against all G query heads, and the two halves are added with
//    one lane swap (half_sum). The query words are spread over vector
//    registers and each v_dot2 fetches its word with a DPP row broadcast.
//  * The tile maximum per head is one wave-wide reduction; the running
//    maximum is wave-uniform. Each weight exp2(s - m) is written once, by the
//    lane of half 0 that owns the position, to a small LDS table.
//  * V rows are loaded into registers in the row layout (LPR lanes x 16 bytes
//    per row, 1 KiB contiguous per wave-wide load), and each lane reads the G
//    weights of its row from the table (a broadcast read) for the product.
// Compared with reducing every score across a row's lanes, the arithmetic per
// cached element drops from G*(2 + 4/8) lane-ops + G exps per row group to
// about G/2 dot2 + G/32 exps, which is what matters when G = 4..8.
// At the end of an item the 4 waves combine their partials through LDS, with
// one barrier; the combine area is double-buffered by item parity.
constexpr int kPoRows = 32;

template <int N, class F, int I = 0>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, F, I + 1>(static_cast<F&&>(f));
  }
}

// Hand-scheduled blocks of DPP arithmetic (inline assembly). The compiler
// inserts the wait states gfx950 needs between dependent instructions for the
// code it generates, but it cannot see into inline assembly, so each block
// carries its own. The requirements are those of the wait-state table in
// AMD's CDNA3 / CDNA4 instruction-set reference guides ("Manually Inserted
// Wait States (NOPs)"), which LLVM's AMDGPU hazard recognizer also enforces
// for gfx940 / gfx950 code:
//  * a VALU write of a VGPR followed by a DPP read of that VGPR: two wait states;
//  * a VALU write of a VGPR followed by v_permlane16/32_swap reading it (new
//    in CDNA4): two;
//  * a dot-product (v_dot2c_f32_bf16) result read by any other VALU
//    instruction: three, while the same dot instruction accumulating into
//    that register needs none.
// Every block therefore opens with s_nop 1 (covering whatever the compiler
// wrote just before) and closes with enough wait states for whatever the
// compiler reads just after; inside a block the spacing is explicit. A CPU
// test compiles the kernels and scans the assembly for these rules.

// acc[h] += dot(q_h, k) over the four bf16 pairs of one 16-byte K chunk, for
// G heads: query word e of the chunk for head h is the value that lane L0 + e
// of the caller's 16-lane row holds in qr[h] (row_newbcast source operand).
template <int L0>
__device__ __forceinline__ void dot_chunk2(float (&acc)[2], const uint32_t (&qr)[2], const uint4& k) {
  asm("s_nop 1\n\t"
      "v_dot2c_f32_bf16_dpp %0, %2, %4 row_newbcast:%8 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %1, %3, %4 row_newbcast:%8 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %0, %2, %5 row_newbcast:%9 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %1, %3, %5 row_newbcast:%9 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %0, %2, %6 row_newbcast:%10 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %1, %3, %6 row_newbcast:%10 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %0, %2, %7 row_newbcast:%11 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %1, %3, %7 row_newbcast:%11 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 2"
      : "+v"(acc[0]), "+v"(acc[1])
      : "v"(qr[0]), "v"(qr[1]), "v"(k.x), "v"(k.y), "v"(k.z), "v"(k.w), "i"(L0 + 0), "i"(L0 + 1), "i"(L0 + 2), "i"(L0 + 3));
}

template <int L0>
__device__ __forceinline__ void dot_chunk4(float (&acc)[4], const uint32_t (&qr)[4], const uint4& k) {
  asm("s_nop 1\n\t"
      "v_dot2c_f32_bf16_dpp %0, %4, %8 row_newbcast:%12 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %1, %5, %8 row_newbcast:%12 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %2, %6, %8 row_newbcast:%12 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %3, %7, %8 row_newbcast:%12 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %0, %4, %9 row_newbcast:%13 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %1, %5, %9 row_newbcast:%13 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %2, %6, %9 row_newbcast:%13 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %3, %7, %9 row_newbcast:%13 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %0, %4, %10 row_newbcast:%14 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %1, %5, %10 row_newbcast:%14 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %2, %6, %10 row_newbcast:%14 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %3, %7, %10 row_newbcast:%14 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %0, %4, %11 row_newbcast:%15 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %1, %5, %11 row_newbcast:%15 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %2, %6, %11 row_newbcast:%15 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %3, %7, %11 row_newbcast:%15 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 2"
      : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3])
      : "v"(qr[0]), "v"(qr[1]), "v"(qr[2]), "v"(qr[3]), "v"(k.x), "v"(k.y), "v"(k.z), "v"(k.w), "i"(L0 + 0), "i"(L0 + 1), "i"(L0 + 2), "i"(L0 + 3));
}

template <int L0>
__device__ __forceinline__ void dot_chunk8(float (&acc)[8], const uint32_t (&qr)[8], const uint4& k) {
  asm("s_nop 1\n\t"
      "v_dot2c_f32_bf16_dpp %0, %8, %16 row_newbcast:%20 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %1, %9, %16 row_newbcast:%20 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %2, %10, %16 row_newbcast:%20 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %3, %11, %16 row_newbcast:%20 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %4, %12, %16 row_newbcast:%20 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %5, %13, %16 row_newbcast:%20 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %6, %14, %16 row_newbcast:%20 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %7, %15, %16 row_newbcast:%20 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %0, %8, %17 row_newbcast:%21 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %1, %9, %17 row_newbcast:%21 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %2, %10, %17 row_newbcast:%21 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %3, %11, %17 row_newbcast:%21 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %4, %12, %17 row_newbcast:%21 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %5, %13, %17 row_newbcast:%21 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %6, %14, %17 row_newbcast:%21 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %7, %15, %17 row_newbcast:%21 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %0, %8, %18 row_newbcast:%22 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %1, %9, %18 row_newbcast:%22 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %2, %10, %18 row_newbcast:%22 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %3, %11, %18 row_newbcast:%22 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %4, %12, %18 row_newbcast:%22 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %5, %13, %18 row_newbcast:%22 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %6, %14, %18 row_newbcast:%22 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %7, %15, %18 row_newbcast:%22 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %0, %8, %19 row_newbcast:%23 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %1, %9, %19 row_newbcast:%23 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %2, %10, %19 row_newbcast:%23 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %3, %11, %19 row_newbcast:%23 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %4, %12, %19 row_newbcast:%23 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %5, %13, %19 row_newbcast:%23 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %6, %14, %19 row_newbcast:%23 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %7, %15, %19 row_newbcast:%23 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 2"
      : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3]), "+v"(acc[4]), "+v"(acc[5]), "+v"(acc[6]), "+v"(acc[7])
      : "v"(qr[0]), "v"(qr[1]), "v"(qr[2]), "v"(qr[3]), "v"(qr[4]), "v"(qr[5]), "v"(qr[6]), "v"(qr[7]), "v"(k.x), "v"(k.y), "v"(k.z), "v"(k.w), "i"(L0 + 0), "i"(L0 + 1), "i"(L0 + 2), "i"(L0 + 3));
}

// Maximum over each 32-lane half of N values per lane (four DPP steps inside
// each 16-lane row, then the swap between rows 0-1 and 2-3 of the half). The
// callers' two halves hold the same values (after the half sums every lane
// holds its position's full scores), so this is the maximum over the wave.
__device__ __forceinline__ void wave_max4(float (&x)[4]) {
  float t[4];
  asm("s_nop 1\n\t"
      "v_max_f32_dpp %0, %0, %0 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
      "v_max_f32_dpp %1, %1, %1 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
      "v_max_f32_dpp %2, %2, %2 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
      "v_max_f32_dpp %3, %3, %3 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
      "v_max_f32_dpp %0, %0, %0 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
      "v_max_f32_dpp %1, %1, %1 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
      "v_max_f32_dpp %2, %2, %2 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
      "v_max_f32_dpp %3, %3, %3 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
      "v_max_f32_dpp %0, %0, %0 row_half_mirror row_mask:0xf bank_mask:0xf\n\t"
      "v_max_f32_dpp %1, %1, %1 row_half_mirror row_mask:0xf bank_mask:0xf\n\t"
      "v_max_f32_dpp %2, %2, %2 row_half_mirror row_mask:0xf bank_mask:0xf\n\t"
      "v_max_f32_dpp %3, %3, %3 row_half_mirror row_mask:0xf bank_mask:0xf\n\t"
      "v_max_f32_dpp %0, %0, %0 row_mirror row_mask:0xf bank_mask:0xf\n\t"
      "v_max_f32_dpp %1, %1, %1 row_mirror row_mask:0xf bank_mask:0xf\n\t"
      "v_max_f32_dpp %2, %2, %2 row_mirror row_mask:0xf bank_mask:0xf\n\t"
      "v_max_f32_dpp %3, %3, %3 row_mirror row_mask:0xf bank_mask:0xf\n\t"
      "v_mov_b32 %4, %0\n\t"
      "v_mov_b32 %5, %1\n\t"
      "v_mov_b32 %6, %2\n\t"
      "v_mov_b32 %7, %3\n\t"
      "s_nop 1\n\t"
      "v_permlane16_swap_b32 %0, %4\n\t"
      "v_permlane16_swap_b32 %1, %5\n\t"
      "v_permlane16_swap_b32 %2, %6\n\t"
      "v_permlane16_swap_b32 %3, %7\n\t"
      "v_max_f32 %0, %0, %4\n\t"
      "v_max_f32 %1, %1, %5\n\t"
      "v_max_f32 %2, %2, %6\n\t"
      "v_max_f32 %3, %3, %7\n\t"
      "s_nop 1"
      : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "=&v"(t[0]), "=&v"(t[1]), "=&v"(t[2]), "=&v"(t[3]));
}

__device__ __forceinline__ void wave_max8(float (&x)[8]) {
  float t[8];
  asm("s_nop 1\n\t"
      "v_max_f32_dpp %0, %0, %0 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
      "v_max_f32_dpp %1, %1, %1 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
      "v_max_f32_dpp %2, %2, %2 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
      "v_max_f32_dpp %3, %3, %3 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
      "v_max_f32_dpp %4, %4, %4 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
      "v_max_f32_dpp %5, %5, %5 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
      "v_max_f32_dpp %6, %6, %6 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
      "v_max_f32_dpp %7, %7, %7 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
      "v_max_f32_dpp %0, %0, %0 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
      "v_max_f32_dpp %1, %1, %1 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
      "v_max_f32_dpp %2, %2, %2 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
      "v_max_f32_dpp %3, %3, %3 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
      "v_max_f32_dpp %4, %4, %4 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
      "v_max_f32_dpp %5, %5, %5 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
      "v_max_f32_dpp %6, %6, %6 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
      "v_max_f32_dpp %7, %7, %7 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
      "v_max_f32_dpp %0, %0, %0 row_half_mirror row_mask:0xf bank_mask:0xf\n\t"
      "v_max_f32_dpp %1, %1, %1 row_half_mirror row_mask:0xf bank_mask:0xf\n\t"
      "v_max_f32_dpp %2, %2, %2 row_half_mirror row_mask:0xf bank_mask:0xf\n\t"
      "v_max_f32_dpp %3, %3, %3 row_half_mirror row_mask:0xf bank_mask:0xf\n\t"
      "v_max_f32_dpp %4, %4, %4 row_half_mirror row_mask:0xf bank_mask:0xf\n\t"
      "v_max_f32_dpp %5, %5, %5 row_half_mirror row_mask:0xf bank_mask:0xf\n\t"
      "v_max_f32_dpp %6, %6, %6 row_half_mirror row_mask:0xf bank_mask:0xf\n\t"
      "v_max_f32_dpp %7, %7, %7 row_half_mirror row_mask:0xf bank_mask:0xf\n\t"
      "v_max_f32_dpp %0, %0, %0 row_mirror row_mask:0xf bank_mask:0xf\n\t"
      "v_max_f32_dpp %1, %1, %1 row_mirror row_mask:0xf bank_mask:0xf\n\t"
      "v_max_f32_dpp %2, %2, %2 row_mirror row_mask:0xf bank_mask:0xf\n\t"
      "v_max_f32_dpp %3, %3, %3 row_mirror row_mask:0xf bank_mask:0xf\n\t"
      "v_max_f32_dpp %4, %4, %4 row_mirror row_mask:0xf bank_mask:0xf\n\t"
      "v_max_f32_dpp %5, %5, %5 row_mirror row_mask:0xf bank_mask:0xf\n\t"
      "v_max_f32_dpp %6, %6, %6 row_mirror row_mask:0xf bank_mask:0xf\n\t"
      "v_max_f32_dpp %7, %7, %7 row_mirror row_mask:0xf bank_mask:0xf\n\t"
      "v_mov_b32 %8, %0\n\t"
      "v_mov_b32 %9, %1\n\t"
      "v_mov_b32 %10, %2\n\t"
      "v_mov_b32 %11, %3\n\t"
      "v_mov_b32 %12, %4\n\t"
      "v_mov_b32 %13, %5\n\t"
      "v_mov_b32 %14, %6\n\t"
      "v_mov_b32 %15, %7\n\t"
      "s_nop 1\n\t"
      "v_permlane16_swap_b32 %0, %8\n\t"
      "v_permlane16_swap_b32 %1, %9\n\t"
      "v_permlane16_swap_b32 %2, %10\n\t"
      "v_permlane16_swap_b32 %3, %11\n\t"
      "v_permlane16_swap_b32 %4, %12\n\t"
      "v_permlane16_swap_b32 %5, %13\n\t"
      "v_permlane16_swap_b32 %6, %14\n\t"
      "v_permlane16_swap_b32 %7, %15\n\t"
      "v_max_f32 %0, %0, %8\n\t"
      "v_max_f32 %1, %1, %9\n\t"
      "v_max_f32 %2, %2, %10\n\t"
      "v_max_f32 %3, %3, %11\n\t"
      "v_max_f32 %4, %4, %12\n\t"
      "v_max_f32 %5, %5, %13\n\t"
      "v_max_f32 %6, %6, %14\n\t"
      "v_max_f32 %7, %7, %15\n\t"
      "s_nop 1"
      : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), "+v"(x[5]), "+v"(x[6]), "+v"(x[7]), "=&v"(t[0]), "=&v"(t[1]), "=&v"(t[2]), "=&v"(t[3]), "=&v"(t[4]), "=&v"(t[5]), "=&v"(t[6]), "=&v"(t[7]));
}

template <int L0>
__device__ __forceinline__ void dot_chunk1(float (&acc)[1], const uint32_t (&qr)[1], const uint4& k) {
  asm("s_nop 1\n\t"
      "v_dot2c_f32_bf16_dpp %0, %1, %2 row_newbcast:%6 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %0, %1, %3 row_newbcast:%7 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %0, %1, %4 row_newbcast:%8 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %0, %1, %5 row_newbcast:%9 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 2"
      : "+v"(acc[0])
      : "v"(qr[0]), "v"(k.x), "v"(k.y), "v"(k.z), "v"(k.w), "i"(L0 + 0), "i"(L0 + 1), "i"(L0 + 2), "i"(L0 + 3));
}

__device__ __forceinline__ void half_sum1(float (&x)[1]) {
  float t[1];
  asm(
      "v_mov_b32 %1, %0\n\t"
      "s_nop 1\n\t"
      "v_permlane32_swap_b32 %0, %1\n\t"
      "s_nop 1\n\t"
      "v_add_f32 %0, %0, %1\n\t"
      "s_nop 1"
      : "+v"(x[0]), "=&v"(t[0]));
}

__device__ __forceinline__ void half_sum2(float (&x)[2]) {
  float t[2];
  asm(
      "v_mov_b32 %2, %0\n\t"
      "v_mov_b32 %3, %1\n\t"
      "s_nop 1\n\t"
      "v_permlane32_swap_b32 %0, %2\n\t"
      "v_permlane32_swap_b32 %1, %3\n\t"
      "s_nop 1\n\t"
      "v_add_f32 %0, %0, %2\n\t"
      "v_add_f32 %1, %1, %3\n\t"
      "s_nop 1"
      : "+v"(x[0]), "+v"(x[1]), "=&v"(t[0]), "=&v"(t[1]));
}

__device__ __forceinline__ void half_sum4(float (&x)[4]) {
  float t[4];
  asm(
      "v_mov_b32 %4, %0\n\t"
      "v_mov_b32 %5, %1\n\t"
      "v_mov_b32 %6, %2\n\t"
      "v_mov_b32 %7, %3\n\t"
      "s_nop 1\n\t"
      "v_permlane32_swap_b32 %0, %4\n\t"
      "v_permlane32_swap_b32 %1, %5\n\t"
      "v_permlane32_swap_b32 %2, %6\n\t"
      "v_permlane32_swap_b32 %3, %7\n\t"
      "s_nop 1\n\t"
      "v_add_f32 %0, %0, %4\n\t"
      "v_add_f32 %1, %1, %5\n\t"
      "v_add_f32 %2, %2, %6\n\t"
      "v_add_f32 %3, %3, %7\n\t"
      "s_nop 1"
      : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "=&v"(t[0]), "=&v"(t[1]), "=&v"(t[2]), "=&v"(t[3]));
}

__device__ __forceinline__ void half_sum8(float (&x)[8]) {
  float t[8];
  asm(
      "v_mov_b32 %8, %0\n\t"
      "v_mov_b32 %9, %1\n\t"
      "v_mov_b32 %10, %2\n\t"
      "v_mov_b32 %11, %3\n\t"
      "v_mov_b32 %12, %4\n\t"
      "v_mov_b32 %13, %5\n\t"
      "v_mov_b32 %14, %6\n\t"
      "v_mov_b32 %15, %7\n\t"
      "s_nop 1\n\t"
      "v_permlane32_swap_b32 %0, %8\n\t"
      "v_permlane32_swap_b32 %1, %9\n\t"
      "v_permlane32_swap_b32 %2, %10\n\t"
      "v_permlane32_swap_b32 %3, %11\n\t"
      "v_permlane32_swap_b32 %4, %12\n\t"
      "v_permlane32_swap_b32 %5, %13\n\t"
      "v_permlane32_swap_b32 %6, %14\n\t"
      "v_permlane32_swap_b32 %7, %15\n\t"
      "s_nop 1\n\t"
      "v_add_f32 %0, %0, %8\n\t"
      "v_add_f32 %1, %1, %9\n\t"
      "v_add_f32 %2, %2, %10\n\t"
      "v_add_f32 %3, %3, %11\n\t"
      "v_add_f32 %4, %4, %12\n\t"
      "v_add_f32 %5, %5, %13\n\t"
      "v_add_f32 %6, %6, %14\n\t"
      "v_add_f32 %7, %7, %15\n\t"
      "s_nop 1"
      : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), "+v"(x[5]), "+v"(x[6]), "+v"(x[7]), "=&v"(t[0]), "=&v"(t[1]), "=&v"(t[2]), "=&v"(t[3]), "=&v"(t[4]), "=&v"(t[5]), "=&v"(t[6]), "=&v"(t[7]));
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int D, int G, bool SPLIT>
__global__ __launch_bounds__(kThreads) void gqa_partial_po_kernel(const GqaArgs a) {
  const uint16_t* __restrict__ q = static_cast<const uint16_t*>(a.q);
  // Not restrict: a decode step writes one row of each cache before reading.
  const uint16_t* kc = static_cast<const uint16_t*>(a.k);
  const uint16_t* vc = static_cast<const uint16_t*>(a.v);
  float* __restrict__ part_out = a.part_out;
  float* __restrict__ part_lse = a.part_lse;
  const int h_kv = a.h_kv, T_max = a.T_max, P = a.P, NP = a.NP;
  const float qk_scale_log2 = a.qk_scale_log2;
  constexpr int TR = kPoRows;
  constexpr int CH = D / 8;              // 16-byte chunks per row
  constexpr int HC = CH / 2;             // chunks per half row
  constexpr int LPR = CH;                // lanes per row in the V layout
  constexpr int RPI = 64 / LPR;          // rows per wave-wide V load
  constexpr int NV = TR / RPI;           // V loads per tile
  constexpr int KBYTES = TR * D * 2;
  constexpr int NK = KBYTES / 1024;      // K copies per tile (one KiB each)
  constexpr int GP = (G + 3) / 4 * 4;   // weight-table row, padded to whole float4s
  constexpr int WPH = D / 4;             // query words per head and half
  constexpr int QR = G * WPH / 16;       // query registers
  static_assert(NK + NV <= 63, "vmcnt range");

  __shared__ __attribute__((aligned(1024))) unsigned char ktile[kWaves][KBYTES];
  __shared__ __attribute__((aligned(16))) float wtab[kWaves][TR][GP];
  // Per-wave partials of an item, double-buffered by item parity: one
  // barrier per item then keeps a wave that runs ahead from overwriting a
  // buffer that is still being combined.
  __shared__ __attribute__((aligned(16))) float comb[2][kWaves][G][D];
  __shared__ float sm_m[2][kWaves][G];
  __shared__ float sm_l[2][kWaves][G];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform
  const int rr = lane / LPR, c = lane % LPR;
  const int hf = lane >> 5, pr = lane & 31;
  const int H = h_kv * G;
  const bool paged = a.block_table != nullptr;
  const uint32_t kt_lds = __builtin_amdgcn_readfirstlane(lds_addr(&ktile[wave][0]));
  float* wt = &wtab[wave][0][0];

  // K tile -> LDS buffer. Copy i moves rows RPC*i .. RPC*i + RPC - 1 of the
  // tile (one KiB); its lane l fills LDS chunk 64*i + l, i.e. row RPC*i + l / CH,
  // stored chunk l % CH, which carries logical chunk (l % CH) ^ (row % CH).
  // K and V loads use the non-temporal cache policy (every row is read once).
  constexpr int RPC = 1024 / (D * 2);           // rows per copy
  constexpr int KPER = (RPC % CH == 0) ? 1 : CH / RPC;
  uint32_t kvoff[KPER];
#pragma unroll
  for (int mm = 0; mm < KPER; ++mm) {
    const int rl = lane / CH, pc = lane % CH;
    const int lc = pc ^ ((RPC * mm + rl) % CH);
    kvoff[mm] = (uint32_t)(rl * D + lc * 8) * 2u;
  }
  // (M0 is reserved to the compiler, which warns about the clobber; it is
  // kept so that no value of the compiler's own is assumed to survive.)
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
  auto copy_k = [&](const __amdgpu_buffer_rsrc_t& kr, uint32_t tile_off) {
    const uint32_t dst = kt_lds;
#pragma unroll
    for (int i = 0; i < NK; ++i) {
      const uint32_t soff = tile_off + 1024u * i;
      asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen nt lds"
                   ::"s"(dst + 1024u * i), "v"(kvoff[i % KPER]), "s"(kr), "s"(soff)
                   : "memory", "m0");
    }
  };
#pragma clang diagnostic pop
  // V rows -> registers (row layout): load i brings rows i*RPI .. i*RPI+RPI-1.
  const uint32_t vvoff = (uint32_t)(rr * D + c * 8) * 2u;
  auto load_v = [&](const __amdgpu_buffer_rsrc_t& vr_, uint32_t tile_off, int i) {
    const u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(vr_, vvoff, tile_off + 1024u * i, kLoadNonTemporal);
    return make_uint4(w.x, w.y, w.z, w.w);
  };

  // Query words of this lane's half: half-local word w of head h (w < D/4)
  // sits in register (h * D/4 + w) / 16 of lane w % 16 of every 16-lane row of
  // that half, and each dot product fetches it with a row broadcast.
  uint32_t qd[QR];
  int qb = -1, qj = -1;  // (sequence, KV head) whose query qd holds
  int par = 0;           // parity of the current item

  // Tile resources for (sequence bb, KV head jj, attended length nn), tile t0.
  // Contiguous cache: the slab, limited to the sequence's valid rows (a read
  // at or past row nn returns zeros). Paged cache: the tile's 32 rows, which
  // lie in one page (page_size is a multiple of 32 and tiles start at
  // multiples of 32); a table entry outside [0, num_pages) reads as zeros.
  auto rsrc_at = [&](int bb, int jj, int nn, int t0, __amdgpu_buffer_rsrc_t& kr, __amdgpu_buffer_rsrc_t& vr_,
                     uint32_t& toff) {
    if (!paged) {
      const size_t head_off = ((size_t)bb * h_kv + jj) * (size_t)T_max * D;
      kr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(kc + head_off), 0, nn * (D * 2), kBufWord3);
      vr_ = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(vc + head_off), 0, nn * (D * 2), kBufWord3);
      toff = (uint32_t)t0 * (D * 2);
      return;
    }
    const int phys = a.block_table[(size_t)bb * a.max_pages + (t0 >> a.page_shift)];
    const bool ok = phys >= 0 && phys < a.num_pages;
    const int rows = ok ? min(TR, nn - t0) : 0;
    const size_t off = (((size_t)(ok ? phys : 0) * h_kv + jj) * a.page_size + (t0 & (a.page_size - 1))) * D;
    kr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(kc + off), 0, rows * (D * 2), kBufWord3);
    vr_ = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(vc + off), 0, rows * (D * 2), kBufWord3);
    toff = 0;
  };
  // Whether this wave's first K tile of the current item was already
  // requested before the previous item's combine.
  bool k_ahead = false;

  for (items::ItemRun run = items::first_item(a); run.left > 0 && run.b < a.B;) {
    const int b = run.b, j = run.j, p = run.p;
    // Units (or partitions) of (b, j) this item covers: split mode takes all
    // of the run's remaining units of the pair at once.
    const int len = SPLIT ? (int)min((long long)(run.np - run.p), run.left) : 1;
    const int len0 = a.seq_lens[b];
    const int n = attended_len(len0, a.k_new ? 1 : 0, T_max);
    const int start = window_lo(n, a.window) + p * P;
    const int end = min(n - start, len * P) + start;
    if (a.k_new) {  // decode step: the work-group that reads the new row writes it first
      const int pos = max(len0, 0);
      if (pos < T_max && pos >= start && pos < end) {
        const size_t row = (((size_t)b * h_kv + j) * (size_t)T_max + pos) * D;
        const size_t src = ((size_t)b * h_kv + j) * D;
        write_row_then_sync<D * 2>(const_cast<uint16_t*>(kc) + row, static_cast<const uint16_t*>(a.k_new) + src);
        write_row_then_sync<D * 2>(const_cast<uint16_t*>(vc) + row, static_cast<const uint16_t*>(a.v_new) + src);
      }
    }

    if (b != qb || j != qj) {
      const uint32_t* qw = reinterpret_cast<const uint32_t*>(q + ((size_t)b * H + (size_t)j * G) * D);
#pragma unroll
      for (int r = 0; r < QR; ++r) {
        const int wl = 16 * r + (lane & 15);
        qd[r] = qw[(wl / WPH) * (D / 2) + hf * WPH + wl % WPH];
      }
      qb = b;
      qj = j;
      // Wait here, in a form the compiler's own wait counting sees: a query
      // load still counted as pending inside the tile loop would make it wait
      // for the K prefetch as well. (vmcnt(0); the other counters at maximum.)
      __builtin_amdgcn_s_waitcnt(0x0F70);
    }

    float m[G], lpart[G], acc[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      m[h] = kNegInf;
      lpart[h] = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
    }

    for (int t0 = start + wave * TR; t0 < end; t0 += kWaves * TR) {
      __amdgpu_buffer_rsrc_t krt, vrt;
      uint32_t toff;
      rsrc_at(b, j, n, t0, krt, vrt, toff);
      if (!k_ahead) copy_k(krt, toff);
      k_ahead = false;
      uint4 vr[NV];
#pragma unroll
      for (int i = 0; i < NV; ++i) vr[i] = load_v(vrt, toff, i);
      // The K copies were issued first: once at most NV memory operations of
      // this wave are outstanding, they have all landed.
      if constexpr (NV == 8) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(4)" ::: "memory");

      // ---- scores: lane (hf, pr) dots half hf of position t0 + pr.
      const unsigned char* krow = &ktile[wave][0] + pr * (D * 2);
      float s[G];
#pragma unroll
      for (int h = 0; h < G; ++h) s[h] = 0.f;
      constexpr int KS = (G >= 4 && HC >= 8) ? 2 : 1;
      constexpr int CS = HC / KS;
      static_for<KS>([&](auto ks_) {
        constexpr int ks = decltype(ks_)::value;
        uint4 kk[CS];
#pragma unroll
        for (int u = 0; u < CS; ++u)
          kk[u] = *reinterpret_cast<const uint4*>(krow + 16 * ((hf * HC + ks * CS + u) ^ (pr % CH)));
        static_for<CS>([&](auto u_) {
          constexpr int u = decltype(u_)::value;
          constexpr int jc = ks * CS + u;        // chunk within the half
          constexpr int l0 = 4 * (jc % 4);
          uint32_t qr[G];
#pragma unroll
          for (int h = 0; h < G; ++h) qr[h] = qd[(h * WPH + 4 * jc) / 16];
          if constexpr (G == 1) dot_chunk1<l0>(s, qr, kk[u]);
          else if constexpr (G == 2) dot_chunk2<l0>(s, qr, kk[u]);
          else if constexpr (G == 4) dot_chunk4<l0>(s, qr, kk[u]);
          else dot_chunk8<l0>(s, qr, kk[u]);
        });
        __builtin_amdgcn_sched_barrier(0);
      });
      // The K area is rewritten by the next tile's copy: all its reads are done.
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      // Request this wave's next K tile of the item now, so that it overlaps
      // the softmax and the V products below. First wait, in a form the
      // compiler sees, for this tile's V rows (issued with its K): later
      // waits it would place for them could not tell the new copies apart.
      if (t0 + kWaves * TR < end) {
        __builtin_amdgcn_s_waitcnt(0x0F70);
        __amdgpu_buffer_rsrc_t krn, vrn;
        uint32_t toffn;
        rsrc_at(b, j, n, t0 + kWaves * TR, krn, vrn, toffn);
        copy_k(krn, toffn);
        k_ahead = true;
      }
      if constexpr (G == 1) half_sum1(s);
      else if constexpr (G == 2) half_sum2(s);
      else if constexpr (G == 4) half_sum4(s);
      else half_sum8(s);

      const bool valid = t0 + pr < end;
      bool need = false;
      float mx[G];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        s[h] = valid ? s[h] * qk_scale_log2 : kNegInf;
        mx[h] = s[h];
      }
      if constexpr (G == 4) {
        wave_max4(mx);
      } else if constexpr (G == 8) {
        wave_max8(mx);
      } else {
#pragma unroll
        for (int h = 0; h < G; ++h) mx[h] = wave_max(mx[h]);
      }
#pragma unroll
      for (int h = 0; h < G; ++h) need |= mx[h] > m[h] + kTau;
      if (need) {  // wave-uniform: the maxima are wave-wide
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const bool nh = mx[h] > m[h] + kTau;
          const float f = nh ? fast_exp2(m[h] - mx[h]) : 1.f;
          m[h] = nh ? mx[h] : m[h];
          lpart[h] *= f;
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[h][e] *= f;
        }
      }
      // Both halves hold every score; the lanes of half 0 own the weights.
      // A position past the end has score -inf and weight exp2(-inf) = 0 (m
      // is finite: every tile starts at a valid position). Both halves add
      // the same weights to lpart; the final sum is halved (exactly: the two
      // halves reduce identical values in the same order).
      float w[GP];
#pragma unroll
      for (int h = 0; h < GP; ++h) {
        w[h] = h < G ? fast_exp2(s[h < G ? h : 0] - m[h < G ? h : 0]) : 0.f;
        if (h < G) lpart[h] += w[h];
      }
      if (hf == 0) {
#pragma unroll
        for (int h = 0; h < GP; h += 4)
          *reinterpret_cast<float4*>(wt + pr * GP + h) = make_float4(w[h], w[h + 1], w[h + 2], w[h + 3]);
      }

      // ---- output: lane (rr, c) accumulates rows i*RPI + rr, dims 8c .. 8c+7
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const float* wr = wt + (i * RPI + rr) * GP;
        float wv[GP];
#pragma unroll
        for (int h = 0; h < GP; h += 4) {
          const float4 t = *reinterpret_cast<const float4*>(wr + h);
          wv[h] = t.x;
          wv[h + 1] = t.y;
          wv[h + 2] = t.z;
          wv[h + 3] = t.w;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t wd = word(vr[i], e >> 1);
          const float x = (e & 1) ? bf16_hi(wd) : bf16_lo(wd);
#pragma unroll
          for (int h = 0; h < G; ++h) acc[h][e] = fmaf(wv[h], x, acc[h][e]);
        }
      }
    }

    // Request the K rows of this wave's first tile of the next item now, so
    // the copy overlaps the combine below (not in a decode step, whose next
    // item may first have to write its new row).
    items::ItemRun nrun = run;
    bool have_next = run.left > len;
    if (have_next) {
      nrun.p = run.p + len - 1;
      items::next_item(nrun, a);
      have_next = nrun.b < a.B;
    }
    if (have_next && !a.k_new) {
      const int nlen = SPLIT ? (int)min((long long)(nrun.np - nrun.p), run.left - len) : 1;
      const int nn = attended_len(a.seq_lens[nrun.b], 0, T_max);
      const int nstart = window_lo(nn, a.window) + nrun.p * P;
      const int nend = min(nn - nstart, nlen * P) + nstart;
      if (nstart + wave * TR < nend) {
        __amdgpu_buffer_rsrc_t krt, vrt;
        uint32_t toff;
        rsrc_at(nrun.b, nrun.j, nn, nstart + wave * TR, krt, vrt, toff);
        copy_k(krt, toff);
        k_ahead = true;
      }
    }

    // All lanes of a wave share m: the row groups add up (lane swaps, no
    // LDS), the per-position sums add up.
    float L[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      L[h] = 0.5f * wave_sum(lpart[h]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float x = acc[h][e];
        if constexpr (LPR == 8) x += __shfl_xor(x, 8, 64);
        acc[h][e] = xor32_sum(xor16_sum(x));
      }
    }

    // Combine the waves through LDS and write this partition's partial.
    if (lane < LPR) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float4* dst = reinterpret_cast<float4*>(&comb[par][wave][h][c * 8]);
        dst[0] = make_float4(acc[h][0], acc[h][1], acc[h][2], acc[h][3]);
        dst[1] = make_float4(acc[h][4], acc[h][5], acc[h][6], acc[h][7]);
        if (c == 0) {
          sm_m[par][wave][h] = m[h];
          sm_l[par][wave][h] = L[h];
        }
      }
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < G * D; idx += kThreads) {
      const int h = idx / D, d = idx % D;
      float M = sm_m[par][0][h];
#pragma unroll
      for (int w2 = 1; w2 < kWaves; ++w2) M = fmaxf(M, sm_m[par][w2][h]);
      float Ls = 0.f, A = 0.f;
#pragma unroll
      for (int w2 = 0; w2 < kWaves; ++w2) {
        const float mw = sm_m[par][w2][h];
        const float f = (mw == kNegInf) ? 0.f : fast_exp2(mw - M);
        Ls += sm_l[par][w2][h] * f;
        A += comb[par][w2][h][d] * f;
      }
      const size_t row = SPLIT ? (size_t)(blockIdx.x + (long long)b * h_kv + j) * G + h
                               : ((size_t)b * H + (size_t)j * G + h) * NP + p;
      part_out[row * D + d] = A / Ls;
      if (d == 0) part_lse[row] = M + fast_log2(Ls);
    }
    par ^= 1;
    if (!have_next) break;
    nrun.left = run.left - len;
    run = nrun;
  }
}

// Compute units of the current device (looked up once per device).
int device_cus() {
  static std::atomic<int> cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64 && cus[dev].load(std::memory_order_relaxed) > 0) return cus[dev].load(std::memory_order_relaxed);
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (dev < 64) cus[dev].store(n, std::memory_order_relaxed);
  return n;
}

// Work-groups of the persistent kernel one CU holds at once.
template <int D, int G, bool SPLIT>
int po_per_cu() {
  static const int per_cu = [] {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &nb, reinterpret_cast<const void*>(&gqa_partial_po_kernel<D, G, SPLIT>), kThreads, 0) != hipSuccess ||
        nb < 1)
      nb = 1;
    return nb;
  }();
  return per_cu;
}

// The persistent kernel is launched with as many work-groups as the device
// holds at once (never more than there are partitions); each takes an equal
// share of the non-empty partitions.
template <int D, int G>
hipError_t launch_po(const GqaArgs& a, hipStream_t stream) {
  const int cus = device_cus();
  if (cus <= 0) return hipErrorInvalidDevice;
  const long long items = (long long)a.B * a.h_kv * a.NP;
  const int grid = (int)std::min<long long>(items, (long long)cus * po_per_cu<D, G, false>());
  hipLaunchKernelGGL((gqa_partial_po_kernel<D, G, false>), dim3(grid), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

static_assert(kSplitUnit == kWaves * kPoRows, "a split unit is one tile per wave");

// Work-groups per CU of the split launch (at most what the CU holds). At
// g = 8 a wave's arithmetic per byte needs two waves per SIMD to keep up with
// the memory stream (one work-group per CU: 248 us for the 70B-shaped layer,
// two: 186 us); at g <= 4 one work-group per CU, with the longest runs and the
// fewest combines, is fastest (8B-shaped layer: 95 us against 98 with two).
template <int D, int G>
int split_groups_dg() {
  const int cus = device_cus();
  if (cus <= 0) return 0;
  return cus * std::min(G >= 8 ? 2 : 1, po_per_cu<D, G, true>());
}

template <class E, int D, int G>
hipError_t launch_one(const GqaArgs& a, int chunks, hipStream_t stream) {
  GqaArgs b = a;
  b.head_chunks = chunks;
  if ((long long)a.h_kv * chunks > 65535) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((gqa_partial_kernel<E, D, G>), dim3(a.NP, a.h_kv * chunks, a.B), dim3(kThreads), 0, stream, b);
  return hipGetLastError();
}

template <class E, int D>
hipError_t launch_d(int G, const GqaArgs& a, hipStream_t s) {
  if constexpr (sizeof(typename E::storage) == 2) {
    switch (bf16_kernel(D, G, a.block_table ? a.page_size : 0)) {
      case BfKernel::kMma16: return launch_gqa_mma16(D, G, a, 0, false, s);
      case BfKernel::kMatrix: return launch_gqa_matrix(D, G, a, 0, false, s);
      case BfKernel::kPo:
        switch (G) {
          case 1: return launch_po<D, 1>(a, s);
          case 2: return launch_po<D, 2>(a, s);
          case 4: return launch_po<D, 4>(a, s);
          default: return launch_po<D, 8>(a, s);
        }
      default: break;
    }
  }
  switch (G) {
    case 1: return launch_one<E, D, 1>(a, 1, s);
    case 2: return launch_one<E, D, 2>(a, 1, s);
    case 3: return launch_one<E, D, 3>(a, 1, s);
    case 4: return launch_one<E, D, 4>(a, 1, s);
    case 5: return launch_one<E, D, 5>(a, 1, s);
    case 6: return launch_one<E, D, 6>(a, 1, s);
    case 7: return launch_one<E, D, 7>(a, 1, s);
    case 8: return launch_one<E, D, 8>(a, 1, s);
    default:  // groups of 16 or more: chunks of 16 heads
      if (G % 16 != 0) return hipErrorInvalidValue;
      return launch_one<E, D, 16>(a, G / 16, s);
  }
}

// One thread per 16-byte piece of the new rows: piece i of row (b, j) goes to
// row seq_lens[b] of head j of both caches. A full cache is left unchanged.
__global__ __launch_bounds__(256) void kv_append_kernel(const unsigned char* __restrict__ k_new,
                                                        const unsigned char* __restrict__ v_new,
                                                        unsigned char* __restrict__ kc,
                                                        unsigned char* __restrict__ vc,
                                                        const int32_t* __restrict__ seq_lens,
                                                        int B, int h_kv, int row_pieces, int T_max) {
  const int64_t total = (int64_t)B * h_kv * row_pieces;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t bj = t / row_pieces;
    const int piece = (int)(t % row_pieces);
    const int b = (int)(bj / h_kv);
    const int pos = max(seq_lens[b], 0);
    if (pos >= T_max) continue;
    const size_t dst = ((size_t)bj * T_max + pos) * row_pieces * 16 + (size_t)piece * 16;
    const size_t src = (size_t)t * 16;
    st16(kc + dst, ld16(k_new + src));
    st16(vc + dst, ld16(v_new + src));
  }
}

}  // namespace

// The kernel that serves a bf16 shape (page_size 0: contiguous cache). Paged
// caches need pages that hold whole tiles of the kernel: 64, 32 or 16 rows
// for the 16 x 16 matrix-core kernel (groups of up to 16, 32, 64 heads), 32
// rows for the position-per-lane and the 32 x 32 matrix-core kernels.
BfKernel bf16_kernel(int D, int group, int page_size) {
  if (!(D == 64 || D == 128) || !gqa_group_supported(group)) return BfKernel::kGeneric;
  if (!pow2(group))  // groups of 3, 5, 6, 7: the 16 x 16 kernel's masked head columns
    return page_size == 0 || page_size % gqa_mma16_tile(group) == 0 ? BfKernel::kMma16 : BfKernel::kGeneric;
  const bool fits32 = page_size == 0 || page_size % kPoRows == 0;
  if (group >= 8 && group <= 64 && (page_size == 0 || page_size % gqa_mma16_tile(group) == 0))
    return BfKernel::kMma16;
  if (group <= 8 && fits32) return BfKernel::kPo;
  if (group >= 16 && group <= 128 && fits32) return BfKernel::kMatrix;
  return BfKernel::kGeneric;
}

static int po_split_groups(int D, int group) {
  switch (D * 16 + group) {
    case 128 * 16 + 1: return split_groups_dg<128, 1>();
    case 128 * 16 + 2: return split_groups_dg<128, 2>();
    case 128 * 16 + 4: return split_groups_dg<128, 4>();
    case 128 * 16 + 8: return split_groups_dg<128, 8>();
    case 64 * 16 + 1: return split_groups_dg<64, 1>();
    case 64 * 16 + 2: return split_groups_dg<64, 2>();
    case 64 * 16 + 4: return split_groups_dg<64, 4>();
    case 64 * 16 + 8: return split_groups_dg<64, 8>();
    default: return 0;
  }
}

int gqa_split_groups(int D, int group, int page_size) {
  switch (bf16_kernel(D, group, page_size)) {
    case BfKernel::kMma16: return gqa_mma16_groups(D, group);
    case BfKernel::kMatrix: return gqa_matrix_groups(D, group);
    case BfKernel::kPo: return po_split_groups(D, group);
    default: return 0;
  }
}

int gqa_split_groups_max(int D, int group) {
  // contiguous caches and pages of 32 rows (the largest page set that can
  // pick a different kernel)
  return std::max(gqa_split_groups(D, group, 0), gqa_split_groups(D, group, kPoRows));
}

hipError_t launch_gqa_split(int D, int group, const GqaArgs& a, int groups, hipStream_t s) {
  if (groups < 1) return hipErrorInvalidValue;
  switch (bf16_kernel(D, group, a.block_table ? a.page_size : 0)) {
    case BfKernel::kMma16: return launch_gqa_mma16(D, group, a, groups, true, s);
    case BfKernel::kMatrix: return launch_gqa_matrix(D, group, a, groups, true, s);
    case BfKernel::kPo: break;
    default: return hipErrorInvalidValue;
  }
  const dim3 grid((unsigned)groups), block(kThreads);
  switch (D * 16 + group) {
    case 128 * 16 + 1: hipLaunchKernelGGL((gqa_partial_po_kernel<128, 1, true>), grid, block, 0, s, a); break;
    case 128 * 16 + 2: hipLaunchKernelGGL((gqa_partial_po_kernel<128, 2, true>), grid, block, 0, s, a); break;
    case 128 * 16 + 4: hipLaunchKernelGGL((gqa_partial_po_kernel<128, 4, true>), grid, block, 0, s, a); break;
    case 128 * 16 + 8: hipLaunchKernelGGL((gqa_partial_po_kernel<128, 8, true>), grid, block, 0, s, a); break;
    case 64 * 16 + 1: hipLaunchKernelGGL((gqa_partial_po_kernel<64, 1, true>), grid, block, 0, s, a); break;
    case 64 * 16 + 2: hipLaunchKernelGGL((gqa_partial_po_kernel<64, 2, true>), grid, block, 0, s, a); break;
    case 64 * 16 + 4: hipLaunchKernelGGL((gqa_partial_po_kernel<64, 4, true>), grid, block, 0, s, a); break;
    case 64 * 16 + 8: hipLaunchKernelGGL((gqa_partial_po_kernel<64, 8, true>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}


hipError_t launch_gqa_partial(int dt, int D, int group, const GqaArgs& a, hipStream_t s) {
  if (dt == 1) {
    if (D == 128) return launch_d<BF16Elem, 128>(group, a, s);
    if (D == 64) return launch_d<BF16Elem, 64>(group, a, s);
  } else if (dt == 0) {
    if (D == 128) return launch_d<F32Elem, 128>(group, a, s);
    if (D == 64) return launch_d<F32Elem, 64>(group, a, s);
  }
  return hipErrorInvalidValue;
}

namespace {

// One thread per 16-byte piece of a new row: piece i of row (b, head) goes to
// row pos % page_size of page block_table[b][pos / page_size] (and of the
// second page array, when there is one).
__global__ __launch_bounds__(256) void append_paged_kernel(
    const unsigned char* __restrict__ new_a, const unsigned char* __restrict__ new_b,
    unsigned char* __restrict__ pages_a, unsigned char* __restrict__ pages_b,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ seq_lens, int B, int heads,
    int row_pieces, int page_size, int max_pages, int num_pages) {
  const int64_t total = (int64_t)B * heads * row_pieces;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t bh = t / row_pieces;
    const int piece = (int)(t % row_pieces);
    const int b = (int)(bh / heads), h = (int)(bh % heads);
    const int pos = max(seq_lens[b], 0);
    if (pos >= max_pages * page_size) continue;
    const int phys = block_table[(size_t)b * max_pages + pos / page_size];
    if (phys < 0 || phys >= num_pages) continue;
    const size_t dst = ((((size_t)phys * heads + h) * page_size + pos % page_size) * row_pieces + piece) * 16;
    st16(pages_a + dst, ld16(new_a + (size_t)t * 16));
    if (pages_b) st16(pages_b + dst, ld16(new_b + (size_t)t * 16));
  }
}

}  // namespace

hipError_t launch_append_paged(const void* new_a, const void* new_b, void* pages_a, void* pages_b,
                               const int32_t* block_table, const int32_t* seq_lens, int B,
                               int heads, int row_bytes, int page_size, int max_pages,
                               int num_pages, hipStream_t s) {
  const int row_pieces = row_bytes / 16;
  const int64_t total = (int64_t)B * heads * row_pieces;
  const int blocks = (int)std::min<int64_t>((total + 255) / 256, 4096);
  hipLaunchKernelGGL(append_paged_kernel, dim3(blocks), dim3(256), 0, s,
                     static_cast<const unsigned char*>(new_a), static_cast<const unsigned char*>(new_b),
                     static_cast<unsigned char*>(pages_a), static_cast<unsigned char*>(pages_b),
                     block_table, seq_lens, B, heads, row_pieces, page_size, max_pages, num_pages);
  return hipGetLastError();
}

hipError_t launch_kv_append(int dt, const void* k_new, const void* v_new, void* k, void* v,
                            const int32_t* seq_lens, int B, int h_kv, int D, int T_max,
                            hipStream_t s) {
  const int row_pieces = D * (dt == 1 ? 2 : 4) / 16;
  const int64_t total = (int64_t)B * h_kv * row_pieces;
  const int blocks = (int)std::min<int64_t>((total + 255) / 256, 4096);
  hipLaunchKernelGGL(kv_append_kernel, dim3(blocks), dim3(256), 0, s,
                     static_cast<const unsigned char*>(k_new), static_cast<const unsigned char*>(v_new),
                     static_cast<unsigned char*>(k), static_cast<unsigned char*>(v), seq_lens, B, h_kv,
                     row_pieces, T_max);
  return hipGetLastError();
}

}  // namespace attn
