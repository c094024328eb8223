// Decode attention for large query groups (16 to 128 query heads per KV
// head, MQA included) on the gfx950 matrix cores.
//
// Every query head of a group scores against the same K row and averages the
// same V rows ("Attention variants: MQA, GQA, and MLA", sections "MQA: one KV
// head for everyone" and "GQA: interpolating with groups"). With 16 or more
// heads per KV head the two products of a 32-position tile are dense
// contractions over the group:
//
//   S^T [32 positions x 32 heads]  = K_tile [32 x D] . Q^T [D x 32]
//   O^T [D dims x 32 heads]       += V_tile^T [D x 32] . P^T [32 x 32]
//
// on v_mfma_f32_32x32x16_bf16 (the same operand layouts as the absorbed-MLA
// kernel: a lane works for one head, l % 32, and holds 16 of the tile's 32
// positions; lane l ^ 32 holds the other 16). Groups of 16 fill half of the
// 32 head columns; the other half multiplies zeros and is never stored.
//
// A work-group streams K and V tiles of one (sequence, KV head) from HBM once,
// through a ring of four LDS buffers (direct buffer-to-LDS copies, three tiles
// ahead), and all its waves read every tile: a wave owns one block of 32
// heads and some of the D / 32 output tiles of those heads (it recomputes the
// block's scores, which costs D / 16 products per tile, to avoid an exchange
// through LDS). The waves meet once per tile, to recycle the buffers.
//
// Work distribution is that of the persistent position-per-lane kernel
// (split_items.h): resident work-groups take equal runs of 128-position
// units, and each run's part of a (sequence, KV head) row is one partial,
// merged by split_merge_kernel; or, for the explicit-partition entry point,
// runs of whole partitions. The tile stream of a work-group crosses from one
// segment to the next without draining, except when the query block changes.
//
// The weights enter the second product as a pair of bf16 values hi + lo (two
// products on the same V fragment), about 16 significant bits; accumulation
// is fp32. Online softmax in the exp2 domain with the lazy rescale of the
// other kernels (the running maximum moves only when a tile exceeds it by
// more than 8).
//
// LDS layouts (per buffer: the K tile, then the V tile, 32 rows of 2D bytes
// each). 16-byte chunk c of row r is stored at chunk c ^ swk(r) (K) or
// c ^ swv(r) (V). The score reads take one chunk of each of 16 rows per 16
// lanes; swk spreads them over all 64 banks. The transposed V reads
// (ds_read_b64_tr_b16) take 64 bytes of each of 4 rows per 32 lanes; swv puts
// the four 64-byte pieces in different bank quarters.

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

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kTile = 32;   // positions per tile
constexpr int kRing = 4;    // tile buffers; the copy of tile i + 3 overlaps tile i
constexpr float kTau = 8.0f;

template <int D, int G>
struct MxCfg {
  static constexpr int kNH = G <= 32 ? 1 : G / 32;            // 32-head blocks
  static constexpr int kHV = G < 32 ? G : 32;                 // valid heads per block
  static constexpr int kCh = D / 8;                           // 16-byte chunks per row
  static constexpr int kOTiles = D / 32;                      // 32-dim output tiles
  static constexpr int kNDW = (4 / kNH < kOTiles) ? 4 / kNH : kOTiles;  // waves per head block
  static constexpr int kWaves = kNH * kNDW;
  static constexpr int kOT = kOTiles / kNDW;                  // output tiles per wave
  static constexpr int kKSteps = D / 16;                      // k-steps of the score product
  static constexpr int kHalfBytes = kTile * D * 2;            // the K (or V) part of a buffer
  static constexpr int kBufBytes = 2 * kHalfBytes;
  static constexpr int kBlocks = kBufBytes / 1024;            // 1 KiB copies per tile
  static constexpr int kPerWave = kBlocks / kWaves;
  static constexpr int kRowsPerBlock = 1024 / (2 * D);
  static_assert(kBlocks % kWaves == 0 && kPerWave % 2 == 0, "every wave copies as many K as V blocks");
  static_assert(kOTiles % kNDW == 0, "output tiles split evenly over a head block's waves");
};

template <int D>
__device__ __forceinline__ int swk(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
template <int D>
__device__ __forceinline__ int swv(int r) { return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }

// Two fp32 -> packed bf16 pair, round to nearest even.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// The value held by lane l ^ 32.
__device__ __forceinline__ float partner_half(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return (threadIdx.x & 32) ? __uint_as_float(r[0]) : __uint_as_float(r[1]);
}

template <int D, int G, bool SPLIT>
__global__ __launch_bounds__((64 * MxCfg<D, G>::kWaves)) void gqa_matrix_kernel(const GqaArgs a) {
  using C = MxCfg<D, G>;
  const uint16_t* __restrict__ q = static_cast<const uint16_t*>(a.q);
  // Not restrict: a decode step writes one row of each cache before reading it.
  const uint16_t* kc = static_cast<const uint16_t*>(a.k);
  const uint16_t* vc = static_cast<const uint16_t*>(a.v);
  float* __restrict__ part_out = a.part_out;
  float* __restrict__ part_lse = a.part_lse;
  const int h_kv = a.h_kv, T_max = a.T_max, NP = a.NP;
  const int H = h_kv * G;
  const float qk_scale_log2 = a.qk_scale_log2;
  const bool paged = a.block_table != nullptr;

  __shared__ __attribute__((aligned(1024))) unsigned char bufs[kRing][C::kBufBytes];

  items::Cursor cc;  // the tile being computed
  items::cursor_init<SPLIT>(cc, a);
  if (!cc.ok) return;  // an empty run (fewer items than work-groups): uniform exit
  items::Cursor pf = cc;      // the tile being copied, three ahead

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hb = wave / C::kNDW;   // this wave's block of 32 heads
  const int dw = wave % C::kNDW;   // its output tiles: [dw * kOT, (dw + 1) * kOT)
  const int half = lane >> 5, col = lane & 31;
  const bool hvalid = col < C::kHV;
  const int hg = hb * 32 + col;    // head within the group

  // Byte offsets (within a tile of the K or V cache) of the 16-byte chunks
  // this lane copies: block k = wave + kWaves * m, K for m < kPerWave / 2.
  uint32_t voff[C::kPerWave];
#pragma unroll
  for (int m = 0; m < C::kPerWave; ++m) {
    const bool isv = m >= C::kPerWave / 2;
    const int k = wave + C::kWaves * m - (isv ? C::kBlocks / 2 : 0);
    const int r = k * C::kRowsPerBlock + lane / C::kCh, pc = lane % C::kCh;
    const int lc = pc ^ (isv ? swv<D>(r) : swk<D>(r));
    voff[m] = (uint32_t)(r * D + 8 * lc) * 2u;
  }

  // Buffer resources of a tile: contiguous cache, the (sequence, KV head)
  // slab limited to its attended rows (reads at or past row n return zeros);
  // paged cache, the tile's 32 rows inside its page. Past the run's end a
  // null resource keeps the number of copies per tile fixed.
  auto tile_src = [&](const items::Cursor& c, __amdgpu_buffer_rsrc_t& kr, __amdgpu_buffer_rsrc_t& vr,
                      uint32_t& soff) {
    if (!c.ok) {
      kr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(kc), 0, 0, kBufWord3);
      vr = kr;
      soff = 0;
      return;
    }
    const int b = c.run.b, j = c.run.j;
    if (!paged) {
      const size_t head_off = ((size_t)b * h_kv + j) * (size_t)T_max * D;
      kr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(kc + head_off), 0, c.n * (D * 2), kBufWord3);
      vr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(vc + head_off), 0, c.n * (D * 2), kBufWord3);
      soff = (uint32_t)c.t0 * (D * 2);
      return;
    }
    const int phys = items::sload_i32(a.block_table + (size_t)b * a.max_pages + (c.t0 >> a.page_shift));
    const bool ok = phys >= 0 && phys < a.num_pages;
    const int rows = ok ? min(kTile, c.n - c.t0) : 0;
    const size_t off = (((size_t)(ok ? phys : 0) * h_kv + j) * a.page_size + (c.t0 & (a.page_size - 1))) * D;
    kr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(kc + off), 0, rows * (D * 2), kBufWord3);
    vr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(vc + off), 0, rows * (D * 2), kBufWord3);
    soff = 0;
  };

  // The copies of one tile into a buffer: kPerWave 1 KiB blocks per wave,
  // buffer_load_dwordx4 ... lds (M0 holds the LDS address; the compiler is
  // told M0 is clobbered, and it uses M0 for nothing else here), with the
  // non-temporal cache policy (`nt`: every row is read once per call).
  auto issue_tile = [&](unsigned char* buf, const items::Cursor& c) {
    __amdgpu_buffer_rsrc_t kr, vr;
    uint32_t soff;
    tile_src(c, kr, vr, soff);
    const uint32_t base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)buf;
#pragma unroll
    for (int m = 0; m < C::kPerWave; ++m) {
      const uint32_t dst = __builtin_amdgcn_readfirstlane(base + 1024u * (uint32_t)(wave + C::kWaves * m));
      const __amdgpu_buffer_rsrc_t rs = m < C::kPerWave / 2 ? kr : vr;
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
      asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen nt lds"
                   ::"s"(dst), "v"(voff[m]), "s"(rs), "s"(soff) : "memory", "m0");
#pragma clang diagnostic pop
    }
  };

  // Decode step: the work-group whose segment holds the new row writes it
  // (K and V) before any copy of the segment's tiles is issued.
  auto write_new_row = [&](const items::Cursor& c) {
    if (!a.k_new || !c.ok) return;
    const int pos = max(c.len0, 0);
    if (pos < T_max && pos >= c.start && pos < c.end) {
      const int b = c.run.b, j = c.run.j;
      const size_t row = (((size_t)b * h_kv + j) * (size_t)T_max + pos) * D;
      const size_t src = ((size_t)b * h_kv + j) * D;
      write_row_then_sync<D * 2>(const_cast<uint16_t*>(kc) + row, static_cast<const uint16_t*>(a.k_new) + src);
      write_row_then_sync<D * 2>(const_cast<uint16_t*>(vc) + row, static_cast<const uint16_t*>(a.v_new) + src);
    }
  };
  auto copy_and_advance = [&](unsigned char* buf) {
    issue_tile(buf, pf);
    if (pf.ok && items::cursor_next<SPLIT, kTile>(pf, a) && pf.ok) write_new_row(pf);
  };

  write_new_row(pf);
  copy_and_advance(bufs[0]);
  copy_and_advance(bufs[1]);
  copy_and_advance(bufs[2]);

  // Query fragments of this wave's heads: B operand of the score product,
  // lane l holds dims 16 ks + 8 (l / 32) .. + 7 of head l % 32.
  uint4 qf[C::kKSteps];
  int qb = -1, qj = -1;

  const int g16 = lane >> 4, i16 = lane & 15;
  const int tr_row = 4 * (g16 >> 1) + (i16 >> 2);
  const int tr_col = 16 * (g16 & 1) + 4 * (i16 & 3);

  f32x16 acc[C::kOT];
#pragma unroll
  for (int t = 0; t < C::kOT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[t][r] = 0.f;
  float m = kNegInf, lsum = 0.f;

  int cur = 0;
  while (cc.ok) {
    if (cc.run.b != qb || cc.run.j != qj) {
      qb = cc.run.b;
      qj = cc.run.j;
      const uint16_t* qrow = q + ((size_t)qb * H + (size_t)qj * G + hg) * D + 8 * half;
#pragma unroll
      for (int ks = 0; ks < C::kKSteps; ++ks) qf[ks] = hvalid ? ld16(qrow + 16 * ks) : make_uint4(0u, 0u, 0u, 0u);
      // vmcnt(0) in a form the compiler's wait counting sees (it also waits
      // for the copies in flight: once per query block).
      __builtin_amdgcn_s_waitcnt(0x0F70);
    }
    // This wave's copies of the current tile have landed once at most the
    // next two tiles' copies are outstanding; after the barrier every wave's
    // have, and every wave is done with the buffer the next copy overwrites.
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"i"(2 * C::kPerWave) : "memory");
    copy_and_advance(bufs[(cur + kRing - 1) & (kRing - 1)]);

    const uint16_t* kt = reinterpret_cast<const uint16_t*>(bufs[cur]);
    const uint16_t* vt = reinterpret_cast<const uint16_t*>(bufs[cur] + C::kHalfBytes);
    const int t0 = cc.t0, end = cc.end;

    // ---- scores S^T = K . Q^T over the D dims
    f32x16 s;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < C::kKSteps; ++ks) {
      const uint4 av = *reinterpret_cast<const uint4*>(kt + col * D + 8 * ((2 * ks + half) ^ swk<D>(col)));
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av),
                                                   __builtin_bit_cast(bf16x8, qf[ks]), s, 0, 0, 0);
    }

    // ---- online softmax for head `col` over this tile's positions
    float x[16];
    float mt = kNegInf;
    const bool full = t0 + kTile <= end;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int pos = t0 + 8 * (r >> 2) + 4 * half + (r & 3);
      x[r] = (full || pos < end) ? s[r] * qk_scale_log2 : kNegInf;
      mt = fmaxf(mt, x[r]);
    }
    mt = fmaxf(mt, partner_half(mt));
    const bool need = mt > m + kTau;
    if (__any(need)) {
      const float f = need ? fast_exp2(m - mt) : 1.f;
      m = need ? mt : m;
      lsum *= f;
#pragma unroll
      for (int t = 0; t < C::kOT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[t][r] *= f;
    }
    uint32_t ph[8], pl[8];
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const float p0 = fast_exp2(x[r] - m), p1 = fast_exp2(x[r + 1] - m);
      lsum += p0 + p1;
      const uint32_t h = pack_bf16x2(p0, p1);
      ph[r >> 1] = h;
      pl[r >> 1] = pack_bf16x2(p0 - bf16_lo(h), p1 - bf16_hi(h));
    }

    // ---- O^T += V^T . P^T for this wave's output tiles (two k-steps of 16 positions)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const bf16x8 pbh = __builtin_bit_cast(bf16x8, make_uint4(ph[4 * ks], ph[4 * ks + 1], ph[4 * ks + 2], ph[4 * ks + 3]));
      const bf16x8 pbl = __builtin_bit_cast(bf16x8, make_uint4(pl[4 * ks], pl[4 * ks + 1], pl[4 * ks + 2], pl[4 * ks + 3]));
      const int rlo = 16 * ks + tr_row;
#pragma unroll
      for (int tt = 0; tt < C::kOT; ++tt) {
        const int ce = 32 * (dw * C::kOT + tt) + tr_col;  // logical element of the row
        const uint16_t* plo = vt + rlo * D + 8 * ((ce >> 3) ^ swv<D>(rlo)) + (ce & 7);
        const uint16_t* phi = plo + 8 * D;                 // row + 8: same swizzle
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)plo);
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)phi);
        uint4 av;
        av.x = __builtin_bit_cast(uint2, lo).x;
        av.y = __builtin_bit_cast(uint2, lo).y;
        av.z = __builtin_bit_cast(uint2, hi).x;
        av.w = __builtin_bit_cast(uint2, hi).y;
        const bf16x8 aw = __builtin_bit_cast(bf16x8, av);
        acc[tt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aw, pbh, acc[tt], 0, 0, 0);
        acc[tt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aw, pbl, acc[tt], 0, 0, 0);
      }
    }

    if (t0 + kTile >= end) {
      // ---- end of the segment: normalised partial output and log2-sum-exp
      const float lt = lsum + partner_half(lsum);
      const float inv = 1.f / lt;
      if (hvalid) {
        const int b = cc.run.b, j = cc.run.j;
        const size_t row = SPLIT ? (size_t)(blockIdx.x + (long long)b * h_kv + j) * G + hg
                                 : ((size_t)b * H + (size_t)j * G + hg) * NP + cc.run.p;
#pragma unroll
        for (int tt = 0; tt < C::kOT; ++tt) {
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const int d0 = 32 * (dw * C::kOT + tt) + 8 * g4 + 4 * half;
            *reinterpret_cast<float4*>(part_out + row * D + d0) =
                make_float4(acc[tt][4 * g4] * inv, acc[tt][4 * g4 + 1] * inv, acc[tt][4 * g4 + 2] * inv,
                            acc[tt][4 * g4 + 3] * inv);
          }
        }
        if (dw == 0 && half == 0) part_lse[row] = m + fast_log2(lt);
      }
      m = kNegInf;
      lsum = 0.f;
#pragma unroll
      for (int t = 0; t < C::kOT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[t][r] = 0.f;
    }
    items::cursor_next<SPLIT, kTile>(cc, a);
    cur = (cur + 1) & (kRing - 1);
  }
  // The copies issued for the last tiles (zeros into free buffers) land
  // before the work-group ends.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// Compute units of the current device and resident work-groups per CU of a
// kernel (each read once).
int mx_device_cus() {
  static std::atomic<int> cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64 && cus[dev].load(std::memory_order_relaxed) > 0) return cus[dev].load(std::memory_order_relaxed);
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (dev < 64) cus[dev].store(n, std::memory_order_relaxed);
  return n;
}

template <int D, int G, bool SPLIT>
int mx_per_cu() {
  static const int per_cu = [] {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, reinterpret_cast<const void*>(&gqa_matrix_kernel<D, G, SPLIT>),
                                                     64 * MxCfg<D, G>::kWaves, 0) != hipSuccess ||
        nb < 1)
      nb = 1;
    return nb;
  }();
  return per_cu;
}

template <int D, int G, bool SPLIT>
hipError_t launch_mx(const GqaArgs& a, int groups, hipStream_t s) {
  hipLaunchKernelGGL((gqa_matrix_kernel<D, G, SPLIT>), dim3((unsigned)groups), dim3(64 * MxCfg<D, G>::kWaves), 0,
                     s, a);
  return hipGetLastError();
}

// Calls f with the group size as a compile-time constant (16, 32, 64 or 128).
template <class F>
auto by_group(int group, F&& f) {
  switch (group) {
    case 16: return f(std::integral_constant<int, 16>{});
    case 32: return f(std::integral_constant<int, 32>{});
    case 64: return f(std::integral_constant<int, 64>{});
    default: return f(std::integral_constant<int, 128>{});
  }
}

}  // namespace

int gqa_matrix_groups(int D, int group) {
  const int cus = mx_device_cus();
  if (cus <= 0 || !gqa_matrix(1, D, group)) return 0;
  auto f = [&](auto g) {
    constexpr int G = decltype(g)::value;
    return D == 128 ? cus * mx_per_cu<128, G, true>() : cus * mx_per_cu<64, G, true>();
  };
  return by_group(group, f);
}

hipError_t launch_gqa_matrix(int D, int group, const GqaArgs& a, int groups, bool split, hipStream_t s) {
  if (!gqa_matrix(1, D, group)) return hipErrorInvalidValue;
  if (groups <= 0) {  // fixed partitions: as many work-groups as the device holds, at most one per item
    const int cus = mx_device_cus();
    if (cus <= 0) return hipErrorInvalidDevice;
    auto f = [&](auto g) {
      constexpr int G = decltype(g)::value;
      return D == 128 ? mx_per_cu<128, G, false>() : mx_per_cu<64, G, false>();
    };
    const long long items = (long long)a.B * a.h_kv * a.NP;
    groups = (int)std::min<long long>(items, (long long)cus * by_group(group, f));
  }
  auto f = [&](auto g) {
    constexpr int G = decltype(g)::value;
    if (D == 128) return split ? launch_mx<128, G, true>(a, groups, s) : launch_mx<128, G, false>(a, groups, s);
    return split ? launch_mx<64, G, true>(a, groups, s) : launch_mx<64, G, false>(a, groups, s);
  };
  return by_group(group, f);
}

}  // namespace attn
