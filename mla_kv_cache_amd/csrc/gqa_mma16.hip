// Decode attention for the GQA family on 16 x 16 matrix-core tiles (gfx950),
// groups of 1 to 64 query heads per KV head (bf16).
//
// Every query head of a group scores against the same K rows and averages the
// same V rows ("Attention variants: MQA, GQA, and MLA", sections "GQA:
// interpolating with groups" and "MQA: one KV head for everyone"). For a
// sub-tile of 16 cached positions and a block of 16 heads of the group:
//
//   S^T [16 positions x 16 heads]  = K [16 x D] . Q^T [D x 16]    (16x16x32 bf16, D / 32 steps)
//   O^T [D x 16 heads]            += V^T [D x 16] . P^T [16 x 16]  (16x16x16 bf16, D / 16 tiles)
//
// A group of fewer than 16 heads fills part of the head columns (the rest
// multiply zeros and are never stored); on these tiles the products cost a
// few hundred matrix-core cycles per 8 KiB of K and V, far below the time
// HBM takes to deliver them, and the softmax handles 4 values per lane.
//
// Work-group: 4 waves (8 at G = 32); nb = max(1, G / 16) blocks of 16 heads,
// ns = waves / nb sub-tiles per tile. A tile is 16 ns positions of one (sequence, KV head),
// copied from HBM once into a ring of four LDS buffers (buffer-to-LDS copies,
// three tiles ahead), and wave w takes head block w % nb and sub-tile w / nb:
// every score and weight is computed once. The waves meet once per tile, to
// recycle the buffers, and at the end of a segment the ns waves of a head
// block combine their (max, sum, accumulator) through LDS.
//
// Work distribution and partials are those of the other persistent GQA
// kernels (split_items.h): the work-balanced split (one partial per
// work-group and (sequence, KV head) segment, merged by split_merge_kernel)
// or fixed partitions.
//
// Weights enter the second product as bf16 hi + lo (about 16 significant
// bits); accumulation is fp32; online softmax in the exp2 domain with the
// lazy rescale of the other kernels (the running maximum moves only when a
// tile exceeds it by more than 8).
//
// LDS: each buffer holds the tile's K rows, then its V rows (2D bytes each).
// 16-byte chunk c of row r is stored at c ^ swk(r) (K) or c ^ swv(r) (V):
// the score reads (one chunk of 16 rows per 16 lanes) and the transposed V
// reads (32 bytes of 8 rows per 32 lanes, ds_read_b64_tr_b16) then each
// touch all 64 banks once.

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
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kRing = 4;
constexpr float kTau = 8.0f;

template <int D, int G>
struct M16 {
  // Waves per work-group: 4, or 8 at G = 32 (one work-group per CU with two
  // waves per SIMD, 64-position tiles).
  static constexpr int kWaves = G == 32 ? 8 : 4;
  static constexpr int kNB = G <= 16 ? 1 : G / 16;      // blocks of 16 heads
  static constexpr int kHV = G < 16 ? G : 16;           // valid heads per block
  static constexpr int kNS = kWaves / kNB;              // 16-position sub-tiles per tile
  static constexpr int kTP = 16 * kNS;                  // positions per tile
  static constexpr int kCh = D / 8;                     // 16-byte chunks per row
  static constexpr int kKSteps = D / 32;                // 16x16x32 steps of the score product
  static constexpr int kOT = D / 16;                    // 16-dim output tiles
  static constexpr int kHalfBytes = kTP * D * 2;        // K (or V) part of a buffer
  static constexpr int kBufBytes = 2 * kHalfBytes;
  static constexpr int kBlocks = kBufBytes / 1024;      // 1 KiB copies per tile
  static constexpr int kPerWave = kBlocks / kWaves;
  static constexpr int kRowsPerBlock = 1024 / (2 * D);
  static constexpr int kPitch = D * 4 + 16;             // combine-area row (fp32, padded)
  static constexpr int kAreas = kNS == 4 ? 2 : (kNS == 2 ? 1 : 0);  // the head blocks of ns = 2 take turns
  static_assert(kNB * kNS == kWaves, "waves = head blocks x sub-tiles");
  static_assert(kBlocks % kWaves == 0, "every wave copies the same number of blocks");
};

template <int D>
__device__ __forceinline__ int swk(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
template <int D>
__device__ __forceinline__ int swv(int r) { return D == 128 ? 2 * (r & 7) : 2 * ((r >> 1) & 3); }

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Maximum / sum over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (the lanes of one head).
__device__ __forceinline__ float head_max(float x) { return xor32_max(xor16_max(x)); }
__device__ __forceinline__ float head_sum(float x) { return xor32_sum(xor16_sum(x)); }

template <int D, int G, bool SPLIT>
__global__ __launch_bounds__((64 * M16<D, G>::kWaves)) void gqa_mma16_kernel(const GqaArgs a) {
  using C = M16<D, G>;
  constexpr int kWaves = C::kWaves;
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
  __shared__ __attribute__((aligned(16))) unsigned char area[C::kAreas > 0 ? C::kAreas : 1][16 * C::kPitch];
  __shared__ float sm_m[kWaves][16], sm_l[kWaves][16];

  items::Cursor cc;
  items::cursor_init<SPLIT>(cc, a);
  if (!cc.ok) return;  // an empty run: uniform exit
  items::Cursor pf = cc;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hb = wave % C::kNB;    // head block
  const int st = wave / C::kNB;    // sub-tile within the tile
  const int col = lane & 15, grp = lane >> 4;
  const bool hvalid = col < C::kHV;
  const int hg = hb * 16 + col;    // head within the group

  // Copy offsets: block k = wave + kWaves * m of the tile (K blocks first).
  uint32_t voff[C::kPerWave];
  bool visv[C::kPerWave];
#pragma unroll
  for (int m = 0; m < C::kPerWave; ++m) {
    const int k0 = wave + kWaves * m;
    const bool isv = k0 >= C::kBlocks / 2;
    const int k = isv ? k0 - C::kBlocks / 2 : k0;
    const int r = k * C::kRowsPerBlock + lane / C::kCh, pc = lane % C::kCh;
    const int lc = pc ^ (isv ? swv<D>(r) : swk<D>(r));
    voff[m] = (uint32_t)(r * D + 8 * lc) * 2u;
    visv[m] = isv;
  }

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
    // Paged: page_size is a multiple of the tile, so the tile lies in one page.
    const int phys = items::sload_i32(a.block_table + (size_t)b * a.max_pages + (c.t0 >> a.page_shift));
    const bool ok = phys >= 0 && phys < a.num_pages;
    const int rows = ok ? min(C::kTP, c.n - c.t0) : 0;
    const size_t off = (((size_t)(ok ? phys : 0) * h_kv + j) * a.page_size + (c.t0 & (a.page_size - 1))) * D;
    kr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(kc + off), 0, rows * (D * 2), kBufWord3);
    vr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(vc + off), 0, rows * (D * 2), kBufWord3);
    soff = 0;
  };

  // The copies of one tile into a buffer, with the non-temporal cache policy
  // (`nt`: every row is read once per call).
  auto issue_tile = [&](unsigned char* buf, const items::Cursor& c) {
    __amdgpu_buffer_rsrc_t kr, vr;
    uint32_t soff;
    tile_src(c, kr, vr, soff);
    const uint32_t base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)buf;
#pragma unroll
    for (int m = 0; m < C::kPerWave; ++m) {
      const uint32_t dst = __builtin_amdgcn_readfirstlane(base + 1024u * (uint32_t)(wave + kWaves * m));
      const __amdgpu_buffer_rsrc_t rs = visv[m] ? vr : kr;
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
      asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen nt lds"
                   ::"s"(dst), "v"(voff[m]), "s"(rs), "s"(soff) : "memory", "m0");
#pragma clang diagnostic pop
    }
  };

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
    if (pf.ok && items::cursor_next<SPLIT, C::kTP>(pf, a) && pf.ok) write_new_row(pf);
  };

  write_new_row(pf);
  copy_and_advance(bufs[0]);
  copy_and_advance(bufs[1]);
  copy_and_advance(bufs[2]);

  // Query of this wave's heads: B operand of the score product, lane l holds
  // dims 32 ks + 8 (l / 16) .. + 7 of head l % 16 of the block.
  uint4 qf[C::kKSteps];
  int qb = -1, qj = -1;

  f32x4 acc[C::kOT];
#pragma unroll
  for (int t = 0; t < C::kOT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = kNegInf, lsum = 0.f;

  // Transposed V read of lane (grp, i): row 4 grp + i / 4 of the sub-tile,
  // elements 4 (i % 4) .. + 3 of each 16-dim output tile.
  const int vrow = 16 * st + 4 * grp + (col >> 2);
  const int krow = 16 * st + col;

  int cur = 0;
  while (cc.ok) {
    if (cc.run.b != qb || cc.run.j != qj) {
      qb = cc.run.b;
      qj = cc.run.j;
      const uint16_t* qrow = q + ((size_t)qb * H + (size_t)qj * G + hg) * D + 8 * grp;
#pragma unroll
      for (int ks = 0; ks < C::kKSteps; ++ks) qf[ks] = hvalid ? ld16(qrow + 32 * ks) : make_uint4(0u, 0u, 0u, 0u);
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), seen by the compiler (once per query block)
    }
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"i"(2 * C::kPerWave) : "memory");
    copy_and_advance(bufs[(cur + kRing - 1) & (kRing - 1)]);

    const unsigned char* kt = bufs[cur];
    const unsigned char* vt = bufs[cur] + C::kHalfBytes;
    const int t0 = cc.t0 + 16 * st, end = cc.end;

    if (t0 < end) {  // this wave's sub-tile holds positions
      // ---- scores S^T = K . Q^T
      f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < C::kKSteps; ++ks) {
        const uint4 av = *reinterpret_cast<const uint4*>(kt + krow * (2 * D) + 16 * ((4 * ks + grp) ^ swk<D>(krow)));
        s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av),
                                                     __builtin_bit_cast(bf16x8, qf[ks]), s, 0, 0, 0);
      }
      // ---- online softmax for head `col` over the sub-tile's 16 positions
      float x[4];
      float mt = kNegInf;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int pos = t0 + 4 * grp + r;
        x[r] = pos < end ? s[r] * qk_scale_log2 : kNegInf;
        mt = fmaxf(mt, x[r]);
      }
      mt = head_max(mt);
      const bool need = mt > m + kTau;
      if (__any(need)) {
        const float f = need ? fast_exp2(m - mt) : 1.f;
        m = need ? mt : m;
        lsum *= f;
#pragma unroll
        for (int t = 0; t < C::kOT; ++t) acc[t] *= f;
      }
      float p[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[r] = fast_exp2(x[r] - m);
        lsum += p[r];
      }
      const uint32_t h01 = pack_bf16x2(p[0], p[1]), h23 = pack_bf16x2(p[2], p[3]);
      const uint32_t l01 = pack_bf16x2(p[0] - bf16_lo(h01), p[1] - bf16_hi(h01));
      const uint32_t l23 = pack_bf16x2(p[2] - bf16_lo(h23), p[3] - bf16_hi(h23));
      const i16x4 pbh = __builtin_bit_cast(i16x4, make_uint2(h01, h23));
      const i16x4 pbl = __builtin_bit_cast(i16x4, make_uint2(l01, l23));

      // ---- O^T += V^T . P^T, one 16-dim output tile per product pair
#pragma unroll
      for (int t = 0; t < C::kOT; ++t) {
        const int ce = 16 * t + 4 * (col & 3);
        const i16x4 av = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)(vt + vrow * (2 * D) + 16 * ((ce >> 3) ^ swv<D>(vrow)) + 2 * (ce & 7)));
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, pbh, acc[t], 0, 0, 0);
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, pbl, acc[t], 0, 0, 0);
      }
    }

    if (cc.t0 + C::kTP >= end) {
      // ---- end of the segment: the ns waves of each head block combine
      const float lt = head_sum(lsum);
      if (grp == 0) {
        sm_m[wave][col] = m;
        sm_l[wave][col] = lt;
      }
      __syncthreads();
      float M = kNegInf;
#pragma unroll
      for (int s2 = 0; s2 < C::kNS; ++s2) M = fmaxf(M, sm_m[hb + C::kNB * s2][col]);
      float L = 0.f;
#pragma unroll
      for (int s2 = 0; s2 < C::kNS; ++s2) {
        const float mw = sm_m[hb + C::kNB * s2][col];
        L += mw == kNegInf ? 0.f : sm_l[hb + C::kNB * s2][col] * fast_exp2(mw - M);
      }
      const float f = (m == kNegInf ? 0.f : fast_exp2(m - M)) / L;
#pragma unroll
      for (int t = 0; t < C::kOT; ++t) acc[t] *= f;
      // acc now holds this wave's share of the normalised output.
      auto put = [&](int ar) {
        unsigned char* base = area[ar] + col * C::kPitch + 16 * grp;
#pragma unroll
        for (int t = 0; t < C::kOT; ++t) *reinterpret_cast<f32x4*>(base + 64 * t) = acc[t];
      };
      auto add = [&](int ar) {
        const unsigned char* base = area[ar] + col * C::kPitch + 16 * grp;
#pragma unroll
        for (int t = 0; t < C::kOT; ++t) acc[t] += *reinterpret_cast<const f32x4*>(base + 64 * t);
      };
      if constexpr (C::kNS == 4 && C::kNB == 1) {
        if (st >= 2) put(st - 2);
        __syncthreads();
        if (st < 2) add(st);
        __syncthreads();
        if (st == 1) put(0);
        __syncthreads();
        if (st == 0) add(0);
      } else if constexpr (C::kNS == 4) {
        // two areas, the head blocks in turn
#pragma unroll
        for (int hb2 = 0; hb2 < C::kNB; ++hb2) {
          if (hb == hb2 && st >= 2) put(st - 2);
          __syncthreads();
          if (hb == hb2 && st < 2) add(st);
          __syncthreads();
          if (hb == hb2 && st == 1) put(0);
          __syncthreads();
          if (hb == hb2 && st == 0) add(0);
          __syncthreads();
        }
      } else if constexpr (C::kNS == 2) {
        // one area, the head blocks in turn (keeps two work-groups per CU)
#pragma unroll
        for (int hb2 = 0; hb2 < C::kNB; ++hb2) {
          if (st == 1 && hb == hb2) put(0);
          __syncthreads();
          if (st == 0 && hb == hb2) add(0);
          __syncthreads();
        }
      }
      if (st == 0 && hvalid) {
        const int b = cc.run.b, j = cc.run.j;
        const size_t row = SPLIT ? (size_t)(blockIdx.x + (long long)b * h_kv + j) * G + hg
                                 : ((size_t)b * H + (size_t)j * G + hg) * NP + cc.run.p;
        // lane (grp, col) holds dims 16 t + 4 grp .. + 3 of head hg
#pragma unroll
        for (int t = 0; t < C::kOT; ++t)
          *reinterpret_cast<f32x4*>(part_out + row * D + 16 * t + 4 * grp) = acc[t];
        if (grp == 0) part_lse[row] = M + fast_log2(L);
      }
      // The combine area and the (max, sum) table are reused by the next
      // segment only after the next tile's barrier.
      m = kNegInf;
      lsum = 0.f;
#pragma unroll
      for (int t = 0; t < C::kOT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    items::cursor_next<SPLIT, C::kTP>(cc, a);
    cur = (cur + 1) & (kRing - 1);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

int m16_device_cus() {
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
int m16_per_cu() {
  static const int per_cu = [] {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, reinterpret_cast<const void*>(&gqa_mma16_kernel<D, G, SPLIT>),
                                                     64 * M16<D, G>::kWaves, 0) != hipSuccess ||
        nb < 1)
      nb = 1;
    return nb;
  }();
  return per_cu;
}

template <class F>
auto by_group16(int group, F&& f) {
  switch (group) {
    case 1: return f(std::integral_constant<int, 1>{});
    case 2: return f(std::integral_constant<int, 2>{});
    case 3: return f(std::integral_constant<int, 3>{});
    case 4: return f(std::integral_constant<int, 4>{});
    case 5: return f(std::integral_constant<int, 5>{});
    case 6: return f(std::integral_constant<int, 6>{});
    case 7: return f(std::integral_constant<int, 7>{});
    case 8: return f(std::integral_constant<int, 8>{});
    case 16: return f(std::integral_constant<int, 16>{});
    case 32: return f(std::integral_constant<int, 32>{});
    default: return f(std::integral_constant<int, 64>{});
  }
}

}  // namespace

int gqa_mma16_tile(int group) {
  return by_group16(group, [](auto g) { return M16<128, decltype(g)::value>::kTP; });
}

int gqa_mma16_groups(int D, int group) {
  const int cus = m16_device_cus();
  if (cus <= 0) return 0;
  auto f = [&](auto g) {
    constexpr int G = decltype(g)::value;
    return D == 128 ? cus * m16_per_cu<128, G, true>() : cus * m16_per_cu<64, G, true>();
  };
  return by_group16(group, f);
}

hipError_t launch_gqa_mma16(int D, int group, const GqaArgs& a, int groups, bool split, hipStream_t s) {
  if (groups <= 0) {
    const int cus = m16_device_cus();
    if (cus <= 0) return hipErrorInvalidDevice;
    auto f = [&](auto g) {
      constexpr int G = decltype(g)::value;
      return D == 128 ? m16_per_cu<128, G, false>() : m16_per_cu<64, G, false>();
    };
    const long long items = (long long)a.B * a.h_kv * a.NP;
    groups = (int)std::min<long long>(items, (long long)cus * by_group16(group, f));
  }
  auto f = [&](auto g) {
    constexpr int G = decltype(g)::value;
    const dim3 grid((unsigned)groups), block(64 * M16<128, G>::kWaves);
    if (D == 128) {
      if (split) hipLaunchKernelGGL((gqa_mma16_kernel<128, G, true>), grid, block, 0, s, a);
      else hipLaunchKernelGGL((gqa_mma16_kernel<128, G, false>), grid, block, 0, s, a);
    } else {
      if (split) hipLaunchKernelGGL((gqa_mma16_kernel<64, G, true>), grid, block, 0, s, a);
      else hipLaunchKernelGGL((gqa_mma16_kernel<64, G, false>), grid, block, 0, s, a);
    }
    return hipGetLastError();
  };
  return by_group16(group, f);
}

}  // namespace attn
