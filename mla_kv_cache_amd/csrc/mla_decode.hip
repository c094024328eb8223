// Absorbed multi-head latent attention, split-KV decode, on gfx950 MFMA.
//
// After the key up-projection is absorbed into the query, every head scores
// against the SAME cached row per token (latent c of d_c = 512 values, then
// a decoupled rotary key of d_r = 64 values) and averages the latents
// ("Attention variants: MQA, GQA, and MLA", section "MLA: cache a latent,
// not the keys and values"). Many heads share one wide row, so the two
// products are dense contractions and run on the matrix cores:
//
//   S^T [32 positions x 32 heads]  = L_tile [32 x 576] . Q^T [576 x 32]
//   O^T [512 dims x 32 heads]     += L_tile^T [512 x 32] . P^T [32 x 32]
//
// One work-group owns (sequence b, head block of up to 128 heads, partition
// p) and runs one wave per 32 heads (four for 128 heads, one per SIMD). Each
// wave does the whole 576-wide score contraction and all 512 output dims for
// its heads, so waves never exchange scores; they meet once per tile, to
// recycle the tile buffers. A wave holds its 36 query fragments (144 VGPRs)
// and 16 output tiles (256 AGPRs) for the whole partition.
//
// The latent tile (32 positions x 576) is copied from HBM straight into LDS
// (buffer loads with the lds flag, no register staging) into a ring of four
// buffers: the copies of the next three tiles are in flight while one is
// computed, their blocks issued between the output products. HBM
// sees every cached row of the partition once. Rows are 1152 bytes with
// 16-byte chunks XOR-swizzled per row, which keeps both read patterns below
// free of bank conflicts on the 64-bank LDS.
//
// MFMA 32x32x16 bf16 operand layout (lane l): A[m][k] holds m = l % 32,
// k = 8*(l/32) + j; B[k][n] holds n = l % 32, k = 8*(l/32) + j; result
// register r holds row 8*(r/4) + 4*(l/32) + r%4, column l % 32. So in S^T
// and O^T every lane works for exactly one head (l % 32): the softmax state
// is lane-local apart from one exchange with lane l ^ 32, which holds the
// other 16 positions of the same head.
//
// P^T enters the second product as the B operand straight from the S^T
// result registers: over the positions the contraction index may be
// permuted, provided A uses the same order, and A = L^T is read with the
// LDS transpose load (ds_read_b64_tr_b16), whose 16-lane groups deliver
// lane i, slot j from source lane 4j + i/4, slot i%4.
//
// The weights enter the second product as a pair of bf16 values hi + lo
// (two MFMAs on the same latent fragment), so they carry about 16 significant
// bits instead of bf16's 8; accumulation is fp32 throughout. Online softmax in
// the exp2 domain with the same lazy rescale rule as the GQA kernel (only when
// a tile's maximum exceeds the running one by more than 8).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_util.h"
#include "launch.h"

namespace attn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kDc = 512;
constexpr int kDr = 64;
constexpr int kRow = kDc + kDr;            // 576 bf16 per cached token
constexpr int kTile = 32;                  // positions per tile
constexpr int kSteps = kRow / 16;          // 36 k-steps of the score product
constexpr int kOTiles = kDc / 32;          // 16 output tiles of 32 latent dims
constexpr float kTau = 8.0f;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// The value held by lane l ^ 32 (v_permlane32_swap exchanges the two halves of
// the wave; each lane ends with its own value and its partner's).
__device__ __forceinline__ float partner_half(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const float a = __uint_as_float(r[0]), b = __uint_as_float(r[1]);
  return (threadIdx.x & 32) ? a : b;
}

// Tile layout in LDS: rows of 72 16-byte chunks (1152 bytes, no padding),
// logical chunk c of row r stored at chunk c ^ sw(r), with sw(r) the
// bit-reversed value of (r / 2) % 8. On the 64-bank LDS this spreads both
// read patterns: the score reads (one chunk of each of 32 rows) and the
// transposed output reads (64 bytes of each of 4 rows per half-wave).
__device__ __forceinline__ int tile_sw(int r) {
  const int x = (r >> 1) & 7;
  return ((x & 1) << 2) | (x & 2) | ((x >> 2) & 1);
}
constexpr int kRowChunks = kRow / 8;                     // 72
constexpr int kTileBlocks = kTile * kRowChunks / 64;     // 36 blocks of 1 KiB

// Copy blocks per tile for a work-group of NWAVES waves: rounded up so every
// wave issues the same number of copies (the extra blocks land in slack space
// at the end of the buffer); the per-wave count is what s_waitcnt vmcnt waits on.
template <int NWAVES>
struct TileCopy {
  static constexpr int kPerWave = (kTileBlocks + NWAVES - 1) / NWAVES;
  static constexpr int kBlocks = kPerWave * NWAVES;
  static constexpr int kBufBytes = kBlocks * 1024;
};

// Copy block k of a latent tile (32 rows from byte offset `soff` of the
// buffer `rsrc`) into an LDS buffer. Lane i of block k fills LDS chunk 64k + i
// = (row, pc) from logical chunk pc ^ sw(row) of that row; voff is that
// chunk's byte offset within the tile (tile_voffsets). Rows at or past the
// resource's num_records bytes arrive as zeros.
//
// The copy uses the non-temporal cache policy (`nt`: every latent row is read
// once per call) and is issued as buffer_load_dwordx4 ... lds in inline assembly: it
// writes no register, only LDS, and M0 holds the block's LDS address (no
// other code in these kernels uses M0). Written this way the compiler does not
// insert a wait for the copy before every later LDS read (it cannot prove that
// the reads touch another buffer); the kernel waits for the copies itself
// (s_waitcnt vmcnt before the barrier that opens a tile).
// M0 is a reserved register to the compiler, which warns when an assembly
// block names it as clobbered; the clobber is kept so that the compiler never
// assumes a value of its own survives the block.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
template <int NWAVES>
__device__ __forceinline__ void copy_block(unsigned char* buf, __amdgpu_buffer_rsrc_t rsrc, uint32_t soff,
                                           uint32_t voff, int wave, int k) {
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)buf;
  const uint32_t dst = __builtin_amdgcn_readfirstlane(lds0 + 1024u * (uint32_t)(wave + NWAVES * k));
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen nt lds"
               ::"s"(dst), "v"(voff), "s"(rsrc), "s"(soff) : "memory", "m0");
}
#pragma clang diagnostic pop

template <int NWAVES>
__device__ __forceinline__ void copy_tile(unsigned char* buf, __amdgpu_buffer_rsrc_t rsrc, uint32_t soff,
                                          const uint32_t (&voff)[TileCopy<NWAVES>::kPerWave], int wave) {
#pragma unroll
  for (int k = 0; k < TileCopy<NWAVES>::kPerWave; ++k) copy_block<NWAVES>(buf, rsrc, soff, voff[k], wave, k);
}

// Byte offsets within a tile of the chunks this lane copies (see copy_block);
// lanes of slack blocks past the tile read row 0 into the slack space.
template <int NWAVES>
__device__ __forceinline__ void tile_voffsets(uint32_t (&voff)[TileCopy<NWAVES>::kPerWave], int wave, int lane) {
#pragma unroll
  for (int k = 0; k < TileCopy<NWAVES>::kPerWave; ++k) {
    const int ci = 64 * (wave + NWAVES * k) + lane;
    const int row = ci / kRowChunks, pc = ci % kRowChunks;
    voff[k] = row < kTile ? (uint32_t)(row * kRow + 8 * (pc ^ tile_sw(row))) * 2u : 0u;
  }
}

// Wait until this wave's copies of the current tile have landed while the
// copies of the next two tiles (N of them, issued later) may still be in
// flight, then barrier: afterwards every wave's copies of the current tile are
// in LDS and every wave is done with the tile before it. The counter holds at
// most 63; a smaller bound only waits longer.
template <int N>
__device__ __forceinline__ void wait_tile_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"i"(N > 63 ? 63 : N) : "memory");
}

// acc *= f on an accumulator tile that lives in AGPRs, in place, through one
// temporary VGPR. Written as assembly because the compiler, asked for a
// vector multiply of the whole tile, keeps VGPR copies of all 16 tiles and
// spills; the caller waits out the matrix-core write latency first.
__device__ __forceinline__ void scale_acc(f32x16& acc, float f) {
  float e[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) e[r] = acc[r];
  float t;
#pragma unroll
  for (int r = 0; r < 16; r += 4)
    asm volatile(
        "v_accvgpr_read_b32 %4, %0\n\tv_mul_f32 %4, %4, %5\n\tv_accvgpr_write_b32 %0, %4\n\t"
        "v_accvgpr_read_b32 %4, %1\n\tv_mul_f32 %4, %4, %5\n\tv_accvgpr_write_b32 %1, %4\n\t"
        "v_accvgpr_read_b32 %4, %2\n\tv_mul_f32 %4, %4, %5\n\tv_accvgpr_write_b32 %2, %4\n\t"
        "v_accvgpr_read_b32 %4, %3\n\tv_mul_f32 %4, %4, %5\n\tv_accvgpr_write_b32 %3, %4\n\t"
        "s_nop 1"
        : "+a"(e[r]), "+a"(e[r + 1]), "+a"(e[r + 2]), "+a"(e[r + 3]), "=&v"(t) : "v"(f));
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = e[r];
}

// Read-ahead depths of the two products (operand reads issued before the
// products that consume them; limited by the registers left beside the query
// fragments and the accumulators).
constexpr int kQkAhead = 6;
constexpr int kPvAhead = 3;
// Tile buffers in the ring: tile i sits in buffer i % 4, and the copy of tile
// i + 3 goes into the buffer of tile i - 1.
constexpr int kRing = 4;

// One wave per 32 heads, each with the whole 576-wide score contraction and
// all 512 output dims (see the file comment). NW waves (NW * 32 heads) share
// each latent tile; the kernel runs one wave per SIMD, and the matrix cores
// are kept busy by operand reads issued ahead of the products.
template <int NW, bool PAGED>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mla_partial_kernel(const MlaArgs a) {
  const uint16_t* __restrict__ q_nope = static_cast<const uint16_t*>(a.q_nope);
  const uint16_t* __restrict__ q_rope = static_cast<const uint16_t*>(a.q_rope);
  // Not restrict: a decode step writes one row of the cache before reading.
  const uint16_t* lat = static_cast<const uint16_t*>(a.latent);
  float* __restrict__ part_out = a.part_out;
  float* __restrict__ part_lse = a.part_lse;
  const int H = a.H, T_max = a.T_max, P = a.P, NP = a.NP;
  const float qk_scale_log2 = a.qk_scale_log2;
  using TC = TileCopy<NW>;
  __shared__ __attribute__((aligned(1024))) unsigned char bufs[kRing][TC::kBufBytes];

  // Work-group L of the 1-D grid serves (partition p, head block hb,
  // sequence b). Work-groups are handed to the 8 XCDs in turn (L % 8), each
  // with its own L2; when the grid allows, the NP partitions of one
  // (sequence, head block) get consecutive slots of one XCD, so the query
  // block they all read comes from that L2 after the first read.
  const int L = blockIdx.x, NHBK = H / (32 * NW);
  int p, hb, b;
  if (gridDim.x % (8 * NP) == 0) {
    const int x = L % 8, slot = L / 8;
    const int g = (slot / NP) * 8 + x;
    p = slot % NP;
    hb = g % NHBK;
    b = g / NHBK;
  } else {
    p = L % NP;
    hb = (L / NP) % NHBK;
    b = L / (NP * NHBK);
  }
  const int len0 = a.seq_lens[b];
  const int n = attended_len(len0, a.lat_new ? 1 : 0, T_max);
  const int start = p * P;
  if (start >= n) return;
  const int end = min(start, n - P) + P;
  if (a.lat_new) {  // decode step: every work-group that reads the new row writes it first
    const int pos = max(len0, 0);
    if (pos < T_max && pos >= start && pos < end)
      write_row_then_sync<kRow * 2>(const_cast<uint16_t*>(lat) + ((size_t)b * T_max + pos) * kRow,
                                    static_cast<const uint16_t*>(a.lat_new) + (size_t)b * kRow);
  }

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;          // which 16 of a tile's 32 positions this lane holds
  const int col = lane & 31;           // this lane's head within the wave's 32
  const int head = hb * (32 * NW) + wave * 32 + col;

  // Latent tiles are read through a buffer resource. Contiguous cache: the
  // sequence's rows up to its attended length n (rows past n arrive as zeros),
  // tile t0 at byte offset 1152 t0. Paged cache: the tile's rows inside its
  // page (pages hold whole tiles: page_size and P are multiples of 32).
  uint32_t voff[TC::kPerWave];
  tile_voffsets<NW>(voff, wave, lane);
  const __amdgpu_buffer_rsrc_t lat_rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(lat + (PAGED ? 0 : (size_t)b * T_max * kRow)), 0,
                                        PAGED ? 0 : n * (kRow * 2), kBufWord3);
  // Resource and offset for the copy of the tile at t0. Past the partition's
  // end: a null resource (num_records 0), whose copy only writes zeros into a
  // free buffer, so that every tile issues the same number of copies.
  auto tile_src = [&](int t0, __amdgpu_buffer_rsrc_t& r, uint32_t& soff) {
    if (t0 >= end) {
      r = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(lat), 0, 0, kBufWord3);
      soff = 0;
    } else if constexpr (PAGED) {
      // The table entry is read with a scalar load (waited for at once):
      // as a vector load, the compiler's wait for it would also wait for
      // every tile copy in flight, which it does not know about.
      const int32_t* ent = a.block_table + (size_t)b * a.max_pages + (t0 >> a.page_shift);
      int raw;
      asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(raw) : "s"(ent) : "memory");
      const int phys = min(max(raw, 0), a.num_pages - 1);
      const uint16_t* base = lat + ((size_t)phys * a.page_size + (t0 & (a.page_size - 1))) * kRow;
      r = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base), 0, min(kTile, n - t0) * (kRow * 2),
                                            kBufWord3);
      soff = 0;
    } else {
      r = lat_rsrc;
      soff = (uint32_t)t0 * (kRow * 2);
    }
  };

  {  // the first three tiles, in flight together with the query loads
    __amdgpu_buffer_rsrc_t r;
    uint32_t soff;
    tile_src(start, r, soff);
    copy_tile<NW>(bufs[0], r, soff, voff, wave);
    tile_src(start + kTile, r, soff);
    copy_tile<NW>(bufs[1], r, soff, voff, wave);
    tile_src(start + 2 * kTile, r, soff);
    copy_tile<NW>(bufs[2], r, soff, voff, wave);
  }

  // Query fragments for all 576 score dims.
  uint4 qf[kSteps];
  {
    const uint16_t* qn = q_nope + ((size_t)b * H + head) * kDc;
    const uint16_t* qr = q_rope + ((size_t)b * H + head) * kDr;
#pragma unroll
    for (int ks = 0; ks < kSteps; ++ks) {
      const int d = 16 * ks + 8 * half;
      qf[ks] = d < kDc ? ld16(qn + d) : ld16(qr + (d - kDc));
    }
    // Wait for the query (and this wave's first copies) here, in a form the
    // compiler's own wait counting sees (vmcnt(0), the other counters at
    // maximum): otherwise it waits for the query inside the tile loop with
    // counts that also cover the tile copies in flight, which would stall
    // every tile on its successors' copies.
    __builtin_amdgcn_s_waitcnt(0x0F70);
  }
  f32x16 acc[kOTiles];
#pragma unroll
  for (int t = 0; t < kOTiles; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[t][r] = 0.f;
  float m = kNegInf, lsum = 0.f;


  const int g16 = lane >> 4, i16 = lane & 15;
  const int tr_row = 4 * (g16 >> 1) + (i16 >> 2);
  const int tr_col = 16 * (g16 & 1) + 4 * (i16 & 3);
  // Swizzle offsets (bf16 units) that depend on the lane only. The score read
  // of step ks takes qoff[ks % 4]; the output read of tile t and row half h
  // (rows + 8h) takes poff[h][t % 2]. Rows 16ks + tr_row + 8h have the same
  // swizzle for both ks.
  int qoff[4], poff[2][2];
#pragma unroll
  for (int k3 = 0; k3 < 4; ++k3) qoff[k3] = 8 * ((2 * k3 + half) ^ tile_sw(col));
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int t1 = 0; t1 < 2; ++t1)
      poff[h][t1] = 8 * ((4 * t1 + (tr_col >> 3)) ^ tile_sw(8 * h + tr_row)) + (tr_col & 7);

  auto tile = [&](const unsigned char* __restrict__ cur_b, unsigned char* __restrict__ nxt_b, int t0) {
    const uint16_t* cur = reinterpret_cast<const uint16_t*>(cur_b);
    wait_tile_barrier<(kRing - 2) * TC::kPerWave>();
    // The copy of the tile three ahead (a null copy past the end) goes into
    // the buffer of the tile before this one; its blocks are issued between
    // the output products below.
    __amdgpu_buffer_rsrc_t r3;
    uint32_t soff3;
    tile_src(t0 + 3 * kTile, r3, soff3);

    // ---- scores S^T = L . Q^T over all 576 dims
    f32x16 s;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.f;
    const uint16_t* arow = cur + col * kRow;
    // The operand reads run kQkAhead steps ahead of the products that use
    // them: the schedule below asks for reads, then one product per read.
#pragma unroll
    for (int ks = 0; ks < kSteps; ++ks) {
      // chunk 2ks + half of row col sits at 8 * (ks / 4) + qoff[ks % 4]
      const uint4 av = *reinterpret_cast<const uint4*>(arow + 64 * (ks >> 2) + qoff[ks & 3]);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av),
                                                   __builtin_bit_cast(bf16x8, qf[ks]), s, 0, 0, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, kQkAhead, 0);
#pragma unroll
    for (int i = 0; i < kSteps - kQkAhead; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, kQkAhead, 0);
    __builtin_amdgcn_sched_barrier(0);

    // ---- online softmax for head `col` over this tile's positions
    float x[16];
    float mt = kNegInf;
    if (t0 + kTile <= end) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        x[r] = s[r] * qk_scale_log2;
        mt = fmaxf(mt, x[r]);
      }
    } else {  // the last tile of the partition: positions past `end` get no weight
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int pos = t0 + 8 * (r >> 2) + 4 * half + (r & 3);
        x[r] = pos < end ? s[r] * qk_scale_log2 : kNegInf;
        mt = fmaxf(mt, x[r]);
      }
    }
    mt = fmaxf(mt, partner_half(mt));
    const bool need = mt > m + kTau;
    if (__any(need)) {
      const float f = need ? fast_exp2(m - mt) : 1.f;
      // Before a head's first weight its accumulators are still zero (m is
      // -inf); the first tile needs no rescale.
      const bool scale = __any(need && m != kNegInf);
      m = need ? mt : m;
      lsum *= f;
      if (scale) {
        // Matrix-core results are read back only after the wait states the
        // hardware requires (this path is rare; see scale_acc).
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
        for (int t = 0; t < kOTiles; ++t) scale_acc(acc[t], f);
      }
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

    // ---- O^T += L^T . P^T over all 512 output dims (two k-steps of 16 positions)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const bf16x8 pbh = __builtin_bit_cast(bf16x8, make_uint4(ph[4 * ks], ph[4 * ks + 1], ph[4 * ks + 2], ph[4 * ks + 3]));
      const bf16x8 pbl = __builtin_bit_cast(bf16x8, make_uint4(pl[4 * ks], pl[4 * ks + 1], pl[4 * ks + 2], pl[4 * ks + 3]));
      const uint16_t* base = cur + (16 * ks + tr_row) * kRow;
      const uint16_t* base_hi = base + 8 * kRow;
#pragma unroll
      for (int t = 0; t < kOTiles; ++t) {
        // chunk 4t + tr_col / 8 of the row sits at 8 * (t / 2) + poff[.][t % 2]
        const uint16_t* plo = base + 64 * (t >> 1) + poff[0][t & 1];
        const uint16_t* phi = base_hi + 64 * (t >> 1) + poff[1][t & 1];
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)plo);
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)phi);
        // Copy block j goes out after the reads of output step
        // kPvAhead + 29 j / kPerWave: LDS reads do not cross the copies (asm
        // statements), so each lands between two pairs of products and the
        // copy path never stalls the wave for a whole tile's worth of copies.
#pragma unroll
        for (int j = 0; j < TC::kPerWave; ++j)
          if (kPvAhead + (j * (2 * kOTiles - kPvAhead)) / TC::kPerWave == kOTiles * ks + t)
            copy_block<NW>(nxt_b, r3, soff3, voff[j], wave, j);
        uint4 av;
        av.x = __builtin_bit_cast(uint2, lo).x;
        av.y = __builtin_bit_cast(uint2, lo).y;
        av.z = __builtin_bit_cast(uint2, hi).x;
        av.w = __builtin_bit_cast(uint2, hi).y;
        const bf16x8 aw = __builtin_bit_cast(bf16x8, av);
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aw, pbh, acc[t], 0, 0, 0);
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aw, pbl, acc[t], 0, 0, 0);
      }
      // The operand reads of kPvAhead output tiles run ahead of the products.
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * kPvAhead, 0);
#pragma unroll
      for (int i = 0; i < kOTiles - kPvAhead; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 2 * kPvAhead, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // The copy of tile i + 3 goes into the buffer of tile i - 1, which every
  // wave has finished with at tile i's barrier.
  int cur = 0;
  for (int t0 = start; t0 < end; t0 += kTile) {
    const int nxt = (cur + kRing - 1) & (kRing - 1);
    tile(bufs[cur], bufs[nxt], t0);
    cur = (cur + 1) & (kRing - 1);
  }
  // The copies issued during the last three tiles (zeros into free buffers)
  // land before the work-group can end.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // Lanes l and l^32 share a head and a running maximum; add their sums.
  lsum += partner_half(lsum);
  const float inv = 1.f / lsum;
  const size_t prow = ((size_t)b * H + head) * NP + p;

  // The partial output goes out through LDS, one 32-dim slice at a time, so
  // that every store instruction writes whole 128-byte lines (8 heads x 32
  // dims) instead of 32-byte pieces of 32 rows. The stores use the default
  // cache policy: the merge that runs next reads them back faster than after
  // non-temporal stores (measured 15.6 against 17.1 us per merge; the bytes
  // it fetches past the L2 are the same, so the gain lies beyond the L2, most
  // likely in the last-level cache).
  // The staging area is this wave's own blocks of the buffer after the last
  // tile's: no other wave reads that buffer any more, and this wave's copies
  // into it have landed. In block k, head 8k + c holds the eight 16-byte
  // pieces of its 32 dims in chunks 8c .. 8c + 7, piece x at chunk
  // 8c + (x ^ phi(8k + c)): with phi below, the 16 lanes of each write
  // group (16 heads, one piece each) land in 16 different bank groups.
  static_assert(TC::kPerWave >= 4, "the staging area is four of this wave's copy blocks");
  unsigned char* stage = bufs[cur];
  auto phi = [](int c) { return ((c >> 1) & 3) | (((c >> 3) & 1) << 2); };
  const int sh = lane >> 3, sc = lane & 7;  // the head (within 8) and stored piece this lane reads
  const int wphi = phi(col);
  const size_t prow0 = ((size_t)b * H + hb * (32 * NW) + wave * 32) * NP + p;
#pragma unroll
  for (int t = 0; t < kOTiles; ++t) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      float4* dst = reinterpret_cast<float4*>(stage + 1024 * (wave + NW * (col >> 3)) +
                                              16 * (8 * (col & 7) + ((2 * g + half) ^ wphi)));
      *dst = make_float4(acc[t][4 * g] * inv, acc[t][4 * g + 1] * inv, acc[t][4 * g + 2] * inv,
                         acc[t][4 * g + 3] * inv);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(stage + 1024 * (wave + NW * k) + 16 * lane);
      float* po = part_out + (prow0 + (size_t)(8 * k + sh) * NP) * kDc + 32 * t + 4 * (sc ^ phi(8 * k + sh));
      *reinterpret_cast<f32x4*>(po) = v;
    }
  }
  if (half == 0) part_lse[prow] = m + fast_log2(lsum);
}

}  // namespace


template <bool PAGED>
hipError_t launch_mla_nhb(const MlaArgs& a, hipStream_t stream) {
  const int nhb = a.H >= 128 ? 4 : a.H / 32;  // 32-head blocks (waves) per work-group
  const long long groups = (long long)a.NP * (a.H / (32 * nhb)) * a.B;
  if (groups > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)groups);
  switch (nhb) {
    case 4: hipLaunchKernelGGL((mla_partial_kernel<4, PAGED>), grid, dim3(256), 0, stream, a); break;
    case 3: hipLaunchKernelGGL((mla_partial_kernel<3, PAGED>), grid, dim3(192), 0, stream, a); break;
    case 2: hipLaunchKernelGGL((mla_partial_kernel<2, PAGED>), grid, dim3(128), 0, stream, a); break;
    default: hipLaunchKernelGGL((mla_partial_kernel<1, PAGED>), grid, dim3(64), 0, stream, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_mla_partial(const MlaArgs& a, hipStream_t stream) {
  return a.block_table ? launch_mla_nhb<true>(a, stream) : launch_mla_nhb<false>(a, stream);
}

namespace {

// One thread per 16-byte piece of the new rows: row b goes to row seq_lens[b]
// of sequence b. A full cache is left unchanged.
__global__ __launch_bounds__(256) void latent_append_kernel(const unsigned char* __restrict__ lat_new,
                                                            unsigned char* __restrict__ lat,
                                                            const int32_t* __restrict__ seq_lens,
                                                            int B, int row_pieces, int T_max) {
  const int64_t total = (int64_t)B * row_pieces;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * blockDim.x) {
    const int b = (int)(t / row_pieces);
    const int piece = (int)(t % row_pieces);
    const int pos = max(seq_lens[b], 0);
    if (pos >= T_max) continue;
    st16(lat + ((size_t)b * T_max + pos) * row_pieces * 16 + (size_t)piece * 16, ld16(lat_new + (size_t)t * 16));
  }
}

}  // namespace

hipError_t launch_latent_append(const void* lat_new, void* latent, const int32_t* seq_lens, int B,
                                int row_elems, int T_max, hipStream_t stream) {
  const int row_pieces = row_elems * 2 / 16;
  const int64_t total = (int64_t)B * row_pieces;
  const int blocks = (int)((total + 255) / 256 < 4096 ? (total + 255) / 256 : 4096);
  hipLaunchKernelGGL(latent_append_kernel, dim3(blocks), dim3(256), 0, stream,
                     static_cast<const unsigned char*>(lat_new), static_cast<unsigned char*>(latent),
                     seq_lens, B, row_pieces, T_max);
  return hipGetLastError();
}

}  // namespace attn
