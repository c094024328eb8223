// The two per-head matrix products on either side of the absorbed MLA decode
// ("Attention variants: MQA, GQA, and MLA", section "MLA: cache a latent, not
// the keys and values", decode sketch), on the gfx950 matrix cores:
//
//   absorb:  q_lat[b, h, c] = sum_d q[b, h, d]     * W_UK[h, c, d]    (W_UK [H, d_c, d_h])
//   up:      o[b, h, d]     = sum_c o_lat[b, h, c] * W_UV[h, c, d]    (W_UV [H, d_c, d_v])
//
// Both are batched over heads with the decode batch B as the M dimension.
// v_mfma_f32_32x32x16_bf16 operands (lane l): A[m][k] holds m = l % 32,
// k = 8*(l/32) + j; B[k][n] holds n = l % 32, k = 8*(l/32) + j; result
// register r holds row 8*(r/4) + 4*(l/32) + r%4, column l % 32.
//
// absorb: A = q rows (k = d contiguous) and B = W_UK rows (k = d contiguous):
// 16-byte fragments, W_UK's straight from memory, q's from rows staged in LDS
// (shared by the work-group's waves).
// up: A = o_lat rows (k = c contiguous), but B = W_UV is contiguous along n
// (= d), not along the contraction. Tiles of W_UV go to LDS, and the B
// fragments are read back transposed with ds_read_b64_tr_b16 (in each
// 16-lane group, output lane i, slot j comes from source lane 4j + i/4,
// slot i % 4: a lane addressing row k0 + s/4, columns n0 + 4*(s%4) .. + 3
// delivers, to lane i, column n0 + i of rows k0 .. k0 + 3).
// Accumulation is fp32; outputs are bf16, rounded to nearest even.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_util.h"
#include "launch.h"

namespace attn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kWavesPerGroup = 4;
constexpr int kMTilesPerPass = 2;  // 32-row M tiles accumulated at once (64 registers)
constexpr int kChunk = 8;          // k-steps whose operand loads are issued together

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& u) { return __builtin_bit_cast(bf16x8, u); }

__device__ __forceinline__ void store_tile(uint16_t* __restrict__ out, const f32x16& acc, int mt, int B,
                                           size_t row_stride, int n0, int lane) {
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int m = mt * 32 + 8 * (r / 4) + 4 * (lane / 32) + (r % 4);
    if (m < B) out[(size_t)m * row_stride + n0 + (lane % 32)] = f32_to_bf16_rne(acc[r]);
  }
}

// Query rows staged per work-group: kMTilesPerPass tiles of 32 rows, one
// chunk of the contraction (kChunk k-steps of 16) at a time; the row pitch is
// padded by 16 bytes so that the 16-byte fragment reads of 16 consecutive
// rows fall on 64 distinct banks.
constexpr int kAqPitch = 16 * kChunk * 2 + 16;
// 16-byte query pieces each thread stages per chunk
constexpr int kAqStage = 32 * kMTilesPerPass * 2 * kChunk / (64 * kWavesPerGroup);
static_assert(kAqStage * 64 * kWavesPerGroup == 32 * kMTilesPerPass * 2 * kChunk, "whole pieces per thread");

// One wave per 32 latent columns c of one head; all of B in passes of
// kMTilesPerPass tiles of 32 rows. The four waves of a work-group share the
// head's query rows, which are staged in LDS once per chunk (with the
// W_UK fragment loads of every wave already in flight) instead of being read
// by each wave. Rows past B read zeros and are not stored.
__global__ __launch_bounds__(64 * kWavesPerGroup) void absorb_q_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ w_uk, uint16_t* __restrict__ q_lat,
    int B, int H, int d_h, int d_c) {
  __shared__ __attribute__((aligned(16))) unsigned char qs[32 * kMTilesPerPass * kAqPitch];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int h = blockIdx.y;
  const int n0 = (blockIdx.x * kWavesPerGroup + wave) * 32;
  const bool active = n0 < d_c;  // waves past d_c still take part in the staging
  const int ko = 8 * (lane / 32);
  const uint16_t* wrow = w_uk + ((size_t)h * d_c + n0 + (lane % 32)) * d_h + ko;
  bool staged = false;
  for (int mt0 = 0; mt0 * 32 < B; mt0 += kMTilesPerPass) {
    f32x16 acc[kMTilesPerPass];
#pragma unroll
    for (int t = 0; t < kMTilesPerPass; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[t][r] = 0.f;
    for (int kb = 0; kb < d_h; kb += 16 * kChunk) {
      uint4 bw[kChunk];
#pragma unroll
      for (int i = 0; i < kChunk; ++i) {
        const int k0 = kb + 16 * i;
        bw[i] = (active && k0 < d_h) ? ld16(wrow + k0) : make_uint4(0, 0, 0, 0);
      }
      // this thread's query pieces: every load issued before the first store
      // (one memory round trip, not one per piece)
      uint4 qv[kAqStage];
#pragma unroll
      for (int it = 0; it < kAqStage; ++it) {
        const int i = threadIdx.x + it * 64 * kWavesPerGroup;
        const int r = i / (2 * kChunk), c = i % (2 * kChunk);
        const int m = mt0 * 32 + r, k = kb + 8 * c;
        qv[it] = (m < B && k < d_h) ? ld16(q + ((size_t)m * H + h) * d_h + k) : make_uint4(0, 0, 0, 0);
      }
      if (staged) __syncthreads();  // the previous chunk's reads are done
#pragma unroll
      for (int it = 0; it < kAqStage; ++it) {
        const int i = threadIdx.x + it * 64 * kWavesPerGroup;
        const int r = i / (2 * kChunk), c = i % (2 * kChunk);
        *reinterpret_cast<uint4*>(qs + r * kAqPitch + 16 * c) = qv[it];
      }
      __syncthreads();
      staged = true;
      if (active) {
#pragma unroll
        for (int i = 0; i < kChunk; ++i) {
          if (kb + 16 * i >= d_h) break;
#pragma unroll
          for (int t = 0; t < kMTilesPerPass; ++t) {
            const uint4 aq = *reinterpret_cast<const uint4*>(qs + (t * 32 + lane % 32) * kAqPitch + 2 * (16 * i + ko));
            acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(aq), as_bf16x8(bw[i]), acc[t], 0, 0, 0);
          }
        }
      }
    }
    if (active) {
#pragma unroll
      for (int t = 0; t < kMTilesPerPass; ++t)
        if ((mt0 + t) * 32 < B) store_tile(q_lat + (size_t)h * d_c, acc[t], mt0 + t, B, (size_t)H * d_c, n0, lane);
    }
  }
}

constexpr int kUpColW = 2;                      // 32-column halves of a work-group's columns
constexpr int kUpKSplit = 4;                    // parts of the contraction, one wave each
constexpr int kUpWaves = kUpColW * kUpKSplit;   // waves per work-group (two per SIMD)
constexpr int kUpCols = 32 * kUpColW;           // W_UV columns per work-group (128-byte row pieces)
constexpr int kUpPitch = kUpCols * 2 + 32;      // bytes per LDS row: padding spreads the transposed reads
constexpr int kUpMaxRows = 512;                 // the whole contraction of one head fits in LDS
constexpr int kUpPartSteps = kUpMaxRows / 16 / kUpKSplit;  // 16-row k-steps of a wave's part (at most)
// 16-byte W_UV pieces each thread stages per piece of the contraction (at most)
constexpr int kUpStage = kUpMaxRows * (kUpCols / 8) / (64 * kUpWaves);
static_assert(kUpStage * 64 * kUpWaves == kUpMaxRows * (kUpCols / 8), "whole pieces per thread");

// One work-group per (head, 64 output columns); wave w takes the 32 columns
// of half w % 2 and part w / 2 of the contraction. The head's W_UV slice
// [d_c x 64] goes to LDS at once, with every wave's o_lat fragment loads
// already in flight (one memory round trip for both), each wave multiplies
// its part, and the four parts of a column half are added in LDS in a fixed
// order (part 0 + 1 + 2 + 3) by the part-0 wave, which stores the result.
// d_c > 512 takes the slice in pieces of 512 rows.
__global__ __launch_bounds__(64 * kUpWaves) void up_v_kernel(
    const uint16_t* __restrict__ o_lat, const uint16_t* __restrict__ w_uv, uint16_t* __restrict__ out,
    int B, int H, int d_c, int d_v) {
  __shared__ __attribute__((aligned(16))) unsigned char wt[kUpMaxRows * kUpPitch];
  // partial sums of parts 1..3: [half][part - 1][M tile][register][lane]
  __shared__ __attribute__((aligned(16))) float red[kUpColW][kUpKSplit - 1][kMTilesPerPass][16][64];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int ch = wave % kUpColW, kq = wave / kUpColW;
  const int h = blockIdx.y;
  const int cols = min(kUpCols, d_v - blockIdx.x * kUpCols);   // a multiple of 32
  const int c0 = blockIdx.x * kUpCols;                           // first output column of the group
  const int n0 = ch * 32;                                        // this wave's columns within the group
  const bool active = n0 < cols;
  const int ko = 8 * (lane / 32);
  // transposed-read source address inside a 16-row step (see the file comment)
  const int g = lane >> 4, s = lane & 15;
  const int tr_row = 8 * (g >> 1) + (s >> 2);
  const int tr_col = n0 + 16 * (g & 1) + 4 * (s & 3);
  const uint16_t* wsrc = w_uv + (size_t)h * d_c * d_v + c0;

  for (int mt0 = 0; mt0 * 32 < B; mt0 += kMTilesPerPass) {
    f32x16 acc[kMTilesPerPass];
#pragma unroll
    for (int t = 0; t < kMTilesPerPass; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[t][r] = 0.f;
    for (int kc = 0; kc < d_c; kc += kUpMaxRows) {
      const int rows = min(kUpMaxRows, d_c - kc);   // a multiple of 16
      const int per = (rows / 16 + kUpKSplit - 1) / kUpKSplit;
      const int k_lo = kq * per * 16, k_hi = min(rows, k_lo + per * 16);
      // this wave's o_lat fragments (issued before the staging below waits)
      uint4 ao[kUpPartSteps][kMTilesPerPass];
#pragma unroll
      for (int i = 0; i < kUpPartSteps; ++i) {
        const int k0 = k_lo + 16 * i;
#pragma unroll
        for (int t = 0; t < kMTilesPerPass; ++t) {
          const int m = (mt0 + t) * 32 + (lane % 32);
          ao[i][t] = (active && m < B && k0 < k_hi) ? ld16(o_lat + ((size_t)m * H + h) * d_c + kc + k0 + ko)
                                                    : make_uint4(0, 0, 0, 0);
        }
      }
      const bool stage = mt0 == 0 || d_c > kUpMaxRows;
      // this thread's W_UV pieces: every load issued before the first store
      // (one memory round trip, not one per piece)
      uint4 wv[kUpStage];
      if (stage) {
#pragma unroll
        for (int it = 0; it < kUpStage; ++it) {
          const int i = threadIdx.x + it * 64 * kUpWaves;
          const int r = i / (cols / 8), c8 = i % (cols / 8);
          wv[it] = i < rows * (cols / 8) ? ld16(wsrc + (size_t)(kc + r) * d_v + c8 * 8) : make_uint4(0, 0, 0, 0);
        }
      }
      if (mt0 > 0 || kc > 0) __syncthreads();       // the previous piece's reads are done
      if (stage) {
#pragma unroll
        for (int it = 0; it < kUpStage; ++it) {
          const int i = threadIdx.x + it * 64 * kUpWaves;
          const int r = i / (cols / 8), c8 = i % (cols / 8);
          if (i < rows * (cols / 8)) *reinterpret_cast<uint4*>(wt + r * kUpPitch + c8 * 16) = wv[it];
        }
        __syncthreads();
      }
      if (active) {
#pragma unroll
        for (int i = 0; i < kUpPartSteps; ++i) {
          const int k0 = k_lo + 16 * i;
          if (k0 >= k_hi) break;
          const unsigned char* base = wt + (k0 + tr_row) * kUpPitch + tr_col * 2;
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base));
          const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + 4 * kUpPitch));
          const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
          const uint4 bw = make_uint4(l2.x, l2.y, h2.x, h2.y);
#pragma unroll
          for (int t = 0; t < kMTilesPerPass; ++t)
            acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ao[i][t]), as_bf16x8(bw), acc[t], 0, 0, 0);
        }
      }
    }
    // add the parts of each column half: part 0 + part 1 + part 2 + part 3
    if (active && kq > 0) {
#pragma unroll
      for (int t = 0; t < kMTilesPerPass; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) red[ch][kq - 1][t][r][lane] = acc[t][r];
    }
    __syncthreads();
    if (active && kq == 0) {
#pragma unroll
      for (int q2 = 0; q2 < kUpKSplit - 1; ++q2)
#pragma unroll
        for (int t = 0; t < kMTilesPerPass; ++t)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[t][r] += red[ch][q2][t][r][lane];
#pragma unroll
      for (int t = 0; t < kMTilesPerPass; ++t)
        if ((mt0 + t) * 32 < B) store_tile(out + (size_t)h * d_v + c0, acc[t], mt0 + t, B, (size_t)H * d_v, n0, lane);
    }
  }
}

}  // namespace


hipError_t launch_absorb_q(const void* q, const void* w_uk, void* q_lat, int B, int H, int d_h, int d_c,
                           hipStream_t stream) {
  const dim3 grid((d_c / 32 + kWavesPerGroup - 1) / kWavesPerGroup, H);
  hipLaunchKernelGGL(absorb_q_kernel, grid, dim3(64 * kWavesPerGroup), 0, stream,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(w_uk),
                     static_cast<uint16_t*>(q_lat), B, H, d_h, d_c);
  return hipGetLastError();
}

hipError_t launch_up_v(const void* o_lat, const void* w_uv, void* out, int B, int H, int d_c, int d_v,
                       hipStream_t stream) {
  const dim3 grid((d_v + kUpCols - 1) / kUpCols, H);
  hipLaunchKernelGGL(up_v_kernel, grid, dim3(64 * kUpWaves), 0, stream,
                     static_cast<const uint16_t*>(o_lat), static_cast<const uint16_t*>(w_uv),
                     static_cast<uint16_t*>(out), B, H, d_c, d_v);
  return hipGetLastError();
}

}  // namespace attn
