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
// both fragments are 16-byte loads straight from memory, no LDS.
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

// One wave per 32 latent columns c of one head; all of B in passes of
// kMTilesPerPass tiles of 32 rows. Rows past B read zeros and are not stored.
__global__ __launch_bounds__(64 * kWavesPerGroup) void absorb_q_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ w_uk, uint16_t* __restrict__ q_lat,
    int B, int H, int d_h, int d_c) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int h = blockIdx.y;
  const int n0 = (blockIdx.x * kWavesPerGroup + wave) * 32;
  if (n0 >= d_c) return;
  const int ko = 8 * (lane / 32);
  const uint16_t* wrow = w_uk + ((size_t)h * d_c + n0 + (lane % 32)) * d_h + ko;
  for (int mt0 = 0; mt0 * 32 < B; mt0 += kMTilesPerPass) {
    f32x16 acc[kMTilesPerPass];
#pragma unroll
    for (int t = 0; t < kMTilesPerPass; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[t][r] = 0.f;
    // Eight k-steps at a time: every fragment load of the chunk is issued
    // before its products, so the chunk costs one memory round trip.
    for (int kb = 0; kb < d_h; kb += 16 * kChunk) {
      uint4 bw[kChunk], aq[kChunk][kMTilesPerPass];
#pragma unroll
      for (int i = 0; i < kChunk; ++i) {
        const int k0 = kb + 16 * i;
        bw[i] = k0 < d_h ? ld16(wrow + k0) : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int t = 0; t < kMTilesPerPass; ++t) {
          const int m = (mt0 + t) * 32 + (lane % 32);
          aq[i][t] = (m < B && k0 < d_h) ? ld16(q + ((size_t)m * H + h) * d_h + k0 + ko) : make_uint4(0, 0, 0, 0);
        }
      }
#pragma unroll
      for (int i = 0; i < kChunk; ++i)
#pragma unroll
        for (int t = 0; t < kMTilesPerPass; ++t)
          acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(aq[i][t]), as_bf16x8(bw[i]), acc[t], 0, 0, 0);
    }
#pragma unroll
    for (int t = 0; t < kMTilesPerPass; ++t)
      if ((mt0 + t) * 32 < B) store_tile(q_lat + (size_t)h * d_c, acc[t], mt0 + t, B, (size_t)H * d_c, n0, lane);
  }
}

constexpr int kUpWaves = 2;                     // waves per work-group, 32 output columns each
constexpr int kUpCols = 32 * kUpWaves;          // W_UV columns per work-group (128-byte row pieces)
constexpr int kUpPitch = kUpCols * 2 + 32;      // bytes per LDS row: padding spreads the transposed reads
constexpr int kUpMaxRows = 512;                 // the whole contraction of one head fits in LDS

// One work-group per (head, 64 output columns), one wave per 32 of them. The
// head's whole W_UV slice [d_c x 64] is loaded into LDS at once (every load in
// flight together, one barrier), then each wave runs the full contraction.
// d_c > 512 takes the slice in pieces of 512 rows.
__global__ __launch_bounds__(64 * kUpWaves) void up_v_kernel(
    const uint16_t* __restrict__ o_lat, const uint16_t* __restrict__ w_uv, uint16_t* __restrict__ out,
    int B, int H, int d_c, int d_v) {
  __shared__ __attribute__((aligned(16))) unsigned char wt[kUpMaxRows * kUpPitch];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int h = blockIdx.y;
  const int cols = min(kUpCols, d_v - blockIdx.x * kUpCols);   // a multiple of 32
  const int c0 = blockIdx.x * kUpCols;                           // first output column of the group
  const int n0 = wave * 32;                                      // this wave's columns within the group
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
      if (mt0 > 0 || kc > 0) __syncthreads();       // the previous piece's reads are done
      if (mt0 == 0 || d_c > kUpMaxRows) {
        for (int i = threadIdx.x; i < rows * (cols / 8); i += blockDim.x) {
          const int r = i / (cols / 8), c8 = i % (cols / 8);
          *reinterpret_cast<uint4*>(wt + r * kUpPitch + c8 * 16) = ld16(wsrc + (size_t)(kc + r) * d_v + c8 * 8);
        }
        __syncthreads();
      }
      if (active) {
        // Eight k-steps at a time: the o_lat fragment loads of the chunk are
        // issued together, then the products (one memory round trip per chunk).
        for (int kb = 0; kb < rows; kb += 16 * kChunk) {
          uint4 ao[kChunk][kMTilesPerPass];
#pragma unroll
          for (int i = 0; i < kChunk; ++i) {
            const int k0 = kb + 16 * i;
#pragma unroll
            for (int t = 0; t < kMTilesPerPass; ++t) {
              const int m = (mt0 + t) * 32 + (lane % 32);
              ao[i][t] = (m < B && k0 < rows) ? ld16(o_lat + ((size_t)m * H + h) * d_c + kc + k0 + ko)
                                               : make_uint4(0, 0, 0, 0);
            }
          }
#pragma unroll
          for (int i = 0; i < kChunk; ++i) {
            const int k0 = kb + 16 * i;
            if (k0 >= rows) break;
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
    }
    if (active) {
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
