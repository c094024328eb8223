// Work items of the persistent GQA partial kernels: which (sequence, KV head,
// positions) each resident work-group takes. Shared by the position-per-lane
// kernel (gqa_decode.hip) and the matrix-core kernel (gqa_matrix.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_util.h"
#include "launch.h"

namespace attn {
namespace items {

// Work items of the persistent partial kernel: (sequence b, KV head j,
// partition p) for every partition that holds at least one attended
// position, numbered sequence-major (b, then j, then p). Work-group w of G
// takes the contiguous run [w * N / G, (w + 1) * N / G) of the N items, so
// every work-group gets the same number of partitions (give or take one)
// whatever the mix of sequence lengths, and consecutive items mostly share
// one query and one KV head.
//
// Split mode: the items are units of kSplitUnit positions (one 32-row tile
// per wave), and a work-group treats the consecutive units of its run that
// belong to one (b, j) as one segment, with one partial output. Every
// work-group then streams the same number of units (give or take one), and
// a (b, j) row is split between work-groups only where a run boundary falls.
// The partial of work-group w's segment of pair (b, j) goes to slot
// w + b * h_kv + j: along a run both w and the pair index only grow, so the
// slots are distinct, and the segments of one pair sit in consecutive slots
// (those of the work-groups whose run meets its units).
struct ItemRun {
  long long left;  // items still to do, the current one included
  int b, j, p;     // current item
  int np;          // partitions of sequence b
};

__device__ __forceinline__ int partitions_of(const GqaArgs& a, int b) {
  const int n = attended_len(a.seq_lens[b], a.k_new ? 1 : 0, a.T_max);
  return (int)(((long long)n - window_lo(n, a.window) + a.P - 1) / a.P);
}

__device__ __forceinline__ long long wave_sum_ll(long long x) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) x += __shfl_xor(x, off, 64);
  return x;
}

__device__ __forceinline__ long long wave_incl_scan_ll(long long x, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const long long y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  return x;
}

__device__ __forceinline__ long long uniform_ll(long long x) {
  const uint64_t u = (uint64_t)x;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return (long long)(((uint64_t)hi << 32) | lo);
}

// This work-group's first item and item count. Every wave computes the same
// (uniform) answer from the sequence lengths, 64 sequences at a time.
__device__ __forceinline__ ItemRun first_item(const GqaArgs& a) {
  const int lane = threadIdx.x & 63;
  ItemRun r{0, 0, 0, 0, 0};
  long long total = 0;
  for (int b0 = 0; b0 < a.B; b0 += 64) {
    const int b = b0 + lane;
    total += wave_sum_ll(b < a.B ? (long long)partitions_of(a, b) : 0);
  }
  total = uniform_ll(total * a.h_kv);
  const long long lo = total * blockIdx.x / gridDim.x;
  const long long hi = total * (blockIdx.x + 1) / gridDim.x;
  if (hi <= lo) return r;
  long long base = 0;
  for (int b0 = 0; b0 < a.B; b0 += 64) {
    const int b = b0 + lane;
    const int np = b < a.B ? partitions_of(a, b) : 0;
    const long long cnt = (long long)np * a.h_kv;
    const long long incl = base + wave_incl_scan_ll(cnt, lane);
    const uint64_t hit = __ballot(incl > lo);
    if (hit) {
      const int l0 = __builtin_amdgcn_readfirstlane(__ffsll((unsigned long long)hit) - 1);
      const long long excl = uniform_ll(__shfl(incl - cnt, l0, 64));
      r.np = __builtin_amdgcn_readfirstlane(__shfl(np, l0, 64));
      r.b = b0 + l0;
      const long long off = lo - excl;
      r.j = (int)(off / r.np);
      r.p = (int)(off % r.np);
      r.left = hi - lo;
      return r;
    }
    base = uniform_ll(__shfl(incl, 63, 64));
  }
  return r;
}

// The item after the current one (sequences without partitions are skipped).
__device__ __forceinline__ void next_item(ItemRun& r, const GqaArgs& a) {
  if (++r.p < r.np) return;
  r.p = 0;
  if (++r.j < a.h_kv) return;
  r.j = 0;
  do {
    ++r.b;
  } while (r.b < a.B && (r.np = partitions_of(a, r.b)) == 0);
}

// A wave-uniform 32-bit load through the scalar cache (read-only data: the
// sequence lengths and the block table). Waited for at once: as a vector
// load, the compiler's wait for it would also wait for every tile copy in
// flight, which it does not know about. p must be wave-uniform.
__device__ __forceinline__ int sload_i32(const int32_t* p) {
  int v;
  asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(p) : "memory");
  return v;
}

// Position in a work-group's tile stream: the current item (segment) and
// the first position of the current tile. Every wave holds the same values.
struct Cursor {
  items::ItemRun run;
  int len;          // units (or partitions) of the segment
  int len0;         // seq_lens[b] as stored
  int n;            // attended length of sequence b
  int start, end;   // positions [start, end) of the segment
  int t0;           // current tile
  bool ok;          // a tile remains
};

__device__ __forceinline__ int parts_of_len(const GqaArgs& a, int len0) {
  const int n = attended_len(len0, a.k_new ? 1 : 0, a.T_max);
  return (int)(((long long)n - window_lo(n, a.window) + a.P - 1) / a.P);
}

template <bool SPLIT>
__device__ __forceinline__ void set_item(Cursor& c, const GqaArgs& a) {
  c.len = SPLIT ? (int)min((long long)(c.run.np - c.run.p), c.run.left) : 1;
  c.len0 = sload_i32(a.seq_lens + c.run.b);
  c.n = attended_len(c.len0, a.k_new ? 1 : 0, a.T_max);
  c.start = window_lo(c.n, a.window) + c.run.p * a.P;
  c.end = min(c.n - c.start, c.len * a.P) + c.start;
  c.t0 = c.start;
}

template <bool SPLIT>
__device__ __forceinline__ void cursor_init(Cursor& c, const GqaArgs& a) {
  c.run = items::first_item(a);
  c.ok = c.run.left > 0 && c.run.b < a.B;
  if (c.ok) set_item<SPLIT>(c, a);
}

// Moves to the next tile of TILE positions; returns true when that tile opens a new segment.
template <bool SPLIT, int TILE>
__device__ __forceinline__ bool cursor_next(Cursor& c, const GqaArgs& a) {
  c.t0 += TILE;
  if (c.t0 < c.end) return false;
  if (c.run.left <= c.len) {
    c.ok = false;
    return true;
  }
  items::ItemRun r = c.run;
  r.left -= c.len;
  r.p += c.len;
  if (r.p >= r.np) {  // the pair is done: next KV head, then the next sequence with positions
    r.p = 0;
    if (++r.j >= a.h_kv) {
      r.j = 0;
      do {
        ++r.b;
      } while (r.b < a.B && (r.np = parts_of_len(a, sload_i32(a.seq_lens + r.b))) == 0);
    }
  }
  c.run = r;
  c.ok = r.b < a.B;
  if (c.ok) set_item<SPLIT>(c, a);
  return true;
}

}  // namespace items
}  // namespace attn
