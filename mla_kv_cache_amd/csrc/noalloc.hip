// attn_decode_gqa_noalloc: attn_decode_gqa with the library's own scratch
// memory in place of a caller-provided workspace, for callers that cannot
// allocate device memory.
//
// The scratch is one file-scope device array. In host code its name is only a
// stand-in for the symbol, not a device address: the address is looked up
// once per device with hipGetSymbolAddress (with that device current) and
// kept; kernels receive that pointer as their workspace. The decode kernels
// write every partial they later read, so the scratch needs no clearing
// between calls. Calls on one device share it: calls that overlap in time on
// one device (different streams, or different host threads without ordering)
// race on it.

#include <hip/hip_runtime.h>

#include <atomic>

#include "attn_decode.h"

namespace {

constexpr size_t kScratchBytes = ATTN_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Device address of this device's scratch array (looked up on the first call
// on each device; nullptr if the lookup fails).
void* scratch_ptr() {
  static std::atomic<void*> ptrs[kMaxDevices];
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = ptrs[dev].load(std::memory_order_acquire);
  if (p) return p;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
  ptrs[dev].store(p, std::memory_order_release);
  return p;
}

}  // namespace

extern "C" {

int attn_decode_gqa_noalloc(const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* seq_lens, int B, int h_q, int h_kv, int D, int T_max,
                            float scale, attn_dtype dt, void* out, hipStream_t stream) {
  int P = 0, NP = 0;
  size_t need = 0;
  const int st = attn_decode_gqa_plan(B, h_q, h_kv, D, T_max, dt, &P, &NP, &need);
  if (st != ATTN_OK) return st;
  if (need > kScratchBytes) return ATTN_ERR_WORKSPACE;  // the shape needs more than the static scratch
  void* ws = scratch_ptr();
  if (!ws) return ATTN_ERR_HIP;
  return attn_decode_gqa(q, k_cache, v_cache, seq_lens, B, h_q, h_kv, D, T_max, scale, dt, out, ws,
                         kScratchBytes, stream);
}

}  // extern "C"
