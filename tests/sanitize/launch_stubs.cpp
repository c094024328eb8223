// Host-only stand-ins for the kernel launchers, for a sanitizer build of the
// C ABI's host code (attn_decode.cpp) on a machine without a GPU. The argument
// checks under test return before any launch; a launch that is reached
// anyway fails loudly (the entry point then returns ATTN_ERR_HIP) and is
// counted, so the test can tell it happened.

#include <stdint.h>

#include "launch.h"

extern "C" {
int attn_sanitize_launches = 0;
}

namespace attn {

static hipError_t reached() {
  ++attn_sanitize_launches;
  return hipErrorNotSupported;
}

// No device: the work-balanced split is not planned (as on a host without a GPU).
int gqa_split_groups(int, int, int) { return 0; }
int gqa_split_groups_max(int, int) { return 0; }

hipError_t launch_gqa_partial(int, int, int, const GqaArgs&, hipStream_t) { return reached(); }
hipError_t launch_gqa_split(int, int, const GqaArgs&, int, hipStream_t) { return reached(); }
hipError_t launch_split_merge(int, const float*, const float*, const int32_t*, int, int, int, int, int,
                              int, int, int, void*, hipStream_t) { return reached(); }
hipError_t launch_kv_append(int, const void*, const void*, void*, void*, const int32_t*, int, int, int,
                            int, hipStream_t) { return reached(); }
hipError_t launch_merge(int, const float*, const float*, const int32_t*, int, int, int, int, int, int,
                        int, int, void*, hipStream_t) { return reached(); }
hipError_t launch_mla_partial(const MlaArgs&, hipStream_t) { return reached(); }
hipError_t launch_latent_append(const void*, void*, const int32_t*, int, int, int, hipStream_t) {
  return reached();
}
hipError_t launch_append_paged(const void*, const void*, void*, void*, const int32_t*, const int32_t*,
                               int, int, int, int, int, int, hipStream_t) { return reached(); }
hipError_t launch_absorb_q(const void*, const void*, void*, int, int, int, int, hipStream_t) {
  return reached();
}
hipError_t launch_up_v(const void*, const void*, void*, int, int, int, int, hipStream_t) {
  return reached();
}

}  // namespace attn
