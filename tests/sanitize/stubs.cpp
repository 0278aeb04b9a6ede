// Stand-ins for the attention launchers and the hipBLASLt GEMM, for the
// host-only sanitizer build of the C ABI (tests/test_sanitize_host.py; the
// layout, loss and norm sources are compiled as they are, for their size
// functions).  The checks that build runs fail validation before any launch;
// reaching one of these is a test failure.
#include <cstdio>
#include <cstdlib>

#include "opr_internal.h"

namespace opr {

static void reached(const char *what) {
  std::fprintf(stderr, "sanitizer build: %s reached in a host-only check\n", what);
  std::abort();
}

void launch_rope_order(const opr_attn_in &, const AttnWs &, hipStream_t) { reached("launch_rope_order"); }
void launch_pack_q(const opr_attn_in &, const AttnWs &, hipStream_t) { reached("launch_pack_q"); }
void launch_pack_kv(const opr_attn_in &, const AttnWs &, hipStream_t) { reached("launch_pack_kv"); }
hipError_t launch_attn_fwd_kernel(const opr_attn_in &, float, void *, float *, const AttnWs &, hipStream_t) {
  reached("launch_attn_fwd_kernel");
  return hipSuccess;
}
hipError_t launch_attn_bwd_kernels(const opr_attn_in &, float, const void *, const float *, const void *, float *,
                                   float *, float *, const AttnWs &, hipStream_t, hipEvent_t *) {
  reached("launch_attn_bwd_kernels");
  return hipSuccess;
}
bool gemm_bf16(bool, bool, int64_t, int64_t, int64_t, const void *, const void *, void *, bool, void *, size_t,
               hipStream_t) {
  reached("gemm_bf16");
  return false;
}
}  // namespace opr
