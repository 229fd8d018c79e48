// Launcher stubs for the host-only sanitizer build of api.cpp: the driver only makes
// calls that are rejected (or empty) before any launch, so reaching a launcher, or the
// HIP runtime, is itself a failure.
#include <cstdio>
#include <cstdlib>

#include "../../paged_kv_cache_95_amd/csrc/internal.h"

namespace {
[[noreturn]] void reached(const char* what) {
  std::fprintf(stderr, "stub reached: %s (a call expected to fail validation launched)\n", what);
  std::abort();
}
}  // namespace

namespace pa {
int launch_store(const pa_kv_pool_t&, const void*, const void*, int, int64_t, int64_t, int64_t,
                 int64_t, int64_t, const int64_t*, hipStream_t) { reached("launch_store"); }
int launch_copy_blocks(const pa_kv_pool_t&, const int32_t*, const int32_t*, int, hipStream_t) {
  reached("launch_copy_blocks");
}
int launch_decode(const pa_kv_pool_t&, const DecodeArgs&, hipStream_t) { reached("launch_decode"); }
int launch_decode_step(const pa_kv_pool_t&, const DecodeArgs&, const StepRows&, hipStream_t) {
  reached("launch_decode_step");
}
int launch_rope_store(const pa_kv_pool_t&, const RopeArgs&, int, hipStream_t) {
  reached("launch_rope_store");
}
int launch_prefill(const pa_kv_pool_t&, const PrefillArgs&, hipStream_t) { reached("launch_prefill"); }
int noalloc_scratch(void**, hipStream_t) { reached("noalloc_scratch"); }
int validate_decode(const pa_kv_pool_t&, const int32_t*, int, const int32_t*, int, int,
                    const int64_t*, hipStream_t) { reached("validate_decode"); }
int validate_tokens(const pa_kv_pool_t&, const int64_t*, int64_t, const int64_t*, int64_t,
                    hipStream_t) { reached("validate_tokens"); }
int validate_varlen(const pa_kv_pool_t&, const PrefillArgs&, hipStream_t) {
  reached("validate_varlen");
}
int debug_gate(hipStream_t) { reached("debug_gate"); }
int debug_take(hipStream_t, int32_t*, int64_t*) { reached("debug_take"); }
}  // namespace pa

extern "C" hipError_t hipStreamSynchronize(hipStream_t) { reached("hipStreamSynchronize"); }
