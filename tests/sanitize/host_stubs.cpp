// Device-side entry points of the library replaced for the host-only
// sanitizer build of tq_host.cpp: the driver below exercises only paths that
// return before any launch, so reaching one of these is itself a failure.
#include <cstdio>
#include <cstdlib>

#include "tq_internal.h"

namespace tq {
[[noreturn]] static void reached(const char *what) {
  std::fprintf(stderr, "host driver reached %s\n", what);
  std::abort();
}
hipError_t noalloc_scratch(void **) { reached("noalloc_scratch"); }
hipError_t launch_encode(const EncodeArgs &, hipStream_t) { reached("launch_encode"); }
hipError_t launch_decode(const DecodeArgs &, hipStream_t) { reached("launch_decode"); }
hipError_t launch_prefill(const DecodeArgs &, hipStream_t) { reached("launch_prefill"); }
hipError_t launch_step_prep(const EncodeArgs *, const DecodeArgs &, hipStream_t) { reached("launch_step_prep"); }
}  // namespace tq
