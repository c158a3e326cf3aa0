// Test-only stand-ins for the device half of libcsmla.so, linked with the host
// sources into a host-only library built with AddressSanitizer and
// UndefinedBehaviorSanitizer (tests/test_host_sanitizers.py).  The host ABI
// tests never reach a launch; if one did, it gets an error back, never a
// silent result.
#include <stddef.h>
#include <stdint.h>

#include "../../sparse_compressed_mla_amd/csrc/csmla_indexer_internal.h"
#include "../../sparse_compressed_mla_amd/csrc/csmla_internal.h"

namespace {
constexpr int kNoDevice = 100;   // hipErrorNoDevice
}

namespace csmla {
int noalloc_scratch(void** ptr, void*) {
  *ptr = nullptr;
  return kNoDevice;
}
int launch_forward(const KArgs&, void*) { return kNoDevice; }
int launch_debug_resolve(const KArgs&, int32_t*, int32_t*, int32_t, int, void*) { return kNoDevice; }
}  // namespace csmla

namespace csmla_idx {
int launch_indexer(const IArgs&, int, int, void*) { return kNoDevice; }
}  // namespace csmla_idx
