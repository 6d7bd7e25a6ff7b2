// Grouped (MoE expert) FC: not yet implemented; run_grouped reports
// FC_GGUF_EUNSUPPORTED until the grouped kernel lands.
#include "common.h"
#include "internal.h"

namespace fcg {

size_t moe_workspace_bytes(int E, int T, int top_k) {
  (void)E; (void)T; (void)top_k;
  return 0;
}

hipError_t launch_moe(int, const uint8_t*, size_t, int, int, int, const f16*, int, int,
                      const int32_t*, int, f16*, void*, int, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace fcg
