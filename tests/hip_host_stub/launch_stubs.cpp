// The device-side entry points of the library (kernel launches and the
// no-alloc scratch lookup) for the host-only sanitizer build: host-only
// handles never launch, so each aborts if reached.
#include "kernels.h"

namespace spkv {

hipError_t launch_append(const AppendArgs&, hipStream_t) { hip_host_stub_called("launch_append"); }
hipError_t launch_expand(const PlanArgs&, hipStream_t) { hip_host_stub_called("launch_expand"); }
hipError_t launch_attention(const AttnArgs&, hipStream_t) {
  hip_host_stub_called("launch_attention");
}
hipError_t launch_attention_batch(const AttnArgs*, int, hipStream_t) {
  hip_host_stub_called("launch_attention_batch");
}
hipError_t scratch_address(void**) { hip_host_stub_called("scratch_address"); }

}  // namespace spkv
