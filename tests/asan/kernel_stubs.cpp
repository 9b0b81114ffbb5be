// Stand-ins for the kernel-side entry points that the ABI implementation
// calls, for the sanitizer build of its host code: that build compiles no
// device code, and its driver never gets past the device check to a launch.
// Each reports "no device".
#include "gqa_kernels.h"

namespace gqa {

hipError_t enqueue_kv_append(const AppendArgs&, int, int, hipStream_t) { return hipErrorNoDevice; }
int balanced_grid_size(int, int, int) { return 0; }
hipError_t enqueue_decode_step(const StepArgs&, int, int, hipStream_t, hipEvent_t) {
  return hipErrorNoDevice;
}
int paged_balanced_grid_size(int, int, int) { return 0; }
hipError_t no_alloc_scratch(int, void**) { return hipErrorNoDevice; }
hipError_t enqueue_paged_decode_step(const StepArgs&, int, int, hipStream_t, hipEvent_t) {
  return hipErrorNoDevice;
}

}  // namespace gqa
