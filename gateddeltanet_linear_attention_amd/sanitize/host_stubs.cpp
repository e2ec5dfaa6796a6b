// Launch stubs for the host-only sanitizer build of the C ABI (gdn_api.cpp): every
// launcher refuses with hipErrorNoDevice, as the real ones do on a machine without a
// GPU, so argument validation, the transaction planner and the size arithmetic run
// unchanged under AddressSanitizer / UndefinedBehaviorSanitizer while no kernel, and no
// HIP runtime call, is ever reached.  Never part of libgdn.so itself.
#include "gdn_internal.h"

namespace gdn {

hipError_t launch_recurrent(const RecurrentArgs &, int, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_select(const SelectArgs &, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_chunked(const ChunkArgs &, int, int, hipStream_t) { return hipErrorNoDevice; }
hipError_t static_workspace(void **ptr, size_t *bytes) {
  *ptr = nullptr;
  *bytes = 0;
  return hipErrorNoDevice;
}
hipError_t launch_commit(const CommitArgs &, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_fold(const FoldArgs &, int, hipStream_t) { return hipErrorNoDevice; }

}  // namespace gdn
