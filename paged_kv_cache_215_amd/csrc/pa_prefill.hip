// Chunked-prefill attention against the paged cache (matrix-core path).
#include "pa_device.hpp"
#include "pa_internal.hpp"

namespace pa {

int prefill_kv_splits(int, int, int, int) { return 1; }

hipError_t launch_prefill(const PrefillArgs&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace pa
