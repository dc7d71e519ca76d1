// Stand-ins for the device-side launchers, for a host-only build of the
// C-ABI under AddressSanitizer / UndefinedBehaviorSanitizer (test
// infrastructure: the sanitized driver exercises only host logic, so every
// launch reports "not supported" if it were ever reached).
#include "pkv_internal.h"

namespace pkv {
hipError_t launch_compress(const CompressJob&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_compress_batch(const CompressBatch&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_compress_tri(const CompressJob&, hipStream_t, hipEvent_t, hipEvent_t) {
  return hipErrorNotSupported;
}
hipError_t launch_prefill_dense(const CacheGeom&, const void*, const void*, int64_t, int64_t, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_chunk_dense(const CacheGeom&, const void*, const void*, int64_t, int64_t, int64_t, int64_t,
                              hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_table_fill(const CacheGeom&, int64_t, int64_t, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_table_set(const CacheGeom&, int64_t, int32_t, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_append(const CacheGeom&, const void*, const void*, int64_t, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_partial(const CacheGeom&, const AttnJob&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_partial_batch(const CacheGeom*, const int64_t*, const int64_t*, const int*, int, const AttnJob&,
                                hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_merge(const CacheGeom&, const AttnJob&, hipStream_t) { return hipErrorNotSupported; }
hipError_t noalloc_scratch(void** ptr) {
  *ptr = nullptr;
  return hipErrorNotSupported;
}
hipError_t launch_merge_batch(const CacheGeom*, int, const AttnJob&, const AttnJob*, const int*, hipStream_t) {
  return hipErrorNotSupported;
}
int decode_default_splits(const CacheGeom&, int64_t, int64_t) { return 1; }
bool batched_kernel(const CacheGeom&) { return true; }
int decode_batch_splits(const CacheGeom&, const int64_t*, int n, int* ns) {
  for (int i = 0; i < n; ++i) ns[i] = 1;
  return 1;
}
}  // namespace pkv
