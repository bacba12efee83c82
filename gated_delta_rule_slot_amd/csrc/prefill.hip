// prefill.hip -- chunked prefill (placeholder until the MFMA kernels land).
#include "common.hpp"

namespace gdn {
size_t prefill_record_bytes(const gdn_pool *) { return 92160; }
size_t prefill_carry_bytes(const gdn_pool *p, int batch) {
  return size_t(batch) * p->d.heads * p->d.head_v * p->d.head_k * 4;
}
hipError_t launch_prefill(const gdn_pool *, const PrefillArgs &, hipStream_t) {
  return hipErrorNotSupported;
}
}  // namespace gdn
