// Chunked prefill (placeholder until the MFMA kernels land).
#include "common.hpp"
#include "launch.hpp"

namespace gdn {

size_t prefill_chunked_workspace_bytes(int B, int T, int Hk, int Hv) {
  (void)B; (void)T; (void)Hk; (void)Hv;
  return 0;
}

hipError_t launch_prefill_chunked(const void*, int64_t, const void*, int64_t, const void*, int64_t,
                                  const void*, const void*, int, const float*, const float*,
                                  const float*, float*, void*, int, int, int, int, float, void*,
                                  hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace gdn
