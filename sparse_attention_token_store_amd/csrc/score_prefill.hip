// Chunked-prefill scoring (fp8 queries x fp8 keys on the fp8 matrix cores).
#include "common.hpp"
#include "launch.hpp"

namespace dsa {

hipError_t launch_score_prefill(const uint8_t*, const float*, const float*, const KCache&,
                                const Rows&, float*, int64_t, bool, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace dsa
