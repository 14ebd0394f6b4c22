// Matrix-core (MFMA) GQA-path decode: not built yet; every shape takes the generic path.
#include "common.hpp"
#include "launch.hpp"

namespace mla {
bool gqa_decode_mfma_supported(const mla_shape_t&) { return false; }
hipError_t launch_gqa_decode_mfma(const mla_shape_t&, const void*, const void*, const void*,
                                  const void*, const int32_t*, const int32_t*, float*, float*,
                                  hipStream_t) {
  return hipErrorNotSupported;
}
}  // namespace mla
