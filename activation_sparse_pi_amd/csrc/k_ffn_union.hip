// Batch > 1 union-mask FFN on MFMA (placeholder until the MFMA kernels land).
#include "device_common.h"
#include "internal.h"

namespace pi {

hipError_t launch_ffn_union(const pi_ffn_desc&, const FfnPlan&, const uint16_t*, int,
                            const int32_t*, const int32_t*, const uint32_t*, int, float*, char*,
                            hipStream_t) {
    return hipErrorNotSupported;
}

}  // namespace pi
