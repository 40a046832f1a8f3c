// fp8 path: placeholder until the e4m3 kernels are in place.
#include "common.h"
#include "fwd_params.h"

namespace attn {
hipError_t launch_fwd_fp8(const FwdParams&, int, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_fp8_prepare(const void*, const void*, const void*, int, int, int, int, int,
                              const int8_t*, void*, void*, void*, hipStream_t) {
    return hipErrorNotSupported;
}
}  // namespace attn
