// Paged mounted decode on gfx950 (kernels follow).
#include "device_common.h"
#include "kernels.h"

namespace octo {

hipError_t launch_decode_bf16(int, int, int, int, int, float, const void*, const void*,
                              const void*, int, const int32_t*, const int32_t*,
                              const int32_t*, const int32_t*, int, void*, float*, float*,
                              hipStream_t) {
    return hipErrorNotSupported;
}

}  // namespace octo
