// placeholder, replaced by the decode GEMV kernel
#include "qk_internal.h"
namespace qk {
hipError_t launch_gemv(const void*, int32_t, const MatArgs&, void*, hipStream_t, const char** variant) {
    *variant = "none";
    return hipErrorNotSupported;
}
}  // namespace qk
