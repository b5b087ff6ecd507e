#include "isd_internal.h"
namespace isd {
hipError_t launch_lm_head(const uint16_t *, const uint16_t *, int, int, int, uint16_t *, hipStream_t) {
    return hipErrorNotSupported;
}
}  // namespace isd
