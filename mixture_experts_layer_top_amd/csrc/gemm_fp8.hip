// Grouped expert GEMMs with block-scaled fp8 weights (placeholder until the fp8 kernels land).
#include "common.h"
#include "kernels.h"

namespace moe {

hipError_t launch_gemms_fp8(const SelectOut&, int, int, hipStream_t) { return hipErrorNotSupported; }

}  // namespace moe
