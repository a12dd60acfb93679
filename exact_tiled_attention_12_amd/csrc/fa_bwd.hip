// Attention backward for gfx950 (placeholder until the kernels land).
#include "fa_kernels.h"

namespace fa {
hipError_t launch_bwd(DType, int, int, BwdArgs, int, int, hipStream_t) { return hipErrorNotSupported; }
}  // namespace fa
