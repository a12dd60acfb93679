// fp8 quantisation and forward for gfx950 (placeholder until the kernels land).
#include "fa_kernels.h"

namespace fa {
hipError_t launch_quant_fp8(int, QuantArgs, int, int, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_fwd_fp8(int, int, Fp8FwdArgs, int, int, hipStream_t) { return hipErrorNotSupported; }
}  // namespace fa
