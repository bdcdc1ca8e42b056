// rpbh_quantize kernels for Hadamard blocks of 4096 (one instantiation unit per block size, so that
// the kernel variants compile in parallel).
#include "rpbh_quantize_kernel.h"

namespace orbq {
namespace rq {
template hipError_t launch_block<4096>(QuantMode, int, const QuantKernelArgs&, int, size_t, hipStream_t);
}  // namespace rq
}  // namespace orbq
