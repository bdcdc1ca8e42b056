// lut_gemm kernels for 2-bit activation codes (one translation unit per activation bit width).
#include "lut_gemm_kernel.h"

namespace orbq {
namespace lg {

hipError_t launch_gemm_a2(int bw, int cfg, bool out_bf16, const GemmArgs& a, int grid, size_t lds, hipStream_t st) {
  return launch_ba<2>(bw, cfg, out_bf16, a, grid, lds, st);
}

}  // namespace lg
}  // namespace orbq
