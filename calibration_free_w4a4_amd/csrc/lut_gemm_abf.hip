// lut_gemm kernels for activations already decoded to bf16 centroids (the layer's path for 6-bit
// activation codes; one translation unit per activation format).
#include "lut_gemm_kernel.h"

namespace orbq {
namespace lg {

hipError_t launch_gemm_abf(int bw, int cfg, bool out_bf16, const GemmArgs& a, int grid, size_t lds, hipStream_t st) {
  return launch_ba<16>(bw, cfg, out_bf16, a, grid, lds, st);
}

}  // namespace lg
}  // namespace orbq
