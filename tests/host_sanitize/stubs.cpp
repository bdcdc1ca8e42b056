// Stand-ins for the GPU side of liborbq in the host-only sanitizer build of api.cpp and
// codebook.cpp: every kernel launcher aborts, so a host path that reaches a launch fails the
// test loudly; hipGetErrorString is the one HIP runtime call the host layer makes.
#include <cstdio>
#include <cstdlib>

#include "../../calibration_free_w4a4_amd/csrc/internal.h"

namespace {
[[noreturn]] void reached(const char* what) {
  std::fprintf(stderr, "host-only build reached a GPU launch: %s\n", what);
  std::abort();
}
}  // namespace

namespace orbq {
int launch_rpbh_quantize(QuantMode, const uint16_t*, int64_t, int64_t, const RotArgs&, const QuantParams*, float,
                         uint8_t*, void*, float*, hipStream_t) {
  reached("launch_rpbh_quantize");
}
int launch_quantize_t(const float*, int64_t, const QuantParams&, uint8_t*, hipStream_t) { reached("launch_quantize_t"); }
int launch_lut_gemm(const uint8_t*, const float*, const DecodeParams&, const uint8_t*, const uint16_t*,
                    const DecodeParams&, int64_t, int64_t, int64_t, void*, int, int64_t, int, hipStream_t) {
  reached("launch_lut_gemm");
}
int launch_a16_gemm(const uint16_t*, int, int64_t, const uint8_t*, const uint16_t*, const DecodeParams&, int64_t,
                    void*, int, int64_t, hipStream_t) {
  reached("launch_a16_gemm");
}
int launch_flatness(const uint16_t*, int64_t, int, int64_t, float*, float*, hipStream_t) { reached("launch_flatness"); }
int noalloc_scratch(void**) { reached("noalloc_scratch"); }
int launch_mfma_probe(int, int, float*, hipStream_t) { reached("launch_mfma_probe"); }
int launch_a16_gemm_rot(const uint16_t*, int64_t, int, int64_t, const int32_t*, const int8_t*, int32_t, const uint8_t*,
                        const uint16_t*, const DecodeParams&, int64_t, void*, int, int64_t, hipStream_t) {
  reached("launch_a16_gemm_rot");
}
double mfma_probe_flops(int, int) { return 0.0; }
int device_cus() { return 256; }
}  // namespace orbq

extern "C" const char* hipGetErrorString(hipError_t) { return "(host-only build)"; }
