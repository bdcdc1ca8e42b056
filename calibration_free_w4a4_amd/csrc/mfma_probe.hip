// mfma_probe: the sustained rate of the bf16 matrix cores on this device, for reading the
// product kernel's MFMA figures against what the chip delivers under load rather than only
// against its data-sheet peak.
//
// Each workgroup is laid out like the product kernel (512 threads, two waves per SIMD) and each
// wave runs a long chain of v_mfma_f32_32x32x16_bf16 into 9 independent accumulators, as many
// as the product's 384 x 192 tile holds per wave.  The operands are held in registers (no
// memory, no LDS, no decode): four A and four B fragments per lane with pseudo-random signs and
// mantissas, cycled so that every MFMA sees new operand bits.  The matrix cores' power, and so
// the clock they sustain, depends on how many operand bits switch; constant operands run near
// the data-sheet rate and random ones well below it, so the random form is the ceiling a GEMM on
// real data can be held against.
#include <hip/hip_runtime.h>

#include <stdint.h>

namespace orbq {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kProbeThreads = 512;
constexpr int kProbeAcc = 9;

// an integer hash (xor-shift / multiply rounds) for the operand bits
__device__ __forceinline__ uint32_t mix32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

__global__ __launch_bounds__(kProbeThreads) void k_mfma_probe(float* sink, int iters) {
  const uint32_t gid = blockIdx.x * kProbeThreads + threadIdx.x;
  bf16x8_t fa[4], fb[4];
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t h = mix32(gid * 64u + 8u * k + i);
      // sign and the low 8 bits of exponent and mantissa random: |v| in [2^-7, 2^-5), so the
      // accumulators stay finite over any number of steps
      fa[k][i] = __builtin_bit_cast(__bf16, static_cast<unsigned short>(0x3C00u | (h & 0x80FFu)));
      fb[k][i] = __builtin_bit_cast(__bf16, static_cast<unsigned short>(0x3C00u | ((h >> 16) & 0x80FFu)));
    }
  f32x16_t acc[kProbeAcc];
#pragma unroll
  for (int j = 0; j < kProbeAcc; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.0f;
  for (int it = 0; it < iters; it += 4) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int j = 0; j < kProbeAcc; ++j)
        acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[(j + u) & 3], fb[(j + 2 * u) & 3], acc[j], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < kProbeAcc; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[j][r];
  sink[gid] = s;  // keeps every MFMA live
}

}  // namespace

double mfma_probe_flops(int workgroups, int iters) {
  return 2.0 * 32 * 32 * 16 * kProbeAcc * static_cast<double>(iters) * (kProbeThreads / 64) * workgroups;
}

int launch_mfma_probe(int workgroups, int iters, float* sink, hipStream_t stream) {
  hipLaunchKernelGGL(k_mfma_probe, dim3(workgroups), dim3(kProbeThreads), 0, stream, sink, iters);
  return static_cast<int>(hipGetLastError());
}

}  // namespace orbq
