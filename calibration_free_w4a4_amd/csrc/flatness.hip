// flatness: the O(d) check on bf16 rows that tells whether fewer composed randomized Hadamard
// transforms suffice: rho3 = sqrt(d) ||x||_3^3 / ||x||_2^3 and rhoinf = sqrt(d) ||x||_inf /
// ||x||_2 per row (1 for a constant row, sqrt(d) for a one-hot row, 0 for a zero row).
//
// Method: "Quantizing With Randomized Hadamard Transforms" (gist.science), "Method", adaptive
// check: the l3 norm governs scalar quantization (the Berry-Esseen bound of a randomized
// Hadamard sum), the l_inf norm vector quantization.
//
// One wave per row: coalesced 16-byte loads, fp32 sums of x^2 and |x|^3 and the running max,
// reduced across the wave with DPP / permute shuffles.  HBM-bound (2 d bytes in, 8 out).
#include <hip/hip_runtime.h>

#include <algorithm>

#include "internal.h"

namespace orbq {
namespace {

constexpr int kWaves = 4;

__device__ __forceinline__ void accumulate(uint32_t pair, float& s2, float& s3, float& mx) {
  const float lo = __builtin_bit_cast(float, pair << 16), hi = __builtin_bit_cast(float, pair & 0xFFFF0000u);
  const float alo = __builtin_fabsf(lo), ahi = __builtin_fabsf(hi);
  s2 = __builtin_fmaf(lo, lo, s2);
  s2 = __builtin_fmaf(hi, hi, s2);
  s3 = __builtin_fmaf(alo * alo, alo, s3);
  s3 = __builtin_fmaf(ahi * ahi, ahi, s3);
  mx = __builtin_fmaxf(mx, __builtin_fmaxf(alo, ahi));
}

__global__ __launch_bounds__(64 * kWaves) void k_flatness(const uint16_t* X, int64_t n, int32_t d, int64_t ldx,
                                                          float* rho3, float* rhoinf) {
  const int lane = threadIdx.x & 63;
  const int64_t wave0 = static_cast<int64_t>(blockIdx.x) * kWaves + (threadIdx.x >> 6);
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kWaves;
  const float sqrt_d = __builtin_sqrtf(static_cast<float>(d));
  for (int64_t row = wave0; row < n; row += stride) {
    const uint4* src = reinterpret_cast<const uint4*>(X + row * ldx);
    float s2 = 0.0f, s3 = 0.0f, mx = 0.0f;
    for (int c = lane; c < d / 8; c += 64) {
      const uint4 v = src[c];
      accumulate(v.x, s2, s3, mx);
      accumulate(v.y, s2, s3, mx);
      accumulate(v.z, s2, s3, mx);
      accumulate(v.w, s2, s3, mx);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      s2 += __shfl_xor(s2, off);
      s3 += __shfl_xor(s3, off);
      mx = __builtin_fmaxf(mx, __shfl_xor(mx, off));
    }
    if (lane == 0) {
      const float l2 = __builtin_sqrtf(s2);
      rho3[row] = s2 > 0.0f ? sqrt_d * s3 / (s2 * l2) : 0.0f;
      rhoinf[row] = s2 > 0.0f ? sqrt_d * mx / l2 : 0.0f;
    }
  }
}

}  // namespace

int launch_flatness(const uint16_t* X, int64_t n, int32_t d, int64_t ldx, float* rho3, float* rhoinf,
                    hipStream_t stream) {
  const int cus = device_cus();
  const int64_t want = (n + kWaves - 1) / kWaves;
  const int grid = static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(want, static_cast<int64_t>(cus) * 8)));
  hipLaunchKernelGGL(k_flatness, dim3(grid), dim3(64 * kWaves), 0, stream, X, n, d, ldx, rho3, rhoinf);
  return static_cast<int>(hipGetLastError());
}

}  // namespace orbq
