// Internal declarations shared by the host layer and the kernels of liborbq.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace orbq {

constexpr int kMaxPosBoundaries = 31;  // 6-bit codebooks: N/2 - 1 positive decision boundaries
constexpr int kMaxTableHalf = 256;     // quantizer table holds buckets -J..J-1, J <= 256
// 2-, 3- and 4-bit codebooks: the quantize kernel's table covers every bucket of t' in
// [-2^k, 2^k] (2^(k+1) + 4 entries of 8 bytes), so 2^k is capped at 1024 (16 KB of LDS).  Every
// Lloyd-Max codebook of f_d up to d = 16384 needs 2^k <= 1024.
constexpr int kMaxFullScale = 1024;

// Decision thresholds of one codebook in the scaled coordinate t' = t * 2^k.
//
// Positive centroids c_{N/2+p} (p = 0..N/2-1) are separated by the exact midpoints
// B_p = (c_{N/2+p} + c_{N/2+p+1}) / 2.  For fp32 t':
//   t' > 0 : rank = #{p : t' > B_p}            (ties -> lower index -> lower rank)
//   t' <= 0: rank = #{p : |t'| >= B_p}         (ties -> lower index -> higher rank)
// thr_gt[p] = largest float <= B_p * 2^k, so  t' > B_p  <=>  t' > thr_gt[p];
// thr_ge[p] = largest float <  B_p * 2^k, so  u >= B_p  <=>  u > thr_ge[p].
// 2^k is chosen so that neighbouring thresholds are at least 1.5 apart: every unit
// bucket of t' then holds at most one threshold, which lets the kernels decide with one
// table lookup and one compare per coordinate.
struct QuantParams {
  float scale;  // 2^k
  int32_t J;    // buckets j = floor(-t') are clamped to [-J, J-1]
  int32_t nb;   // number of positive boundaries, N/2 - 1
  int32_t bits;
  float thr_gt[kMaxPosBoundaries + 1];
  float thr_ge[kMaxPosBoundaries + 1];
  uint16_t vals[64];  // bf16 of the signed centroid of each code (QuantMode::kDecoded only)
};

// Host: builds QuantParams from an ascending, antisymmetric fp32 codebook.
// Returns 0 on success, nonzero when no power-of-two scale separates the thresholds.
int build_quant_params(const float* centroids, int bits, QuantParams* qp);

// Host: float64 Lloyd-Max for f_d (codebook.cpp).
int lloyd_max_host(int d, int bits, double* out);

// Decode tables for the product: bf16 bit patterns of the centroid magnitudes, by rank.
struct DecodeParams {
  int32_t bits;
  uint16_t mag[32];  // bf16(|c_{N/2+r}|), r = 0..N/2-1
};
void build_decode_params(const float* centroids, int bits, DecodeParams* dp);

uint16_t f32_to_bf16_rne(float x);

// Launchers (return hipError_t as int).
struct RotArgs {
  int32_t d, block;
  const int32_t* perm;
  const int8_t* signs;
  int32_t passes;  // composed passes (1..3); perm and signs hold passes * d entries
};

// kDecoded: activations written as the bf16 centroids of their codes (qp.vals), [n][d] bf16 with
// the 8 values of each aligned group of 8 positions in the order 0,2,4,6,1,3,5,7 (the order in
// which the product stages its operands), for a product that stages them without decoding.
// kRotateBf16: the rotated rows x' = Pi x (no quantization) as bf16, rounded to nearest even,
// in the same order within each group of 8 positions, for the weight-only product.
enum class QuantMode { kActivations, kWeights, kRotateOnly, kDecoded, kRotateBf16 };

int launch_rpbh_quantize(QuantMode mode, const uint16_t* X, int64_t n, int64_t ldx, const RotArgs& rot,
                         const QuantParams* qp, float eps, uint8_t* codes, void* norms, float* x_rot,
                         hipStream_t stream);

// The current device's compute-unit count (256 if the runtime cannot say), cached per device
// and host thread.
int device_cus();

// Weight-only product (bf16 activations, rotated in fp32): K-range splits and launcher.
// x_rot [nt][d] bf16 (QuantMode::kRotateBf16) with nt <= 16; d % 128 == 0.
void a16_splits(int64_t d, int* splits, int* ss_per_split);
int launch_a16_gemm(const uint16_t* x_rot, int nt, int64_t d, const uint8_t* w_codes, const uint16_t* w_norms,
                    const DecodeParams& dw, int64_t m, void* Y, int y_bf16, int64_t ldy, hipStream_t stream);

int launch_flatness(const uint16_t* X, int64_t n, int32_t d, int64_t ldx, float* rho3, float* rhoinf,
                    hipStream_t stream);

int launch_quantize_t(const float* t, int64_t count, const QuantParams& qp, uint8_t* codes,
                      hipStream_t stream);

// The current device's fixed workspace for orbq_linear_noalloc (noalloc.hip).
int noalloc_scratch(void** ptr);

int launch_lut_gemm(const uint8_t* x_codes, const float* x_norms, const DecodeParams& da,
                    const uint8_t* w_codes, const uint16_t* w_norms, const DecodeParams& dw,
                    int64_t n, int64_t m, int64_t d, void* Y, int y_bf16, int64_t ldy,
                    int act, hipStream_t stream);

}  // namespace orbq
