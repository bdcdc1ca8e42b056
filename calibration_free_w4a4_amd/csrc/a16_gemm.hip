// a16_gemm: the weight-only product with bf16 activations (W{2,3,4,6}A16).
#include "lut_gemm_kernel.h"

namespace orbq {
namespace lg {
namespace {

// ============================================================================ A16 (weight-only)
// Y[t][j] = r'_j sum_k bf16(x'_tk) bf16(C_w[w_jk]) for a few tokens (t < 16 per launch):
// x' = Pi x in fp32 (the rotate-only pass of rpbh_quantize), codes streamed from HBM once.
// Workgroup = 4 waves; each wave owns 64 weight rows (four 16-row MFMA column blocks) and one
// split of the K range; v_mfma_f32_16x16x32_bf16 with the tokens as the M side (rows past the
// token count read as zero).  A super-step covers 128 codes: lane (m = l % 16, g = l / 16)
// holds codes 32 g .. 32 g + 31 of it, i.e. one 16-byte (4-bit) load per row block, and takes
// them 8 at a time in four MFMAs.  The k order inside each 8 (0,2,4,6,1,3,5,7, the decoders'
// order) is applied to x' as well.  Partial sums of each split go to a workspace; a second
// kernel adds the splits and applies r'.
// A buffer resource from wave-uniform values, forced into scalar registers: the compiler keeps
// values derived from 64-bit compares and selects in VGPRs, which would wrap every load that
// uses the resource in a waterfall loop.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t uniform_rsrc(const void* base, uint32_t bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b >> 32));
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo), 0,
                                           __builtin_amdgcn_readfirstlane(bytes), kBufWord3);
}

constexpr int kA16Waves = 4;
constexpr int kA16Rows = 64;                  // weight rows per wave
constexpr int kA16SS = 128;                   // codes per super-step

struct A16Args {
  const float* xr;       // x' [nt][d] fp32
  const uint8_t* wc;
  float* part;           // [splits][nt][m]
  int64_t m;
  int32_t d, nt, rb;     // rb = code bytes per weight row
  int32_t ss_per_split, nss, row_blocks;
  uint32_t xr_bytes;     // nt * d * 4
  uint32_t lt_lo, lt_hi, ht_lo, ht_hi;
  uint16_t mag[32];
};

template <int BW>
struct CodesA16;  // the 32 codes of one (row, super-step) lane slot and their decode

template <>
struct CodesA16<4> {
  uint4 w;
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
    w = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
  }
  __device__ __forceinline__ uint4 get(int s, const Tab4& t, const void*) const {
    const uint32_t x = s == 0 ? w.x : s == 1 ? w.y : s == 2 ? w.z : w.w;
    return decode4_b(x, decode4_a(x, t));
  }
};

template <>
struct CodesA16<2> {
  v2u_t w;
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
    w = __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, 0);
  }
  __device__ __forceinline__ uint4 get(int s, const Tab4& t, const void*) const {
    const uint32_t x = ((s < 2 ? w.x : w.y) >> (16 * (s & 1))) & 0xFFFFu;
    return decode2_b(decode2_a(x, t), t);
  }
};

template <>
struct CodesA16<3> {
  v2u_t a;
  uint32_t b;
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
    a = __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, 0);
    b = __builtin_amdgcn_raw_buffer_load_b32(rs, off + 8, 0, 0);
  }
  __device__ __forceinline__ uint4 get(int s, const Tab4& t, const void*) const {
    // 24 bits per 8 codes: s = 0 -> a.x [0, 24), 1 -> (a.x, a.y) [24, 48), 2 -> (a.y, b) [48, 72), 3 -> b [72, 96)
    const uint32_t x = s == 0 ? a.x : s == 1 ? __builtin_amdgcn_alignbit(a.y, a.x, 24)
                     : s == 2 ? __builtin_amdgcn_alignbit(b, a.y, 16) : (b >> 8);
    return decode3_b(decode3_a(x, t), t);
  }
};

template <>
struct CodesA16<6> {
  uint4 a;
  v2u_t b;
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
    a = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
    b = __builtin_amdgcn_raw_buffer_load_b64(rs, off + 16, 0, 0);
  }
  __device__ __forceinline__ uint4 get(int s, const Tab4&, const void* lut) const {
    // 48 bits per 8 codes: s = 0 -> (a.x, a.y lo), 1 -> (a.y hi, a.z), 2 -> (a.w, b.x lo), 3 -> (b.x hi, b.y)
    uint32_t lo, hi;
    if (s == 0) { lo = a.x; hi = a.y & 0xFFFFu; }
    else if (s == 1) { lo = __builtin_amdgcn_alignbit(a.z, a.y, 16); hi = a.z >> 16; }
    else if (s == 2) { lo = a.w; hi = b.x & 0xFFFFu; }
    else { lo = __builtin_amdgcn_alignbit(b.y, b.x, 16); hi = b.y >> 16; }
    return decode6(lo, hi, static_cast<const uint32_t*>(lut));
  }
};

template <int BW>
__global__ __launch_bounds__(64 * kA16Waves) void k_a16_partial(A16Args a) {
  __shared__ __align__(16) unsigned char lut[BW == 6 ? 4096 * 4 : 16];
  __shared__ uint16_t mags[32];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if constexpr (needs_lut(BW)) {
    if (tid < 32) mags[tid] = a.mag[tid];
    __syncthreads();
    build_lut<BW, 64 * kA16Waves>(mags, lut, tid);
    __syncthreads();
  }
  const Tab4 tw{a.lt_lo, a.lt_hi, a.ht_lo, a.ht_hi};
  const int rblk = blockIdx.x % a.row_blocks, split = blockIdx.x / a.row_blocks;
  const int ss0 = split * a.ss_per_split;
  const int ss1 = min(a.nss, ss0 + a.ss_per_split);
  const int m16 = lane & 15, g = lane >> 4;
  const int64_t row_base = (static_cast<int64_t>(rblk) * kA16Waves + wave) * kA16Rows;

  // x' rows past nt read as zero; code rows past m read as zero (never stored)
  const __amdgpu_buffer_rsrc_t xs = uniform_rsrc(a.xr, a.xr_bytes);
  const int64_t rows_left = a.m - row_base;
  const uint32_t wc_bytes = rows_left <= 0 ? 0u : static_cast<uint32_t>(min<int64_t>(rows_left, kA16Rows) * a.rb);
  const __amdgpu_buffer_rsrc_t ws = uniform_rsrc(a.wc + (rows_left > 0 ? row_base * a.rb : 0), wc_bytes);
  const uint32_t xoff = static_cast<uint32_t>(m16 < a.nt ? m16 * a.d * 4 : 0x7FFFFFF0) ;
  f32x4_t acc[4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) acc[cb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  for (int ss = ss0; ss < ss1; ++ss) {
    const int k0 = ss * kA16SS + 32 * g;
    // A: 32 consecutive x' values of token m16
    float xv[32];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const uint4 v = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
          xs, xoff + static_cast<uint32_t>((k0 + 4 * c) * 4), 0, 0));
      xv[4 * c] = __builtin_bit_cast(float, v.x);
      xv[4 * c + 1] = __builtin_bit_cast(float, v.y);
      xv[4 * c + 2] = __builtin_bit_cast(float, v.z);
      xv[4 * c + 3] = __builtin_bit_cast(float, v.w);
    }
    CodesA16<BW> cw[4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
      cw[cb].load(ws, static_cast<uint32_t>((16 * cb + m16) * a.rb + k0 * BW / 8));
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const float* x8 = xv + 8 * s;
      const bf16x8_t av = {static_cast<__bf16>(x8[0]), static_cast<__bf16>(x8[2]), static_cast<__bf16>(x8[4]),
                           static_cast<__bf16>(x8[6]), static_cast<__bf16>(x8[1]), static_cast<__bf16>(x8[3]),
                           static_cast<__bf16>(x8[5]), static_cast<__bf16>(x8[7])};
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        const uint4 bw = cw[cb].get(s, tw, lut);
        acc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8_t, bw), acc[cb], 0, 0, 0);
      }
    }
  }
  // D[t][n]: t = 4 (lane / 16) + i, n = lane % 16 of column block cb
  float* part = a.part + static_cast<int64_t>(split) * a.nt * a.m;
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) {
    const int64_t row = row_base + 16 * cb + m16;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 4 * g + i;
      if (t < a.nt && row < a.m) part[static_cast<int64_t>(t) * a.m + row] = acc[cb][i];
    }
  }
}

template <bool OUT_BF16>
__global__ __launch_bounds__(256) void k_a16_reduce(const float* part, int splits, int nt, int64_t m,
                                                    const uint16_t* wn, void* Y, int64_t ldy) {
  const int64_t total = static_cast<int64_t>(nt) * m;
  for (int64_t e = blockIdx.x * 256ll + threadIdx.x; e < total; e += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t t = e / m, j = e - t * m;
    float acc = 0.0f;
    for (int s = 0; s < splits; ++s) acc += part[(static_cast<int64_t>(s) * nt + t) * m + j];
    const float v = acc * __builtin_bit_cast(float, static_cast<uint32_t>(wn[j]) << 16);
    if constexpr (OUT_BF16) reinterpret_cast<__bf16*>(Y)[t * ldy + j] = static_cast<__bf16>(v);
    else reinterpret_cast<float*>(Y)[t * ldy + j] = v;
  }
}

}  // namespace
}  // namespace lg

using namespace lg;

// Splits of the K range for the weight-only product: enough workgroups to stream the codes
// from every compute unit (about 1024), each split a whole number of 128-code super-steps.
void a16_splits(int64_t m, int64_t d, int* splits, int* ss_per_split, int* row_blocks) {
  const int64_t rb = (m + kA16Waves * kA16Rows - 1) / (kA16Waves * kA16Rows);
  const int nss = static_cast<int>(d / kA16SS);
  const int64_t want = std::max<int64_t>(1, std::min<int64_t>(nss, (1024 + rb - 1) / rb));
  const int per = static_cast<int>((nss + want - 1) / want);
  *ss_per_split = per;
  *splits = (nss + per - 1) / per;
  *row_blocks = static_cast<int>(rb);
}

int launch_a16_gemm(const float* x_rot, int nt, int64_t d, const uint8_t* w_codes, const uint16_t* w_norms,
                    const DecodeParams& dw, int64_t m, float* part, void* Y, int y_bf16, int64_t ldy,
                    hipStream_t stream) {
  A16Args a{};
  a.xr = x_rot;
  a.wc = w_codes;
  a.part = part;
  a.m = m;
  a.d = static_cast<int32_t>(d);
  a.nt = nt;
  a.rb = static_cast<int32_t>(d * dw.bits / 8);
  a.nss = static_cast<int32_t>(d / kA16SS);
  int splits = 1;
  a16_splits(m, d, &splits, &a.ss_per_split, &a.row_blocks);
  a.xr_bytes = static_cast<uint32_t>(static_cast<int64_t>(nt) * d * 4);
  tab4(dw, &a.lt_lo, &a.lt_hi, &a.ht_lo, &a.ht_hi);
  for (int i = 0; i < 32; ++i) a.mag[i] = dw.mag[i];
  const int grid = a.row_blocks * splits;
  switch (dw.bits) {
    case 2: hipLaunchKernelGGL(k_a16_partial<2>, dim3(grid), dim3(64 * kA16Waves), 0, stream, a); break;
    case 3: hipLaunchKernelGGL(k_a16_partial<3>, dim3(grid), dim3(64 * kA16Waves), 0, stream, a); break;
    case 4: hipLaunchKernelGGL(k_a16_partial<4>, dim3(grid), dim3(64 * kA16Waves), 0, stream, a); break;
    default: hipLaunchKernelGGL(k_a16_partial<6>, dim3(grid), dim3(64 * kA16Waves), 0, stream, a); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return static_cast<int>(e);
  const int64_t total = static_cast<int64_t>(nt) * m;
  const int rgrid = static_cast<int>(std::min<int64_t>((total + 255) / 256, 4096));
  if (y_bf16)
    hipLaunchKernelGGL(k_a16_reduce<true>, dim3(rgrid), dim3(256), 0, stream, part, splits, nt, m, w_norms, Y, ldy);
  else
    hipLaunchKernelGGL(k_a16_reduce<false>, dim3(rgrid), dim3(256), 0, stream, part, splits, nt, m, w_norms, Y, ldy);
  return static_cast<int>(hipGetLastError());
}


}  // namespace orbq
