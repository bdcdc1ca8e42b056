// a16_gemm: the weight-only product with bf16 activations (W{2,3,4,6}A16).
#include <algorithm>

#include "lut_gemm_kernel.h"

namespace orbq {
namespace lg {
namespace {

// ============================================================================ A16 (weight-only)
// Y[t][j] = r'_j sum_k bf16(x'_tk) bf16(C_w[w_jk]) for a few tokens (t < 16 per launch):
// x' = Pi x computed in fp32 and stored as bf16 by the rotate pass of rpbh_quantize, in the
// decoders' k order, so that 16 bytes of a row are one MFMA operand; codes streamed from HBM once.
// A workgroup owns 16 CB weight rows (CB 16-row MFMA column blocks, 2 to 5); each of its waves takes one
// split of the K range, with v_mfma_f32_16x16x32_bf16 and the tokens as the M side (rows past
// the token count read as zero).  A super-step covers 128 codes: lane (m = l % 16, g = l / 16)
// holds codes 32 g .. 32 g + 31 of it, i.e. one 16-byte (4-bit) load per row block, and takes
// them 8 at a time in four MFMAs, each with the matching 16 bytes of x' (already in the
// decoders' k order 0,2,4,6,1,3,5,7 within each 8).  The waves' partial sums meet in LDS, where they are added
// in split order and scaled by r'.
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

constexpr int kA16MaxSplits = 16;            // waves per workgroup, one K split each
constexpr int kA16MaxCB = 5;                  // 16-row MFMA column blocks per workgroup (2 to 5)
constexpr int kA16SS = 128;                   // codes per super-step

struct A16Args {
  const uint16_t* xr;    // x' [nt][d] bf16, k order 0,2,4,6,1,3,5,7 within each 8
  const uint8_t* wc;
  const uint16_t* wn;    // r' bf16 [m]
  void* Y;
  int64_t ldy;
  int64_t m;
  int32_t d, nt, rb;     // rb = code bytes per weight row
  int32_t ss_per_split, nss, splits;
  uint32_t xr_bytes;     // nt * d * 2
  uint32_t lt_lo, lt_hi, ht_lo, ht_hi;
  uint16_t mag[32];
  // rotation inside the product (ROT): each wave computes x' for its own K split from X, perm and
  // signs (one RPBH pass, h = 64 or 128) into LDS, at byte offset slice_off of the dynamic LDS
  const uint16_t* X;     // [nt][ldx] bf16
  int64_t ldx;
  const int32_t* perm;
  const int8_t* signs;
  int32_t h;
  float inv_scale;       // 1 / sqrt(h)
  uint32_t x_bytes;      // nt * ldx * 2 (< 2^31)
  uint32_t slice_off;
};

// x[i] += sgn * (x[i] in the DPP partner lane), for 8 registers, one v_fmac_f32_dpp each; the
// leading s_nop 4 covers the VALU-write -> DPP-read and EXEC-write -> DPP hazards of whatever
// the compiler placed before the block
#define ORBQ_A16_DPP_FMAC8(CTRL, X, S)                                                             \
  asm("s_nop 4\n"                                                                                 \
      "v_fmac_f32_dpp %0, %0, %8 " CTRL " row_mask:0xf bank_mask:0xf\n"                            \
      "v_fmac_f32_dpp %1, %1, %8 " CTRL " row_mask:0xf bank_mask:0xf\n"                            \
      "v_fmac_f32_dpp %2, %2, %8 " CTRL " row_mask:0xf bank_mask:0xf\n"                            \
      "v_fmac_f32_dpp %3, %3, %8 " CTRL " row_mask:0xf bank_mask:0xf\n"                            \
      "v_fmac_f32_dpp %4, %4, %8 " CTRL " row_mask:0xf bank_mask:0xf\n"                            \
      "v_fmac_f32_dpp %5, %5, %8 " CTRL " row_mask:0xf bank_mask:0xf\n"                            \
      "v_fmac_f32_dpp %6, %6, %8 " CTRL " row_mask:0xf bank_mask:0xf\n"                            \
      "v_fmac_f32_dpp %7, %7, %8 " CTRL " row_mask:0xf bank_mask:0xf\n"                            \
      : "+v"((X)[0]), "+v"((X)[1]), "+v"((X)[2]), "+v"((X)[3]), "+v"((X)[4]), "+v"((X)[5]),       \
        "+v"((X)[6]), "+v"((X)[7])                                                                 \
      : "v"(S))

__device__ __forceinline__ float a16_dot2(uint32_t a, uint32_t b) {
  float r;
  asm("v_dot2_f32_bf16 %0, %1, %2, 0" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float a16_dot2_neghi(uint32_t a, uint32_t b) {
  float r;
  asm("v_dot2_f32_bf16 %0, %1, %2, 0 neg_hi:[0,1,0]" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// One wave's slice of x' = Pi x (OrbitQuant summary, "Randomized Permuted Block-Hadamard (RPBH)
// Rotation"): positions p0 .. p0 + P - 1 of the nt tokens, written as bf16 (nearest even) to
// xl[t][p - p0], each aligned group of 8 in the decoders' order 0,2,4,6,1,3,5,7.  A lane takes 8
// consecutive positions 8 b .. 8 b + 7 of one Hadamard block of one token; the block's h / 8
// lanes hold b = M i over GF(2) (b0 = i0 ^ i2, b1 = i1 ^ i2, b2 = i2 ^ i3, b3 = i3), so that the
// butterfly partners b xor 1, 2, 4, 8 are the quad_perm [1,0,3,2], quad_perm [2,3,0,1],
// row_half_mirror and row_mirror lanes.  The arithmetic is rpbh_quantize's, stage for stage: the
// signs and the first stage as two v_dot2_f32_bf16 per pair, the stages on position bits 1 and 2
// as register adds, the rest as x += sgn * partner (which leaves upper lanes negated; that sign
// folds into the scale), then x * (sign / sqrt(h)) rounded to bf16.  So x' is bit for bit the
// rotate pass's.
__device__ __forceinline__ void a16_rotate_slice(const A16Args& a, int lane, int p0, int P, unsigned char* xl) {
  const int lpb = a.h >> 3;  // lanes per block: 8 or 16
  const int nblk = P / a.h, items = a.nt * nblk;
  const int li = lane & (lpb - 1);
  const int b = li ^ (((li >> 2) & 1) * 3) ^ (((li >> 3) & 1) * 4);
  const float sc = a.inv_scale * ((__builtin_popcount(b) & 1) ? -1.0f : 1.0f);
  const float s1 = (b & 1) ? -1.0f : 1.0f, s2 = (b & 2) ? -1.0f : 1.0f;
  const float s3 = (b & 4) ? -1.0f : 1.0f, s4 = (b & 8) ? -1.0f : 1.0f;
  const __amdgpu_buffer_rsrc_t xsrc = uniform_rsrc(a.X, a.x_bytes);
  const uint32_t dm1 = static_cast<uint32_t>(a.d - 1);
  for (int q0 = 0; q0 < items; q0 += 64 / lpb) {
    const int bi = q0 + lane / lpb;
    const bool valid = bi < items;
    const int t = valid ? bi / nblk : 0;
    const int jl = (valid ? bi - t * nblk : 0) * a.h + 8 * b;  // position within the slice
    const int j0 = p0 + jl;                                    // position within the row
    const int4 pa = *reinterpret_cast<const int4*>(a.perm + j0);
    const int4 pb = *reinterpret_cast<const int4*>(a.perm + j0 + 4);
    const uint2 sg = *reinterpret_cast<const uint2*>(a.signs + j0);
    const int pv[8] = {pa.x, pa.y, pa.z, pa.w, pb.x, pb.y, pb.z, pb.w};
    const uint32_t rowoff = static_cast<uint32_t>(t) * static_cast<uint32_t>(a.ldx);
    float y[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b16(
          xsrc, (rowoff + min(static_cast<uint32_t>(pv[2 * i]), dm1)) * 2u, 0, 0);
      const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b16(
          xsrc, (rowoff + min(static_cast<uint32_t>(pv[2 * i + 1]), dm1)) * 2u, 0, 0);
      const uint32_t x2 = (lo & 0xFFFFu) | (hi << 16);
      const uint32_t sb = (i < 2 ? sg.x : sg.y) >> (16 * (i & 1));  // the signs of positions 2i, 2i + 1
      const uint32_t smask = 0x3F803F80u | ((sb & 0x80u) << 8) | ((sb & 0x8000u) << 16);
      y[2 * i] = a16_dot2(x2, smask);
      y[2 * i + 1] = a16_dot2_neghi(x2, smask);
    }
#pragma unroll
    for (int st = 2; st < 8; st <<= 1) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (i & st) continue;
        const float u0 = y[i], u1 = y[i + st];
        y[i] = u0 + u1;
        y[i + st] = u0 - u1;
      }
    }
    ORBQ_A16_DPP_FMAC8("quad_perm:[1,0,3,2]", y, s1);
    ORBQ_A16_DPP_FMAC8("quad_perm:[2,3,0,1]", y, s2);
    ORBQ_A16_DPP_FMAC8("row_half_mirror", y, s3);
    if (lpb == 16) ORBQ_A16_DPP_FMAC8("row_mirror", y, s4);
    auto pair = [&](int lo, int hi) {
      typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
      const bf16x2_t p = {static_cast<__bf16>(y[lo] * sc), static_cast<__bf16>(y[hi] * sc)};
      return __builtin_bit_cast(uint32_t, p);
    };
    const uint4 w = make_uint4(pair(0, 2), pair(4, 6), pair(1, 3), pair(5, 7));
    if (valid) *reinterpret_cast<uint4*>(xl + (static_cast<uint32_t>(t) * P + jl) * 2u) = w;
  }
}

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

template <int BW, bool OUT_BF16, int CB, bool ROT>
__global__ __launch_bounds__(64 * kA16MaxSplits) void k_a16(A16Args a) {
  constexpr int kA16Rows = 16 * CB;  // weight rows of this workgroup
  __shared__ __align__(16) unsigned char lut[BW == 6 ? 4096 * 4 : 16];
  __shared__ uint16_t mags[32];
  extern __shared__ float red[];  // [splits][nt][16 CB] partial sums
  const int tid = threadIdx.x, lane = tid & 63, split = tid >> 6, nthreads = blockDim.x;
  if constexpr (needs_lut(BW)) {
    if (tid < 32) mags[tid] = a.mag[tid];
    __syncthreads();
    build_lut<BW>(mags, lut, tid, nthreads);
    __syncthreads();
  }
  const Tab4 tw{a.lt_lo, a.lt_hi, a.ht_lo, a.ht_hi};
  const int ss0 = split * a.ss_per_split;
  const int ss1 = min(a.nss, ss0 + a.ss_per_split);
  const int m16 = lane & 15, g = lane >> 4;
  const int64_t row_base = static_cast<int64_t>(blockIdx.x) * kA16Rows;

  // x' rows past nt read as zero; code rows past m read as zero (never stored)
  const __amdgpu_buffer_rsrc_t xs = uniform_rsrc(a.xr, a.xr_bytes);
  const int64_t rows_left = a.m - row_base;
  const uint32_t wc_bytes = rows_left <= 0 ? 0u : static_cast<uint32_t>(min<int64_t>(rows_left, kA16Rows) * a.rb);
  const __amdgpu_buffer_rsrc_t ws = uniform_rsrc(a.wc + (rows_left > 0 ? row_base * a.rb : 0), wc_bytes);
  const uint32_t xoff = static_cast<uint32_t>(m16 < a.nt ? m16 * a.d * 2 : 0x7FFFFFF0);
  f32x4_t acc[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) acc[cb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  // ROT: this wave's x' slice [nt][P] in LDS (the splits' slices follow one another)
  const int P = kA16SS * (ss1 - ss0);
  unsigned char* xl = reinterpret_cast<unsigned char*>(red) + a.slice_off +
                      static_cast<uint32_t>(a.nt) * (2u * kA16SS) * static_cast<uint32_t>(ss0);
  const uint32_t lrow = static_cast<uint32_t>(m16 < a.nt ? m16 : 0) * static_cast<uint32_t>(P) * 2u;
  CodesA16<BW> cw[CB];
  if constexpr (ROT) {
    // the first super-step's codes are in flight while the wave rotates its slice
    if (ss0 < ss1) {
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
        cw[cb].load(ws, static_cast<uint32_t>((16 * cb + m16) * a.rb + (ss0 * kA16SS + 32 * g) * BW / 8));
    }
    a16_rotate_slice(a, lane, kA16SS * ss0, P, xl);
    __syncthreads();
  }
  for (int ss = ss0; ss < ss1; ++ss) {
    const int k0 = ss * kA16SS + 32 * g;
    // A: the 32 x' values of token m16 that match the lane's codes, as four MFMA operands
    bf16x8_t xv[4];
    if constexpr (ROT) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint4 v = *reinterpret_cast<const uint4*>(xl + lrow + static_cast<uint32_t>((k0 - kA16SS * ss0 + 8 * c) * 2));
        xv[c] = __builtin_bit_cast(bf16x8_t, m16 < a.nt ? v : make_uint4(0, 0, 0, 0));
      }
      if (ss > ss0) {
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
          cw[cb].load(ws, static_cast<uint32_t>((16 * cb + m16) * a.rb + k0 * BW / 8));
      }
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c)
        xv[c] = __builtin_bit_cast(bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(
            xs, xoff + static_cast<uint32_t>((k0 + 8 * c) * 2), 0, 0));
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
        cw[cb].load(ws, static_cast<uint32_t>((16 * cb + m16) * a.rb + k0 * BW / 8));
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const bf16x8_t av = xv[s];
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const uint4 bw = cw[cb].get(s, tw, lut);
        acc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8_t, bw), acc[cb], 0, 0, 0);
      }
    }
  }
  // D[t][n]: t = 4 (lane / 16) + i, n = lane % 16 of column block cb
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 4 * g + i;
      if (t < a.nt) red[(split * a.nt + t) * kA16Rows + 16 * cb + m16] = acc[cb][i];
    }
  __syncthreads();
  for (int e = tid; e < a.nt * kA16Rows; e += nthreads) {
    const int t = e / kA16Rows, rr = e - t * kA16Rows;
    const int64_t j = row_base + rr;
    if (j >= a.m) continue;
    float sum = 0.0f;
    for (int sp = 0; sp < a.splits; ++sp) sum += red[(sp * a.nt + t) * kA16Rows + rr];
    const float v = sum * __builtin_bit_cast(float, static_cast<uint32_t>(a.wn[j]) << 16);
    if constexpr (OUT_BF16) reinterpret_cast<__bf16*>(a.Y)[t * a.ldy + j] = static_cast<__bf16>(v);
    else reinterpret_cast<float*>(a.Y)[t * a.ldy + j] = v;
  }
}

}  // namespace
}  // namespace lg

using namespace lg;

// Splits of the K range for the weight-only product: up to 16, one wave each, every split a
// whole number of 128-code super-steps; a workgroup holds its weight rows and all their splits.
void a16_splits(int64_t d, int* splits, int* ss_per_split) {
  const int nss = static_cast<int>(d / kA16SS);
  const int per = (nss + kA16MaxSplits - 1) / kA16MaxSplits;
  *ss_per_split = per;
  *splits = (nss + per - 1) / per;
}

namespace {

// 16-row column blocks per workgroup, 2 to 5.  The smallest count whose workgroups fit one per
// compute unit: each workgroup then has its compute unit to itself, and a wave's x' loads serve
// as many MFMAs as that allows.  The partial sums [splits][nt][16 CB] floats must fit the 64 KB
// of dynamic LDS.  When no count fits one workgroup per compute unit (m > 80 per CU), the count
// of 4 or 2 that puts the fewest rows on the busiest compute unit, 4 on ties.  Measured on 256
// compute units (same outputs bit for bit for every count): 16 x 3072 -> 18432 took 14.2 us with
// 5 blocks (231 workgroups) against 16.4, 18.1 and 18.8 with 3, 4 and 2; 2 x 3072 -> 18432
// 3-4 % less with 5 than with 2; 16 x 3072 -> 12288 13.6 with 3 (256 workgroups), 13.5 with 4.
int a16_column_blocks(int64_t m, int nt, int splits) {
  const int cus = device_cus();
  const int lds_cap = static_cast<int>(65536 / (static_cast<int64_t>(splits) * nt * 16 * sizeof(float)));
  const int top = std::min(kA16MaxCB, lds_cap);
  for (int cb = 2; cb <= top; ++cb)
    if ((m + 16 * cb - 1) / (16 * cb) <= cus) return cb;
  int best = 4;
  int64_t best_rows = INT64_MAX;
  for (int cb = 4; cb >= 2; cb /= 2) {
    const int64_t wg = (m + 16 * cb - 1) / (16 * cb);
    const int64_t rows = (wg + cus - 1) / cus * 16 * cb;
    if (rows < best_rows) {
      best_rows = rows;
      best = cb;
    }
  }
  return best;
}

template <int CB, bool ROT>
void launch_k_a16(int bits, bool out_bf16, dim3 grid, dim3 blk, size_t lds, hipStream_t st, const A16Args& a) {
  if (out_bf16) {
    switch (bits) {
      case 2: hipLaunchKernelGGL((k_a16<2, true, CB, ROT>), grid, blk, lds, st, a); break;
      case 3: hipLaunchKernelGGL((k_a16<3, true, CB, ROT>), grid, blk, lds, st, a); break;
      case 4: hipLaunchKernelGGL((k_a16<4, true, CB, ROT>), grid, blk, lds, st, a); break;
      default: hipLaunchKernelGGL((k_a16<6, true, CB, ROT>), grid, blk, lds, st, a); break;
    }
  } else {
    switch (bits) {
      case 2: hipLaunchKernelGGL((k_a16<2, false, CB, ROT>), grid, blk, lds, st, a); break;
      case 3: hipLaunchKernelGGL((k_a16<3, false, CB, ROT>), grid, blk, lds, st, a); break;
      case 4: hipLaunchKernelGGL((k_a16<4, false, CB, ROT>), grid, blk, lds, st, a); break;
      default: hipLaunchKernelGGL((k_a16<6, false, CB, ROT>), grid, blk, lds, st, a); break;
    }
  }
}

template <bool ROT>
void launch_cb(int cb, int bits, bool out_bf16, dim3 grid, dim3 blk, size_t lds, hipStream_t st, const A16Args& a) {
  switch (cb) {
    case 2: launch_k_a16<2, ROT>(bits, out_bf16, grid, blk, lds, st, a); break;
    case 3: launch_k_a16<3, ROT>(bits, out_bf16, grid, blk, lds, st, a); break;
    case 4: launch_k_a16<4, ROT>(bits, out_bf16, grid, blk, lds, st, a); break;
    default: launch_k_a16<5, ROT>(bits, out_bf16, grid, blk, lds, st, a); break;
  }
}

void a16_setup(A16Args& a, int nt, int64_t d, const uint8_t* w_codes, const uint16_t* w_norms, const DecodeParams& dw,
               int64_t m, void* Y, int64_t ldy) {
  a.wc = w_codes;
  a.wn = w_norms;
  a.Y = Y;
  a.ldy = ldy;
  a.m = m;
  a.d = static_cast<int32_t>(d);
  a.nt = nt;
  a.rb = static_cast<int32_t>(d * dw.bits / 8);
  a.nss = static_cast<int32_t>(d / kA16SS);
  a16_splits(d, &a.splits, &a.ss_per_split);
  tab4(dw, &a.lt_lo, &a.lt_hi, &a.ht_lo, &a.ht_hi);
  for (int i = 0; i < 32; ++i) a.mag[i] = dw.mag[i];
}

size_t round16(size_t x) { return (x + 15) & ~size_t(15); }

}  // namespace

int launch_a16_gemm(const uint16_t* x_rot, int nt, int64_t d, const uint8_t* w_codes, const uint16_t* w_norms,
                    const DecodeParams& dw, int64_t m, void* Y, int y_bf16, int64_t ldy, hipStream_t stream) {
  A16Args a{};
  a16_setup(a, nt, d, w_codes, w_norms, dw, m, Y, ldy);
  a.xr = x_rot;
  a.xr_bytes = static_cast<uint32_t>(static_cast<int64_t>(nt) * d * 2);
  const int cb = a16_column_blocks(m, nt, a.splits);
  const dim3 grid(static_cast<unsigned>((m + 16 * cb - 1) / (16 * cb))), blk(64 * a.splits);
  const size_t red = static_cast<size_t>(a.splits) * nt * 16 * cb * sizeof(float);
  launch_cb<false>(cb, dw.bits, y_bf16 != 0, grid, blk, red, stream, a);
  return static_cast<int>(hipGetLastError());
}

// The weight-only product with the rotation inside it (one launch): each workgroup's waves rotate
// their own K splits of the nt tokens into LDS (a16_rotate_slice) and stream the codes against
// them.  Every workgroup repeats the rotation, on its critical path, so this pays only while a
// wave's share is small: at most 8 (token, super-step) pairs, i.e. one or two gather passes per
// wave.  Measured against the rotation launch then the product (same outputs bit for bit):
// 2 x 3072 -> 18432 11.1-11.3 against 12.7-13.2 us, 5 x 1536 -> 8960 (h = 64) 9.1-9.5 against
// 11.8-12.4; with 3 passes (2 x 12288 -> 3072) 18.7 against 16.6, with 8 (16 x 3072 -> 18432)
// 24.0 against 14.1.  For one RPBH pass with a permutation and h = 64 or 128, when X's extent
// stays below 2^31 bytes and the x' slices (nt d bf16) fit in LDS beside the partial sums;
// otherwise returns hipErrorNotSupported and the caller rotates in a launch of its own.
int launch_a16_gemm_rot(const uint16_t* X, int64_t ldx, int nt, int64_t d, const int32_t* perm, const int8_t* signs,
                        int32_t h, const uint8_t* w_codes, const uint16_t* w_norms, const DecodeParams& dw, int64_t m,
                        void* Y, int y_bf16, int64_t ldy, hipStream_t stream) {
  if (!perm || (h != 64 && h != 128) || d % 128 || static_cast<int64_t>(nt) * ldx * 2 >= (int64_t(1) << 31))
    return static_cast<int>(hipErrorNotSupported);
  A16Args a{};
  a16_setup(a, nt, d, w_codes, w_norms, dw, m, Y, ldy);
  if (nt * a.ss_per_split > 8) return static_cast<int>(hipErrorNotSupported);
  const int cb = a16_column_blocks(m, nt, a.splits);
  const size_t red = round16(static_cast<size_t>(a.splits) * nt * 16 * cb * sizeof(float));
  const size_t slices = static_cast<size_t>(nt) * d * 2;
  const size_t fixed = (dw.bits == 6 ? 4096 * 4 : 16) + 64;  // the kernel's static LDS
  if (red + slices + fixed > 160 * 1024) return static_cast<int>(hipErrorNotSupported);
  a.X = X;
  a.ldx = ldx;
  a.perm = perm;
  a.signs = signs;
  a.h = h;
  a.inv_scale = 1.0f / __builtin_sqrtf(static_cast<float>(h));
  a.x_bytes = static_cast<uint32_t>(static_cast<int64_t>(nt) * ldx * 2);
  a.slice_off = static_cast<uint32_t>(red);
  const dim3 grid(static_cast<unsigned>((m + 16 * cb - 1) / (16 * cb))), blk(64 * a.splits);
  launch_cb<true>(cb, dw.bits, y_bf16 != 0, grid, blk, red + slices, stream, a);
  return static_cast<int>(hipGetLastError());
}

}  // namespace orbq
