#pragma once
// rpbh_quantize kernel (shared by the per-block-size instantiation units rpbh_quantize_b*.hip and
// the host side in rpbh_quantize.hip).
//
// rpbh_quantize: one pass over bf16 token rows that applies the RPBH rotation, takes the row
// norm, normalises and quantizes every coordinate to a Lloyd-Max codebook, and packs the codes.
//
// Method: OrbitQuant summary (picx.dev), "Online Activation Quantization" (rotate, normalise,
// quantize) and "Randomized Permuted Block-Hadamard (RPBH) Rotation"
// (Pi = blkdiag(H_h D_i) P_pi, O(d log h) by the fast Walsh-Hadamard transform).  The same
// kernel folds weight rows ("Offline Weight Quantization") with bf16 norms.
//
// Work layout (gfx950, wave64):
//   * 16 post-permutation positions of one token per lane; a Hadamard block of h = 128 spans 8
//     lanes (h = 64: 4 lanes).  A workgroup holds `tg` tokens (up to 1024 threads) and loops over
//     token groups (persistent grid sized by the kernel's occupancy).  Short rows per lane keep the
//     registers low, so six or more waves share each SIMD and hide the load / LDS / barrier
//     latencies.
//   * Staging: the lanes of a token load its bf16 row with coalesced 16-byte loads (lane q takes
//     chunks q and q + L), prefetched one token group ahead in registers, store it to LDS and add
//     the squares into a partial norm (sum of squares is invariant under Pi).  The LDS row is
//     double-buffered: every 128 positions own 512 bytes, the first 256 for even token groups and
//     the second 256 for odd ones, so the buffer is an immediate offset of every LDS access (the
//     loop body is unrolled for the two buffers) and one barrier per token group suffices.
//   * Norm: the partial sums are reduced over each wave (or over aligned lane segments when
//     tokens share a wave) with DPP adds; after the barrier every lane reads up to 16 partials of
//     its token (zero-padded) and adds them with four more DPP adds.
//   * Compute: each lane gathers its 16 permuted positions x[perm[j]] from LDS as bf16 pairs (a
//     16-bit read into each half of a register; addresses precomputed once from perm) and runs
//     the block FWHT: the Rademacher signs, the first butterfly stage and the bf16 -> fp32
//     widening are two v_dot2_f32_bf16 per bf16 pair against the pair's signs (the second with
//     the high sign negated), the next three stages run in registers, the last log2(h/16) stages
//     across lanes with v_fmac_f32_dpp (lanes placed so that every partner is a quad_perm or
//     row_half_mirror lane).
//   * Quantization uses the power-of-two-scaled coordinate t' = t * 2^k: one table lookup on
//     floor(-t') and one fp32 compare give the exact nearest-centroid decision (QuantParams).
//   * Codes are packed in registers and written with one 4/8/12-byte store per lane.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <type_traits>

#include "internal.h"

namespace orbq {
namespace rq {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));

constexpr int kE = 16;       // positions per lane
constexpr int kCH = kE / 8;  // 16-byte input chunks staged per lane
constexpr int kNP = 16;      // norm partials read per token after the barrier (zero-padded)
constexpr uint32_t kGroupBytes = 256;  // LDS bytes per 128 positions of a staged row
constexpr int kHostTableHalf = 32;     // decision tables with J <= 32 are built on the host

struct QuantKernelArgs {
  const uint16_t* X;
  int64_t n;
  int64_t ldx;
  const int32_t* perm;
  const int8_t* signs;
  uint8_t* codes;
  void* norms;
  float* x_rot;
  int32_t d;
  int32_t lpt;      // lanes per token = d / 16
  int32_t tg;       // tokens per workgroup iteration
  int32_t seg;      // power-of-two lane segment reduced with DPP (64 when tg == 1)
  int32_t seg_lev;  // log2(seg)
  int32_t nseg;     // partial sums per token
  int32_t row_reduce;  // 1: lpt % 16 == 0 and nseg <= 16 (partials added by a 16-lane DPP tree)
  uint32_t div_magic;  // tid / lpt == (tid * div_magic) >> 32 for tid < 1024
  int32_t ngroups;
  float eps;
  float inv_scale;  // 2^k / sqrt(h) (quantize) or 1 / sqrt(h) (rotate only)
  uint32_t codes_bytes, norms_bytes, rot_bytes;  // buffer extents (< 2^31) for bounds-dropped stores
  uint32_t x_bytes;                              // extent of X in this launch (< 2^31)
  uint32_t row_lds;                              // LDS bytes per staged token row
  uint32_t tbl_off, part_off, part_stride;       // LDS byte offsets: table, partials; floats per token
  int32_t passes;                                // composed RPBH passes (1..3)
  uint32_t xf_off;                               // LDS byte offset of the fp32 rows (passes > 1)
  float rsqrt_h;                                 // 1 / sqrt(h), the scale of each earlier pass
  int32_t host_tbl;                              // 1: htbl holds the decision table (J <= 32)
  int32_t full;                                  // 1: the full-range table (2-, 3-, 4-bit, one pass)
  int32_t jf;                                    // table half-size: buckets -jf..jf-1 (2^k + 2 when full, else J)
  int32_t pipe;                                  // 1: software-pipelined loop, staging and partials double-buffered
  QuantParams qp;
  float2 htbl[2 * kHostTableHalf];               // buckets -J..J-1 as build_table makes them
};

typedef int v4i_t __attribute__((ext_vector_type(4)));
typedef uint32_t v2u_t __attribute__((ext_vector_type(2)));
constexpr uint32_t kBufWord3 = 0x00020000u;  // raw (untyped) buffer resource, gfx9 family
constexpr uint32_t kDropped = 0xFFFFFF00u;   // offset past every extent: the access is discarded

__device__ __forceinline__ float dot2_acc(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c, false);
}


// x[i] += sgn * (x[i] in the lane whose index differs in bit 0 / bit 1), for 8 registers, with
// v_fmac_f32_dpp (one instruction per element).  The leading s_nop 4 covers the VALU-write ->
// DPP-read and EXEC-write -> DPP hazards for whatever the compiler placed before the block.
#define ORBQ_DPP_FMAC8(CTRL, X, S)                                                                  \
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

// floor(-x) as an int: one v_cvt_flr_i32_f32 with a negated source (the compiler's own lowering of
// floorf then a conversion takes two instructions)
__device__ __forceinline__ int floor_neg_to_int(float x) {
  int r;
  asm("v_cvt_flr_i32_f32_e64 %0, -%1" : "=v"(r) : "v"(x));
  return r;
}

__device__ __forceinline__ int med3_i32(int x, int lo, int hi) {
  int r;
  asm("v_med3_i32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "s"(lo), "v"(hi));
  return r;
}

// (c << sh) | w in one instruction (the compiler otherwise builds shift-or trees of two ops per
// pair of codes)
__device__ __forceinline__ uint32_t lshl_or(uint32_t c, uint32_t sh, uint32_t w) {
  uint32_t r;
  asm("v_lshl_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(c), "i"(sh), "v"(w));
  return r;
}

__device__ __forceinline__ uint16_t bf16_rne_dev(float x) {
  uint32_t u = __builtin_bit_cast(uint32_t, x);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Builds the per-bucket table: entry for bucket j = floor(-t') in [-J, J-1] is
// (threshold, base code); the code is base + (|t'| > threshold).  The loop over the BITS-bit
// codebook's positive boundaries is unrolled so that the thresholds are read from the kernel
// arguments once (scalar loads with constant offsets), and the body has no branches.
template <int BITS, bool DEC = false>
__device__ void build_table(const QuantParams& qp, float2* tbl, int tid, int nthreads) {
  constexpr int NB = (1 << (BITS - 1)) - 1, HALF = 1 << (BITS - 1);
  const int J = qp.J;
  for (int e = tid; e < 2 * J; e += nthreads) {
    const int j = e - J;
    const bool pos = j < 0;  // t' in (i, i + 1] with i = -j - 1; else |t'| in [j, j + 1), t' <= 0
    const float lo = static_cast<float>(pos ? -j - 1 : j), hi = lo + 1.0f;
    float thr = __builtin_inff();
    int base = pos ? 0 : HALF;
    // (not unrolled for 6-bit codebooks: 31 boundaries unrolled would set the register budget of
    // the whole kernel)
#pragma unroll 8
    for (int p = 0; p < NB; ++p) {
      const float b = pos ? qp.thr_gt[p] : qp.thr_ge[p];
      const bool below = pos ? (b <= lo) : (b < lo);
      base += below ? 1 : 0;
      thr = (!below && b < hi) ? b : thr;
    }
    if constexpr (DEC) {  // the bf16 centroids of codes base and base + 1 (base + 1 only when thr is finite)
      const uint32_t lo = qp.vals[base], hi = qp.vals[min(base + 1, 2 * HALF - 1)];
      tbl[e] = make_float2(thr, __builtin_bit_cast(float, lo | (hi << 16)));
    } else {
      tbl[e] = make_float2(thr, __builtin_bit_cast(float, base));
    }
  }
}

template <bool CLAMP = true>
__device__ __forceinline__ uint32_t quantize_one(float tp, const float2* tbl, int J) {
  // CLAMP = false: the table covers every bucket |t'| <= 2^k (1 + 1e-6) can reach, so no clamp
  const int j = CLAMP ? med3_i32(floor_neg_to_int(tp), -J, J - 1) : floor_neg_to_int(tp);
  const float2 e = tbl[j];  // tbl points at bucket 0
  return static_cast<uint32_t>(__builtin_bit_cast(int, e.y)) + (__builtin_fabsf(tp) > e.x ? 1u : 0u);
}

// Codes of four coordinates: the four table reads are issued together, then decided
template <bool CLAMP>
__device__ __forceinline__ void quantize4(const float* y, float inv_s, const float2* tbl, int J, uint32_t (&c)[4]) {
  float t[4];
  float2 e[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    t[k] = y[k] * inv_s;
    const int j = CLAMP ? med3_i32(floor_neg_to_int(t[k]), -J, J - 1) : floor_neg_to_int(t[k]);
    e[k] = tbl[j];
  }
#pragma unroll
  for (int k = 0; k < 4; ++k)
    c[k] = static_cast<uint32_t>(__builtin_bit_cast(int, e[k].y)) + (__builtin_fabsf(t[k]) > e[k].x ? 1u : 0u);
}

// The same decision against a table of centroid pairs: the bf16 centroid of the code (low 16 bits)
__device__ __forceinline__ uint32_t quantize_value(float tp, const float2* tbl, int J) {
  const int j = med3_i32(floor_neg_to_int(tp), -J, J - 1);
  const float2 e = tbl[j];
  const uint32_t vp = __builtin_bit_cast(uint32_t, e.y);
  return __builtin_fabsf(tp) > e.x ? (vp >> 16) : (vp & 0xFFFFu);
}

// bf16 pair dot product with a zero accumulator, second operand in a VGPR (VOP3P form)
__device__ __forceinline__ float dot2_v(uint32_t a, uint32_t b) {
  float r;
  asm("v_dot2_f32_bf16 %0, %1, %2, 0" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// bf16 pair dot product with the high half of the second operand negated (VOP3P neg_hi)
__device__ __forceinline__ float dot2_neghi(uint32_t a, uint32_t b) {
  float r;
  asm("v_dot2_f32_bf16 %0, %1, %2, 0 neg_hi:[0,1,0]" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_add(float x) {
  return x + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, ROWS, 0xF, false));
}

// Sum over aligned segments of 2^lev lanes (lev <= 6, uniform); the last lane of each segment
// holds the segment's sum (for lev <= 4 every lane does).  The levels nest, so that each test is
// one scalar branch on the uniform level count.
__device__ __forceinline__ float segment_sum(float x, int lev) {
  if (lev >= 4) {
    x = dpp_add<0xB1, 0xF>(x);   // quad_perm [1,0,3,2]
    x = dpp_add<0x4E, 0xF>(x);   // quad_perm [2,3,0,1]
    x = dpp_add<0x141, 0xF>(x);  // row_half_mirror: 8 lanes
    x = dpp_add<0x140, 0xF>(x);  // row_mirror: 16 lanes
    if (lev >= 5) {
      // row_bcast:15 into rows 1 and 3 (32 lanes), then row_bcast:31 into rows 2 and 3 (64
      // lanes); rows outside the row mask keep their value, so each step is one instruction.
      // s_nop 1: the VALU-write -> DPP-read hazard.
      asm("s_nop 1\n v_add_f32_dpp %0, %0, %0 row_bcast:15 row_mask:0xa bank_mask:0xf" : "+v"(x));
      if (lev >= 6) asm("s_nop 1\n v_add_f32_dpp %0, %0, %0 row_bcast:31 row_mask:0xc bank_mask:0xf" : "+v"(x));
    }
  } else {
    if (lev >= 1) x = dpp_add<0xB1, 0xF>(x);
    if (lev >= 2) x = dpp_add<0x4E, 0xF>(x);
    if (lev >= 3) x = dpp_add<0x141, 0xF>(x);
  }
  return x;
}

// Sum over each row of 16 lanes, in every lane of the row
__device__ __forceinline__ float row16_sum(float x) {
  x = dpp_add<0xB1, 0xF>(x);
  x = dpp_add<0x4E, 0xF>(x);
  x = dpp_add<0x141, 0xF>(x);
  return dpp_add<0x140, 0xF>(x);
}

// Two bf16 values from LDS into the halves of one register: a 16-bit read into the low half and
// one into the high half (ds_read_u16_d16 / ds_read_u16_d16_hi), no repacking.
__device__ __forceinline__ uint32_t lds_pair(const unsigned char* base, uint32_t a0, uint32_t a1) {
  u16x2_t v;
  v.x = *reinterpret_cast<const unsigned short*>(base + a0);
  v.y = *reinterpret_cast<const unsigned short*>(base + a1);
  return __builtin_bit_cast(uint32_t, v);
}

// LDS byte offset of position p in a staged row
__device__ __forceinline__ uint32_t row_pos(uint32_t p) { return (p >> 7) * kGroupBytes + (p & 127u) * 2u; }

// MULTI: the rotation is the composition Pi_P ... Pi_1 of a.passes RPBH passes, pass p with its
// own permutation and signs at perm + p d, signs + p d (RHT page, composed randomized Hadamard
// transforms).  Between passes the fp32 rotated row goes through LDS for the next gather (or
// stays in registers when the permutations are the identity).
//
// FULL (2-, 3- and 4-bit codes, chosen on the host when each workgroup runs enough token groups to
// amortise filling it): the decision table covers every bucket t' can reach, so the per-coordinate
// clamp of the bucket index goes away.
//
// PIPE (one pass, quantizing; chosen on the host for large workgroups that run several token
// groups): one barrier per group instead of two, with the staged rows and the norm partials
// double-buffered in LDS (the loop at the end of the kernel says why that is safe).
//
// At most 80 VGPRs (six waves per SIMD) for one pass with blocks up to 256: a workgroup of 9 or 12
// waves (d = 8960, 12288) then places two workgroups on a compute unit; at five waves per SIMD
// (85 VGPRs, measured: 249 against 196 us at 32760 x 8960) fewer fit.  Composed passes and the
// 512- and 1024-wide blocks (more live values in the cross-lane stages) would spill under the cap.
template <int H, int BITS, QuantMode MODE, bool PERM, bool MULTI, bool FULL, bool PIPE>
__global__ __launch_bounds__(1024) __attribute__((amdgpu_waves_per_eu((MULTI || H > 256) ? 1 : 6))) void k_rpbh_quantize(QuantKernelArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int d = a.d;
  const int tid = threadIdx.x;
  // token slot and lane within the token (tid / lpt by a multiply-high)
  const int slot_raw = static_cast<int>((static_cast<uint64_t>(tid) * a.div_magic) >> 32);
  const bool active = slot_raw < a.tg;
  const int slot = active ? slot_raw : 0;
  const int q = active ? tid - slot_raw * a.lpt : 0;
  const int J = a.qp.J;
  float2* tbl_all = reinterpret_cast<float2*>(smem + a.tbl_off);
  float* part = reinterpret_cast<float*>(smem + a.part_off);  // [2][tg][part_stride]
  // Lane -> positions: a Hadamard block of h spans h / 16 consecutive lanes; lane i of a block
  // holds the 16 positions 16 b .. 16 b + 15 of the block with b = M i over GF(2):
  //   b0 = i0 ^ i2,  b1 = i1 ^ i2,  b2 = i2 ^ i3,  b3 = i3,  b4 = i4,  b5 = i5,
  // so that the partners of the cross-lane butterfly stages b xor 1, 2, 4, 8 are the DPP
  // quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror (i xor 7) and row_mirror
  // (i xor 15) lanes, and b xor 16, 32 the lanes i xor 16 (ds_swizzle) and i xor 32.
  constexpr int LPB = H / kE;  // lanes per Hadamard block (4 .. 64)
  const int li = q & (LPB - 1);
  const int bl = li ^ (((li >> 2) & 1) * 3) ^ (((li >> 3) & 1) * 4);
  const int j0 = H * (q / LPB) + kE * bl;

  // X is read through a buffer resource that ends at the last row of the launch: rows past the
  // end read as zero (and are never stored); idle lanes read nothing (their loads are dropped)
  const __amdgpu_buffer_rsrc_t x_rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(a.X), 0, a.x_bytes, kBufWord3);
  const uint32_t ldx_bytes = static_cast<uint32_t>(a.ldx) * 2u;
  const uint32_t lane_off = static_cast<uint32_t>(slot) * ldx_bytes + static_cast<uint32_t>(16 * q);
  const uint32_t chunk_step = static_cast<uint32_t>(16 * a.lpt);
  const uint32_t group_step = static_cast<uint32_t>(a.tg) * ldx_bytes;
  // idle lanes: 2^31 plus the chunk step stays past every extent (< 2^31) without wrapping
  auto load_group = [&](int g, uint4 v[kCH]) {
    const uint32_t off = active ? static_cast<uint32_t>(g) * group_step + lane_off : 0x80000000u;
#pragma unroll
    for (int c = 0; c < kCH; ++c)
      v[c] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(x_rs, off + static_cast<uint32_t>(c) * chunk_step, 0, 0));
  };
  uint4 v[kCH];
  load_group(blockIdx.x, v);  // first group in flight during the set-up

  constexpr bool kRotate = MODE == QuantMode::kRotateOnly || MODE == QuantMode::kRotateBf16;
  // 2-, 3- and 4-bit codes: the table covers buckets -jf..jf-1, every bucket floor(-t') can reach
  // (the buckets past +-J repeat the outermost ones); 6-bit codes clamp the bucket to -J..J-1
  constexpr bool kFull = FULL && BITS <= 4 && !kRotate && MODE != QuantMode::kDecoded;
  const int TH = kFull ? a.jf : J;  // half-size of the table in LDS
  if constexpr (!kRotate) {
    if (a.host_tbl) {  // copied from the kernel arguments (per-lane loads from the kernarg segment)
#if defined(__HIP_DEVICE_COMPILE__)
      typedef __attribute__((address_space(4))) const QuantKernelArgs KArgs;
      KArgs* ka = (KArgs*)__builtin_amdgcn_kernarg_segment_ptr();
      // buckets past +-J lie beyond every boundary: no threshold inside, and all NB boundaries
      // below (base NB for t' > 0, 2^(b-1) + NB for t' <= 0)
      constexpr int NB = (1 << (BITS - 1)) - 1, HALF = 1 << (BITS - 1);
      const float2 out_pos = make_float2(__builtin_inff(), __builtin_bit_cast(float, NB));
      const float2 out_neg = make_float2(__builtin_inff(), __builtin_bit_cast(float, HALF + NB));
      for (int e = tid; e < 2 * TH; e += blockDim.x) {
        const int j = e - TH;
        const float2 in = ka->htbl[min(max(j, -J), J - 1) + J];  // a value select, not a pointer one
        tbl_all[e] = j < -J ? out_pos : j >= J ? out_neg : in;
      }
#endif
    } else {
      build_table<BITS, MODE == QuantMode::kDecoded>(a.qp, tbl_all + (TH - J), tid, blockDim.x);
      if (kFull) {  // the outer buckets repeat the outermost built ones
        __syncthreads();
        for (int e = tid; e < 2 * TH; e += blockDim.x)
          if (e < TH - J || e >= TH + J) tbl_all[e] = tbl_all[min(max(e - TH, -J), J - 1) + TH];
      }
    }
  }
  const float2* tbl = tbl_all + TH;
  // zero the padding of the partial sums (entries nseg .. 15 of each token are never written)
  if (a.row_reduce)
    for (int e = tid; e < (PIPE ? 2 : 1) * a.tg * kNP; e += blockDim.x)
      if ((e & (kNP - 1)) >= a.nseg) part[e] = 0.0f;

  // ---- set-up: gather addresses x[perm[j]] (LDS byte offsets) and sign masks of this lane
  const uint32_t rowbase = static_cast<uint32_t>(slot) * a.row_lds;
  uint32_t gaddr[kE];
  uint32_t smask[kE / 2];  // bf16 pairs (s_2i, s_2i+1) of the Rademacher signs
  {
    if constexpr (PERM) {
      const int4* pp = reinterpret_cast<const int4*>(a.perm + j0);
      const uint32_t dm1 = static_cast<uint32_t>(d - 1);
#pragma unroll
      for (int c = 0; c < kE / 4; ++c) {
        const int4 p4 = pp[c];
        const int pv[4] = {p4.x, p4.y, p4.z, p4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) gaddr[4 * c + e] = rowbase + row_pos(min(static_cast<uint32_t>(pv[e]), dm1));
      }
    } else {
#pragma unroll
      for (int e = 0; e < kE; ++e) gaddr[e] = 0u;
    }
    const uint4 s0 = *reinterpret_cast<const uint4*>(a.signs + j0);  // kE = 16 signs
    const uint32_t sw[4] = {s0.x, s0.y, s0.z, s0.w};
#pragma unroll
    for (int i = 0; i < kE / 2; ++i) {  // int8 signs 2i, 2i+1 -> bf16 (s_2i, s_2i+1)
      const uint32_t b = sw[i >> 1] >> (16 * (i & 1));
      smask[i] = 0x3F803F80u | ((b & 0x80u) << 8) | ((b & 0x8000u) << 16);
    }
  }
  // cross-lane butterflies leave the result negated in lanes with an odd number of "upper"
  // positions; fold that sign into the per-token scale
  const float lane_sign = (__builtin_popcount(bl) & 1) ? -1.0f : 1.0f;
  const float sgn1 = (bl & 1) ? -1.0f : 1.0f;
  const float sgn2 = (bl & 2) ? -1.0f : 1.0f;
  const float sgn3 = (bl & 4) ? -1.0f : 1.0f;
  const float sgn4 = (bl & 8) ? -1.0f : 1.0f;
  const float sgn5 = (bl & 16) ? -1.0f : 1.0f;
  const float sgn6 = (bl & 32) ? -1.0f : 1.0f;
  // staging addresses of this lane's two 16-byte chunks (chunks q and q + lpt, 8 positions each)
  const uint32_t cq0 = static_cast<uint32_t>(q), cq1 = static_cast<uint32_t>(q + a.lpt);
  const uint32_t st0 = rowbase + (cq0 >> 4) * kGroupBytes + (cq0 & 15u) * 16u;
  const uint32_t st1 = rowbase + (cq1 >> 4) * kGroupBytes + (cq1 & 15u) * 16u;
  const uint32_t idaddr = rowbase + row_pos(static_cast<uint32_t>(j0));  // identity: 16 contiguous positions
  // partial-sum slot written by the last lane of each segment, and the one this lane reads
  // (one token per workgroup: lane 63 of every wave, idle lanes of the last wave included)
  const bool pwriter = a.tg == 1 ? (tid & 63) == 63 : (active && (q & (a.seg - 1)) == a.seg - 1);
  const uint32_t pw_off =
      (static_cast<uint32_t>(slot) * a.part_stride + static_cast<uint32_t>(a.tg == 1 ? tid >> 6 : q >> a.seg_lev)) * 4u;
  const uint32_t pr_off = static_cast<uint32_t>(slot) * a.part_stride * 4u;

  // Stores go through buffer resources: lanes with nothing to store (rows past the end, idle
  // lanes) get an offset past the extent and the hardware drops the store.  The loop body has no
  // branches around memory operations, so the compiler's wait counts stay exact (on gfx9 vmcnt
  // also counts stores: a conservative wait would stall on the previous group's stores).
  const __amdgpu_buffer_rsrc_t codes_rs = __builtin_amdgcn_make_buffer_rsrc(a.codes, 0, a.codes_bytes, kBufWord3);
  const __amdgpu_buffer_rsrc_t norms_rs = __builtin_amdgcn_make_buffer_rsrc(a.norms, 0, a.norms_bytes, kBufWord3);
  const __amdgpu_buffer_rsrc_t rot_rs = __builtin_amdgcn_make_buffer_rsrc(a.x_rot, 0, a.rot_bytes, kBufWord3);
  const uint32_t row_bytes = static_cast<uint32_t>(d * BITS / 8);
  const int stride = static_cast<int>(gridDim.x);

  // ---- one token group: stage (rows into LDS buffer sb, next group's loads issued), rotate
  // (gather, norm partials into buffer pb, FWHT), finish (token norm, quantize, store)
  float y[kE];
  const uint32_t stbuf = static_cast<uint32_t>(a.tg) * a.row_lds;         // second staging buffer
  const uint32_t pbuf = static_cast<uint32_t>(a.tg) * a.part_stride * 4u;  // second partials buffer
  auto stage = [&](int g, uint32_t sb) {
    if (active) {
      *reinterpret_cast<uint4*>(smem + sb + st0) = v[0];
      *reinterpret_cast<uint4*>(smem + sb + st1) = v[1];
    }
    // prefetch the next group (the last iteration reloads its own group: no branch)
    load_group(g + stride < a.ngroups ? g + stride : g, v);
  };
  auto rotate = [&](uint32_t sb, uint32_t pb) {
    // ---- gather the 16 permuted positions as bf16 pairs; partial sum of squares over them;
    // signs, FWHT stage 1 (+ widening).  The norm is summed over the gathered (rotation-order)
    // values, so it does not depend on the order the row is stored in: a row stored permuted and
    // rotated without the permutation gives the same bits.
    float ss = 0.0f;
    if constexpr (PERM) {
#pragma unroll
      for (int i = 0; i < kE / 2; ++i) {
        const uint32_t x2 = lds_pair(smem + sb, gaddr[2 * i], gaddr[2 * i + 1]);
        ss = dot2_acc(x2, x2, ss);
        y[2 * i] = dot2_v(x2, smask[i]);
        y[2 * i + 1] = dot2_neghi(x2, smask[i]);
      }
    } else {  // identity permutation (block RHT): the lane's 16 positions are contiguous
      const uint4 c0 = *reinterpret_cast<const uint4*>(smem + sb + idaddr);
      const uint4 c1 = *reinterpret_cast<const uint4*>(smem + sb + idaddr + 16u);
      const uint32_t x2s[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
#pragma unroll
      for (int i = 0; i < kE / 2; ++i) {
        ss = dot2_acc(x2s[i], x2s[i], ss);
        y[2 * i] = dot2_v(x2s[i], smask[i]);
        y[2 * i + 1] = dot2_neghi(x2s[i], smask[i]);
      }
    }
    if (!active) ss = 0.0f;  // idle lanes gathered slot 0's values
    ss = segment_sum(ss, a.seg_lev);
    if (pwriter) *reinterpret_cast<float*>(smem + a.part_off + pb + pw_off) = ss;
    // ---- FWHT stages 2..4 in registers, then the cross-lane stages
    auto fwht_tail = [&](float (&y)[kE]) {
#pragma unroll
      for (int st = 2; st < kE; st <<= 1) {
#pragma unroll
        for (int i = 0; i < kE; ++i) {
          if (i & st) continue;
          const float u0 = y[i], u1 = y[i + st];
          y[i] = u0 + u1;
          y[i + st] = u0 - u1;
        }
      }
      // ---- remaining stages across the lanes of the block: x += sgn * partner
      if constexpr (LPB >= 2) {
        ORBQ_DPP_FMAC8("quad_perm:[1,0,3,2]", y, sgn1);
        ORBQ_DPP_FMAC8("quad_perm:[1,0,3,2]", y + 8, sgn1);
      }
      if constexpr (LPB >= 4) {
        ORBQ_DPP_FMAC8("quad_perm:[2,3,0,1]", y, sgn2);
        ORBQ_DPP_FMAC8("quad_perm:[2,3,0,1]", y + 8, sgn2);
      }
      if constexpr (LPB >= 8) {
        ORBQ_DPP_FMAC8("row_half_mirror", y, sgn3);
        ORBQ_DPP_FMAC8("row_half_mirror", y + 8, sgn3);
      }
      if constexpr (LPB >= 16) {
        ORBQ_DPP_FMAC8("row_mirror", y, sgn4);
        ORBQ_DPP_FMAC8("row_mirror", y + 8, sgn4);
      }
      if constexpr (LPB >= 32) {  // partner lane i xor 16 (within 32 lanes): ds_swizzle bit mode
#pragma unroll
        for (int e = 0; e < kE; ++e)
          y[e] = __builtin_fmaf(sgn5, __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, y[e]), 0x401F)), y[e]);
      }
      if constexpr (LPB >= 64) {  // partner lane i xor 32
        const int pa = (static_cast<int>(threadIdx.x & 63) ^ 32) << 2;
#pragma unroll
        for (int e = 0; e < kE; ++e)
          y[e] = __builtin_fmaf(sgn6, __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(pa, __builtin_bit_cast(int, y[e]))), y[e]);
      }
      // Blocks of 2048 and 4096 span 2 and 4 waves: their last one or two stages pair lanes of
      // different waves (block lane i xor 64, xor 128; positions j0 xor 1024, xor 2048).  Each
      // goes through the token's fp32 row in LDS: every lane writes its 16 values, a barrier,
      // the partner's 16 are read back, and a barrier before the row is written again.
#pragma unroll
      for (int k = 6; (1 << k) < LPB; ++k) {
        float* xrow = reinterpret_cast<float*>(smem + a.xf_off) + slot * d;
        if (active) {
#pragma unroll
          for (int c = 0; c < kE / 4; ++c)
            *reinterpret_cast<float4*>(xrow + j0 + 4 * c) = make_float4(y[4 * c], y[4 * c + 1], y[4 * c + 2], y[4 * c + 3]);
        }
        __syncthreads();
        const float sg = (bl >> k) & 1 ? -1.0f : 1.0f;
        const float* prow = xrow + (j0 ^ (kE << k));
#pragma unroll
        for (int c = 0; c < kE / 4; ++c) {
          const float4 pv = *reinterpret_cast<const float4*>(prow + 4 * c);
          y[4 * c] = __builtin_fmaf(sg, pv.x, y[4 * c]);
          y[4 * c + 1] = __builtin_fmaf(sg, pv.y, y[4 * c + 1]);
          y[4 * c + 2] = __builtin_fmaf(sg, pv.z, y[4 * c + 2]);
          y[4 * c + 3] = __builtin_fmaf(sg, pv.w, y[4 * c + 3]);
        }
        __syncthreads();
      }
    };
    fwht_tail(y);

    if constexpr (MULTI) {
      // passes 2.. : y holds pass p's output at positions j0 + e (unscaled, sign lane_sign)
      float* xrow = reinterpret_cast<float*>(smem + a.xf_off) + slot * d;
      for (int p = 1; p < a.passes; ++p) {
        const float sc = lane_sign * a.rsqrt_h;
#pragma unroll
        for (int e = 0; e < kE; ++e) y[e] *= sc;
        float gv[kE];
        if constexpr (PERM) {
          if (p > 1) __syncthreads();  // the previous pass's gathers from xrow are done
          if (active) {  // idle lanes alias slot 0's first positions
#pragma unroll
            for (int c = 0; c < kE / 4; ++c)
              *reinterpret_cast<float4*>(xrow + j0 + 4 * c) = make_float4(y[4 * c], y[4 * c + 1], y[4 * c + 2], y[4 * c + 3]);
          }
          __syncthreads();
          const int4* pp = reinterpret_cast<const int4*>(a.perm + static_cast<int64_t>(p) * d + j0);
#pragma unroll
          for (int c = 0; c < kE / 4; ++c) {
            const int4 p4 = pp[c];
            gv[4 * c] = xrow[min(max(p4.x, 0), d - 1)];
            gv[4 * c + 1] = xrow[min(max(p4.y, 0), d - 1)];
            gv[4 * c + 2] = xrow[min(max(p4.z, 0), d - 1)];
            gv[4 * c + 3] = xrow[min(max(p4.w, 0), d - 1)];
          }
        } else {
#pragma unroll
          for (int e = 0; e < kE; ++e) gv[e] = y[e];
        }
        // signs of pass p (sign bit of each int8 into the fp32 sign), then FWHT stage 1
        const uint4 sv = *reinterpret_cast<const uint4*>(a.signs + static_cast<int64_t>(p) * d + j0);
        const uint32_t sw4[4] = {sv.x, sv.y, sv.z, sv.w};
#pragma unroll
        for (int e = 0; e < kE; ++e)
          gv[e] = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, gv[e]) ^ (((sw4[e >> 2] >> (8 * (e & 3) + 7)) & 1u) << 31));
#pragma unroll
        for (int i = 0; i < kE / 2; ++i) {
          y[2 * i] = gv[2 * i] + gv[2 * i + 1];
          y[2 * i + 1] = gv[2 * i] - gv[2 * i + 1];
        }
        fwht_tail(y);
      }
    }
  };
  auto finish = [&](int g, uint32_t pb) {
    const int64_t row = static_cast<int64_t>(g) * a.tg + slot;
    const bool valid = active && row < a.n;
    // ---- token norm: the partial sums of the token's lane segments, added in a fixed order
    float s2;
    const float* prow = reinterpret_cast<const float*>(smem + a.part_off + pb + pr_off);
    if (a.row_reduce) {
      s2 = row16_sum(prow[threadIdx.x & (kNP - 1)]);
    } else {
      s2 = 0.0f;
      for (int k = 0; k < a.nseg; ++k) s2 += prow[k];
    }
    // hardware square root and reciprocal (1 ulp): s is reported to fp32 accuracy and t' only
    // needs fp32 accuracy; the correctly rounded forms cost ~20 instructions per lane
    const float s = __builtin_amdgcn_sqrtf(s2);
    const uint32_t lane_row = static_cast<uint32_t>(row);  // < n < 2^31 within a launch chunk

    if constexpr (MODE == QuantMode::kRotateOnly) {
      const float sc = a.inv_scale * lane_sign;
      const uint32_t off = valid ? (lane_row * static_cast<uint32_t>(d) + j0) * 4u : kDropped;
#pragma unroll
      for (int c = 0; c < kE / 4; ++c) {
        const v4i_t w = {__builtin_bit_cast(int, y[4 * c] * sc), __builtin_bit_cast(int, y[4 * c + 1] * sc),
                         __builtin_bit_cast(int, y[4 * c + 2] * sc), __builtin_bit_cast(int, y[4 * c + 3] * sc)};
        __builtin_amdgcn_raw_buffer_store_b128(w, rot_rs, off + 16u * c, 0, 0);
      }
      __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, s), norms_rs,
                                            (valid && q == 0) ? lane_row * 4u : kDropped, 0, 0);
    } else if constexpr (MODE == QuantMode::kRotateBf16) {
      // bf16 (nearest even), 16 positions = two groups of 8 in the order 0,2,4,6,1,3,5,7
      const float sc = a.inv_scale * lane_sign;
      const uint32_t off = valid ? (lane_row * static_cast<uint32_t>(d) + j0) * 2u : kDropped;
#pragma unroll
      for (int gi = 0; gi < 2; ++gi) {
        const float* vv = y + 8 * gi;
        auto pair = [&](int lo, int hi) {
          const bf16x2_t p = {static_cast<__bf16>(vv[lo] * sc), static_cast<__bf16>(vv[hi] * sc)};
          return __builtin_bit_cast(int, p);
        };
        const v4i_t w = {pair(0, 2), pair(4, 6), pair(1, 3), pair(5, 7)};
        __builtin_amdgcn_raw_buffer_store_b128(w, rot_rs, off + 16u * gi, 0, 0);
      }
      __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, s), norms_rs,
                                            (valid && q == 0) ? lane_row * 4u : kDropped, 0, 0);
    } else {
      const float inv_s = lane_sign * a.inv_scale * __builtin_amdgcn_rcpf(s + a.eps);
      const uint32_t off = valid ? lane_row * row_bytes + static_cast<uint32_t>(j0 * BITS / 8) : kDropped;
      if constexpr (MODE == QuantMode::kDecoded) {
        // bf16 centroids, 16 positions = two groups of 8 in the order 0,2,4,6,1,3,5,7
        const uint32_t doff = valid ? (lane_row * static_cast<uint32_t>(d) + static_cast<uint32_t>(j0)) * 2u : kDropped;
#pragma unroll
        for (int gi = 0; gi < 2; ++gi) {
          uint32_t cv[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) cv[i] = quantize_value(y[8 * gi + i] * inv_s, tbl, J);
          const v4i_t w = {static_cast<int>(cv[0] | (cv[2] << 16)), static_cast<int>(cv[4] | (cv[6] << 16)),
                           static_cast<int>(cv[1] | (cv[3] << 16)), static_cast<int>(cv[5] | (cv[7] << 16))};
          __builtin_amdgcn_raw_buffer_store_b128(w, codes_rs, doff + 16u * gi, 0, 0);
        }
      } else if constexpr (BITS == 4) {
        // codes decided four at a time (their table reads in flight together), then shift-or'ed in
        uint32_t w[2];
#pragma unroll
        for (int b4 = 0; b4 < 4; ++b4) {
          uint32_t c[4];
          quantize4<!kFull>(y + 4 * b4, inv_s, tbl, J, c);
          uint32_t& ww = w[b4 >> 1];
          const int sh0 = 16 * (b4 & 1);
          ww = sh0 ? lshl_or(c[0], sh0, ww) : c[0];
#pragma unroll
          for (int k = 1; k < 4; ++k) ww = lshl_or(c[k], sh0 + 4 * k, ww);
        }
        const v2u_t wv = {w[0], w[1]};
        __builtin_amdgcn_raw_buffer_store_b64(wv, codes_rs, off, 0, 0);
      } else if constexpr (BITS == 2) {
        uint32_t w = 0;
#pragma unroll
        for (int b4 = 0; b4 < 4; ++b4) {
          uint32_t c[4];
          quantize4<!kFull>(y + 4 * b4, inv_s, tbl, J, c);
#pragma unroll
          for (int k = 0; k < 4; ++k) w = (b4 | k) ? lshl_or(c[k], 8 * b4 + 2 * k, w) : c[0];
        }
        __builtin_amdgcn_raw_buffer_store_b32(static_cast<int>(w), codes_rs, off, 0, 0);
      } else if constexpr (BITS == 3) {
        // 48 bits at a 2-byte aligned offset (6 bytes per lane): three 16-bit stores.  Code i sits
        // at bit 3 i; code 10 straddles the two words (its low 2 bits end word 0).  Each code is
        // shifted-or'ed in as it is made, so only the partial words stay live.
        uint32_t c[kE];
        uint32_t w[2];
#pragma unroll
        for (int b4 = 0; b4 < 4; ++b4) {
          uint32_t c4[4];
          quantize4<!kFull>(y + 4 * b4, inv_s, tbl, J, c4);
#pragma unroll
          for (int k = 0; k < 4; ++k) c[4 * b4 + k] = c4[k];
          if (b4 == 0) {
            w[0] = c[0];
#pragma unroll
            for (int i = 1; i < 4; ++i) w[0] = lshl_or(c[i], 3 * i, w[0]);
          } else if (b4 == 1) {
#pragma unroll
            for (int i = 4; i < 8; ++i) w[0] = lshl_or(c[i], 3 * i, w[0]);
          } else if (b4 == 2) {
            w[0] = lshl_or(c[8], 24, w[0]);
            w[0] = lshl_or(c[9], 27, w[0]);
            w[0] = lshl_or(c[10], 30, w[0]);
            w[1] = lshl_or(c[11], 1, c[10] >> 2);
          } else {
#pragma unroll
            for (int i = 12; i < kE; ++i) w[1] = lshl_or(c[i], 3 * i - 32, w[1]);
          }
        }
        __builtin_amdgcn_raw_buffer_store_b16(static_cast<short>(w[0] & 0xFFFFu), codes_rs, off, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b16(static_cast<short>(w[0] >> 16), codes_rs, off + 2u, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b16(static_cast<short>(w[1] & 0xFFFFu), codes_rs, off + 4u, 0, 0);
      } else {
        // 96 bits: code i at bit 6 i; codes 5 and 10 straddle words (their low 2 and 4 bits end
        // words 0 and 1).  Shift-or'ed in as they are made, as for 3 bits.
        uint32_t c[kE];
        uint32_t w[3];
#pragma unroll
        for (int b4 = 0; b4 < 4; ++b4) {
          uint32_t c4[4];
          quantize4<!kFull>(y + 4 * b4, inv_s, tbl, J, c4);
#pragma unroll
          for (int k = 0; k < 4; ++k) c[4 * b4 + k] = c4[k];
          if (b4 == 0) {
            w[0] = c[0];
#pragma unroll
            for (int i = 1; i < 4; ++i) w[0] = lshl_or(c[i], 6 * i, w[0]);
          } else if (b4 == 1) {
            w[0] = lshl_or(c[4], 24, w[0]);
            w[0] = lshl_or(c[5], 30, w[0]);
            w[1] = lshl_or(c[6], 4, c[5] >> 2);
            w[1] = lshl_or(c[7], 10, w[1]);
          } else if (b4 == 2) {
            w[1] = lshl_or(c[8], 16, w[1]);
            w[1] = lshl_or(c[9], 22, w[1]);
            w[1] = lshl_or(c[10], 28, w[1]);
            w[2] = lshl_or(c[11], 2, c[10] >> 4);
          } else {
#pragma unroll
            for (int i = 12; i < kE; ++i) w[2] = lshl_or(c[i], 6 * i - 64, w[2]);
          }
        }
        const v2u_t w01 = {w[0], w[1]};
        __builtin_amdgcn_raw_buffer_store_b64(w01, codes_rs, off, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b32(static_cast<int>(w[2]), codes_rs, off + 8u, 0, 0);
      }
      if constexpr (MODE == QuantMode::kWeights)
        __builtin_amdgcn_raw_buffer_store_b16(static_cast<short>(bf16_rne_dev(s)), norms_rs,
                                              (valid && q == 0) ? lane_row * 2u : kDropped, 0, 0);
      else
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, s), norms_rs,
                                              (valid && q == 0) ? lane_row * 4u : kDropped, 0, 0);
    }
  };

  // Pipelined (PIPE, workgroups that run several token groups): one barrier per group.  The
  // staged rows and the norm partials alternate between two buffers, and group g is quantized
  // after the barrier of the next group: a wave stages group g + 1 into the buffer last gathered
  // from by group g - 1 (before the previous barrier), and writes group g + 1's partials into
  // the buffer group g - 1's were read from (also before it).
  // Otherwise two barriers per group, on one buffer: staged rows visible, then partials visible
  // (every gather of the group done before the next staging).
  int g = blockIdx.x;
  if constexpr (!PIPE) {
    for (; g < a.ngroups; g += stride) {
      stage(g, 0u);
      __syncthreads();
      rotate(0u, 0u);
      __syncthreads();
      finish(g, 0u);
    }
  } else if (g < a.ngroups) {
    stage(g, 0u);
    __syncthreads();
    rotate(0u, 0u);
    uint32_t sb = 0u, pb = 0u;
    for (int gn = g + stride; gn < a.ngroups; gn += stride) {
      const uint32_t sbn = sb ^ stbuf, pbn = pb ^ pbuf;
      stage(gn, sbn);
      __syncthreads();
      finish(g, pb);
      rotate(sbn, pbn);
      g = gn;
      sb = sbn;
      pb = pbn;
    }
    __syncthreads();
    finish(g, pb);
  }
}

// Balanced persistent grid: every workgroup runs the same number of token groups, and all of
// them are resident at once (as many workgroups per CU as the kernel's occupancy allows).
template <int H, int BITS, QuantMode MODE, bool PERM, bool MULTI, bool FULL, bool PIPE = false>
hipError_t launch_typed(const QuantKernelArgs& a, int threads, size_t lds, hipStream_t st) {
  static thread_local int cached_threads = -1, cached_occ = 1;
  static thread_local size_t cached_lds = 0;
  if (threads != cached_threads || lds != cached_lds) {
    int occ = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, k_rpbh_quantize<H, BITS, MODE, PERM, MULTI, FULL, PIPE>, threads, lds) != hipSuccess ||
        occ < 1)
      occ = 1;
    cached_threads = threads;
    cached_lds = lds;
    cached_occ = occ;
  }
  const int max_grid = device_cus() * cached_occ;
  const int iters = (a.ngroups + max_grid - 1) / max_grid;
  const int grid = (a.ngroups + iters - 1) / iters;
  hipLaunchKernelGGL((k_rpbh_quantize<H, BITS, MODE, PERM, MULTI, FULL, PIPE>), dim3(grid), dim3(threads), lds, st, a);
  return hipGetLastError();
}

// one pass, quantizing: the pipelined loop or the two-barrier one (chosen on the host)
template <int H, int BITS, QuantMode MODE, bool PERM, bool FULL>
hipError_t launch_pipe(const QuantKernelArgs& a, int threads, size_t lds, hipStream_t st) {
  return a.pipe ? launch_typed<H, BITS, MODE, PERM, false, FULL, true>(a, threads, lds, st)
                : launch_typed<H, BITS, MODE, PERM, false, FULL, false>(a, threads, lds, st);
}

template <int H, QuantMode MODE, bool PERM, bool MULTI>
hipError_t launch_perm(int bits, const QuantKernelArgs& a, int threads, size_t lds, hipStream_t st) {
  if constexpr (MODE == QuantMode::kRotateOnly || MODE == QuantMode::kRotateBf16) {
    return launch_typed<H, 4, MODE, PERM, MULTI, false>(a, threads, lds, st);
  } else if constexpr (MODE == QuantMode::kDecoded) {
    return launch_typed<H, 6, MODE, PERM, MULTI, false>(a, threads, lds, st);
  } else if constexpr (MULTI) {
    switch (bits) {
      case 2: return launch_typed<H, 2, MODE, PERM, MULTI, false>(a, threads, lds, st);
      case 3: return launch_typed<H, 3, MODE, PERM, MULTI, false>(a, threads, lds, st);
      case 4: return launch_typed<H, 4, MODE, PERM, MULTI, false>(a, threads, lds, st);
      default: return launch_typed<H, 6, MODE, PERM, MULTI, false>(a, threads, lds, st);
    }
  } else {
    switch (bits) {
      case 2:
        return a.full ? launch_pipe<H, 2, MODE, PERM, true>(a, threads, lds, st)
                      : launch_pipe<H, 2, MODE, PERM, false>(a, threads, lds, st);
      case 3:
        return a.full ? launch_pipe<H, 3, MODE, PERM, true>(a, threads, lds, st)
                      : launch_pipe<H, 3, MODE, PERM, false>(a, threads, lds, st);
      case 4:
        return a.full ? launch_pipe<H, 4, MODE, PERM, true>(a, threads, lds, st)
                      : launch_pipe<H, 4, MODE, PERM, false>(a, threads, lds, st);
      default: return launch_pipe<H, 6, MODE, PERM, false>(a, threads, lds, st);
    }
  }
}

template <int H, QuantMode MODE>
hipError_t launch_bits(int bits, const QuantKernelArgs& a, int threads, size_t lds, hipStream_t st) {
  if (a.passes > 1)
    return a.perm ? launch_perm<H, MODE, true, true>(bits, a, threads, lds, st)
                  : launch_perm<H, MODE, false, true>(bits, a, threads, lds, st);
  return a.perm ? launch_perm<H, MODE, true, false>(bits, a, threads, lds, st)
                : launch_perm<H, MODE, false, false>(bits, a, threads, lds, st);
}

// every mode of one Hadamard block size (each size is instantiated in its own source file)
template <int H>
hipError_t launch_block(QuantMode mode, int bits, const QuantKernelArgs& a, int threads, size_t lds, hipStream_t st) {
  switch (mode) {
    case QuantMode::kActivations: return launch_bits<H, QuantMode::kActivations>(bits, a, threads, lds, st);
    case QuantMode::kWeights: return launch_bits<H, QuantMode::kWeights>(bits, a, threads, lds, st);
    case QuantMode::kRotateBf16: return launch_bits<H, QuantMode::kRotateBf16>(4, a, threads, lds, st);
    case QuantMode::kDecoded:
      return bits == 6 ? launch_bits<H, QuantMode::kDecoded>(bits, a, threads, lds, st) : hipErrorInvalidValue;
    default: return launch_bits<H, QuantMode::kRotateOnly>(4, a, threads, lds, st);
  }
}

}  // namespace rq
}  // namespace orbq
