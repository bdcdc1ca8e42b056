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
//     registers at ~80, so six waves share each SIMD and hide the load / LDS / barrier latencies.
//   * Staging: the lanes of a token load its bf16 row with coalesced 16-byte loads (lane q takes
//     chunks q and q + L), prefetched one token group ahead in registers, store it to LDS and add
//     the squares into a partial norm (sum of squares is invariant under Pi), reduced over aligned
//     lane segments with DPP adds and across segments through LDS.
//   * Compute: each lane gathers its 16 permuted positions x[perm[j]] from LDS with 16-bit reads
//     (addresses precomputed once from perm) and runs the block FWHT: the Rademacher signs, the
//     first butterfly stage and the bf16 -> fp32 widening are two v_dot2_f32_bf16 per bf16 pair
//     against the pair's signs (the second with the high sign negated), the next three stages
//     run in registers, the last log2(h/16) stages across lanes with v_fmac_f32_dpp (lanes placed
//     so that every partner is a quad_perm or row_half_mirror lane).
//   * Quantization uses the power-of-two-scaled coordinate t' = t * 2^k: one table lookup on
//     floor(-t') and one fp32 compare give the exact nearest-centroid decision (QuantParams).
//   * Codes are packed in registers and written with one 4/8/12-byte store per lane.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>

#include "internal.h"

namespace orbq {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));

constexpr int kE = 16;  // positions per lane
constexpr int kCH = kE / 8;  // 16-byte input chunks staged per lane

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
  int32_t lpt;     // lanes per token = d / 32
  int32_t tg;      // tokens per workgroup iteration
  int32_t seg;     // power-of-two lane segment reduced with shuffles
  int32_t nseg;    // segments per token
  int32_t ngroups;
  float eps;
  float inv_scale; // 2^k / sqrt(h) (quantize) or 1 / sqrt(h) (rotate only)
  uint32_t codes_bytes, norms_bytes, rot_bytes;  // buffer extents (< 2^31) for bounds-dropped stores
  uint32_t x_bytes;                              // extent of X in this launch (< 2^31)
  int32_t passes;                                // composed RPBH passes (1..3)
  uint32_t xf_off;                               // LDS byte offset of the fp32 rows (passes > 1)
  float rsqrt_h;                                 // 1 / sqrt(h), the scale of each earlier pass
  QuantParams qp;
};

typedef int v4i_t __attribute__((ext_vector_type(4)));
typedef uint32_t v2u_t __attribute__((ext_vector_type(2)));
constexpr uint32_t kBufWord3 = 0x00020000u;  // raw (untyped) buffer resource, gfx9 family
constexpr uint32_t kDropped = 0xFFFFFF00u;   // offset past every extent: the store is discarded

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
#pragma unroll
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

__device__ __forceinline__ uint32_t quantize_one(float tp, const float2* tbl, int J) {
  const int j = med3_i32(floor_neg_to_int(tp), -J, J - 1);
  const float2 e = tbl[j];  // tbl points at bucket 0
  return static_cast<uint32_t>(__builtin_bit_cast(int, e.y)) + (__builtin_fabsf(tp) > e.x ? 1u : 0u);
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

// Sum over aligned segments of `seg` lanes (a power of two <= 64, uniform); the last lane of
// each segment holds the segment's sum (for seg <= 16 every lane does).
__device__ __forceinline__ float segment_sum(float x, int seg) {
  if (seg >= 2) x = dpp_add<0xB1, 0xF>(x);   // quad_perm [1,0,3,2]
  if (seg >= 4) x = dpp_add<0x4E, 0xF>(x);   // quad_perm [2,3,0,1]
  if (seg >= 8) x = dpp_add<0x141, 0xF>(x);  // row_half_mirror: 8 lanes
  if (seg >= 16) x = dpp_add<0x140, 0xF>(x); // row_mirror: 16 lanes
  if (seg >= 32) x = dpp_add<0x142, 0xA>(x); // row_bcast:15 into rows 1 and 3: 32 lanes
  if (seg >= 64) x = dpp_add<0x143, 0xC>(x); // row_bcast:31 into rows 2 and 3: 64 lanes
  return x;
}

// MULTI: the rotation is the composition Pi_P ... Pi_1 of a.passes RPBH passes, pass p with its
// own permutation and signs at perm + p d, signs + p d (RHT page, composed randomized Hadamard
// transforms).  Between passes the fp32 rotated row goes through LDS for the next gather (or
// stays in registers when the permutations are the identity).
template <int H, int BITS, QuantMode MODE, bool PERM, bool MULTI>
__global__ __launch_bounds__(1024) void k_rpbh_quantize(QuantKernelArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int d = a.d;
  uint16_t* xs = reinterpret_cast<uint16_t*>(smem);                                    // [tg][d]
  float2* tbl_all = reinterpret_cast<float2*>(smem + ((static_cast<size_t>(a.tg) * d * 2 + 15) & ~size_t(15)));
  float* part = reinterpret_cast<float*>(tbl_all + 2 * a.qp.J);                       // [tg][nseg]
  const int tid = threadIdx.x;
  const int nact = a.tg * a.lpt;
  const bool active = tid < nact;
  const int slot = active ? tid / a.lpt : 0;
  const int q = active ? tid - slot * a.lpt : 0;
  const int J = a.qp.J;
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
  // end read as zero (and are never stored); idle lanes read the group's first row
  const __amdgpu_buffer_rsrc_t x_rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(a.X), 0, a.x_bytes, kBufWord3);
  const uint32_t ldx_bytes = static_cast<uint32_t>(a.ldx) * 2u;
  const uint32_t lane_off = static_cast<uint32_t>(16 * q);
  auto load_group = [&](int g, uint4 v[kCH]) {
    const uint32_t off = (static_cast<uint32_t>(g) * static_cast<uint32_t>(a.tg) + slot) * ldx_bytes + lane_off;
#pragma unroll
    for (int c = 0; c < kCH; ++c)
      v[c] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(x_rs, off + static_cast<uint32_t>(c * 16 * a.lpt), 0, 0));
  };
  uint4 v[kCH];
  load_group(blockIdx.x, v);  // first group in flight during the set-up

  constexpr bool kRotate = MODE == QuantMode::kRotateOnly || MODE == QuantMode::kRotateBf16;
  if constexpr (!kRotate) build_table<BITS, MODE == QuantMode::kDecoded>(a.qp, tbl_all, tid, blockDim.x);
  const float2* tbl = tbl_all + J;

  // ---- set-up: gather addresses x[perm[j]] (LDS byte offsets) and sign masks of this lane
  uint32_t gaddr[kE];
  uint32_t smask[kE / 2];  // bf16 pairs (s_2i, s_2i+1) of the Rademacher signs
  {
    if constexpr (PERM) {
    const int4* pp = reinterpret_cast<const int4*>(a.perm + j0);
    const uint32_t rowbase = static_cast<uint32_t>(slot * d);
#pragma unroll
    for (int c = 0; c < kE / 4; ++c) {
      const int4 p4 = pp[c];
      const int pv[4] = {p4.x, p4.y, p4.z, p4.w};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        gaddr[4 * c + e] = (rowbase + static_cast<uint32_t>(min(max(pv[e], 0), d - 1))) * 2u;
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
  uint4* stage_dst[kCH];
#pragma unroll
  for (int c = 0; c < kCH; ++c) stage_dst[c] = reinterpret_cast<uint4*>(xs + slot * d + 8 * (q + c * a.lpt));

  // Stores go through buffer resources: lanes with nothing to store (rows past the end, idle
  // lanes) get an offset past the extent and the hardware drops the store.  The loop body has no
  // branches around memory operations, so the compiler's wait counts stay exact (on gfx9 vmcnt
  // also counts stores: a conservative wait would stall on the previous group's stores).
  const __amdgpu_buffer_rsrc_t codes_rs = __builtin_amdgcn_make_buffer_rsrc(a.codes, 0, a.codes_bytes, kBufWord3);
  const __amdgpu_buffer_rsrc_t norms_rs = __builtin_amdgcn_make_buffer_rsrc(a.norms, 0, a.norms_bytes, kBufWord3);
  const __amdgpu_buffer_rsrc_t rot_rs = __builtin_amdgcn_make_buffer_rsrc(a.x_rot, 0, a.rot_bytes, kBufWord3);
  const uint32_t row_bytes = static_cast<uint32_t>(d * BITS / 8);

  for (int g = blockIdx.x; g < a.ngroups; g += gridDim.x) {
    const int64_t row = static_cast<int64_t>(g) * a.tg + slot;
    const bool valid = active && row < a.n;

    __syncthreads();  // the previous group's gathers from xs are done
    // ---- stage this lane's chunks; partial sum of squares
    float ss = 0.0f;
    if (active) {
#pragma unroll
      for (int c = 0; c < kCH; ++c) *stage_dst[c] = v[c];
    }
#pragma unroll
    for (int c = 0; c < kCH; ++c) {
      ss = dot2_acc(v[c].x, v[c].x, ss);
      ss = dot2_acc(v[c].y, v[c].y, ss);
      ss = dot2_acc(v[c].z, v[c].z, ss);
      ss = dot2_acc(v[c].w, v[c].w, ss);
    }
    // prefetch the next group (the last iteration reloads its own group: no branch)
    load_group(g + static_cast<int>(gridDim.x) < a.ngroups ? g + static_cast<int>(gridDim.x) : g, v);
    ss = segment_sum(ss, a.seg);
    if (active && (q & (a.seg - 1)) == a.seg - 1) part[slot * a.nseg + q / a.seg] = ss;
    __syncthreads();

    // ---- gather the 32 permuted positions as bf16 pairs, signs, FWHT stage 1 (+ widening)
    float y[kE];
    if constexpr (PERM) {
#pragma unroll
      for (int i = 0; i < kE / 2; ++i) {
        const uint32_t lo = *reinterpret_cast<const uint16_t*>(smem + gaddr[2 * i]);
        const uint32_t hi = *reinterpret_cast<const uint16_t*>(smem + gaddr[2 * i + 1]);
        const uint32_t x2 = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
        y[2 * i] = dot2_v(x2, smask[i]);
        y[2 * i + 1] = dot2_neghi(x2, smask[i]);
      }
    } else {  // identity permutation (block RHT): the lane's 16 positions are contiguous
      const uint4* src = reinterpret_cast<const uint4*>(xs + slot * d + j0);
      const uint4 c0 = src[0], c1 = src[1];
      const uint32_t x2s[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
#pragma unroll
      for (int i = 0; i < kE / 2; ++i) {
        y[2 * i] = dot2_v(x2s[i], smask[i]);
        y[2 * i + 1] = dot2_neghi(x2s[i], smask[i]);
      }
    }
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
    };
    fwht_tail(y);

    if constexpr (MULTI) {
      // passes 2.. : y holds pass p's output at positions j0 + e (unscaled, sign lane_sign)
      float* xrow = reinterpret_cast<float*>(smem + a.xf_off) + slot * d;
      for (int p = 1; p < a.passes; ++p) {
        const float sc = lane_sign * a.rsqrt_h;
#pragma unroll
        for (int e = 0; e < kE; ++e) y[e] *= sc;
        float g[kE];
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
            g[4 * c] = xrow[min(max(p4.x, 0), d - 1)];
            g[4 * c + 1] = xrow[min(max(p4.y, 0), d - 1)];
            g[4 * c + 2] = xrow[min(max(p4.z, 0), d - 1)];
            g[4 * c + 3] = xrow[min(max(p4.w, 0), d - 1)];
          }
        } else {
#pragma unroll
          for (int e = 0; e < kE; ++e) g[e] = y[e];
        }
        // signs of pass p (sign bit of each int8 into the fp32 sign), then FWHT stage 1
        const uint4 sv = *reinterpret_cast<const uint4*>(a.signs + static_cast<int64_t>(p) * d + j0);
        const uint32_t sw4[4] = {sv.x, sv.y, sv.z, sv.w};
#pragma unroll
        for (int e = 0; e < kE; ++e)
          g[e] = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, g[e]) ^ (((sw4[e >> 2] >> (8 * (e & 3) + 7)) & 1u) << 31));
#pragma unroll
        for (int i = 0; i < kE / 2; ++i) {
          y[2 * i] = g[2 * i] + g[2 * i + 1];
          y[2 * i + 1] = g[2 * i] - g[2 * i + 1];
        }
        fwht_tail(y);
      }
    }

    // ---- token norm: the lane segments' partial sums, added in a fixed order
    float s2 = 0.0f;
    for (int k = 0; k < a.nseg; ++k) s2 += part[slot * a.nseg + k];
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
        const float* v = y + 8 * gi;
        auto pair = [&](int lo, int hi) {
          const bf16x2_t p = {static_cast<__bf16>(v[lo] * sc), static_cast<__bf16>(v[hi] * sc)};
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
          uint32_t v[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) v[i] = quantize_value(y[8 * gi + i] * inv_s, tbl, J);
          const v4i_t w = {static_cast<int>(v[0] | (v[2] << 16)), static_cast<int>(v[4] | (v[6] << 16)),
                           static_cast<int>(v[1] | (v[3] << 16)), static_cast<int>(v[5] | (v[7] << 16))};
          __builtin_amdgcn_raw_buffer_store_b128(w, codes_rs, doff + 16u * gi, 0, 0);
        }
      } else if constexpr (BITS == 4) {
        uint32_t w[2] = {0, 0};
#pragma unroll
        for (int i = 0; i < kE; ++i) w[i >> 3] |= quantize_one(y[i] * inv_s, tbl, J) << (4 * (i & 7));
        const v2u_t wv = {w[0], w[1]};
        __builtin_amdgcn_raw_buffer_store_b64(wv, codes_rs, off, 0, 0);
      } else if constexpr (BITS == 2) {
        uint32_t w = 0;
#pragma unroll
        for (int i = 0; i < kE; ++i) w |= quantize_one(y[i] * inv_s, tbl, J) << (2 * i);
        __builtin_amdgcn_raw_buffer_store_b32(static_cast<int>(w), codes_rs, off, 0, 0);
      } else if constexpr (BITS == 3) {
        // 48 bits at a 2-byte aligned offset (6 bytes per lane): three 16-bit stores
        uint32_t w[2] = {0, 0};
#pragma unroll
        for (int i = 0; i < kE; ++i) {
          const uint32_t c = quantize_one(y[i] * inv_s, tbl, J);
          const int bit = 3 * i, wi = bit >> 5, sh = bit & 31;
          w[wi] |= c << sh;
          if (sh > 29) w[wi + 1] |= c >> (32 - sh);
        }
        __builtin_amdgcn_raw_buffer_store_b16(static_cast<short>(w[0] & 0xFFFFu), codes_rs, off, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b16(static_cast<short>(w[0] >> 16), codes_rs, off + 2u, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b16(static_cast<short>(w[1] & 0xFFFFu), codes_rs, off + 4u, 0, 0);
      } else {
        uint32_t w[3] = {0, 0, 0};
#pragma unroll
        for (int i = 0; i < kE; ++i) {
          const uint32_t c = quantize_one(y[i] * inv_s, tbl, J);
          const int bit = 6 * i, wi = bit >> 5, sh = bit & 31;
          w[wi] |= c << sh;
          if (sh > 26) w[wi + 1] |= c >> (32 - sh);
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
  }
}

__global__ void k_quantize_t(const float* t, int64_t count, QuantParams qp, uint8_t* codes) {
  __shared__ float2 tbl_all[2 * kMaxTableHalf];
  switch (qp.bits) {
    case 2: build_table<2>(qp, tbl_all, threadIdx.x, blockDim.x); break;
    case 3: build_table<3>(qp, tbl_all, threadIdx.x, blockDim.x); break;
    case 4: build_table<4>(qp, tbl_all, threadIdx.x, blockDim.x); break;
    default: build_table<6>(qp, tbl_all, threadIdx.x, blockDim.x); break;
  }
  __syncthreads();
  const float2* tbl = tbl_all + qp.J;
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < count;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x)
    codes[i] = static_cast<uint8_t>(quantize_one(t[i] * qp.scale, tbl, qp.J));
}

int device_cu_count();

// Balanced persistent grid: every workgroup runs the same number of token groups, and all of
// them are resident at once (as many workgroups per CU as the kernel's occupancy allows).
template <int H, int BITS, QuantMode MODE, bool PERM, bool MULTI>
hipError_t launch_typed(const QuantKernelArgs& a, int threads, size_t lds, hipStream_t st) {
  static thread_local int cached_threads = -1, cached_occ = 1;
  static thread_local size_t cached_lds = 0;
  if (threads != cached_threads || lds != cached_lds) {
    int occ = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, k_rpbh_quantize<H, BITS, MODE, PERM, MULTI>, threads, lds) != hipSuccess ||
        occ < 1)
      occ = 1;
    cached_threads = threads;
    cached_lds = lds;
    cached_occ = occ;
  }
  const int max_grid = device_cu_count() * cached_occ;
  const int iters = (a.ngroups + max_grid - 1) / max_grid;
  const int grid = (a.ngroups + iters - 1) / iters;
  hipLaunchKernelGGL((k_rpbh_quantize<H, BITS, MODE, PERM, MULTI>), dim3(grid), dim3(threads), lds, st, a);
  return hipGetLastError();
}

template <int H, QuantMode MODE, bool PERM, bool MULTI>
hipError_t launch_perm(int bits, const QuantKernelArgs& a, int threads, size_t lds, hipStream_t st) {
  if constexpr (MODE == QuantMode::kRotateOnly || MODE == QuantMode::kRotateBf16) {
    return launch_typed<H, 4, MODE, PERM, MULTI>(a, threads, lds, st);
  } else if constexpr (MODE == QuantMode::kDecoded) {
    return launch_typed<H, 6, MODE, PERM, MULTI>(a, threads, lds, st);
  } else {
    switch (bits) {
      case 2: return launch_typed<H, 2, MODE, PERM, MULTI>(a, threads, lds, st);
      case 3: return launch_typed<H, 3, MODE, PERM, MULTI>(a, threads, lds, st);
      case 4: return launch_typed<H, 4, MODE, PERM, MULTI>(a, threads, lds, st);
      default: return launch_typed<H, 6, MODE, PERM, MULTI>(a, threads, lds, st);
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

template <QuantMode MODE>
hipError_t launch_mode(int block, int bits, const QuantKernelArgs& a, int threads, size_t lds, hipStream_t st) {
  switch (block) {
    case 64: return launch_bits<64, MODE>(bits, a, threads, lds, st);
    case 128: return launch_bits<128, MODE>(bits, a, threads, lds, st);
    case 256: return launch_bits<256, MODE>(bits, a, threads, lds, st);
    case 512: return launch_bits<512, MODE>(bits, a, threads, lds, st);
    default: return launch_bits<1024, MODE>(bits, a, threads, lds, st);
  }
}

int device_cu_count() {
  static thread_local int cached_dev = -1, cached_cus = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (dev != cached_dev) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    cached_dev = dev;
    cached_cus = cus;
  }
  return cached_cus;
}

}  // namespace

int launch_rpbh_quantize(QuantMode mode, const uint16_t* X, int64_t n, int64_t ldx, const RotArgs& rot,
                         const QuantParams* qp, float eps, uint8_t* codes, void* norms, float* x_rot,
                         hipStream_t stream) {
  QuantKernelArgs a{};
  a.X = X;
  a.n = n;
  a.ldx = ldx;
  a.perm = rot.perm;
  a.signs = rot.signs;
  a.passes = rot.passes < 1 ? 1 : rot.passes;
  a.codes = codes;
  a.norms = norms;
  a.x_rot = x_rot;
  a.d = rot.d;
  a.lpt = rot.d / kE;
  a.eps = eps;
  if (qp) a.qp = *qp;
  else {
    a.qp.J = 0;
    a.qp.bits = 4;
  }
  // tokens per workgroup: least idle lanes, then the workgroup closest to 256 threads
  int best_tg = 1, best_threads = 0;
  double best_score = 1e30;
  for (int tg = 1; tg * a.lpt <= 1024; ++tg) {
    const int act = tg * a.lpt, thr = (act + 63) / 64 * 64;
    const double waste = static_cast<double>(thr - act) / thr;
    const double score = waste * 10.0 + std::abs(std::log2(thr / 256.0)) * 0.01;
    if (score < best_score) {
      best_score = score;
      best_tg = tg;
      best_threads = thr;
    }
  }
  a.tg = best_tg;
  int seg = 1;
  while (seg < 64 && (a.lpt % (seg * 2)) == 0) seg *= 2;
  a.seg = seg;
  a.nseg = a.lpt / seg;
  const float rsqrt_h = 1.0f / __builtin_sqrtf(static_cast<float>(rot.block));
  const bool rotate = mode == QuantMode::kRotateOnly || mode == QuantMode::kRotateBf16;
  a.inv_scale = rotate ? rsqrt_h : static_cast<float>(static_cast<double>(a.qp.scale) /
                                                                                 std::sqrt(static_cast<double>(rot.block)));
  size_t lds = ((static_cast<size_t>(a.tg) * rot.d * 2 + 15) & ~size_t(15)) +
               sizeof(float2) * 2 * a.qp.J + sizeof(float) * a.tg * a.nseg;
  a.rsqrt_h = rsqrt_h;
  if (a.passes > 1 && a.perm) {  // fp32 rows for the gathers of the later passes
    lds = (lds + 15) & ~size_t(15);
    a.xf_off = static_cast<uint32_t>(lds);
    lds += sizeof(float) * a.tg * rot.d;
  }
  // rows per launch: every buffer extent (input rows, codes, norms, rotated rows) stays below 2^31 bytes
  const int64_t bytes_per_row = std::max<int64_t>(std::max<int64_t>(rot.d * 4, rot.d), ldx * 2);
  const int64_t chunk_rows = std::max<int64_t>(a.tg, ((int64_t(1) << 31) - 4096) / bytes_per_row / a.tg * a.tg);
  hipError_t e = hipSuccess;
  const int bits = a.qp.bits;
  for (int64_t r0 = 0; r0 < n && e == hipSuccess; r0 += chunk_rows) {
    QuantKernelArgs c = a;
    const int64_t rows = std::min<int64_t>(chunk_rows, n - r0);
    c.n = rows;
    c.X = X + r0 * ldx;
    c.x_bytes = static_cast<uint32_t>((rows - 1) * ldx * 2 + static_cast<int64_t>(rot.d) * 2);
    const int out_bits = mode == QuantMode::kRotateOnly ? 4 : mode == QuantMode::kDecoded ? 16 : a.qp.bits;
    const int64_t cb = static_cast<int64_t>(rot.d) * out_bits / 8;
    if (codes) c.codes = codes + r0 * cb;
    c.codes_bytes = static_cast<uint32_t>(rows * cb);
    const int64_t nb = mode == QuantMode::kWeights ? 2 : 4;
    c.norms = static_cast<unsigned char*>(norms) + r0 * nb;
    c.norms_bytes = static_cast<uint32_t>(rows * nb);
    const int64_t rot_esz = mode == QuantMode::kRotateBf16 ? 2 : 4;  // bytes per rotated coordinate
    if (x_rot) c.x_rot = reinterpret_cast<float*>(reinterpret_cast<unsigned char*>(x_rot) + r0 * rot.d * rot_esz);
    c.rot_bytes = x_rot ? static_cast<uint32_t>(rows * rot.d * rot_esz) : 0u;
    c.ngroups = static_cast<int>((rows + a.tg - 1) / a.tg);
    switch (mode) {
      case QuantMode::kActivations:
        e = launch_mode<QuantMode::kActivations>(rot.block, bits, c, best_threads, lds, stream);
        break;
      case QuantMode::kWeights:
        e = launch_mode<QuantMode::kWeights>(rot.block, bits, c, best_threads, lds, stream);
        break;
      case QuantMode::kRotateBf16:
        e = launch_mode<QuantMode::kRotateBf16>(rot.block, 4, c, best_threads, lds, stream);
        break;
      case QuantMode::kDecoded:
        e = bits == 6 ? launch_mode<QuantMode::kDecoded>(rot.block, bits, c, best_threads, lds, stream)
                      : hipErrorInvalidValue;
        break;
      default:
        e = launch_mode<QuantMode::kRotateOnly>(rot.block, 4, c, best_threads, lds, stream);
        break;
    }
  }
  return static_cast<int>(e);
}

int launch_quantize_t(const float* t, int64_t count, const QuantParams& qp, uint8_t* codes, hipStream_t stream) {
  const int threads = 256;
  int64_t blocks = (count + threads - 1) / threads;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(k_quantize_t, dim3(static_cast<unsigned>(blocks)), dim3(threads), 0, stream, t, count, qp, codes);
  return static_cast<int>(hipGetLastError());
}

}  // namespace orbq
