// Shared device code of the codes x codes product (lut_gemm) and the weight-only product
// (a16_gemm): operand decoders, the K2 kernel template and its launch templates.  Included by
// lut_gemm_a{2,3,4,6}.hip, which instantiate the kernels for one activation bit width each
// (so that the instantiations compile in parallel), and by a16_gemm.hip.
//
// lut_gemm: Y = diag(s) * (C_a[codes_x] C_w[codes_w]^T) * diag(r') for packed Lloyd-Max codes.
//
// Method: OrbitQuant summary (picx.dev), "Online Activation Quantization": x^' = s Q(x~'),
// W^' = diag(r') Q(W~') ("Offline Weight Quantization"), and W^' x^' approximates W x because the
// rotation cancels.  The product is a dense contraction over d, so it runs on the matrix cores.
//
// Kernel layout (gfx950, wave64, 512 threads = 8 waves, two per SIMD):
//   * workgroup tile BM tokens x BN weight rows (384 x 192 or 256 x 256, chosen on the host so
//     that the tiles fill the compute units in whole rounds), K tile of 64; the waves form a
//     4 x 2 grid, each computing (BM/4) x (BN/2) with v_mfma_f32_32x32x16_bf16 and fp32
//     accumulators.
//   * staging: a K tile holds (BM + BN) code rows of 64 codes, i.e. (BM + BN) * 8 units of 8
//     codes.  Thread t owns unit column t % 8 of rows t / 8 + 64 i, i < (BM + BN) / 64, so every
//     thread decodes the same number of units.  Code rows are read with buffer loads (rows past
//     the end read as zero and are never stored), two K tiles ahead in registers.
//   * decode of 4-bit codes: v_perm_b32 byte lookups into the 8 bf16 magnitudes (held in four
//     registers) plus the sign bit; 2- and 3-bit codes the same into the 4 or 8 signed values;
//     6-bit codes use a 4096-entry LDS table per code pair.  Activations already decoded to bf16
//     centroids (the layer's path for 6-bit activations) are staged by direct-to-LDS loads.
//     Every decoder writes the 8 values of a 16-byte chunk in the order k = 0,2,4,6,1,3,5,7, so
//     A and B agree on k.
//   * LDS: two stages of [BM + BN][64] bf16, 128-byte rows whose 16-byte chunks are xor-swizzled
//     by (row >> 1) & 7; the MFMA fragment reads (32 rows at one chunk) and the staging stores
//     (8 rows x 8 chunks per wave) are free of bank conflicts.  One barrier per K tile.
//   * schedule: a K tile is 4 k-steps of TI x TJ MFMAs.  The decode of the next K tile (half a
//     unit after two of every three MFMAs, with its LDS store) fills the first three k-steps;
//     the fragment reads of the next k-step are spread over the first MFMAs of the current one.
//     The K tile's one barrier sits before its last k-step, whose MFMAs then cover the reads of
//     the next K tile's first fragments: no wave starts a K tile waiting for LDS.
//   * epilogue: Y = act(acc * s_i * r'_j) in fp32, stored as fp32 or bf16 (round to nearest
//     even); act is the identity or GELU (tanh or erf form), the activation an MLP applies
//     between its up- and down-projection (Nunchaku / SVDQuant in Diffusers, ai-papers.net,
//     on fusing GELU with the MLP).
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>

#include "internal.h"

namespace orbq {
namespace lg {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int v2u_t __attribute__((ext_vector_type(2)));

constexpr int KT = 64;          // K tile (codes)
constexpr int kRow = KT * 2;    // bytes of one staged bf16 row
constexpr int kThreads = 512;
constexpr uint32_t kBufWord3 = 0x00020000u;  // raw (untyped) buffer resource, gfx9 family
// Cache policy of the full-tile Y stores: sc0 sc1, system-scope coherence.  Each Y line goes
// through L2 to memory (the memory-side Infinity Cache, where the next layer finds it) as it is
// written, instead of waiting dirty in L2 until a later access evicts it; no Y line is read again
// by this kernel.  Measured 0.6-0.9 % faster per step than the default policy on one box.
constexpr int kYStorePolicy = 1 | 16;

template <int BM_, int BN_>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_;
  static constexpr int TM = BM / 4, TN = BN / 2;    // per-wave tile (4 x 2 waves)
  static constexpr int TI = TM / 32, TJ = TN / 32;  // 32 x 32 MFMA blocks per wave
  static constexpr int U = (BM + BN) / 64;          // 8-code units per thread per K tile
  static constexpr int UA = BM / 64;                // of which in the token tile
  static constexpr int NM = TI * TJ;                // MFMAs per wave per 16-deep k step
  static constexpr int SA = BM * kRow, SB = BN * kRow;  // bytes of one stage of A / B
  static constexpr int LDS = 2 * (SA + SB);
  static_assert(2 * U == 4 * NM / 2, "one half-unit of decode per two MFMAs");
};

struct GemmArgs {
  const uint8_t* xc;
  const float* xs;
  const uint8_t* wc;
  const uint16_t* wn;
  void* Y;
  int64_t n, m, ldy;
  int32_t xrow_bytes, wrow_bytes;
  int32_t nk;  // K tiles
  int32_t tiles_n, tiles_m;
  int32_t act;  // kActNone, kActGeluTanh, kActGeluErf
  int32_t group_n;  // token tiles per group of the XCD order (0: the plain band order)
  // 4-bit decode tables: low / high bytes of the 8 bf16 magnitudes, 4 per register
  uint32_t lt_lo_a, lt_hi_a, ht_lo_a, ht_hi_a;
  uint32_t lt_lo_w, lt_hi_w, ht_lo_w, ht_hi_w;
  uint16_t mag_a[32], mag_w[32];
};

// ----------------------------------------------------------------------------- decoders
struct Tab4 {
  uint32_t lt_lo, lt_hi, ht_lo, ht_hi;
};

// 4-bit, in two halves: (1) magnitude bytes of the even and odd codes, (2) signs and bf16 pairs
struct Half4 {
  uint32_t le, he, lo, ho;
};

__device__ __forceinline__ Half4 decode4_a(uint32_t X, const Tab4& t) {
  const uint32_t se = X & 0x07070707u;
  const uint32_t so = (X >> 4) & 0x07070707u;
  Half4 h;
  h.le = __builtin_amdgcn_perm(t.lt_hi, t.lt_lo, se);
  h.he = __builtin_amdgcn_perm(t.ht_hi, t.ht_lo, se);
  h.lo = __builtin_amdgcn_perm(t.lt_hi, t.lt_lo, so);
  h.ho = __builtin_amdgcn_perm(t.ht_hi, t.ht_lo, so);
  return h;
}

__device__ __forceinline__ uint4 decode4_b(uint32_t X, Half4 h) {
  const uint32_t he = h.he | ((X << 4) & 0x80808080u);  // sign = bit 3 of each code
  const uint32_t ho = h.ho | (X & 0x80808080u);
  uint4 r;
  r.x = __builtin_amdgcn_perm(he, h.le, 0x05010400u);  // (e0, e2)
  r.y = __builtin_amdgcn_perm(he, h.le, 0x07030602u);  // (e4, e6)
  r.z = __builtin_amdgcn_perm(ho, h.lo, 0x05010400u);  // (e1, e3)
  r.w = __builtin_amdgcn_perm(ho, h.lo, 0x07030602u);  // (e5, e7)
  return r;
}

// 2-bit, in two halves, by v_perm_b32 byte lookups into the 4 signed bf16 values (their low
// bytes in t.lt_lo, their high bytes in t.ht_lo).  16 bits hold 8 codes; u = x | x << 12 has
// e0, e4, e2, e6 in the low two bits of bytes 0..3 and e1, e5, e3, e7 two bits above them.
struct Half2 {
  uint32_t le, he, od;
};

__device__ __forceinline__ Half2 decode2_a(uint32_t x16, const Tab4& t) {
  const uint32_t u = (x16 << 12) | x16;
  const uint32_t ev = u & 0x03030303u;
  Half2 h;
  h.od = (u >> 2) & 0x03030303u;
  h.le = __builtin_amdgcn_perm(t.lt_lo, t.lt_lo, ev);
  h.he = __builtin_amdgcn_perm(t.ht_lo, t.ht_lo, ev);
  return h;
}

__device__ __forceinline__ uint4 decode2_b(Half2 h, const Tab4& t) {
  const uint32_t lo = __builtin_amdgcn_perm(t.lt_lo, t.lt_lo, h.od);
  const uint32_t ho = __builtin_amdgcn_perm(t.ht_lo, t.ht_lo, h.od);
  uint4 r;
  r.x = __builtin_amdgcn_perm(h.he, h.le, 0x06020400u);  // (e0, e2)
  r.y = __builtin_amdgcn_perm(h.he, h.le, 0x07030501u);  // (e4, e6)
  r.z = __builtin_amdgcn_perm(ho, lo, 0x06020400u);      // (e1, e3)
  r.w = __builtin_amdgcn_perm(ho, lo, 0x07030501u);      // (e5, e7)
  return r;
}

// 6-bit, in two halves: (1) the four lookups of code pairs in lut6[i] = (bf16 c(i & 63),
// bf16 c(i >> 6)), issued a half-step before (2) their use, so that the wait for them does not
// also wait for the fragment reads issued in between; 48 bits (lo 32 + hi 16) hold 8 codes.
struct Half6 {
  uint32_t p01, p23, p45, p67;
};

__device__ __forceinline__ Half6 decode6_a(uint32_t lo, uint32_t hi, const uint32_t* lut6) {
  Half6 h;
  h.p01 = lut6[lo & 0xFFF];
  h.p23 = lut6[(lo >> 12) & 0xFFF];
  h.p45 = lut6[((lo >> 24) | (hi << 8)) & 0xFFF];
  h.p67 = lut6[(hi >> 4) & 0xFFF];
  return h;
}

__device__ __forceinline__ uint4 decode6_b(const Half6& h) {
  uint4 r;
  r.x = __builtin_amdgcn_perm(h.p23, h.p01, 0x05040100u);  // (e0, e2)
  r.y = __builtin_amdgcn_perm(h.p67, h.p45, 0x05040100u);  // (e4, e6)
  r.z = __builtin_amdgcn_perm(h.p23, h.p01, 0x07060302u);  // (e1, e3)
  r.w = __builtin_amdgcn_perm(h.p67, h.p45, 0x07060302u);  // (e5, e7)
  return r;
}

__device__ __forceinline__ uint4 decode6(uint32_t lo, uint32_t hi, const uint32_t* lut6) {
  return decode6_b(decode6_a(lo, hi, lut6));
}

// 3-bit, in two halves, by v_perm_b32 byte lookups into the 8 signed bf16 values (low bytes in
// t.lt_lo / t.lt_hi, high bytes in t.ht_lo / t.ht_hi).  The low 24 bits of x hold 8 codes (bits
// above are ignored); y has e0..e3 in its low half and e4..e7 in its high half, 12 bits each,
// from which e0, e2, e4, e6 (then e1, e3, e5, e7) are moved to the low bits of bytes 0..3.
struct Half3 {
  uint32_t y, le, he;
};

__device__ __forceinline__ Half3 decode3_a(uint32_t x, const Tab4& t) {
  Half3 h;
  h.y = (x & 0xFFFu) | ((x << 4) & ~0xFFFu);  // bits 12..15 and 28..31 are never read
  const uint32_t ev = (h.y & 0x00070007u) | ((h.y << 2) & 0x07000700u);
  h.le = __builtin_amdgcn_perm(t.lt_hi, t.lt_lo, ev);
  h.he = __builtin_amdgcn_perm(t.ht_hi, t.ht_lo, ev);
  return h;
}

__device__ __forceinline__ uint4 decode3_b(const Half3& h, const Tab4& t) {
  const uint32_t od = ((h.y >> 3) & 0x00070007u) | ((h.y >> 1) & 0x07000700u);
  const uint32_t lo = __builtin_amdgcn_perm(t.lt_hi, t.lt_lo, od);
  const uint32_t ho = __builtin_amdgcn_perm(t.ht_hi, t.ht_lo, od);
  uint4 r;
  r.x = __builtin_amdgcn_perm(h.he, h.le, 0x05010400u);  // (e0, e2)
  r.y = __builtin_amdgcn_perm(h.he, h.le, 0x07030602u);  // (e4, e6)
  r.z = __builtin_amdgcn_perm(ho, lo, 0x05010400u);      // (e1, e3)
  r.w = __builtin_amdgcn_perm(ho, lo, 0x07030602u);      // (e5, e7)
  return r;
}

__device__ __forceinline__ uint16_t mag_signed(const uint16_t* mag, uint32_t code, int bits) {
  const uint32_t half = 1u << (bits - 1);
  return static_cast<uint16_t>(mag[code & (half - 1)] | ((code & half) ? 0x8000u : 0u));
}

constexpr int lut_bytes_dev(int bits) { return bits == 6 ? 4096 * 4 : 0; }
constexpr bool needs_lut(int bits) { return bits == 6; }

template <int BITS>
__device__ __forceinline__ void build_lut(const uint16_t* mag, unsigned char* p, int tid, int nthreads = kThreads) {
  if constexpr (BITS == 6) {
    uint32_t* l = reinterpret_cast<uint32_t*>(p);
    for (int i = tid; i < 4096; i += nthreads)
      l[i] = mag_signed(mag, i & 63, 6) | (static_cast<uint32_t>(mag_signed(mag, i >> 6, 6)) << 16);
  }
}

// One operand's code unit (8 codes) of a K tile: raw bits in registers, decoded in two halves.
// `off` is the unit's byte offset from the resource base (row * row_bytes + unit column bytes).
template <int B>
struct Unit;

template <>
struct Unit<4> {
  static constexpr int kStep = KT / 2;  // bytes per K tile of a row
  uint32_t w;
  Half4 h;
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
    w = __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0);
  }
  __device__ __forceinline__ void first(const Tab4& t, const void*) { h = decode4_a(w, t); }
  __device__ __forceinline__ uint4 second(const Tab4&, const void*) const { return decode4_b(w, h); }
  static __device__ __forceinline__ uint32_t col_bytes(uint32_t c) { return 4 * c; }
};

template <>
struct Unit<2> {
  static constexpr int kStep = KT / 4;
  uint32_t w;
  Half2 h;
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
    w = __builtin_amdgcn_raw_buffer_load_b16(rs, off, 0, 0);
  }
  __device__ __forceinline__ void first(const Tab4& t, const void*) { h = decode2_a(w, t); }
  __device__ __forceinline__ uint4 second(const Tab4& t, const void*) const { return decode2_b(h, t); }
  static __device__ __forceinline__ uint32_t col_bytes(uint32_t c) { return 2 * c; }
};

template <>
struct Unit<3> {
  static constexpr int kStep = KT * 3 / 8;  // 24 bytes per K tile of a row
  v2u_t w;        // 8 bytes read from a 4-byte aligned offset; the unit starts 0..3 bytes in
  uint32_t sh;    // 8 * (3 c mod 4): bit offset of the unit in w
  Half3 h;
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
    w = __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, 0);
  }
  __device__ __forceinline__ void first(const Tab4& t, const void*) {
    h = decode3_a(__builtin_amdgcn_alignbit(w.y, w.x, sh), t);
  }
  __device__ __forceinline__ uint4 second(const Tab4& t, const void*) const { return decode3_b(h, t); }
  static __device__ __forceinline__ uint32_t col_bytes(uint32_t c) { return (3 * c) & ~3u; }
};

template <>
struct Unit<6> {
  static constexpr int kStep = KT * 6 / 8;
  v2u_t w;        // 8 bytes read from a 4-byte aligned offset; the unit starts 0 or 2 bytes in
  uint32_t sh;    // 0 or 16: bit offset of the unit in w
  Half6 h;
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
    w = __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, 0);
  }
  __device__ __forceinline__ void first(const Tab4&, const void* lut) {
    const uint32_t lo = __builtin_amdgcn_alignbit(w.y, w.x, sh);
    const uint32_t hi = (w.y >> sh) & 0xFFFFu;
    h = decode6_a(lo, hi, static_cast<const uint32_t*>(lut));
  }
  __device__ __forceinline__ uint4 second(const Tab4&, const void*) const { return decode6_b(h); }
  static __device__ __forceinline__ uint32_t col_bytes(uint32_t c) { return (6 * c) & ~3u; }
};

// bf16 operand rows (activations already decoded to their centroids, in the staged k order):
// staged by direct-to-LDS loads, nothing held in registers and nothing to decode
template <>
struct Unit<16> {
  static constexpr int kStep = KT * 2;
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t, uint32_t) {}
  __device__ __forceinline__ void first(const Tab4&, const void*) {}
  __device__ __forceinline__ uint4 second(const Tab4&, const void*) const { return make_uint4(0, 0, 0, 0); }
  static __device__ __forceinline__ uint32_t col_bytes(uint32_t c) { return 16 * c; }
};

// 16 bytes per lane from a buffer straight into LDS (buffer_load_dwordx4 ... lds): lane l's bytes
// land at lds + 16 l.  The LDS base goes through M0 and must be wave-uniform.
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t r, unsigned char* lds, uint32_t voff) {
#if __HIP_DEVICE_COMPILE__
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, 0, 0, 0);
#endif
}

// ----------------------------------------------------------------------------- activations
// GELU, tanh form: x/2 (1 + tanh(u)), u = sqrt(2/pi) (x + 0.044715 x^3), rewritten as the
// logistic x / (1 + exp(-2u)) = x / (1 + 2^-z), z = x (k0 + k1 x^2), k0 = 2 sqrt(2/pi) log2(e),
// k1 = 0.044715 k0.  Large negative x gives 2^-z = inf and 0; large positive x gives x.
__device__ __forceinline__ float gelu_tanh(float x) {
  const float z = x * __builtin_fmaf(0.10294324f, x * x, 2.3022082f);
  return x * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-z));
}

// GELU, erf form: x Phi(x).  Phi(-|x|) = erfc(|x|/sqrt 2)/2 by Abramowitz & Stegun 7.1.26:
// erfc(u) = (a1 q + a2 q^2 + a3 q^3 + a4 q^4 + a5 q^5) e^(-u^2), q = 1 / (1 + p u), with an
// absolute error below 1.5e-7 for u >= 0 (the published constants p, a1..a5).  Evaluating
// the small tail Phi(-|x|) directly avoids cancelling 1 - erf for negative x.
__device__ __forceinline__ float gelu_erf(float x) {
  const float ax = __builtin_fabsf(x);
  const float q = __builtin_amdgcn_rcpf(__builtin_fmaf(0.23164189f, ax, 1.0f));  // p / sqrt 2
  float poly = __builtin_fmaf(1.061405429f, q, -1.453152027f);
  poly = __builtin_fmaf(poly, q, 1.421413741f);
  poly = __builtin_fmaf(poly, q, -0.284496736f);
  poly = __builtin_fmaf(poly, q, 0.254829592f);
  const float e = __builtin_amdgcn_exp2f(-0.72134752f * ax * ax);  // e^(-x^2 / 2)
  const float tail = 0.5f * poly * q * e;                           // Phi(-|x|)
  return x * (x >= 0.0f ? 1.0f - tail : tail);
}

constexpr int kActNone = 0, kActGeluTanh = 1, kActGeluErf = 2;

template <int ACT>
__device__ __forceinline__ float activate(float v) {
  if constexpr (ACT == kActGeluTanh) return gelu_tanh(v);
  else if constexpr (ACT == kActGeluErf) return gelu_erf(v);
  else return v;
}

template <int ACT>
struct ActTag {
  static constexpr int value = ACT;
};

// chunk swizzle of a staged row: chunk c of row r sits at c ^ ((r >> 1) & 7)
__device__ __forceinline__ uint32_t swz(uint32_t r) { return (r >> 1) & 7; }

template <int BA, int BW, bool OUT_BF16, int BM, int BN>
__global__ __launch_bounds__(kThreads) void k_lut_gemm(GemmArgs a) {
  using C = Cfg<BM, BN>;
  extern __shared__ __align__(16) unsigned char smem[];
  // LDS: [A stage 0][A stage 1][B stage 0][B stage 1][6-bit tables]
  unsigned char* lut = smem + C::LDS;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 3, wn = wave >> 2;

  // XCD-aware order: workgroups are dealt round-robin to the 8 XCDs.  With group_n > 0 (the
  // weight-column tiles divide by 8) XCD x owns column tiles x cw .. x cw + cw - 1 (cw =
  // tiles_m / 8) and takes them in groups of group_n token tiles x all cw columns, about one
  // group per round of its compute units, so that a round fetches group_n token-row blocks and
  // its own cw weight-row blocks into that XCD's L2 and the weight rows stay there from round to
  // round.  Otherwise each XCD takes a contiguous band of the tiles in tile order.
  const int ntiles = a.tiles_n * a.tiles_m;
  int tn, tm;
  if (a.group_n > 0) {
    const int x = blockIdx.x & 7, l = blockIdx.x >> 3, cw = a.tiles_m >> 3;
    const int span = a.group_n * cw, q = l / span, r = l - q * span;
    const int gn = min(a.group_n, a.tiles_n - q * a.group_n);  // the last group may be shorter
    tn = q * a.group_n + r % gn;
    tm = x * cw + r / gn;
  } else {
    int tile = blockIdx.x;
    if ((ntiles & 7) == 0) tile = (tile & 7) * (ntiles >> 3) + (tile >> 3);
    tn = tile % a.tiles_n;
    tm = tile / a.tiles_n;
  }
  // both orders are bijections onto the tile grid; a workgroup outside it (arguments that do not
  // belong together) leaves before touching memory, all its threads together
  if (tn < 0 || tm < 0 || tn >= a.tiles_n || tm >= a.tiles_m) return;
  const int64_t row0 = static_cast<int64_t>(tn) * BM;  // token rows
  const int64_t col0 = static_cast<int64_t>(tm) * BN;  // weight rows

  // decode table for 6-bit codes, built from the magnitudes (staged through the first
  // bytes of the B region, which the first K tile overwrites only after the next barrier)
  unsigned char* lut_a = lut;
  unsigned char* lut_w = lut + lut_bytes_dev(BA);
  if constexpr (needs_lut(BA) || needs_lut(BW)) {
    uint16_t* mags = reinterpret_cast<uint16_t*>(smem + 2 * C::SA);
#pragma unroll
    for (int r = 0; r < 32; ++r) {
      if (tid == r) mags[r] = a.mag_a[r];
      if (tid == 32 + r) mags[32 + r] = a.mag_w[r];
    }
    __syncthreads();
    build_lut<BA>(mags, lut_a, tid);
    build_lut<BW>(mags + 32, lut_w, tid);
    __syncthreads();
  }
  const Tab4 ta{a.lt_lo_a, a.lt_hi_a, a.ht_lo_a, a.ht_hi_a};
  const Tab4 tw{a.lt_lo_w, a.lt_hi_w, a.ht_lo_w, a.ht_hi_w};

  // ---- staging role: unit column c of rows rr + 64 i of the (A rows, then B rows) tile
  const uint32_t c = tid & 7, rr = tid >> 3;
  const uint32_t xrow = static_cast<uint32_t>(a.xrow_bytes), wrow = static_cast<uint32_t>(a.wrow_bytes);
  const uint32_t xoff0 = rr * xrow + Unit<BA>::col_bytes(c), woff0 = rr * wrow + Unit<BW>::col_bytes(c);
  const uint32_t wofs = rr * kRow + ((c ^ swz(rr)) << 4);  // swz(rr + 64 i) = swz(rr)
  // the odd / even parity of the (virtual) first tile: an odd tile count is padded with a
  // leading all-zero tile so that the loop runs in pairs
  const int odd = a.nk & 1;
  const int nv = a.nk + odd;
  const uint8_t* xbase = a.xc + row0 * xrow;
  const uint8_t* wbase = a.wc + col0 * wrow;
  const int64_t xrem = (a.n - row0) * static_cast<int64_t>(xrow);
  const int64_t wrem = (a.m - col0) * static_cast<int64_t>(wrow);
  auto rsrc = [](const uint8_t* base, int64_t rem, int kt, int step) {
    const int64_t left = rem - static_cast<int64_t>(kt) * step;
    const uint32_t nrec = left > 0xFFFFFFF0ll ? 0xFFFFFFF0u : static_cast<uint32_t>(left);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base + static_cast<int64_t>(kt) * step), 0,
                                             nrec, kBufWord3);
  };
  // real K tile of virtual tile v (clamped into range: loads past the last tile are discarded)
  auto real_tile = [&](int v) { return min(max(v - odd, 0), a.nk - 1); };

  struct Set {
    Unit<BA> ua[C::UA];
    Unit<BW> ub[C::U - C::UA];
  };
  Set s0, s1;
  auto load_set = [&](Set& s, int v) {
    const int kt = real_tile(v);
    const auto rx = rsrc(xbase, xrem, kt, Unit<BA>::kStep);
    const auto rw = rsrc(wbase, wrem, kt, Unit<BW>::kStep);
#pragma unroll
    for (int i = 0; i < C::UA; ++i) s.ua[i].load(rx, xoff0 + 64u * i * xrow);
#pragma unroll
    for (int i = 0; i < C::U - C::UA; ++i) s.ub[i].load(rw, woff0 + 64u * i * wrow);
  };
  // bf16 A rows: each wave's 64 lanes fill 8 whole staged rows (1 KB) per load; lane l takes the
  // 16-byte chunk that belongs in slot l % 8 of row l / 8 (the rows' chunk swizzle)
  auto load_a_lds = [&](int v, int stage) {
    if constexpr (BA == 16) {
      const auto rx = rsrc(xbase, xrem, real_tile(v), KT * 2);
      const uint32_t lrow = (tid >> 3) & 7, slot = tid & 7;
#pragma unroll
      for (int i = 0; i < C::UA; ++i) {
        const uint32_t row = 64u * i + 8u * wave + lrow;
        lds_dma16(rx, smem + stage * C::SA + (64 * i + 8 * wave) * kRow, row * xrow + ((slot ^ swz(row)) << 4));
      }
    }
  };
  if constexpr (BA == 6 || BA == 3) {
    const uint32_t sh = BA == 6 ? (c & 1) * 16 : 8 * ((3 * c) & 3);
#pragma unroll
    for (int i = 0; i < C::UA; ++i) { s0.ua[i].sh = sh; s1.ua[i].sh = sh; }
  }
  if constexpr (BW == 6 || BW == 3) {
    const uint32_t sh = BW == 6 ? (c & 1) * 16 : 8 * ((3 * c) & 3);
#pragma unroll
    for (int i = 0; i < C::U - C::UA; ++i) { s0.ub[i].sh = sh; s1.ub[i].sh = sh; }
  }

  // half-step h (0 <= h < 2U) of the decode of set s into stage buf: unit h / 2, half h % 2
  auto half_step = [&](Set& s, int buf, int h) {
    const int u = h >> 1;
    if (u < C::UA) {
      if constexpr (BA == 16) return;  // staged by the direct loads
      if ((h & 1) == 0) s.ua[u].first(ta, lut_a);
      else {
        const uint4 v = s.ua[u].second(ta, lut_a);
        *reinterpret_cast<uint4*>(smem + buf * C::SA + wofs + u * (64 * kRow)) = v;
      }
    } else {
      const int ub = u - C::UA;
      if ((h & 1) == 0) s.ub[ub].first(tw, lut_w);
      else {
        const uint4 v = s.ub[ub].second(tw, lut_w);
        *reinterpret_cast<uint4*>(smem + 2 * C::SA + buf * C::SB + wofs + ub * (64 * kRow)) = v;
      }
    }
  };

  f32x16_t acc[C::TI][C::TJ];
#pragma unroll
  for (int i = 0; i < C::TI; ++i)
#pragma unroll
    for (int j = 0; j < C::TJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // fragment addresses: row (band + 32 i + l32), chunk (2 ks + g) xor the row swizzle; the
  // swizzle depends only on l32 (bands are multiples of 32 rows), so i, j and the stage are
  // immediate offsets
  const int g = lane >> 5, l32 = lane & 31;
  const uint32_t sw = swz(l32);
  uint32_t a_off[4], b_off[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const uint32_t ch = ((2u * ks + g) ^ sw) << 4;
    a_off[ks] = (wm * C::TM + l32) * kRow + ch;
    b_off[ks] = 2 * C::SA + (wn * C::TN + l32) * kRow + ch;
  }
  struct Frags {
    bf16x8_t fa[C::TI], fb[C::TJ];
  };
  auto read_frags = [&](Frags& f, int buf, int ks) {
#pragma unroll
    for (int i = 0; i < C::TI; ++i)
      f.fa[i] = *reinterpret_cast<const bf16x8_t*>(smem + a_off[ks] + buf * C::SA + i * (32 * kRow));
#pragma unroll
    for (int j = 0; j < C::TJ; ++j)
      f.fb[j] = *reinterpret_cast<const bf16x8_t*>(smem + b_off[ks] + buf * C::SB + j * (32 * kRow));
  };

  // one K tile: MFMAs on stage `buf` (its first fragments already in f[0]); the decode of set
  // `s` into stage 1 - buf runs in the shadow of the first three k-steps, then one barrier, and
  // the last k-step's MFMAs cover the reads of the next tile's first fragments
  auto ktile = [&](int buf, Set& s, Frags (&f)[2], int v) {
    if constexpr (BA == 16) {  // bf16 A of the next K tile, straight into its stage
      if (v + 1 < nv) load_a_lds(v + 1, 1 - buf);
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      if (ks == 3) {
        if constexpr (BA == 16) __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's direct loads landed
        __syncthreads();
      }
#pragma unroll
      for (int p = 0; p < C::NM; ++p) {
        const int i = p / C::TJ, j = p % C::TJ;
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f[ks & 1].fa[i], f[ks & 1].fb[j], acc[i][j], 0, 0, 0);
        if (p < C::TI + C::TJ) {
          Frags& g2 = f[(ks + 1) & 1];
          const int kn = ks < 3 ? ks + 1 : 0;
          const int bn = ks < 3 ? buf : 1 - buf;
          if (p < C::TI)
            g2.fa[p] = *reinterpret_cast<const bf16x8_t*>(smem + a_off[kn] + bn * C::SA + p * (32 * kRow));
          else
            g2.fb[p - C::TI] = *reinterpret_cast<const bf16x8_t*>(smem + b_off[kn] + bn * C::SB + (p - C::TI) * (32 * kRow));
        }
        const int q = ks * C::NM + p;
        if (ks < 3 && (q % 3) != 2) half_step(s, 1 - buf, 2 * (q / 3) + (q % 3));
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // ---- prologue: codes of virtual tiles 0 and 1 in registers, tile 0 staged (all zero when it
  // is the padding tile of an odd tile count)
  load_set(s0, 0);
  load_set(s1, 1);
  if constexpr (BA == 16) {
    if (!odd) load_a_lds(0, 0);
  }
  if (odd) {
#pragma unroll
    for (int u = 0; u < C::UA; ++u)
      *reinterpret_cast<uint4*>(smem + wofs + u * (64 * kRow)) = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int u = 0; u < C::U - C::UA; ++u)
      *reinterpret_cast<uint4*>(smem + 2 * C::SA + wofs + u * (64 * kRow)) = make_uint4(0, 0, 0, 0);
  } else {
#pragma unroll
    for (int h = 0; h < 2 * C::U; ++h) half_step(s0, 0, h);
  }
  if constexpr (BA == 16) __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __syncthreads();

  Frags f[2];
  read_frags(f[0], 0, 0);
  for (int v = 0; v < nv; v += 2) {
    load_set(s0, v + 2);
    ktile(0, s1, f, v);  // MFMAs on tile v, decode of tile v + 1
    load_set(s1, v + 3);
    ktile(1, s0, f, v + 1);  // MFMAs on tile v + 1, decode of tile v + 2
  }

  // ---- epilogue: D[row][col] of a 32x32 tile: col = lane % 32, row = 8*(r/4) + 4*(lane/32) + r%4
  // (the activation is a uniform kernel argument: one branch selects the epilogue's variant)
  auto epilogue = [&](auto tag) {
  constexpr int ACT = decltype(tag)::value;
  const bool full = row0 + BM <= a.n && col0 + BN <= a.m;
  constexpr int esz = OUT_BF16 ? 2 : 4;
  float rn[C::TJ];
  if (full) {
    // whole tile in range: rows of a 32-row block are (r-dependent, uniform) scalar offsets,
    // columns per-lane vector offsets, so the stores need no per-element address arithmetic;
    // bf16 pairs of adjacent rows are rounded together (v_cvt_pk_bf16_f32, nearest even)
    const int64_t ldy = a.ldy;
    unsigned char* ybase = static_cast<unsigned char*>(a.Y) + (row0 * ldy + col0) * esz;
    const __amdgpu_buffer_rsrc_t ys = __builtin_amdgcn_make_buffer_rsrc(ybase, 0, 0xFFFFFFF0u, kBufWord3);
    uint32_t voff[C::TJ];
#pragma unroll
    for (int j = 0; j < C::TJ; ++j) {
      const int col = wn * C::TN + 32 * j + l32;
      rn[j] = __builtin_bit_cast(float, static_cast<uint32_t>(a.wn[col0 + col]) << 16);
      voff[j] = static_cast<uint32_t>(((wm * C::TM + 4 * g) * ldy + col) * esz);
    }
    // the row scales of the next 32-row block are loaded before the current block's stores, so
    // that waiting for them never waits for stores (one counter covers both on gfx9)
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    const float* xsw = a.xs + row0 + wm * C::TM + 4 * g;
    f32x2_t sv[2][8];
    auto load_s = [&](int i, f32x2_t (&dst)[8]) {
#pragma unroll
      for (int r = 0; r < 16; r += 2)
        dst[r >> 1] = *reinterpret_cast<const f32x2_t*>(xsw + 32 * i + 8 * (r >> 2) + (r & 3));
    };
    load_s(0, sv[0]);
#pragma unroll
    for (int i = 0; i < C::TI; ++i) {
      if (i + 1 < C::TI) load_s(i + 1, sv[(i + 1) & 1]);
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const int rr0 = 32 * i + 8 * (r >> 2) + (r & 3);  // row within the wave band (less 4 g)
        const float s0 = sv[i & 1][r >> 1].x, s1 = sv[i & 1][r >> 1].y;
        const int so0 = static_cast<int>(rr0 * ldy * esz), so1 = static_cast<int>((rr0 + 1) * ldy * esz);
#pragma unroll
        for (int j = 0; j < C::TJ; ++j) {
          const float v0 = activate<ACT>(acc[i][j][r] * s0 * rn[j]);
          const float v1 = activate<ACT>(acc[i][j][r + 1] * s1 * rn[j]);
          if constexpr (OUT_BF16) {
            typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
            const bf16x2_t p = {static_cast<__bf16>(v0), static_cast<__bf16>(v1)};
            const uint32_t u = __builtin_bit_cast(uint32_t, p);
            __builtin_amdgcn_raw_buffer_store_b16(static_cast<unsigned short>(u), ys, voff[j], so0, kYStorePolicy);
            __builtin_amdgcn_raw_buffer_store_b16(static_cast<unsigned short>(u >> 16), ys, voff[j], so1, kYStorePolicy);
          } else {
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v0), ys, voff[j], so0, kYStorePolicy);
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v1), ys, voff[j], so1, kYStorePolicy);
          }
        }
      }
    }
    return;
  }
  // edge tile: per-element bounds checks.  The 16 row scales of a 32-row block are loaded
  // first, together (row index clamped), so that their latencies overlap instead of following
  // one another behind the bounds checks.
  int64_t cols[C::TJ];
#pragma unroll
  for (int j = 0; j < C::TJ; ++j) {
    cols[j] = col0 + wn * C::TN + 32 * j + l32;
    rn[j] = __builtin_bit_cast(float, static_cast<uint32_t>(a.wn[min(cols[j], a.m - 1)]) << 16);
  }
#pragma unroll
  for (int i = 0; i < C::TI; ++i) {
    float srow[16];
#pragma unroll
    for (int r = 0; r < 16; ++r)
      srow[r] = a.xs[min(row0 + wm * C::TM + 32 * i + 8 * (r >> 2) + 4 * g + (r & 3), a.n - 1)];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t row = row0 + wm * C::TM + 32 * i + 8 * (r >> 2) + 4 * g + (r & 3);
      if (row >= a.n) continue;
      const float sr = srow[r];
      if constexpr (OUT_BF16) {
        __bf16* yrow = reinterpret_cast<__bf16*>(a.Y) + row * a.ldy;
#pragma unroll
        for (int j = 0; j < C::TJ; ++j)
          if (cols[j] < a.m) yrow[cols[j]] = static_cast<__bf16>(activate<ACT>(acc[i][j][r] * sr * rn[j]));
      } else {
        float* yrow = reinterpret_cast<float*>(a.Y) + row * a.ldy;
#pragma unroll
        for (int j = 0; j < C::TJ; ++j)
          if (cols[j] < a.m) yrow[cols[j]] = activate<ACT>(acc[i][j][r] * sr * rn[j]);
      }
    }
  }
  };
  switch (a.act) {
    case kActGeluTanh: epilogue(ActTag<kActGeluTanh>{}); break;
    case kActGeluErf: epilogue(ActTag<kActGeluErf>{}); break;
    default: epilogue(ActTag<kActNone>{}); break;
  }
}

template <int BA, int BW, int BM, int BN>
inline hipError_t launch_cfg(bool out_bf16, const GemmArgs& a, int grid, size_t lds, hipStream_t st) {
  if (out_bf16)
    hipLaunchKernelGGL((k_lut_gemm<BA, BW, true, BM, BN>), dim3(grid), dim3(kThreads), lds, st, a);
  else
    hipLaunchKernelGGL((k_lut_gemm<BA, BW, false, BM, BN>), dim3(grid), dim3(kThreads), lds, st, a);
  return hipGetLastError();
}

template <int BA, int BW>
inline hipError_t launch_bw(int cfg, bool out_bf16, const GemmArgs& a, int grid, size_t lds, hipStream_t st) {
  return cfg == 0 ? launch_cfg<BA, BW, 384, 192>(out_bf16, a, grid, lds, st)
                  : launch_cfg<BA, BW, 256, 256>(out_bf16, a, grid, lds, st);
}

template <int BA>
inline hipError_t launch_ba(int bw, int cfg, bool out_bf16, const GemmArgs& a, int grid, size_t lds, hipStream_t st) {
  if constexpr (BA == 3) {
    return launch_bw<3, 3>(cfg, out_bf16, a, grid, lds, st);  // 3-bit pairs only with 3-bit
  } else {
    switch (bw) {
      case 2: return launch_bw<BA, 2>(cfg, out_bf16, a, grid, lds, st);
      case 4: return launch_bw<BA, 4>(cfg, out_bf16, a, grid, lds, st);
      default: return launch_bw<BA, 6>(cfg, out_bf16, a, grid, lds, st);
    }
  }
}

inline void tab4(const DecodeParams& dp, uint32_t* lt_lo, uint32_t* lt_hi, uint32_t* ht_lo, uint32_t* ht_hi) {
  uint32_t l[2] = {0, 0}, h[2] = {0, 0};
  if (dp.bits == 4) {
    for (int r = 0; r < 8; ++r) {
      l[r >> 2] |= static_cast<uint32_t>(dp.mag[r] & 0xFF) << (8 * (r & 3));
      h[r >> 2] |= static_cast<uint32_t>(dp.mag[r] >> 8) << (8 * (r & 3));
    }
  } else if (dp.bits == 2 || dp.bits == 3) {  // the signed values: code q = sign bit, then magnitude
    const int half = 1 << (dp.bits - 1);
    for (int q = 0; q < 2 * half; ++q) {
      const uint32_t v = dp.mag[q & (half - 1)] | ((q & half) ? 0x8000u : 0u);
      l[q >> 2] |= (v & 0xFF) << (8 * (q & 3));
      h[q >> 2] |= (v >> 8) << (8 * (q & 3));
    }
  }
  *lt_lo = l[0];
  *lt_hi = l[1];
  *ht_lo = h[0];
  *ht_hi = h[1];
}

// Launchers of one activation bit width (lut_gemm_a<BA>.hip).
hipError_t launch_gemm_a2(int bw, int cfg, bool out_bf16, const GemmArgs& a, int grid, size_t lds, hipStream_t st);
hipError_t launch_gemm_a3(int bw, int cfg, bool out_bf16, const GemmArgs& a, int grid, size_t lds, hipStream_t st);
hipError_t launch_gemm_a4(int bw, int cfg, bool out_bf16, const GemmArgs& a, int grid, size_t lds, hipStream_t st);
hipError_t launch_gemm_a6(int bw, int cfg, bool out_bf16, const GemmArgs& a, int grid, size_t lds, hipStream_t st);
hipError_t launch_gemm_abf(int bw, int cfg, bool out_bf16, const GemmArgs& a, int grid, size_t lds, hipStream_t st);

}  // namespace lg
}  // namespace orbq
