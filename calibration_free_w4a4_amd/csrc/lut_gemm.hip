// lut_gemm: Y = diag(s) * (C_a[codes_x] C_w[codes_w]^T) * diag(r') for packed Lloyd-Max codes.
//
// Method: OrbitQuant summary (picx.dev), "Online Activation Quantization": x^' = s Q(x~'),
// W^' = diag(r') Q(W~') ("Offline Weight Quantization"), and W^' x^' approximates W x because the
// rotation cancels.  The product is a dense contraction over d, so it runs on the matrix cores.
//
// Kernel layout (gfx950, wave64, 512 threads = 8 waves, two per SIMD):
//   * workgroup tile 256 tokens x 256 weight rows, K tile of 32; each wave computes 64 x 128
//     with v_mfma_f32_32x32x16_bf16 and fp32 accumulators (2 x 4 tiles of 32 x 32).
//   * waves 0-3 load the 256 token code rows of the K tile, waves 4-7 the 256 weight code rows
//     (8..24 bytes per thread), decode them to bf16 centroid values and store them to LDS; the
//     MFMA operands are 16-byte LDS reads.  Code rows are prefetched two K tiles ahead in
//     registers; LDS is double buffered, one barrier per K tile.
//   * decode of 4-bit codes: v_perm_b32 byte lookups into the 8 bf16 magnitudes (held in four
//     registers) plus the sign bit; 2-bit codes use a 256-entry LDS table per code byte, 6-bit
//     codes a 4096-entry LDS table per code pair.  Every decoder writes the 8 values of a
//     16-byte chunk in the order k = 0,2,4,6,1,3,5,7, so A and B agree on k.
//   * epilogue: Y = acc * s_i * r'_j in fp32, stored as fp32 or bf16 (round to nearest even).
#include <hip/hip_runtime.h>

#include "internal.h"

namespace orbq {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int BM = 256, BN = 256, KT = 32;
constexpr int kThreads = 512;

struct GemmArgs {
  const uint8_t* xc;
  const float* xs;
  const uint8_t* wc;
  const uint16_t* wn;
  void* Y;
  int64_t n, m, d, ldy;
  int64_t xrow_bytes, wrow_bytes;
  int32_t tiles_n, tiles_m;
  // 4-bit decode tables: low / high bytes of the 8 bf16 magnitudes, 4 per register
  uint32_t lt_lo_a, lt_hi_a, ht_lo_a, ht_hi_a;
  uint32_t lt_lo_w, lt_hi_w, ht_lo_w, ht_hi_w;
  uint16_t mag_a[32], mag_w[32];
};

// ----------------------------------------------------------------------------- decoders
struct Tab4 {
  uint32_t lt_lo, lt_hi, ht_lo, ht_hi;
};

__device__ __forceinline__ uint4 decode4(uint32_t X, const Tab4& t) {
  const uint32_t se = X & 0x07070707u;
  const uint32_t so = (X >> 4) & 0x07070707u;
  const uint32_t le = __builtin_amdgcn_perm(t.lt_hi, t.lt_lo, se);
  uint32_t he = __builtin_amdgcn_perm(t.ht_hi, t.ht_lo, se);
  const uint32_t lo = __builtin_amdgcn_perm(t.lt_hi, t.lt_lo, so);
  uint32_t ho = __builtin_amdgcn_perm(t.ht_hi, t.ht_lo, so);
  he |= (X << 4) & 0x80808080u;  // sign = bit 3 of each code
  ho |= X & 0x80808080u;
  uint4 r;
  r.x = __builtin_amdgcn_perm(he, le, 0x05010400u);  // (e0, e2)
  r.y = __builtin_amdgcn_perm(he, le, 0x07030602u);  // (e4, e6)
  r.z = __builtin_amdgcn_perm(ho, lo, 0x05010400u);  // (e1, e3)
  r.w = __builtin_amdgcn_perm(ho, lo, 0x07030602u);  // (e5, e7)
  return r;
}

// 2-bit: 16 bits hold 8 codes; lut2[b] = {(e0, e2), (e1, e3)} of code byte b
__device__ __forceinline__ uint4 decode2(uint32_t X16, const uint2* lut2) {
  const uint2 p0 = lut2[X16 & 0xFF];
  const uint2 p1 = lut2[(X16 >> 8) & 0xFF];
  return make_uint4(p0.x, p1.x, p0.y, p1.y);
}

// 6-bit: 48 bits (lo 32 + hi 16) hold 8 codes; lut6[i] = (bf16 c(i & 63), bf16 c(i >> 6))
__device__ __forceinline__ uint4 decode6(uint32_t lo, uint32_t hi, const uint32_t* lut6) {
  const uint32_t p01 = lut6[lo & 0xFFF];
  const uint32_t p23 = lut6[(lo >> 12) & 0xFFF];
  const uint32_t p45 = lut6[((lo >> 24) | (hi << 8)) & 0xFFF];
  const uint32_t p67 = lut6[(hi >> 4) & 0xFFF];
  uint4 r;
  r.x = __builtin_amdgcn_perm(p23, p01, 0x05040100u);  // (e0, e2)
  r.y = __builtin_amdgcn_perm(p67, p45, 0x05040100u);  // (e4, e6)
  r.z = __builtin_amdgcn_perm(p23, p01, 0x07060302u);  // (e1, e3)
  r.w = __builtin_amdgcn_perm(p67, p45, 0x07060302u);  // (e5, e7)
  return r;
}

__device__ __forceinline__ uint16_t mag_signed(const uint16_t* mag, uint32_t code, int bits) {
  const uint32_t half = 1u << (bits - 1);
  return static_cast<uint16_t>(mag[code & (half - 1)] | ((code & half) ? 0x8000u : 0u));
}

// Loads the K-tile bytes of one code row and decodes them into 4 chunks of 8 bf16.
template <int B>
struct RowTile;

template <>
struct RowTile<4> {
  uint4 raw;
  __device__ __forceinline__ void load(const uint8_t* row, int kt) {
    raw = *reinterpret_cast<const uint4*>(row + kt * 16);
  }
  __device__ __forceinline__ void decode(uint4 out[4], const Tab4& t, const void*) const {
    out[0] = decode4(raw.x, t);
    out[1] = decode4(raw.y, t);
    out[2] = decode4(raw.z, t);
    out[3] = decode4(raw.w, t);
  }
};

template <>
struct RowTile<2> {
  uint2 raw;
  __device__ __forceinline__ void load(const uint8_t* row, int kt) {
    raw = *reinterpret_cast<const uint2*>(row + kt * 8);
  }
  __device__ __forceinline__ void decode(uint4 out[4], const Tab4&, const void* lut) const {
    const uint2* l = static_cast<const uint2*>(lut);
    out[0] = decode2(raw.x & 0xFFFF, l);
    out[1] = decode2(raw.x >> 16, l);
    out[2] = decode2(raw.y & 0xFFFF, l);
    out[3] = decode2(raw.y >> 16, l);
  }
};

template <>
struct RowTile<6> {
  uint2 r0, r1, r2;  // 24 bytes
  __device__ __forceinline__ void load(const uint8_t* row, int kt) {
    const uint2* p = reinterpret_cast<const uint2*>(row + kt * 24);
    r0 = p[0];
    r1 = p[1];
    r2 = p[2];
  }
  __device__ __forceinline__ void decode(uint4 out[4], const Tab4&, const void* lut) const {
    const uint32_t* l = static_cast<const uint32_t*>(lut);
    // 8 codes per 6 bytes: words w0..w5
    out[0] = decode6(r0.x, r0.y & 0xFFFF, l);
    out[1] = decode6((r0.y >> 16) | (r1.x << 16), r1.x >> 16, l);
    out[2] = decode6(r1.y, r2.x & 0xFFFF, l);
    out[3] = decode6((r2.x >> 16) | (r2.y << 16), r2.y >> 16, l);
  }
};

// Row swizzle of the 16-byte chunks of a [256][32] bf16 tile (64-byte rows): chunk c of row r
// sits at c ^ swz(r).  swz takes distinct values on rows {r, r+2, r+4, r+6} and on rows
// {r, r+4, r+8, r+12}, so 16-byte accesses of any 8 (or 16) consecutive rows at one chunk hit
// distinct banks whether the LDS serves 128 or 256 bytes per clock.
__device__ __forceinline__ uint32_t swz(uint32_t r) { return ((r >> 1) + (r >> 3)) & 3; }

__device__ __forceinline__ uint32_t tile_off(int row, int chunk) {
  return static_cast<uint32_t>(row * 64 + ((chunk ^ swz(row)) << 4));
}

constexpr size_t lut_bytes_dev(int bits) { return bits == 2 ? 256 * 8 : bits == 6 ? 4096 * 4 : 0; }

template <int BITS>
__device__ __forceinline__ void build_lut(const uint16_t* mag, unsigned char* p, int tid) {
  if constexpr (BITS == 2) {
    uint2* l = reinterpret_cast<uint2*>(p);
    for (int b = tid; b < 256; b += kThreads) {
      const uint32_t c0 = mag_signed(mag, b & 3, 2), c1 = mag_signed(mag, (b >> 2) & 3, 2);
      const uint32_t c2 = mag_signed(mag, (b >> 4) & 3, 2), c3 = mag_signed(mag, (b >> 6) & 3, 2);
      l[b] = make_uint2(c0 | (c2 << 16), c1 | (c3 << 16));
    }
  } else if constexpr (BITS == 6) {
    uint32_t* l = reinterpret_cast<uint32_t*>(p);
    for (int i = tid; i < 4096; i += kThreads)
      l[i] = mag_signed(mag, i & 63, 6) | (static_cast<uint32_t>(mag_signed(mag, i >> 6, 6)) << 16);
  }
}

template <int BA, int BW, bool OUT_BF16>
__global__ __launch_bounds__(kThreads, 1) void k_lut_gemm(GemmArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  unsigned char* As = smem;                    // [2][256][32] bf16
  unsigned char* Bs = smem + 2 * BM * KT * 2;  // [2][256][32] bf16
  unsigned char* lut = Bs + 2 * BN * KT * 2;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 3, wn = wave >> 2;     // 64-row band of tokens, 128-row band of weights

  // XCD-aware order: workgroups are dealt round-robin to the 8 XCDs, so give each XCD a
  // contiguous band of tiles (neighbouring tiles share code rows in that XCD's L2)
  const int ntiles = a.tiles_n * a.tiles_m;
  int tile = blockIdx.x;
  if ((ntiles & 7) == 0) tile = (tile & 7) * (ntiles >> 3) + (tile >> 3);
  const int tn = tile % a.tiles_n, tm = tile / a.tiles_n;
  const int64_t row0 = static_cast<int64_t>(tn) * BM;  // token rows
  const int64_t col0 = static_cast<int64_t>(tm) * BN;  // weight rows

  // decode tables: 2- and 6-bit codes decode through LDS tables built from the magnitudes
  uint16_t* mags = reinterpret_cast<uint16_t*>(lut);  // [0, 32): activations, [32, 64): weights
  unsigned char* lut_a = lut + 128;
  unsigned char* lut_w = lut_a + lut_bytes_dev(BA);
  if constexpr (BA != 4 || BW != 4) {
#pragma unroll
    for (int r = 0; r < 32; ++r) {
      if (tid == r) mags[r] = a.mag_a[r];
      if (tid == 32 + r) mags[32 + r] = a.mag_w[r];
    }
    __syncthreads();
    build_lut<BA>(mags, lut_a, tid);
    build_lut<BW>(mags + 32, lut_w, tid);
  }

  // loader role: threads 0-255 stage token row tid, threads 256-511 weight row tid-256
  const bool loads_a = tid < BM;
  const int lrow = loads_a ? tid : tid - BM;
  const uint8_t* arow = a.xc + min(row0 + lrow, a.n - 1) * a.xrow_bytes;  // rows past the end are
  const uint8_t* brow = a.wc + min(col0 + lrow, a.m - 1) * a.wrow_bytes;  // computed and discarded
  const Tab4 ta{a.lt_lo_a, a.lt_hi_a, a.ht_lo_a, a.ht_hi_a};
  const Tab4 tw{a.lt_lo_w, a.lt_hi_w, a.ht_lo_w, a.ht_hi_w};
  const int nk = static_cast<int>(a.d / KT);

  f32x16_t acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int g = lane >> 5, l32 = lane & 31;
  // Fragment addresses: row (band + 32 i + l32), chunk (2 ks + g) xor the row swizzle.  The
  // swizzle depends only on l32, so per lane two bases (ks = 0, 1) per operand suffice and
  // the tile index i / j and the buffer become immediate offsets.
  const uint32_t sw = swz(l32);  // the band offsets are multiples of 32 rows: swz(band + l32) = swz(l32)
  const uint32_t a_base = (wm * 64 + l32) * 64, b_base = (wn * 128 + l32) * 64;
  const uint32_t ch0 = ((0u | g) ^ sw) << 4, ch1 = ((2u | g) ^ sw) << 4;
  const uint32_t a_off[2] = {a_base + ch0, a_base + ch1};
  const uint32_t b_off[2] = {b_base + ch0 + 2 * BM * KT * 2, b_base + ch1 + 2 * BM * KT * 2};
  auto compute = [&](int buf) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8_t fa[2], fb[4];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        fa[i] = *reinterpret_cast<const bf16x8_t*>(smem + a_off[ks] + buf * (BM * KT * 2) + i * (32 * 64));
#pragma unroll
      for (int j = 0; j < 4; ++j)
        fb[j] = *reinterpret_cast<const bf16x8_t*>(smem + b_off[ks] + buf * (BN * KT * 2) + j * (32 * 64));
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
  };

  // Main loop, specialised per loader role (waves 0-3 stage token rows, waves 4-7 weight rows;
  // both paths hit the same barriers).  Two K tiles are in flight in registers; the loop is
  // unrolled by two so that each register set keeps fixed registers.
  auto main_loop = [&](auto& r0, auto& r1, const uint8_t* crow, const Tab4& tab, const void* lutp,
                       unsigned char* tbase) {
    auto stage = [&](int buf, const auto& rt) {
      uint4 cv[4];
      rt.decode(cv, tab, lutp);
      unsigned char* t = tbase + buf * (BM * KT * 2);
#pragma unroll
      for (int c = 0; c < 4; ++c) *reinterpret_cast<uint4*>(t + tile_off(lrow, c)) = cv[c];
    };
    r0.load(crow, 0);
    r1.load(crow, 1);
    __syncthreads();  // decode tables built
    stage(0, r0);
    __syncthreads();
    // d is a multiple of 64, so nk = d / 32 is even and both halves always run.  The loads and
    // stages are unconditional (tile indices clamped; the extra stage at the end writes a buffer
    // nobody reads again) so that the compiler can count outstanding loads exactly and waits only
    // for the tile it decodes, not for the one just issued.
    for (int kt = 0; kt < nk; kt += 2) {
      r0.load(crow, min(kt + 2, nk - 1));
      compute(0);
      stage(1, r1);
      __syncthreads();
      r1.load(crow, min(kt + 3, nk - 1));
      compute(1);
      stage(0, r0);
      __syncthreads();
    }
  };
  if (loads_a) {
    RowTile<BA> r0, r1;
    main_loop(r0, r1, arow, ta, lut_a, As);
  } else {
    RowTile<BW> r0, r1;
    main_loop(r0, r1, brow, tw, lut_w, Bs);
  }

  // epilogue: D[row][col] of a 32x32 tile: col = lane % 32, row = 8*(r/4) + 4*(lane/32) + r%4
  const bool full = row0 + BM <= a.n && col0 + BN <= a.m;
  float rn[4];
  int64_t cols[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    cols[j] = col0 + wn * 128 + 32 * j + l32;
    rn[j] = (full || cols[j] < a.m) ? __builtin_bit_cast(float, static_cast<uint32_t>(a.wn[cols[j]]) << 16) : 0.0f;
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t row = row0 + wm * 64 + 32 * i + 8 * (r >> 2) + 4 * g + (r & 3);
      if (!full && row >= a.n) continue;
      const float sr = a.xs[row];
      if constexpr (OUT_BF16) {
        uint16_t* yrow = reinterpret_cast<uint16_t*>(a.Y) + row * a.ldy;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (!full && cols[j] >= a.m) continue;
          uint32_t u = __builtin_bit_cast(uint32_t, acc[i][j][r] * sr * rn[j]);
          u += 0x7fffu + ((u >> 16) & 1u);
          yrow[cols[j]] = static_cast<uint16_t>(u >> 16);
        }
      } else {
        float* yrow = reinterpret_cast<float*>(a.Y) + row * a.ldy;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (!full && cols[j] >= a.m) continue;
          yrow[cols[j]] = acc[i][j][r] * sr * rn[j];
        }
      }
    }
  }
}

size_t lut_bytes(int bits) { return bits == 2 ? 256 * 8 : bits == 6 ? 4096 * 4 : 0; }

template <int BA, int BW>
hipError_t launch_bw(bool out_bf16, const GemmArgs& a, int grid, size_t lds, hipStream_t st) {
  if (out_bf16)
    hipLaunchKernelGGL((k_lut_gemm<BA, BW, true>), dim3(grid), dim3(kThreads), lds, st, a);
  else
    hipLaunchKernelGGL((k_lut_gemm<BA, BW, false>), dim3(grid), dim3(kThreads), lds, st, a);
  return hipGetLastError();
}

template <int BA>
hipError_t launch_ba(int bw, bool out_bf16, const GemmArgs& a, int grid, size_t lds, hipStream_t st) {
  switch (bw) {
    case 2: return launch_bw<BA, 2>(out_bf16, a, grid, lds, st);
    case 4: return launch_bw<BA, 4>(out_bf16, a, grid, lds, st);
    default: return launch_bw<BA, 6>(out_bf16, a, grid, lds, st);
  }
}

void tab4(const DecodeParams& dp, uint32_t* lt_lo, uint32_t* lt_hi, uint32_t* ht_lo, uint32_t* ht_hi) {
  uint32_t l[2] = {0, 0}, h[2] = {0, 0};
  if (dp.bits == 4) {
    for (int r = 0; r < 8; ++r) {
      l[r >> 2] |= static_cast<uint32_t>(dp.mag[r] & 0xFF) << (8 * (r & 3));
      h[r >> 2] |= static_cast<uint32_t>(dp.mag[r] >> 8) << (8 * (r & 3));
    }
  }
  *lt_lo = l[0];
  *lt_hi = l[1];
  *ht_lo = h[0];
  *ht_hi = h[1];
}

}  // namespace

int launch_lut_gemm(const uint8_t* x_codes, const float* x_norms, const DecodeParams& da, const uint8_t* w_codes,
                    const uint16_t* w_norms, const DecodeParams& dw, int64_t n, int64_t m, int64_t d, void* Y,
                    int y_bf16, int64_t ldy, hipStream_t stream) {
  GemmArgs a{};
  a.xc = x_codes;
  a.xs = x_norms;
  a.wc = w_codes;
  a.wn = w_norms;
  a.Y = Y;
  a.n = n;
  a.m = m;
  a.d = d;
  a.ldy = ldy;
  a.xrow_bytes = d * da.bits / 8;
  a.wrow_bytes = d * dw.bits / 8;
  a.tiles_n = static_cast<int32_t>((n + BM - 1) / BM);
  a.tiles_m = static_cast<int32_t>((m + BN - 1) / BN);
  tab4(da, &a.lt_lo_a, &a.lt_hi_a, &a.ht_lo_a, &a.ht_hi_a);
  tab4(dw, &a.lt_lo_w, &a.lt_hi_w, &a.ht_lo_w, &a.ht_hi_w);
  for (int i = 0; i < 32; ++i) {
    a.mag_a[i] = da.mag[i];
    a.mag_w[i] = dw.mag[i];
  }
  const int grid = a.tiles_n * a.tiles_m;
  const size_t lds = 2 * (BM + BN) * KT * 2 + 128 + lut_bytes(da.bits) + lut_bytes(dw.bits);
  hipError_t e;
  switch (da.bits) {
    case 2: e = launch_ba<2>(dw.bits, y_bf16 != 0, a, grid, lds, stream); break;
    case 4: e = launch_ba<4>(dw.bits, y_bf16 != 0, a, grid, lds, stream); break;
    default: e = launch_ba<6>(dw.bits, y_bf16 != 0, a, grid, lds, stream); break;
  }
  return static_cast<int>(e);
}

}  // namespace orbq
