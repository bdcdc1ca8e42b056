// lut_gemm host side: tile choice, launch chunking and the dispatch over bit widths.  The
// kernel and its design notes are in lut_gemm_kernel.h.
#include "lut_gemm_kernel.h"

namespace orbq {
namespace lg {
namespace {

size_t lut_bytes(int bits) { return bits == 6 ? 4096 * 4 : 0; }

}  // namespace
}  // namespace lg

using namespace lg;

int device_cus() {
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

int launch_lut_gemm(const uint8_t* x_codes, const float* x_norms, const DecodeParams& da, const uint8_t* w_codes,
                    const uint16_t* w_norms, const DecodeParams& dw, int64_t n, int64_t m, int64_t d, void* Y,
                    int y_bf16, int64_t ldy, int act, hipStream_t stream) {
  GemmArgs a{};
  a.act = act;
  a.xs = x_norms;
  a.wn = w_norms;
  a.ldy = ldy;
  a.xrow_bytes = static_cast<int32_t>(d * da.bits / 8);
  a.wrow_bytes = static_cast<int32_t>(d * dw.bits / 8);
  a.nk = static_cast<int32_t>(d / KT);
  tab4(da, &a.lt_lo_a, &a.lt_hi_a, &a.ht_lo_a, &a.ht_hi_a);
  tab4(dw, &a.lt_lo_w, &a.lt_hi_w, &a.ht_lo_w, &a.ht_hi_w);
  for (int i = 0; i < 32; ++i) {
    a.mag_a[i] = da.mag[i];
    a.mag_w[i] = dw.mag[i];
  }
  // tile shape: the one that leaves the least idle work when the tiles are dealt to the
  // compute units in rounds (384 x 192 needs its LDS stages plus the tables to fit in 160 KB)
  const int cus = device_cus();
  const size_t luts = lut_bytes(da.bits) + lut_bytes(dw.bits);
  int cfg = 1;
  {
    double best = 1e300;
    for (int k = 0; k < 2; ++k) {
      const int64_t bm = k == 0 ? 384 : 256, bn = k == 0 ? 192 : 256;
      const size_t lds = (k == 0 ? Cfg<384, 192>::LDS : Cfg<256, 256>::LDS) + luts;
      if (lds > 160 * 1024) continue;
      const int64_t tiles = ((n + bm - 1) / bm) * ((m + bn - 1) / bn);
      const int64_t rounds = (tiles + cus - 1) / cus;
      const double cost = static_cast<double>(rounds) * bm * bn * (k == 0 ? 1.0 : 1.0001);
      if (cost < best) {
        best = cost;
        cfg = k;
      }
    }
  }
  const int bm = cfg == 0 ? 384 : 256, bn = cfg == 0 ? 192 : 256;
  const size_t lds = (cfg == 0 ? Cfg<384, 192>::LDS : Cfg<256, 256>::LDS) + luts;
  // launches over row / column blocks keep every code extent addressable with 32-bit offsets
  const int64_t max_rows_x = std::max<int64_t>(bm, (int64_t(1) << 31) / a.xrow_bytes / bm * bm);
  const int64_t max_rows_w = std::max<int64_t>(bn, (int64_t(1) << 31) / a.wrow_bytes / bn * bn);
  const int64_t esz = y_bf16 ? 2 : 4;
  hipError_t e = hipSuccess;
  for (int64_t r0 = 0; r0 < n && e == hipSuccess; r0 += max_rows_x) {
    for (int64_t c0 = 0; c0 < m && e == hipSuccess; c0 += max_rows_w) {
      GemmArgs b = a;
      b.n = std::min(max_rows_x, n - r0);
      b.m = std::min(max_rows_w, m - c0);
      b.xc = x_codes + r0 * a.xrow_bytes;
      b.xs = x_norms + r0;
      b.wc = w_codes + c0 * a.wrow_bytes;
      b.wn = w_norms + c0;
      b.Y = static_cast<unsigned char*>(Y) + (r0 * ldy + c0) * esz;
      b.tiles_n = static_cast<int32_t>((b.n + bm - 1) / bm);
      b.tiles_m = static_cast<int32_t>((b.m + bn - 1) / bn);
      // grouped XCD order when the column tiles split evenly over the 8 XCDs: groups of token
      // tiles x the XCD's cw column tiles, sized to about one round of its compute units.
      // Measured at 4608 x 3072 -> 12288: fetched bytes 195 -> 109 MB per launch (9216 tokens:
      // 709 -> 212 MB), the time unchanged (285.3 against 285.8 us); outputs identical.
      b.group_n = 0;
      if (b.tiles_m % 8 == 0) {
        const int cw = b.tiles_m / 8;
        b.group_n = std::max(1, (cus / 8) / cw);
      }
      const int grid = b.tiles_n * b.tiles_m;
      switch (da.bits) {
        case 2: e = launch_gemm_a2(dw.bits, cfg, y_bf16 != 0, b, grid, lds, stream); break;
        case 3: e = launch_gemm_a3(dw.bits, cfg, y_bf16 != 0, b, grid, lds, stream); break;
        case 4: e = launch_gemm_a4(dw.bits, cfg, y_bf16 != 0, b, grid, lds, stream); break;
        case 16: e = launch_gemm_abf(dw.bits, cfg, y_bf16 != 0, b, grid, lds, stream); break;
        default: e = launch_gemm_a6(dw.bits, cfg, y_bf16 != 0, b, grid, lds, stream); break;
      }
    }
  }
  return static_cast<int>(e);
}
}  // namespace orbq
