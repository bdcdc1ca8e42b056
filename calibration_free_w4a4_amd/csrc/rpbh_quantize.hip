// rpbh_quantize, host side: the workgroup shape, LDS layout, decision table and launch chunking
// of the kernel in rpbh_quantize_kernel.h, and the test-only decision kernel.
#include "rpbh_quantize_kernel.h"

#include <cstring>

namespace orbq {
namespace rq {
extern template hipError_t launch_block<64>(QuantMode, int, const QuantKernelArgs&, int, size_t, hipStream_t);
extern template hipError_t launch_block<128>(QuantMode, int, const QuantKernelArgs&, int, size_t, hipStream_t);
extern template hipError_t launch_block<256>(QuantMode, int, const QuantKernelArgs&, int, size_t, hipStream_t);
extern template hipError_t launch_block<512>(QuantMode, int, const QuantKernelArgs&, int, size_t, hipStream_t);
extern template hipError_t launch_block<1024>(QuantMode, int, const QuantKernelArgs&, int, size_t, hipStream_t);
extern template hipError_t launch_block<2048>(QuantMode, int, const QuantKernelArgs&, int, size_t, hipStream_t);
extern template hipError_t launch_block<4096>(QuantMode, int, const QuantKernelArgs&, int, size_t, hipStream_t);
}  // namespace rq

using namespace rq;

namespace {

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

size_t align16(size_t x) { return (x + 15) & ~size_t(15); }

// build_table on the host, for the kernel arguments: the same comparisons on the same fp32
// thresholds, so the entries are bit-identical to the device-built ones
void host_table(const QuantParams& qp, float2* out) {
  const int NB = (1 << (qp.bits - 1)) - 1, HALF = 1 << (qp.bits - 1);
  for (int e = 0; e < 2 * qp.J; ++e) {
    const int j = e - qp.J;
    const bool pos = j < 0;
    const float lo = static_cast<float>(pos ? -j - 1 : j), hi = lo + 1.0f;
    float thr = INFINITY;
    int base = pos ? 0 : HALF;
    for (int p = 0; p < NB; ++p) {
      const float b = pos ? qp.thr_gt[p] : qp.thr_ge[p];
      const bool below = pos ? (b <= lo) : (b < lo);
      base += below ? 1 : 0;
      if (!below && b < hi) thr = b;
    }
    float bf;
    std::memcpy(&bf, &base, 4);
    out[e] = make_float2(thr, bf);
  }
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
  const bool quantizes = qp && mode != QuantMode::kRotateOnly && mode != QuantMode::kRotateBf16;
  if (quantizes && mode != QuantMode::kDecoded && a.qp.J <= kHostTableHalf) {
    host_table(a.qp, a.htbl);
    a.host_tbl = 1;
  }
  a.jf = a.qp.J;
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
  // Full-range decision table (2-, 3- and 4-bit codes, one pass): every bucket |t'| <= 2^k (1 + 1e-6)
  // reaches, 2^(k+1) + 4 entries.  Filling it costs each workgroup a few table writes per thread,
  // and it saves one clamp per coordinate, so it pays once a workgroup runs about 8 token groups
  // (estimated with six resident waves per SIMD).  Measured on MI355X: 4608 x 3072 (2 to 3 groups
  // per workgroup) 12.2 us clamped against 13.3 us full; 9216 x 12288 (18 groups) 63.7 against 61.8.
  {
    const int waves = (best_threads + 63) / 64;
    const int64_t resident = static_cast<int64_t>(device_cus()) * std::max(1, 24 / waves);
    const int64_t groups = (n + a.tg - 1) / a.tg;
    a.full = (quantizes && mode != QuantMode::kDecoded && a.qp.bits <= 4 && a.passes == 1 &&
              groups >= 8 * resident) ? 1 : 0;
    if (a.full) a.jf = static_cast<int32_t>(a.qp.scale) + 2;
    // Pipelined loop (one barrier per group, double LDS for the staged rows and partials): it pays
    // where a barrier holds many waves and each workgroup runs several groups.  Measured on MI355X:
    // 9216 x 12288 (12 waves, 18 groups per workgroup) 63.2 -> 60.2 us, 32760 x 8960 (9 waves, 64)
    // 199 -> 188 us; 4608 x 3072 (3 waves, 2 to 3 groups) 11.84 -> 11.97 us and 32760 x 1536
    // (3 waves, 8 groups) 32.95 -> 33.47 us, so those keep two barriers on one buffer.
    a.pipe = (quantizes && mode != QuantMode::kDecoded && a.passes == 1 && waves >= 6 && groups >= 2 * resident) ? 1 : 0;
  }
  // tid / lpt = (tid * magic) >> 32, exact for tid < 1024 (magic = ceil(2^32 / lpt))
  a.div_magic = static_cast<uint32_t>(((uint64_t(1) << 32) + static_cast<uint64_t>(a.lpt) - 1) / static_cast<uint64_t>(a.lpt));
  // norm partials: one per wave when a workgroup holds one token (idle lanes add zeros), else one
  // per aligned power-of-two lane segment inside the token
  if (a.tg == 1) {
    a.seg = 64;
    a.nseg = (a.lpt + 63) / 64;
  } else {
    int seg = 1;
    while (seg < 64 && (a.lpt % (seg * 2)) == 0) seg *= 2;
    a.seg = seg;
    a.nseg = a.lpt / seg;
  }
  a.seg_lev = __builtin_ctz(static_cast<unsigned>(a.seg));
  a.row_reduce = (a.lpt % 16 == 0 && a.nseg <= kNP) ? 1 : 0;
  a.part_stride = static_cast<uint32_t>(std::max(a.nseg, kNP));
  const float rsqrt_h = 1.0f / __builtin_sqrtf(static_cast<float>(rot.block));
  const bool rotate = mode == QuantMode::kRotateOnly || mode == QuantMode::kRotateBf16;
  a.inv_scale = rotate ? rsqrt_h : static_cast<float>(static_cast<double>(a.qp.scale) /
                                                                                 std::sqrt(static_cast<double>(rot.block)));
  // LDS: staged rows [nbuf][tg][ceil(d / 128) x 256 bytes], decision table, partial sums [nbuf][tg][part_stride]
  const int nbuf = a.pipe ? 2 : 1;
  a.row_lds = static_cast<uint32_t>((rot.d + 127) / 128) * kGroupBytes;
  size_t lds = nbuf * static_cast<size_t>(a.tg) * a.row_lds;
  a.tbl_off = static_cast<uint32_t>(lds);
  lds = align16(lds + sizeof(float2) * 2 * a.jf);
  a.part_off = static_cast<uint32_t>(lds);
  lds = align16(lds + nbuf * sizeof(float) * a.tg * a.part_stride);
  a.rsqrt_h = rsqrt_h;
  if ((a.passes > 1 && a.perm) || rot.block > 1024) {  // fp32 rows: later passes' gathers, cross-wave stages
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
    switch (rot.block) {
      case 64: e = launch_block<64>(mode, bits, c, best_threads, lds, stream); break;
      case 128: e = launch_block<128>(mode, bits, c, best_threads, lds, stream); break;
      case 256: e = launch_block<256>(mode, bits, c, best_threads, lds, stream); break;
      case 512: e = launch_block<512>(mode, bits, c, best_threads, lds, stream); break;
      case 1024: e = launch_block<1024>(mode, bits, c, best_threads, lds, stream); break;
      case 2048: e = launch_block<2048>(mode, bits, c, best_threads, lds, stream); break;
      default: e = launch_block<4096>(mode, bits, c, best_threads, lds, stream); break;
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

