// C ABI of liborbq (declared and documented in include/orbq.h): argument checks on the host,
// then asynchronous launches of the rpbh_quantize and lut_gemm kernels.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <vector>

#include "../../include/orbq.h"
#include "internal.h"

#define ORBQ_API extern "C" __attribute__((visibility("default")))

namespace {

thread_local char g_last_error[512] = "";

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_last_error[0] = '\0';
  return ORBQ_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool supported_bits(int b) { return b == 2 || b == 3 || b == 4 || b == 6; }

int check_codebook(const orbq_codebook* cb, int64_t d, const char* what) {
  if (!cb) return fail(ORBQ_ERR_INVALID_ARG, "%s: codebook is NULL", what);
  if (!cb->centroids) return fail(ORBQ_ERR_INVALID_ARG, "%s: codebook centroids are NULL", what);
  if (!supported_bits(cb->bits)) return fail(ORBQ_ERR_UNSUPPORTED, "%s: codebook bits %d not in {2,3,4,6}", what, cb->bits);
  if (d >= 0 && cb->d != d) return fail(ORBQ_ERR_INVALID_ARG, "%s: codebook d=%d but d=%lld", what, cb->d, (long long)d);
  const int n = 1 << cb->bits;
  for (int k = 0; k < n; ++k) {
    if (!std::isfinite(cb->centroids[k])) return fail(ORBQ_ERR_CODEBOOK, "%s: centroid %d not finite", what, k);
    if (k && !(cb->centroids[k] > cb->centroids[k - 1]))
      return fail(ORBQ_ERR_CODEBOOK, "%s: centroids not strictly ascending at %d", what, k);
    if (cb->centroids[n - 1 - k] != -cb->centroids[k])
      return fail(ORBQ_ERR_CODEBOOK, "%s: centroids not antisymmetric at %d", what, k);
  }
  return ORBQ_OK;
}

int check_rot(const orbq_rpbh* rot, int64_t d, const char* what) {
  if (!rot) return fail(ORBQ_ERR_INVALID_ARG, "%s: rotation is NULL", what);
  if (!rot->signs) return fail(ORBQ_ERR_INVALID_ARG, "%s: rotation signs are NULL", what);
  if (rot->d != d) return fail(ORBQ_ERR_INVALID_ARG, "%s: rotation d=%d but d=%lld", what, rot->d, (long long)d);
  if (rot->block < 64 || rot->block > 4096 || (rot->block & (rot->block - 1)))
    return fail(ORBQ_ERR_UNSUPPORTED, "%s: block %d not a power of two in [64, 4096]", what, rot->block);
  if (d % rot->block) return fail(ORBQ_ERR_INVALID_ARG, "%s: d=%lld not a multiple of block %d", what, (long long)d, rot->block);
  if (rot->passes < 0 || rot->passes > 3)
    return fail(ORBQ_ERR_UNSUPPORTED, "%s: %d composed passes (0..3 supported)", what, rot->passes);
  if (rot->passes > 1 && rot->block > 1024)
    return fail(ORBQ_ERR_UNSUPPORTED, "%s: composed passes with blocks above 1024", what);
  if ((rot->perm && !aligned(rot->perm, 16)) || !aligned(rot->signs, 16))
    return fail(ORBQ_ERR_ALIGNMENT, "%s: rotation arrays must be 16-byte aligned", what);
  return ORBQ_OK;
}

int check_dim(int64_t d, const char* what) {
  if (d <= 0) return fail(ORBQ_ERR_INVALID_ARG, "%s: d=%lld must be positive", what, (long long)d);
  if (d > 16384) return fail(ORBQ_ERR_UNSUPPORTED, "%s: d=%lld above 16384", what, (long long)d);
  return ORBQ_OK;
}

int quant_params(const orbq_codebook* cb, orbq::QuantParams* qp, const char* what) {
  if (orbq::build_quant_params(cb->centroids, cb->bits, qp))
    return fail(ORBQ_ERR_CODEBOOK,
                "%s: no power-of-two scale 2^k separates the decision thresholds (at most one per unit of t * 2^k; "
                "2^k <= 1024 for codes of 4 bits or fewer)",
                what);
  return ORBQ_OK;
}

int hip_status(int e, const char* what) {
  if (e != hipSuccess) return fail(ORBQ_ERR_HIP, "%s: %s", what, hipGetErrorString(static_cast<hipError_t>(e)));
  return ok();
}

// shared by orbq_rpbh_quantize and orbq_fold_weights
int quantize_rows(orbq::QuantMode mode, const void* X, int64_t n, int64_t d, int64_t ld, const orbq_rpbh* rot,
                  const orbq_codebook* cb, float eps, uint8_t* codes, void* norms, size_t norm_align,
                  void* stream, const char* what) {
  int s;
  if ((s = check_dim(d, what))) return s;
  if (n < 0) return fail(ORBQ_ERR_INVALID_ARG, "%s: n=%lld negative", what, (long long)n);
  if (ld < d) return fail(ORBQ_ERR_INVALID_ARG, "%s: ld=%lld < d=%lld", what, (long long)ld, (long long)d);
  if ((s = check_rot(rot, d, what))) return s;
  if ((s = check_codebook(cb, d, what))) return s;
  if (!(eps >= 0.0f) || !std::isfinite(eps)) return fail(ORBQ_ERR_INVALID_ARG, "%s: eps must be finite and >= 0", what);
  if (n == 0) return ok();
  if (!X || !codes || !norms) return fail(ORBQ_ERR_INVALID_ARG, "%s: NULL buffer", what);
  if (!aligned(X, 16) || (ld * 2) % 16) return fail(ORBQ_ERR_ALIGNMENT, "%s: input must be 16-byte aligned with a 16-byte pitch", what);
  if (!aligned(codes, 16)) return fail(ORBQ_ERR_ALIGNMENT, "%s: codes must be 16-byte aligned", what);
  if (!aligned(norms, norm_align)) return fail(ORBQ_ERR_ALIGNMENT, "%s: norms misaligned", what);
  orbq::QuantParams qp;
  if ((s = quant_params(cb, &qp, what))) return s;
  if (mode == orbq::QuantMode::kDecoded) {  // the bf16 centroid of each sign-magnitude code, as the product decodes it
    orbq::DecodeParams dp;
    orbq::build_decode_params(cb->centroids, cb->bits, &dp);
    const int half = 1 << (cb->bits - 1);
    for (int q = 0; q < 2 * half; ++q)
      qp.vals[q] = static_cast<uint16_t>(dp.mag[q & (half - 1)] | ((q & half) ? 0x8000u : 0u));
  }
  orbq::RotArgs ra{rot->d, rot->block, rot->perm, rot->signs, rot->passes < 1 ? 1 : rot->passes};
  const int e = orbq::launch_rpbh_quantize(mode, static_cast<const uint16_t*>(X), n, ld, ra, &qp, eps, codes, norms,
                                           nullptr, static_cast<hipStream_t>(stream));
  return hip_status(e, what);
}

}  // namespace

ORBQ_API int orbq_codebook_lloyd_max(int32_t d, int32_t bits, float* centroids_out) {
  if (!centroids_out) return fail(ORBQ_ERR_INVALID_ARG, "orbq_codebook_lloyd_max: output is NULL");
  if (d < 3 || bits < 1 || bits > 8) return fail(ORBQ_ERR_INVALID_ARG, "orbq_codebook_lloyd_max: need d >= 3, 1 <= bits <= 8");
  std::vector<double> c(1u << bits);
  if (orbq::lloyd_max_host(d, bits, c.data())) return fail(ORBQ_ERR_INVALID_ARG, "orbq_codebook_lloyd_max: no convergence");
  for (size_t k = 0; k < c.size(); ++k) centroids_out[k] = static_cast<float>(c[k]);
  return ok();
}

ORBQ_API int orbq_rpbh_validate(int32_t d, int32_t block, const int32_t* perm, const int8_t* signs) {
  const char* what = "orbq_rpbh_validate";
  if (!signs) return fail(ORBQ_ERR_INVALID_ARG, "%s: NULL signs", what);
  int s;
  if ((s = check_dim(d, what))) return s;
  if (block < 64 || block > 4096 || (block & (block - 1)))
    return fail(ORBQ_ERR_UNSUPPORTED, "%s: block %d not a power of two in [64, 4096]", what, block);
  if (d % block) return fail(ORBQ_ERR_INVALID_ARG, "%s: d not a multiple of block", what);
  std::vector<unsigned char> seen(d, 0);
  for (int j = 0; j < d; ++j) {
    if (perm) {
      if (perm[j] < 0 || perm[j] >= d || seen[perm[j]])
        return fail(ORBQ_ERR_INVALID_ARG, "%s: perm is not a permutation (entry %d)", what, j);
      seen[perm[j]] = 1;
    }
    if (signs[j] != 1 && signs[j] != -1) return fail(ORBQ_ERR_INVALID_ARG, "%s: sign %d is not +-1", what, j);
  }
  return ok();
}

ORBQ_API int orbq_codebook_validate(const orbq_codebook* cb) {
  int s = check_codebook(cb, -1, "orbq_codebook_validate");
  if (s) return s;
  orbq::QuantParams qp;
  if ((s = quant_params(cb, &qp, "orbq_codebook_validate"))) return s;
  return ok();
}

ORBQ_API size_t orbq_codes_row_bytes(int64_t d, int32_t bits) {
  if (d <= 0 || bits <= 0 || (d * bits) % 8) return 0;
  return static_cast<size_t>(d * bits / 8);
}

ORBQ_API int orbq_fold_weights(const void* W, int64_t m, int64_t d, int64_t ldw, const orbq_rpbh* rot,
                               const orbq_codebook* cb_w, float eps, uint8_t* w_codes, void* w_norms, void* stream) {
  return quantize_rows(orbq::QuantMode::kWeights, W, m, d, ldw, rot, cb_w, eps, w_codes, w_norms, 2, stream,
                       "orbq_fold_weights");
}

ORBQ_API int orbq_rpbh_quantize(const void* X, int64_t n, int64_t d, int64_t ldx, const orbq_rpbh* rot,
                                const orbq_codebook* cb_a, float eps, uint8_t* x_codes, float* x_norms, void* stream) {
  return quantize_rows(orbq::QuantMode::kActivations, X, n, d, ldx, rot, cb_a, eps, x_codes, x_norms, 4, stream,
                       "orbq_rpbh_quantize");
}

namespace {

int gemm_checks(const uint8_t* x_codes, const float* x_norms, const orbq_codebook* cb_a, const uint8_t* w_codes,
                const void* w_norms, const orbq_codebook* cb_w, int64_t n, int64_t m, int64_t d, void* Y,
                orbq_dtype y_type, int64_t ldy, const char* what, bool check_x) {
  int s;
  if ((s = check_dim(d, what))) return s;
  if (d % 64) return fail(ORBQ_ERR_UNSUPPORTED, "%s: d=%lld not a multiple of 64", what, (long long)d);
  if (n < 0 || m < 0) return fail(ORBQ_ERR_INVALID_ARG, "%s: negative n or m", what);
  if (ldy < m) return fail(ORBQ_ERR_INVALID_ARG, "%s: ldy=%lld < m=%lld", what, (long long)ldy, (long long)m);
  if (y_type != ORBQ_F32 && y_type != ORBQ_BF16) return fail(ORBQ_ERR_INVALID_ARG, "%s: bad y_type", what);
  if ((s = check_codebook(cb_a, d, what))) return s;
  if ((s = check_codebook(cb_w, d, what))) return s;
  if ((cb_a->bits == 3) != (cb_w->bits == 3))
    return fail(ORBQ_ERR_UNSUPPORTED, "%s: 3-bit codes pair only with 3-bit codes (W3A3)", what);
  if (n == 0 || m == 0) return ORBQ_OK;
  if ((check_x && (!x_codes || !x_norms)) || !w_codes || !w_norms || !Y)
    return fail(ORBQ_ERR_INVALID_ARG, "%s: NULL buffer", what);
  if ((check_x && (!aligned(x_codes, 16) || !aligned(x_norms, 4))) || !aligned(w_codes, 16) || !aligned(w_norms, 2))
    return fail(ORBQ_ERR_ALIGNMENT, "%s: codes must be 16-byte aligned, norms naturally aligned", what);
  const int64_t esz = y_type == ORBQ_F32 ? 4 : 2;
  if (!aligned(Y, 16) || (ldy * esz) % 16) return fail(ORBQ_ERR_ALIGNMENT, "%s: Y must be 16-byte aligned with a 16-byte pitch", what);
  return ORBQ_OK;
}

int gemm_launch(const uint8_t* x_codes, const float* x_norms, const orbq_codebook* cb_a, const uint8_t* w_codes,
                const void* w_norms, const orbq_codebook* cb_w, int64_t n, int64_t m, int64_t d, void* Y,
                orbq_dtype y_type, int64_t ldy, int act, void* stream, const char* what) {
  orbq::DecodeParams da, dw;
  orbq::build_decode_params(cb_a->centroids, cb_a->bits, &da);
  orbq::build_decode_params(cb_w->centroids, cb_w->bits, &dw);
  const int e = orbq::launch_lut_gemm(x_codes, x_norms, da, w_codes, static_cast<const uint16_t*>(w_norms), dw, n, m, d,
                                      Y, y_type == ORBQ_BF16, ldy, act, static_cast<hipStream_t>(stream));
  return hip_status(e, what);
}

bool valid_act(int act) { return act == ORBQ_ACT_NONE || act == ORBQ_ACT_GELU_TANH || act == ORBQ_ACT_GELU_ERF; }

// The layer's activation operand in its workspace: packed codes, or for 6-bit activations the
// codes' bf16 centroids (16 bits per coordinate), which the product stages without decoding.
// The product decodes each activation row once per column tile of 192 or 256 weight rows, while
// the centroids cost rpbh_quantize 1.25 more bytes per coordinate to write and the product as
// many more to read; measured on MI355X the centroids win from about 7 column tiles on (W4A6:
// m = 8960 takes 1.0 ms against 1.8 ms, m = 1536 1.22 ms against 1.21 ms).  The workspace is
// sized for the centroids either way.
constexpr int32_t kDecodedBits = 6;
constexpr int64_t kDecodedMinM = 2048;

size_t ws_codes_bytes(int64_t n, int64_t d, int32_t bits) {
  const int64_t row = bits == kDecodedBits ? d * 2 : d * bits / 8;
  return (static_cast<size_t>(n) * static_cast<size_t>(row) + 255) & ~size_t(255);
}

}  // namespace

ORBQ_API int orbq_lut_gemm_act(const uint8_t* x_codes, const float* x_norms, const orbq_codebook* cb_a,
                               const uint8_t* w_codes, const void* w_norms, const orbq_codebook* cb_w, int64_t n,
                               int64_t m, int64_t d, orbq_activation act, void* Y, orbq_dtype y_type, int64_t ldy,
                               void* stream) {
  const char* what = "orbq_lut_gemm_act";
  if (!valid_act(act)) return fail(ORBQ_ERR_INVALID_ARG, "%s: unknown activation %d", what, static_cast<int>(act));
  int s = gemm_checks(x_codes, x_norms, cb_a, w_codes, w_norms, cb_w, n, m, d, Y, y_type, ldy, what, true);
  if (s) return s;
  if (n == 0 || m == 0) return ok();
  return gemm_launch(x_codes, x_norms, cb_a, w_codes, w_norms, cb_w, n, m, d, Y, y_type, ldy, act, stream, what);
}

ORBQ_API int orbq_lut_gemm(const uint8_t* x_codes, const float* x_norms, const orbq_codebook* cb_a,
                           const uint8_t* w_codes, const void* w_norms, const orbq_codebook* cb_w, int64_t n, int64_t m,
                           int64_t d, void* Y, orbq_dtype y_type, int64_t ldy, void* stream) {
  const char* what = "orbq_lut_gemm";
  int s = gemm_checks(x_codes, x_norms, cb_a, w_codes, w_norms, cb_w, n, m, d, Y, y_type, ldy, what, true);
  if (s) return s;
  if (n == 0 || m == 0) return ok();
  return gemm_launch(x_codes, x_norms, cb_a, w_codes, w_norms, cb_w, n, m, d, Y, y_type, ldy, ORBQ_ACT_NONE, stream,
                     what);
}

ORBQ_API size_t orbq_linear_workspace_bytes(int64_t n, int64_t d, int32_t bits_a) {
  if (n < 0 || d <= 0 || !supported_bits(bits_a)) return 0;
  return ws_codes_bytes(n, d, bits_a) + static_cast<size_t>(n) * sizeof(float);
}

namespace {

// the layer's argument checks, workspace aside
int linear_args(const orbq_rpbh* rot, const orbq_codebook* cb_a, const uint8_t* w_codes, const void* w_norms,
                const orbq_codebook* cb_w, int64_t n, int64_t m, int64_t d, int64_t ldx, void* Y, orbq_dtype y_type,
                int64_t ldy, const char* what) {
  int s = gemm_checks(nullptr, nullptr, cb_a, w_codes, w_norms, cb_w, n, m, d, Y, y_type, ldy, what, false);
  if (s) return s;
  if ((s = check_rot(rot, d, what))) return s;
  if (ldx < d) return fail(ORBQ_ERR_INVALID_ARG, "%s: ldx < d", what);
  return ORBQ_OK;
}

int linear_impl(const void* X, int64_t n, int64_t d, int64_t ldx, const orbq_rpbh* rot, const orbq_codebook* cb_a,
                float eps, const uint8_t* w_codes, const void* w_norms, const orbq_codebook* cb_w, int64_t m,
                void* workspace, size_t ws_bytes, int act, void* Y, orbq_dtype y_type, int64_t ldy, void* stream,
                const char* what) {
  int s = linear_args(rot, cb_a, w_codes, w_norms, cb_w, n, m, d, ldx, Y, y_type, ldy, what);
  if (s) return s;
  if (n == 0 || m == 0) return ok();
  const size_t need = orbq_linear_workspace_bytes(n, d, cb_a->bits);
  if (!workspace || ws_bytes < need)
    return fail(ORBQ_ERR_WORKSPACE, "%s: workspace %zu bytes < %zu needed", what, ws_bytes, need);
  if (!aligned(workspace, 256)) return fail(ORBQ_ERR_ALIGNMENT, "%s: workspace must be 256-byte aligned", what);
  uint8_t* codes = static_cast<uint8_t*>(workspace);
  float* norms = reinterpret_cast<float*>(codes + ws_codes_bytes(n, d, cb_a->bits));
  if (cb_a->bits == kDecodedBits && m >= kDecodedMinM) {
    // 6-bit activations: rpbh_quantize writes the bf16 centroids, the product stages them directly
    s = quantize_rows(orbq::QuantMode::kDecoded, X, n, d, ldx, rot, cb_a, eps, codes, norms, 4, stream, what);
    if (s) return s;
    orbq::DecodeParams da{}, dw;
    da.bits = 16;
    orbq::build_decode_params(cb_w->centroids, cb_w->bits, &dw);
    const int e = orbq::launch_lut_gemm(codes, norms, da, w_codes, static_cast<const uint16_t*>(w_norms), dw, n, m, d,
                                        Y, y_type == ORBQ_BF16, ldy, act, static_cast<hipStream_t>(stream));
    return hip_status(e, what);
  }
  s = quantize_rows(orbq::QuantMode::kActivations, X, n, d, ldx, rot, cb_a, eps, codes, norms, 4, stream, what);
  if (s) return s;
  return gemm_launch(codes, norms, cb_a, w_codes, w_norms, cb_w, n, m, d, Y, y_type, ldy, act, stream, what);
}

}  // namespace

ORBQ_API int orbq_linear(const void* X, int64_t n, int64_t d, int64_t ldx, const orbq_rpbh* rot,
                         const orbq_codebook* cb_a, float eps, const uint8_t* w_codes, const void* w_norms,
                         const orbq_codebook* cb_w, int64_t m, void* workspace, size_t ws_bytes, void* Y,
                         orbq_dtype y_type, int64_t ldy, void* stream) {
  return linear_impl(X, n, d, ldx, rot, cb_a, eps, w_codes, w_norms, cb_w, m, workspace, ws_bytes, ORBQ_ACT_NONE, Y,
                     y_type, ldy, stream, "orbq_linear");
}

ORBQ_API int orbq_linear_act(const void* X, int64_t n, int64_t d, int64_t ldx, const orbq_rpbh* rot,
                             const orbq_codebook* cb_a, float eps, const uint8_t* w_codes, const void* w_norms,
                             const orbq_codebook* cb_w, int64_t m, void* workspace, size_t ws_bytes,
                             orbq_activation act, void* Y, orbq_dtype y_type, int64_t ldy, void* stream) {
  const char* what = "orbq_linear_act";
  if (!valid_act(act)) return fail(ORBQ_ERR_INVALID_ARG, "%s: unknown activation %d", what, static_cast<int>(act));
  return linear_impl(X, n, d, ldx, rot, cb_a, eps, w_codes, w_norms, cb_w, m, workspace, ws_bytes, act, Y, y_type,
                     ldy, stream, what);
}

ORBQ_API int orbq_linear_noalloc(const void* X, int64_t n, int64_t d, int64_t ldx, const orbq_rpbh* rot,
                                 const orbq_codebook* cb_a, float eps, const uint8_t* w_codes, const void* w_norms,
                                 const orbq_codebook* cb_w, int64_t m, orbq_activation act, void* Y,
                                 orbq_dtype y_type, int64_t ldy, void* stream) {
  const char* what = "orbq_linear_noalloc";
  if (!valid_act(act)) return fail(ORBQ_ERR_INVALID_ARG, "%s: unknown activation %d", what, static_cast<int>(act));
  // every argument is checked before the scratch is looked up (the lookup is a device call)
  int s = linear_args(rot, cb_a, w_codes, w_norms, cb_w, n, m, d, ldx, Y, y_type, ldy, what);
  if (s) return s;
  const size_t need = orbq_linear_workspace_bytes(n, d, cb_a->bits);
  if (need > ORBQ_NOALLOC_SCRATCH_BYTES)
    return fail(ORBQ_ERR_WORKSPACE, "%s: %lld x %lld at %d bits needs %zu bytes of workspace, above the %u-byte "
                "fixed scratch (use orbq_linear_act with a caller workspace)",
                what, (long long)n, (long long)d, cb_a->bits, need, ORBQ_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if (n > 0 && m > 0) {
    const int e = orbq::noalloc_scratch(&ws);
    if (e != hipSuccess) return hip_status(e, what);
  }
  return linear_impl(X, n, d, ldx, rot, cb_a, eps, w_codes, w_norms, cb_w, m, ws, ORBQ_NOALLOC_SCRATCH_BYTES, act, Y,
                     y_type, ldy, stream, what);
}

namespace orbq {
// a16_gemm.hip: the weight-only product with the rotation inside it (one RPBH pass with a
// permutation, h = 64 or 128); hipErrorNotSupported when that form does not apply
int launch_a16_gemm_rot(const uint16_t* X, int64_t ldx, int nt, int64_t d, const int32_t* perm, const int8_t* signs,
                        int32_t h, const uint8_t* w_codes, const uint16_t* w_norms, const DecodeParams& dw, int64_t m,
                        void* Y, int y_bf16, int64_t ldy, hipStream_t stream);
}  // namespace orbq

namespace {

constexpr int64_t kA16Tokens = 16;  // tokens per weight-only launch

size_t round256(size_t x) { return (x + 255) & ~size_t(255); }

// [x' bf16 nt x d][norms fp32 nt]: the rotated tokens of one 16-token chunk (m does not enter)
size_t a16_ws_bytes(int64_t n, int64_t d, int64_t /*m*/) {
  const int64_t nt = std::min<int64_t>(n, kA16Tokens);
  return round256(static_cast<size_t>(nt * d * 2)) + round256(static_cast<size_t>(nt * 4));
}

}  // namespace

ORBQ_API size_t orbq_linear_a16_workspace_bytes(int64_t n, int64_t d, int64_t m) {
  if (n < 0 || d <= 0 || d % 128 || m < 0) return 0;
  return a16_ws_bytes(std::max<int64_t>(n, 1), d, std::max<int64_t>(m, 1));
}

ORBQ_API int orbq_linear_a16(const void* X, int64_t n, int64_t d, int64_t ldx, const orbq_rpbh* rot,
                             const uint8_t* w_codes, const void* w_norms, const orbq_codebook* cb_w, int64_t m,
                             void* workspace, size_t ws_bytes, void* Y, orbq_dtype y_type, int64_t ldy,
                             void* stream) {
  const char* what = "orbq_linear_a16";
  int s;
  if ((s = check_dim(d, what))) return s;
  if (d % 128) return fail(ORBQ_ERR_UNSUPPORTED, "%s: d=%lld not a multiple of 128", what, (long long)d);
  if ((s = check_rot(rot, d, what))) return s;
  if ((s = check_codebook(cb_w, d, what))) return s;
  if (n < 0 || m < 0 || ldx < d || ldy < m) return fail(ORBQ_ERR_INVALID_ARG, "%s: bad n, m, ldx or ldy", what);
  if (y_type != ORBQ_F32 && y_type != ORBQ_BF16) return fail(ORBQ_ERR_INVALID_ARG, "%s: bad y_type", what);
  if (n == 0 || m == 0) return ok();
  if (!X || !w_codes || !w_norms || !Y) return fail(ORBQ_ERR_INVALID_ARG, "%s: NULL buffer", what);
  if (!aligned(X, 16) || (ldx * 2) % 16 || !aligned(w_codes, 16) || !aligned(w_norms, 2) ||
      !aligned(Y, y_type == ORBQ_BF16 ? 2 : 4))
    return fail(ORBQ_ERR_ALIGNMENT, "%s: misaligned buffer", what);
  const size_t need = a16_ws_bytes(n, d, m);
  if (!workspace || ws_bytes < need)
    return fail(ORBQ_ERR_WORKSPACE, "%s: workspace %zu bytes < %zu needed", what, ws_bytes, need);
  if (!aligned(workspace, 256)) return fail(ORBQ_ERR_ALIGNMENT, "%s: workspace must be 256-byte aligned", what);
  orbq::DecodeParams dw;
  orbq::build_decode_params(cb_w->centroids, cb_w->bits, &dw);
  const int64_t nt_max = std::min<int64_t>(n, kA16Tokens);
  uint16_t* xr = static_cast<uint16_t*>(workspace);
  float* norms = reinterpret_cast<float*>(static_cast<unsigned char*>(workspace) + round256(static_cast<size_t>(nt_max * d * 2)));
  orbq::RotArgs ra{rot->d, rot->block, rot->perm, rot->signs, rot->passes < 1 ? 1 : rot->passes};
  const int64_t esz = y_type == ORBQ_BF16 ? 2 : 4;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  for (int64_t t0 = 0; t0 < n; t0 += kA16Tokens) {
    const int nt = static_cast<int>(std::min<int64_t>(kA16Tokens, n - t0));
    const uint16_t* Xc = static_cast<const uint16_t*>(X) + t0 * ldx;
    void* Yc = static_cast<unsigned char*>(Y) + t0 * ldy * esz;
    // one RPBH pass with a permutation and h <= 128: the product rotates its own K splits
    int e = ra.passes == 1 ? orbq::launch_a16_gemm_rot(Xc, ldx, nt, d, ra.perm, ra.signs, ra.block, w_codes,
                                                         static_cast<const uint16_t*>(w_norms), dw, m, Yc,
                                                         y_type == ORBQ_BF16, ldy, st)
                           : static_cast<int>(hipErrorNotSupported);
    if (e == hipErrorNotSupported) {
      e = orbq::launch_rpbh_quantize(orbq::QuantMode::kRotateBf16, Xc, nt, ldx, ra, nullptr, 0.0f, nullptr, norms,
                                     reinterpret_cast<float*>(xr), st);
      if (e == hipSuccess)
        e = orbq::launch_a16_gemm(xr, nt, d, w_codes, static_cast<const uint16_t*>(w_norms), dw, m, Yc,
                                  y_type == ORBQ_BF16, ldy, st);
    }
    if (e != hipSuccess) return hip_status(e, what);
  }
  return ok();
}

ORBQ_API int orbq_rpbh_flatness(const void* X, int64_t n, int64_t d, int64_t ldx, float* rho3, float* rhoinf,
                                void* stream) {
  const char* what = "orbq_rpbh_flatness";
  int s;
  if ((s = check_dim(d, what))) return s;
  if (d % 8) return fail(ORBQ_ERR_UNSUPPORTED, "%s: d=%lld not a multiple of 8", what, (long long)d);
  if (n < 0 || ldx < d) return fail(ORBQ_ERR_INVALID_ARG, "%s: bad n or ldx", what);
  if (n == 0) return ok();
  if (!X || !rho3 || !rhoinf) return fail(ORBQ_ERR_INVALID_ARG, "%s: NULL buffer", what);
  if (!aligned(X, 16) || (ldx * 2) % 16 || !aligned(rho3, 4) || !aligned(rhoinf, 4))
    return fail(ORBQ_ERR_ALIGNMENT, "%s: input must be 16-byte aligned with a 16-byte pitch", what);
  const int e = orbq::launch_flatness(static_cast<const uint16_t*>(X), n, static_cast<int32_t>(d), ldx, rho3, rhoinf,
                                      static_cast<hipStream_t>(stream));
  return hip_status(e, what);
}

ORBQ_API int32_t orbq_rht_passes(float rho3, float rhoinf, int32_t d, int32_t vector_quantization) {
  if (!(rho3 >= 0.0f) || !(rhoinf >= 0.0f) || d < 2) return ORBQ_ERR_INVALID_ARG;
  // a Gaussian row has rho3 -> E|g|^3 = 2 sqrt(2/pi) and rhoinf ~ sqrt(2 ln(2d))
  const double g3 = 2.0 * std::sqrt(2.0 / 3.14159265358979323846);
  const double ginf = std::sqrt(2.0 * std::log(2.0 * d));
  if (!vector_quantization) return rho3 <= 2.0 * g3 ? 1 : 2;
  if (rhoinf <= ginf) return 1;
  return rhoinf <= 2.0 * ginf ? 2 : 3;
}

ORBQ_API const char* orbq_status_string(int status) {
  switch (status) {
    case ORBQ_OK: return "ORBQ_OK";
    case ORBQ_ERR_INVALID_ARG: return "ORBQ_ERR_INVALID_ARG";
    case ORBQ_ERR_UNSUPPORTED: return "ORBQ_ERR_UNSUPPORTED";
    case ORBQ_ERR_ALIGNMENT: return "ORBQ_ERR_ALIGNMENT";
    case ORBQ_ERR_WORKSPACE: return "ORBQ_ERR_WORKSPACE";
    case ORBQ_ERR_HIP: return "ORBQ_ERR_HIP";
    case ORBQ_ERR_CODEBOOK: return "ORBQ_ERR_CODEBOOK";
    default: return "ORBQ_ERR_UNKNOWN";
  }
}

ORBQ_API const char* orbq_last_error(void) { return g_last_error; }

ORBQ_API int orbq_test_rotate(const void* X, int64_t n, int64_t d, int64_t ldx, const orbq_rpbh* rot, float* x_rot,
                              float* x_norms, void* stream) {
  const char* what = "orbq_test_rotate";
  int s;
  if ((s = check_dim(d, what))) return s;
  if ((s = check_rot(rot, d, what))) return s;
  if (n < 0 || ldx < d) return fail(ORBQ_ERR_INVALID_ARG, "%s: bad n or ldx", what);
  if (n == 0) return ok();
  if (!X || !x_rot || !x_norms) return fail(ORBQ_ERR_INVALID_ARG, "%s: NULL buffer", what);
  if (!aligned(X, 16) || (ldx * 2) % 16 || !aligned(x_rot, 16))
    return fail(ORBQ_ERR_ALIGNMENT, "%s: misaligned buffer", what);
  orbq::RotArgs ra{rot->d, rot->block, rot->perm, rot->signs, rot->passes < 1 ? 1 : rot->passes};
  const int e = orbq::launch_rpbh_quantize(orbq::QuantMode::kRotateOnly, static_cast<const uint16_t*>(X), n, ldx, ra,
                                           nullptr, 0.0f, nullptr, x_norms, x_rot, static_cast<hipStream_t>(stream));
  return hip_status(e, what);
}

ORBQ_API int orbq_test_quantize_t(const float* t, int64_t count, const orbq_codebook* cb, uint8_t* codes, void* stream) {
  const char* what = "orbq_test_quantize_t";
  int s = check_codebook(cb, -1, what);
  if (s) return s;
  if (count < 0) return fail(ORBQ_ERR_INVALID_ARG, "%s: negative count", what);
  if (count == 0) return ok();
  if (!t || !codes) return fail(ORBQ_ERR_INVALID_ARG, "%s: NULL buffer", what);
  orbq::QuantParams qp;
  if ((s = quant_params(cb, &qp, what))) return s;
  return hip_status(orbq::launch_quantize_t(t, count, qp, codes, static_cast<hipStream_t>(stream)), what);
}

namespace orbq {
// mfma_probe.hip: `workgroups` x 512 threads, `iters` (a multiple of 4) MFMA steps per
// accumulator; sink receives workgroups * 512 floats
int launch_mfma_probe(int workgroups, int iters, float* sink, hipStream_t stream);
double mfma_probe_flops(int workgroups, int iters);
}  // namespace orbq

ORBQ_API int orbq_test_mfma_rate(int32_t workgroups, int32_t iters, float* sink, double* flops, void* stream) {
  const char* what = "orbq_test_mfma_rate";
  if (workgroups < 1 || workgroups > 65536 || iters < 4 || iters % 4 || iters > (1 << 24))
    return fail(ORBQ_ERR_INVALID_ARG, "%s: workgroups %d or iters %d out of range", what, workgroups, iters);
  if (!sink || !flops) return fail(ORBQ_ERR_INVALID_ARG, "%s: NULL pointer", what);
  if (!aligned(sink, 4)) return fail(ORBQ_ERR_ALIGNMENT, "%s: misaligned sink", what);
  *flops = orbq::mfma_probe_flops(workgroups, iters);
  return hip_status(orbq::launch_mfma_probe(workgroups, iters, sink, static_cast<hipStream_t>(stream)), what);
}
