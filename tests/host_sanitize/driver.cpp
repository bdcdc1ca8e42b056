// Host-only exercise of liborbq's C ABI under AddressSanitizer and UndefinedBehaviorSanitizer:
// the codebook builder, the validators, the size helpers and every entry point's argument
// checks (each call below is rejected before any GPU work; the launchers are stubs that abort).
// Prints "ok <checks>" and exits 0 when every status is the documented one.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "../../include/orbq.h"

static int g_checks = 0, g_fail = 0;

static void expect(int got, int want, const char* what) {
  ++g_checks;
  if (got != want) {
    ++g_fail;
    std::printf("FAIL %s: status %d, expected %d (%s)\n", what, got, want, orbq_last_error());
  }
}

int main() {
  // ---- Lloyd-Max codebooks: ascending, antisymmetric, inside (-1, 1)
  const int dims[] = {3, 5, 64, 256, 1536, 3072, 12288};
  for (int d : dims)
    for (int bits = 1; bits <= (d <= 256 ? 8 : 6); ++bits) {
      std::vector<float> c(1u << bits);
      expect(orbq_codebook_lloyd_max(d, bits, c.data()), ORBQ_OK, "lloyd_max");
      for (size_t k = 0; k + 1 < c.size(); ++k) {
        ++g_checks;
        if (!(c[k] < c[k + 1]) || c[k] != -c[c.size() - 1 - k] || !(std::fabs(c[k]) < 1.0f)) {
          ++g_fail;
          std::printf("FAIL codebook d=%d bits=%d at %zu: %.9g %.9g mirror %.9g\n", d, bits, k, c[k], c[k + 1],
                      c[c.size() - 1 - k]);
          break;
        }
      }
      if (bits == 2 || bits == 3 || bits == 4 || bits == 6) {
        orbq_codebook cb{d, bits, c.data()};
        if (d >= 64) expect(orbq_codebook_validate(&cb), ORBQ_OK, "codebook_validate");
      }
    }
  {  // d = 3: f_3 is uniform on [-1, 1], whose Lloyd-Max quantizer is the uniform one
    for (int bits = 1; bits <= 8; ++bits) {
      const int N = 1 << bits;
      std::vector<float> c(N);
      expect(orbq_codebook_lloyd_max(3, bits, c.data()), ORBQ_OK, "lloyd_max d = 3");
      for (int k = 0; k < N; ++k) {
        ++g_checks;
        if (std::fabs(c[k] - ((2.0 * k + 1.0) / N - 1.0)) > 1e-6) {
          ++g_fail;
          std::printf("FAIL uniform codebook d=3 bits=%d k=%d: %.9g\n", bits, k, c[k]);
          break;
        }
      }
    }
  }
  float c4[16];
  expect(orbq_codebook_lloyd_max(2, 4, c4), ORBQ_ERR_INVALID_ARG, "lloyd_max d < 3");
  expect(orbq_codebook_lloyd_max(64, 9, c4), ORBQ_ERR_INVALID_ARG, "lloyd_max bits > 8");
  expect(orbq_codebook_lloyd_max(64, 4, nullptr), ORBQ_ERR_INVALID_ARG, "lloyd_max NULL");
  expect(orbq_codebook_lloyd_max(3072, 4, c4), ORBQ_OK, "lloyd_max 3072 x 4");
  {  // a codebook that is not antisymmetric, one that is not ascending
    float bad[16];
    std::memcpy(bad, c4, sizeof bad);
    bad[3] *= 1.01f;
    orbq_codebook cb{3072, 4, bad};
    expect(orbq_codebook_validate(&cb), ORBQ_ERR_CODEBOOK, "codebook not antisymmetric");
    std::memcpy(bad, c4, sizeof bad);
    std::swap(bad[5], bad[6]);
    std::swap(bad[9], bad[10]);
    expect(orbq_codebook_validate(&cb), ORBQ_ERR_CODEBOOK, "codebook not ascending");
  }

  // ---- rotation validator on host arrays
  const int d = 3072;
  std::vector<int32_t> perm(d);
  std::vector<int8_t> signs(d);
  for (int j = 0; j < d; ++j) {
    perm[j] = (j * 1237 + 11) % d;  // 1237 is prime to 3072: a permutation
    signs[j] = (j * 7 % 3) ? 1 : -1;
  }
  for (int block : {64, 128, 256, 512, 1024})
    expect(orbq_rpbh_validate(d, block, perm.data(), signs.data()), ORBQ_OK, "rpbh_validate");
  expect(orbq_rpbh_validate(d, 128, nullptr, signs.data()), ORBQ_OK, "rpbh_validate identity");
  expect(orbq_rpbh_validate(d, 2048, perm.data(), signs.data()), ORBQ_ERR_INVALID_ARG, "block does not divide d");
  expect(orbq_rpbh_validate(d, 96, perm.data(), signs.data()), ORBQ_ERR_UNSUPPORTED, "block not a power of two");
  expect(orbq_rpbh_validate(d, 8192, perm.data(), signs.data()), ORBQ_ERR_UNSUPPORTED, "block too large");
  expect(orbq_rpbh_validate(d, 128, perm.data(), nullptr), ORBQ_ERR_INVALID_ARG, "NULL signs");
  perm[17] = perm[18];
  expect(orbq_rpbh_validate(d, 128, perm.data(), signs.data()), ORBQ_ERR_INVALID_ARG, "repeated perm entry");
  perm[17] = d;
  expect(orbq_rpbh_validate(d, 128, perm.data(), signs.data()), ORBQ_ERR_INVALID_ARG, "perm entry out of range");
  perm[17] = (17 * 1237 + 11) % d;
  signs[5] = 0;
  expect(orbq_rpbh_validate(d, 128, perm.data(), signs.data()), ORBQ_ERR_INVALID_ARG, "sign not +-1");
  signs[5] = 1;

  // ---- size helpers
  ++g_checks;
  if (orbq_codes_row_bytes(3072, 4) != 1536 || orbq_codes_row_bytes(3072, 3) != 1152 ||
      orbq_codes_row_bytes(3072, 6) != 2304 || orbq_codes_row_bytes(3, 3) != 0 || orbq_codes_row_bytes(-1, 4) != 0) {
    ++g_fail;
    std::printf("FAIL codes_row_bytes\n");
  }
  ++g_checks;
  if (orbq_linear_workspace_bytes(4608, 3072, 4) < 4608u * 1536u + 4608u * 4u || orbq_linear_workspace_bytes(4, 64, 5) != 0) {
    ++g_fail;
    std::printf("FAIL linear_workspace_bytes\n");
  }
  for (int s = -6; s <= 0; ++s) {
    ++g_checks;
    if (!orbq_status_string(s) || !*orbq_status_string(s)) {
      ++g_fail;
      std::printf("FAIL status_string(%d)\n", s);
    }
  }
  ++g_checks;
  if (!orbq_status_string(-99)) {
    ++g_fail;
    std::printf("FAIL status_string(-99)\n");
  }

  // ---- every entry point's argument checks (fake device addresses, aligned; nothing launches)
  orbq_rpbh rot{d, 128, reinterpret_cast<const int32_t*>(0x10000), reinterpret_cast<const int8_t*>(0x20000), 1};
  orbq_codebook cba{d, 4, c4}, cbw{d, 4, c4};
  void* X = reinterpret_cast<void*>(0x100000);
  auto* codes = reinterpret_cast<uint8_t*>(0x200000);
  auto* norms = reinterpret_cast<float*>(0x300000);
  void* Y = reinterpret_cast<void*>(0x400000);
  expect(orbq_rpbh_quantize(nullptr, 16, d, d, &rot, &cba, 1e-8f, codes, norms, nullptr), ORBQ_ERR_INVALID_ARG, "quantize NULL X");
  expect(orbq_rpbh_quantize(X, -1, d, d, &rot, &cba, 1e-8f, codes, norms, nullptr), ORBQ_ERR_INVALID_ARG, "quantize n < 0");
  expect(orbq_rpbh_quantize(X, 16, d, d - 1, &rot, &cba, 1e-8f, codes, norms, nullptr), ORBQ_ERR_INVALID_ARG, "quantize ldx < d");
  expect(orbq_rpbh_quantize(reinterpret_cast<char*>(X) + 2, 16, d, d, &rot, &cba, 1e-8f, codes, norms, nullptr),
         ORBQ_ERR_ALIGNMENT, "quantize misaligned X");
  expect(orbq_rpbh_quantize(X, 16, d, d, nullptr, &cba, 1e-8f, codes, norms, nullptr), ORBQ_ERR_INVALID_ARG, "quantize NULL rot");
  {
    orbq_rpbh r2 = rot;
    r2.block = 96;
    expect(orbq_rpbh_quantize(X, 16, d, d, &r2, &cba, 1e-8f, codes, norms, nullptr), ORBQ_ERR_UNSUPPORTED, "quantize block 96");
    r2 = rot;
    r2.d = 1024;
    expect(orbq_rpbh_quantize(X, 16, d, d, &r2, &cba, 1e-8f, codes, norms, nullptr), ORBQ_ERR_INVALID_ARG, "quantize rot d mismatch");
  }
  expect(orbq_fold_weights(X, 16, d, d, &rot, nullptr, 1e-8f, codes, norms, nullptr), ORBQ_ERR_INVALID_ARG, "fold NULL codebook");
  expect(orbq_lut_gemm(codes, norms, &cba, codes, norms, &cbw, 16, 16, d, nullptr, ORBQ_BF16, 16, nullptr),
         ORBQ_ERR_INVALID_ARG, "lut_gemm NULL Y");
  expect(orbq_lut_gemm(codes, norms, &cba, codes, norms, &cbw, 16, 16, d, Y, ORBQ_BF16, 15, nullptr),
         ORBQ_ERR_INVALID_ARG, "lut_gemm ldy < m");
  expect(orbq_lut_gemm_act(codes, norms, &cba, codes, norms, &cbw, 16, 16, d, static_cast<orbq_activation>(9), Y,
                           ORBQ_BF16, 16, nullptr),
         ORBQ_ERR_INVALID_ARG, "lut_gemm_act unknown activation");
  expect(orbq_linear(X, 16, d, d, &rot, &cba, 1e-8f, codes, norms, &cbw, 16, nullptr, 0, Y, ORBQ_BF16, 16, nullptr),
         ORBQ_ERR_WORKSPACE, "linear without workspace");
  expect(orbq_linear_noalloc(X, 16, 4096, 4096, &rot, &cba, 1e-8f, codes, norms, &cbw, 16, ORBQ_ACT_NONE, Y, ORBQ_BF16,
                             16, nullptr),
         ORBQ_ERR_INVALID_ARG, "noalloc rot d mismatch");
  {
    orbq_rpbh r4{4096, 128, rot.perm, rot.signs, 1};
    float c44[16];
    expect(orbq_codebook_lloyd_max(4096, 4, c44), ORBQ_OK, "lloyd_max 4096 x 4");
    orbq_codebook a4{4096, 4, c44};
    expect(orbq_linear_noalloc(X, 8192, 4096, 4096, &r4, &a4, 1e-8f, codes, norms, &a4, 16, ORBQ_ACT_NONE, Y, ORBQ_BF16,
                               16, nullptr),
           ORBQ_ERR_WORKSPACE, "noalloc beyond the scratch");
  }
  {  // matrix-core probe: every rejection before a launch
    double fl = -1.0;
    float* sink = reinterpret_cast<float*>(Y);
    expect(orbq_test_mfma_rate(0, 400, sink, &fl, nullptr), ORBQ_ERR_INVALID_ARG, "probe: no workgroups");
    expect(orbq_test_mfma_rate(1 << 20, 400, sink, &fl, nullptr), ORBQ_ERR_INVALID_ARG, "probe: too many");
    expect(orbq_test_mfma_rate(256, 6, sink, &fl, nullptr), ORBQ_ERR_INVALID_ARG, "probe: iters % 4");
    expect(orbq_test_mfma_rate(256, -4, sink, &fl, nullptr), ORBQ_ERR_INVALID_ARG, "probe: negative iters");
    expect(orbq_test_mfma_rate(256, 400, nullptr, &fl, nullptr), ORBQ_ERR_INVALID_ARG, "probe: NULL sink");
    expect(orbq_test_mfma_rate(256, 400, sink, nullptr, nullptr), ORBQ_ERR_INVALID_ARG, "probe: NULL flops");
    expect(orbq_test_mfma_rate(256, 400, reinterpret_cast<float*>(reinterpret_cast<char*>(sink) + 2), &fl, nullptr),
           ORBQ_ERR_ALIGNMENT, "probe: misaligned sink");
  }
  ++g_checks;
  if (std::strlen(orbq_last_error()) == 0) {
    ++g_fail;
    std::printf("FAIL last_error empty\n");
  }

  if (g_fail) {
    std::printf("%d of %d checks failed\n", g_fail, g_checks);
    return 1;
  }
  std::printf("ok %d\n", g_checks);
  return 0;
}
