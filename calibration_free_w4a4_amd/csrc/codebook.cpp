// Host-side codebook work of liborbq: Lloyd-Max design for f_d, the decision-threshold
// parameters of the quantizer kernels, and the bf16 decode tables of the product.
//
// Lloyd-Max for the marginal f_d of a rotated unit vector: OrbitQuant summary (picx.dev),
// "Theoretical Basis" items 1-2; TurboQuant slides (docswell) "Page. 13"-"Page. 16".
// Cell integrals of w(t) = (1 - t^2)^((d-3)/2) use composite Gauss-Legendre quadrature on
// the part of each cell where the density is not negligible; the normalising constant of
// f_d cancels in every centroid (a ratio of two integrals) and is never formed.
#include <cmath>
#include <cstring>
#include <vector>

#include "internal.h"

namespace orbq {
namespace {

// Gauss-Legendre nodes and weights on [-1, 1] (Newton on P_n, Golub-Welsch not needed).
struct GaussLegendre {
  std::vector<double> x, w;
  explicit GaussLegendre(int n) : x(n), w(n) {
    for (int i = 0; i < n; ++i) {
      double z = std::cos(M_PI * (i + 0.75) / (n + 0.5));
      for (int it = 0; it < 100; ++it) {
        double p0 = 1.0, p1 = z;
        for (int k = 2; k <= n; ++k) {
          double p2 = ((2.0 * k - 1.0) * z * p1 - (k - 1.0) * p0) / k;
          p0 = p1;
          p1 = p2;
        }
        double dp = n * (z * p1 - p0) / (z * z - 1.0);
        double dz = p1 / dp;
        z -= dz;
        if (std::fabs(dz) < 1e-16) break;
      }
      double p0 = 1.0, p1 = z;
      for (int k = 2; k <= n; ++k) {
        double p2 = ((2.0 * k - 1.0) * z * p1 - (k - 1.0) * p0) / k;
        p0 = p1;
        p1 = p2;
      }
      double dp = n * (z * p1 - p0) / (z * z - 1.0);
      x[i] = z;
      w[i] = 2.0 / ((1.0 - z * z) * dp * dp);
    }
  }
};

// integral over [lo, hi] of w(t) and t*w(t), w(t) = exp(a * log1p(-t^2)), with the cell cut to
// where w is above exp(-60) of its value at the cell's inner edge.
void cell_integrals(double lo, double hi, double a, const GaussLegendre& gl, double* m0, double* m1) {
  const double sigma = 1.0 / std::sqrt(2.0 * a + 3.0);
  // density decays away from 0: clip the far end of outer cells at 12 sigma beyond the near end
  if (lo >= 0.0) {
    hi = std::fmin(hi, std::fmin(1.0, lo + 12.0 * sigma));
  } else if (hi <= 0.0) {
    lo = std::fmax(lo, std::fmax(-1.0, hi - 12.0 * sigma));
  }
  const int pieces = 8;
  double s0 = 0.0, s1 = 0.0;
  const double h = (hi - lo) / pieces;
  for (int p = 0; p < pieces; ++p) {
    const double a0 = lo + p * h, half = 0.5 * h, mid = a0 + half;
    for (size_t i = 0; i < gl.x.size(); ++i) {
      const double t = mid + half * gl.x[i];
      const double v = std::exp(a * std::log1p(-t * t)) * gl.w[i] * half;
      s0 += v;
      s1 += t * v;
    }
  }
  *m0 = s0;
  *m1 = s1;
}

}  // namespace

// Lloyd-Max on the positive half (the codebook of an even density is antisymmetric):
// unknowns c_p = c_{N/2+p}, cells [b_{p-1}, b_p] with b_{-1} = 0, b_p = (c_p + c_{p+1})/2 and
// the last cell open to 1.  Plain Lloyd steps c <- T(c) bring the iterate close; Newton steps on
// T(c) - c = 0 with the exact tridiagonal Jacobian of T then converge quadratically:
//   dT_p/db_p     = w(b_p) (b_p - T_p) / M0_p,   dT_p/db_{p-1} = w(b_{p-1}) (T_p - b_{p-1}) / M0_p,
//   db_p/dc_p = db_p/dc_{p+1} = 1/2.
int lloyd_max_host(int d, int bits, double* out) {
  if (d < 3 || bits < 1 || bits > 8) return 1;
  const int n = 1 << bits, H = n / 2;
  const double a = 0.5 * (d - 3);
  const double sd = std::sqrt(static_cast<double>(d));
  static const GaussLegendre gl(24);
  auto w = [a](double t) { return std::exp(a * std::log1p(-t * t)); };
  std::vector<double> c(H), T(H), m0(H), b(H + 1);
  // start: uniform grid over (0, min(2.5 sigma, 1)) (any interior start converges: f_d is
  // log-concave; for d < 7, 2.5 sigma passes the support's end at 1)
  for (int p = 0; p < H; ++p) c[p] = sd > 2.5 ? 2.5 * (p + 0.5) / H / sd : (p + 0.5) / H;
  auto apply = [&]() {
    b[0] = 0.0;
    for (int p = 0; p + 1 < H; ++p) b[p + 1] = 0.5 * (c[p] + c[p + 1]);
    b[H] = 1.0;
    for (int p = 0; p < H; ++p) {
      double s0, s1;
      cell_integrals(b[p], b[p + 1], a, gl, &s0, &s1);
      m0[p] = s0;
      T[p] = s1 / s0;
    }
  };
  // Lloyd until the step is below 1e-7 / sqrt(d), then Newton; Newton stops at the float64 noise
  // floor (step no longer shrinking) or after 12 steps, returning the best fixed-point residual.
  int phase = 0, newton_steps = 0;
  double best = INFINITY;
  std::vector<double> best_c(H);
  for (int it = 0; it < 1000000; ++it) {
    apply();
    double delta = 0.0;
    for (int p = 0; p < H; ++p) delta = std::fmax(delta, std::fabs(T[p] - c[p]));
    if (phase == 1 && delta < best) {
      best = delta;
      best_c = T;
    }
    if (delta * sd < 1e-15 || (phase == 1 && (newton_steps >= 12 || (newton_steps >= 3 && delta >= best)))) {
      const std::vector<double>& r = (phase == 1) ? best_c : T;
      for (int p = 0; p < H; ++p) {
        out[H + p] = r[p];
        out[H - 1 - p] = -r[p];
      }
      return 0;
    }
    if (phase == 0 && delta * sd < 1e-7) phase = 1;
    if (phase == 0 || H == 1) {
      c = T;
      continue;
    }
    ++newton_steps;
    // Newton: (I - J) dc = T - c, J tridiagonal
    std::vector<double> lo(H, 0.0), di(H, 1.0), up(H, 0.0), rhs(H);
    for (int p = 0; p < H; ++p) {
      rhs[p] = T[p] - c[p];
      if (p + 1 < H) {  // upper boundary b_{p+1} moves with c_p and c_{p+1}
        const double g = w(b[p + 1]) * (b[p + 1] - T[p]) / m0[p];
        di[p] -= 0.5 * g;
        up[p] -= 0.5 * g;
      }
      if (p > 0) {      // lower boundary b_p moves with c_{p-1} and c_p
        const double g = w(b[p]) * (T[p] - b[p]) / m0[p];
        di[p] -= 0.5 * g;
        lo[p] -= 0.5 * g;
      }
    }
    for (int p = 1; p < H; ++p) {  // Thomas algorithm
      const double f = lo[p] / di[p - 1];
      di[p] -= f * up[p - 1];
      rhs[p] -= f * rhs[p - 1];
    }
    std::vector<double> dc(H);
    dc[H - 1] = rhs[H - 1] / di[H - 1];
    for (int p = H - 2; p >= 0; --p) dc[p] = (rhs[p] - up[p] * dc[p + 1]) / di[p];
    for (int p = 0; p < H; ++p) c[p] += dc[p];
  }
  return 2;
}

uint16_t f32_to_bf16_rne(float x) {
  uint32_t u;
  std::memcpy(&u, &x, 4);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40);  // NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

namespace {

// largest float <= v (v exactly representable in double)
float float_rd(double v) {
  float f = static_cast<float>(v);
  if (static_cast<double>(f) > v) f = std::nextafter(f, -INFINITY);
  return f;
}

// largest float < v
float float_below(double v) {
  float f = float_rd(v);
  if (static_cast<double>(f) == v) f = std::nextafter(f, -INFINITY);
  return f;
}

}  // namespace

int build_quant_params(const float* c, int bits, QuantParams* qp) {
  const int n = 1 << bits, half = n / 2, nb = half - 1;
  std::memset(qp, 0, sizeof(*qp));
  qp->bits = bits;
  qp->nb = nb;
  double B[kMaxPosBoundaries + 1];
  for (int p = 0; p < nb; ++p)  // exact: two floats of like magnitude sum exactly in double
    B[p] = 0.5 * (static_cast<double>(c[half + p]) + static_cast<double>(c[half + p + 1]));
  double min_gap = INFINITY;
  for (int p = 0; p + 1 < nb; ++p) min_gap = std::fmin(min_gap, B[p + 1] - B[p]);
  if (nb == 1) min_gap = B[0];
  int k = static_cast<int>(std::ceil(std::log2(1.5 / min_gap)));
  for (int attempt = 0; attempt < 4; ++attempt, ++k) {
    const double sc = std::ldexp(1.0, k);
    for (int p = 0; p < nb; ++p) {
      qp->thr_gt[p] = float_rd(B[p] * sc);
      qp->thr_ge[p] = float_below(B[p] * sc);
    }
    // at most one threshold per unit bucket on each side
    bool ok = true;
    for (int p = 0; p + 1 < nb; ++p) {
      if (std::floor(qp->thr_gt[p + 1]) == std::floor(qp->thr_gt[p]) ||
          std::ceil(qp->thr_gt[p + 1]) == std::ceil(qp->thr_gt[p]) ||
          std::floor(qp->thr_ge[p + 1]) == std::floor(qp->thr_ge[p]))
        ok = false;
    }
    const double top = nb ? static_cast<double>(qp->thr_gt[nb - 1]) : 0.0;
    const int J = static_cast<int>(std::floor(top)) + 2;
    if (!ok || J > kMaxTableHalf || (bits <= 4 && sc > kMaxFullScale)) continue;
    qp->scale = static_cast<float>(sc);
    qp->J = J;
    return 0;
  }
  return 1;
}

void build_decode_params(const float* c, int bits, DecodeParams* dp) {
  const int half = 1 << (bits - 1);
  std::memset(dp, 0, sizeof(*dp));
  dp->bits = bits;
  for (int r = 0; r < half; ++r) dp->mag[r] = f32_to_bf16_rne(c[half + r]);
}

}  // namespace orbq
