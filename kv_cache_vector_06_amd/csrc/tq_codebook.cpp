// Host Lloyd-Max codebook for one coordinate of a uniformly random unit vector.
//
// Computes the quantizer of "TurboQuant của Google…" (omelet.tech), section
// "Lloyd-Max quantizer: chia bucket đúng chỗ", eq. C(f,b), for the density of
// section "Trick đầu tiên: xoay ngẫu nhiên trước khi nén", eq. f(x):
//   f_d(x) = C_d (1 - x²)^((d-3)/2) on [-1, 1],  C_d = Γ(d/2) / (√π Γ((d-1)/2)).
//
// Cell integrals use the substitution x = sin φ, under which
//   ∫ f_d dx = C_d ∫ cos^(d-2) φ dφ   and   ∫ x f_d dx = C_d ∫ sin φ cos^(d-2) φ dφ,
// whose integrands are smooth on [-π/2, π/2] for every d >= 2; each cell is
// integrated with composite 16-point Gauss-Legendre quadrature.
#include <cmath>
#include <cstring>
#include <vector>

#include "tq.h"

namespace {

// 16-point Gauss-Legendre nodes/weights on [-1, 1] (positive half).
const double kGLx[8] = {0.0950125098376374401853193, 0.2816035507792589132304605,
                        0.4580167776572273863424194, 0.6178762444026437484466718,
                        0.7554044083550030338951012, 0.8656312023878317438804679,
                        0.9445750230732325760779884, 0.9894009349916499325961542};
const double kGLw[8] = {0.1894506104550684962853967, 0.1826034150449235888667637,
                        0.1691565193950025381893121, 0.1495959888165767320815017,
                        0.1246289712555338720524763, 0.0951585116824927848099251,
                        0.0622535239386478928628438, 0.0271524594117540948517806};

struct Moments {
  double m0, m1, m2;  // ∫ f, ∫ x f, ∫ x² f over the cell
};

class CoordLaw {
 public:
  explicit CoordLaw(int d) : d_(d) {
    logc_ = std::lgamma(d / 2.0) - std::lgamma((d - 1) / 2.0) - 0.5 * std::log(M_PI);
  }

  // Moments over [a, b] ⊂ [-1, 1], with `panels` Gauss-Legendre panels in φ.
  Moments cell(double a, double b, int panels = 48) const {
    const double pa = std::asin(std::max(-1.0, std::min(1.0, a)));
    const double pb = std::asin(std::max(-1.0, std::min(1.0, b)));
    Moments m{0, 0, 0};
    if (pb <= pa) return m;
    const double h = (pb - pa) / panels;
    for (int p = 0; p < panels; ++p) {
      const double mid = pa + (p + 0.5) * h, half = 0.5 * h;
      for (int k = 0; k < 8; ++k) {
        for (int sgn = -1; sgn <= 1; sgn += 2) {
          const double phi = mid + sgn * half * kGLx[k];
          const double c = std::cos(phi);
          const double s = std::sin(phi);
          // C_d cos^(d-2) φ, in log space to stay finite for large d
          const double w = (c > 0) ? std::exp(logc_ + (d_ - 2) * std::log(c)) : (d_ == 2 ? std::exp(logc_) : 0.0);
          const double ww = w * kGLw[k] * half;
          m.m0 += ww;
          m.m1 += ww * s;
          m.m2 += ww * s * s;
        }
      }
    }
    return m;
  }

 private:
  int d_;
  double logc_;
};

}  // namespace

extern "C" int tq_codebook(int d, int bits, double* centroids, double* boundaries, double* mse_unit) {
  if (centroids == nullptr || d < 2) return TQ_ERR_INVALID_ARG;
  if (bits < 0 || bits > 8 || d > 65536) return TQ_ERR_UNSUPPORTED;
  if (bits > 0 && boundaries == nullptr) return TQ_ERR_INVALID_ARG;
  if (bits == 0) {
    centroids[0] = 0.0;
    if (mse_unit) *mse_unit = 1.0;
    return TQ_OK;
  }
  const int K = 1 << bits;
  const CoordLaw law(d);
  const double sd = 1.0 / std::sqrt(static_cast<double>(d));
  // Start: K levels evenly spread over ±2.5 standard deviations of one coordinate.
  std::vector<double> c(K), t(K - 1), lo(K), hi(K);
  for (int i = 0; i < K; ++i) c[i] = sd * 2.5 * (2.0 * (i + 0.5) / K - 1.0);
  const double tol = 1e-13 * sd;
  bool converged = false;
  for (int it = 0; it < 200000 && !converged; ++it) {
    for (int i = 0; i + 1 < K; ++i) t[i] = 0.5 * (c[i] + c[i + 1]);
    double delta = 0.0;
    // Only the upper half is integrated; the law is even, so the lower half
    // mirrors it and the middle boundary stays at 0.
    for (int i = K / 2; i < K; ++i) {
      const double a = (i == K / 2) ? 0.0 : t[i - 1];
      const double b = (i == K - 1) ? 1.0 : t[i];
      const Moments m = law.cell(a, b);
      const double cn = (m.m0 > 0) ? m.m1 / m.m0 : 0.5 * (a + b);
      delta = std::max(delta, std::fabs(cn - c[i]));
      c[i] = cn;
      c[K - 1 - i] = -cn;
    }
    converged = delta < tol;
  }
  if (!converged) return TQ_ERR_NO_CONVERGE;
  for (int i = 0; i + 1 < K; ++i) t[i] = 0.5 * (c[i] + c[i + 1]);
  t[K / 2 - 1] = 0.0;
  std::memcpy(centroids, c.data(), sizeof(double) * K);
  std::memcpy(boundaries, t.data(), sizeof(double) * (K - 1));
  if (mse_unit) {
    double per = 0.0;
    for (int i = K / 2; i < K; ++i) {
      const double a = (i == K / 2) ? 0.0 : t[i - 1];
      const double b = (i == K - 1) ? 1.0 : t[i];
      const Moments m = law.cell(a, b);
      per += 2.0 * (m.m2 - 2.0 * c[i] * m.m1 + c[i] * c[i] * m.m0);
    }
    *mse_unit = per * d;
  }
  return TQ_OK;
}

extern "C" const char* tq_status_string(int status) {
  switch (status) {
    case TQ_OK: return "ok";
    case TQ_ERR_INVALID_ARG: return "invalid argument";
    case TQ_ERR_UNSUPPORTED: return "unsupported configuration";
    case TQ_ERR_HIP: return "HIP runtime error";
    case TQ_ERR_WORKSPACE: return "workspace too small or misaligned";
    case TQ_ERR_NO_CONVERGE: return "Lloyd-Max iteration did not converge";
    default: return "unknown status";
  }
}
