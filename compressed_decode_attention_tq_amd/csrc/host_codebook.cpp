// Lloyd-Max scalar codebooks (host, float64).
//
// "How 0xsero/turboquant works", "Compression Pipeline": keys use a Lloyd-Max
// scalar codebook, precomputed per (dimension, bit width).  "5x Faster LLM
// Inference? ...", "What is TurboQuant-GPU?": Lloyd-Max is MSE-optimal for the
// Gaussian-like rotated coordinates.  "tiny-turboquant 0.18.0", "The algorithm
// in three lines": the exact marginal of a rotated unit vector is a Beta law.
//
// Units: t = sqrt(d) (R k)_j / ||k||.  TQ_DIST_GAUSSIAN: N(0,1).  TQ_DIST_SPHERE:
// t = sqrt(d) u_j with density proportional to (1 - t^2/d)^((d-3)/2) on
// [-sqrt d, sqrt d].
// Lloyd (1957) / Max (1960): boundaries are midpoints of neighbouring centroids,
// centroids are the conditional means of their cells.  Start from the quantile
// midpoints of N(0,1); iterate until max |delta c| < 1e-14.
// Cell moments: closed form (erfc and the density) for the Gaussian; composite
// Gauss-Legendre quadrature for the sphere marginal.
#include <cmath>
#include <vector>

#include "tq_internal.hpp"

namespace tq {
namespace {

constexpr double kInvSqrt2Pi = 0.39894228040143267794;

double phi(double x) { return std::isinf(x) ? 0.0 : kInvSqrt2Pi * std::exp(-0.5 * x * x); }

// P(a < X <= b), X ~ N(0,1); use the upper tail on the positive side.
double gauss_prob(double a, double b) {
  if (a >= 0.0) return 0.5 * std::erfc(a / M_SQRT2) - 0.5 * std::erfc(b / M_SQRT2);
  return 0.5 * std::erfc(-b / M_SQRT2) - 0.5 * std::erfc(-a / M_SQRT2);
}

struct Moments {
  double p, m1, m2;  // integral of f, x f, x^2 f over the cell
};

Moments gauss_moments(double a, double b) {
  Moments m;
  m.p = gauss_prob(a, b);
  m.m1 = phi(a) - phi(b);
  const double xa = std::isinf(a) ? 0.0 : a * phi(a);
  const double xb = std::isinf(b) ? 0.0 : b * phi(b);
  m.m2 = m.p - (xb - xa);
  return m;
}

// n-point Gauss-Legendre nodes/weights on [-1, 1] (Newton iteration on the
// Legendre recurrence, started from the Tricomi approximation cos(pi (i+3/4)/(n+1/2))).
void gauss_legendre(int n, std::vector<double>* x, std::vector<double>* w) {
  x->assign(n, 0.0);
  w->assign(n, 0.0);
  for (int i = 0; i < n; ++i) {
    double z = std::cos(M_PI * (i + 0.75) / (n + 0.5));
    double dp = 1.0;
    for (int it = 0; it < 100; ++it) {
      double p0 = 1.0, p1 = z;
      for (int k = 2; k <= n; ++k) {
        const double p2 = ((2.0 * k - 1.0) * z * p1 - (k - 1.0) * p0) / k;
        p0 = p1;
        p1 = p2;
      }
      dp = n * (z * p1 - p0) / (z * z - 1.0);
      const double dz = p1 / dp;
      z -= dz;
      if (std::fabs(dz) < 1e-16) break;
    }
    (*x)[i] = z;
    (*w)[i] = 2.0 / ((1.0 - z * z) * dp * dp);
  }
}

// Unnormalised moments of (1 - x^2/d)^((d-3)/2) on [a, b] (sphere marginal in
// sqrt(d) units) by composite 24-point Gauss-Legendre on panels of width <= 1/8.
// The normalising constant cancels in the centroid m1/p.
Moments sphere_moments(double a, double b, int d) {
  static std::vector<double> gx, gw;
  if (gx.empty()) gauss_legendre(24, &gx, &gw);
  const double dd = static_cast<double>(d);
  const double lim = std::sqrt(dd);
  if (a < -lim) a = -lim;
  if (b > lim) b = lim;
  const double alpha = 0.5 * (dd - 3.0);
  Moments m{0.0, 0.0, 0.0};
  if (!(b > a)) return m;
  const int panels = static_cast<int>(std::ceil((b - a) * 8.0));
  const double h = (b - a) / panels;
  for (int p = 0; p < panels; ++p) {
    const double lo = a + p * h, mid = lo + 0.5 * h;
    for (size_t i = 0; i < gx.size(); ++i) {
      const double x = mid + 0.5 * h * gx[i];
      const double wv = 1.0 - x * x / dd;
      const double f = (wv > 0.0) ? std::pow(wv, alpha) * 0.5 * h * gw[i] : 0.0;
      m.p += f;
      m.m1 += x * f;
      m.m2 += x * x * f;
    }
  }
  return m;
}

double sphere_total(int d) {
  const double lim = std::sqrt(static_cast<double>(d));
  return sphere_moments(-lim, lim, d).p;
}

// Inverse of the N(0,1) CDF by bisection (used only to pick starting centroids).
double gauss_quantile(double p) {
  double lo = -40.0, hi = 40.0;
  for (int i = 0; i < 200; ++i) {
    const double mid = 0.5 * (lo + hi);
    const double c = (mid < 0.0) ? 0.5 * std::erfc(-mid / M_SQRT2) : 1.0 - 0.5 * std::erfc(mid / M_SQRT2);
    if (c < p) lo = mid; else hi = mid;
  }
  return 0.5 * (lo + hi);
}

}  // namespace

tq_status lloyd_max(int bits, tq_dist dist, int dim, double* centroids, double* boundaries,
                    double* mse) {
  if (bits < 1 || bits > 8) return fail(TQ_ERR_INVALID_ARGUMENT, "codebook bits must be 1..8, got %d", bits);
  if (dist != TQ_DIST_GAUSSIAN && dist != TQ_DIST_SPHERE)
    return fail(TQ_ERR_INVALID_ARGUMENT, "unknown codebook density %d", static_cast<int>(dist));
  if (dist == TQ_DIST_SPHERE && dim < 3)
    return fail(TQ_ERR_INVALID_ARGUMENT, "sphere codebook needs dim >= 3, got %d", dim);
  if (!centroids || !boundaries) return fail(TQ_ERR_INVALID_ARGUMENT, "null codebook output");
  const int L = 1 << bits;
  auto moments = [&](double a, double b) {
    return dist == TQ_DIST_GAUSSIAN ? gauss_moments(a, b) : sphere_moments(a, b, dim);
  };
  std::vector<double> c(L), nc(L), bnd(L - 1), edges(L + 1);
  const double clip = 0.9 * std::sqrt(static_cast<double>(dim));
  for (int i = 0; i < L; ++i) {
    c[i] = gauss_quantile((i + 0.5) / L);
    if (dist == TQ_DIST_SPHERE) c[i] = std::fmax(-clip, std::fmin(clip, c[i]));
  }
  bool converged = false;
  for (int it = 0; it < 200000; ++it) {
    edges[0] = -INFINITY;
    edges[L] = INFINITY;
    for (int i = 0; i + 1 < L; ++i) edges[i + 1] = 0.5 * (c[i] + c[i + 1]);
    double delta = 0.0;
    for (int i = 0; i < L; ++i) {
      const Moments m = moments(edges[i], edges[i + 1]);
      nc[i] = m.m1 / m.p;
    }
    // Both densities are even: keep the iterate exactly symmetric.
    for (int i = 0; i < L / 2; ++i) {
      const double v = 0.5 * (nc[L - 1 - i] - nc[i]);
      nc[i] = -v;
      nc[L - 1 - i] = v;
    }
    for (int i = 0; i < L; ++i) delta = std::fmax(delta, std::fabs(nc[i] - c[i]));
    c.swap(nc);
    if (delta < 1e-14) {
      converged = true;
      break;
    }
  }
  if (!converged) return fail(TQ_ERR_NOT_CONVERGED, "Lloyd-Max did not converge (bits=%d)", bits);
  for (int i = 0; i + 1 < L; ++i) bnd[i] = 0.5 * (c[i] + c[i + 1]);
  for (int i = 0; i < L; ++i) centroids[i] = c[i];
  for (int i = 0; i + 1 < L; ++i) boundaries[i] = bnd[i];
  if (mse) {
    const double z = (dist == TQ_DIST_GAUSSIAN) ? 1.0 : sphere_total(dim);
    double total = 0.0;
    for (int i = 0; i < L; ++i) {
      const double a = (i == 0) ? -INFINITY : bnd[i - 1];
      const double b = (i == L - 1) ? INFINITY : bnd[i];
      const Moments m = moments(a, b);
      total += m.m2 - 2.0 * c[i] * m.m1 + c[i] * c[i] * m.p;
    }
    *mse = total / z;
  }
  return TQ_OK;
}

}  // namespace tq
