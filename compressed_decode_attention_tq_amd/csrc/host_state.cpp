// Host-side random state of a compressed layer: SplitMix64 + Box-Muller streams,
// the Haar-random rotation and the randomised Hadamard rotation.
//
// The method keeps one random orthogonal rotation and one Gaussian projection per
// head, fixed for the life of the cache ("5x Faster LLM Inference? This KV Cache
// Hack Changes Everything", "Example 1: Complete Generation Pipeline"; "How
// 0xsero/turboquant works", "Compression Pipeline").  The pages do not say how
// they are drawn; this library draws them from published generators:
//   SplitMix64 (Steele, Lea, Flood, OOPSLA 2014): Weyl increment 0x9E3779B97F4A7C15
//     followed by the variant-13 64-bit mixer;
//   Box-Muller (1958): u1 in (0,1], u2 in [0,1) -> r cos(2 pi u2), r sin(2 pi u2);
//   Haar rotation (Mezzadri 2007): Householder QR of a Gaussian matrix, column j of
//     Q multiplied by sign(R_jj) so the factorisation is unique.
// Stream key: mix64(mix64(mix64(mix64(seed) ^ layer) ^ head) ^ tag).
#include <cmath>
#include <vector>

#include "tq_internal.hpp"

namespace tq {

uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

uint64_t stream_key(uint64_t seed, uint64_t layer, uint64_t head, uint64_t tag) {
  uint64_t s = mix64(seed);
  s = mix64(s ^ layer);
  s = mix64(s ^ head);
  return mix64(s ^ tag);
}

void gaussians(uint64_t seed, uint64_t layer, uint64_t head, uint64_t tag, size_t count,
               double* out) {
  uint64_t state = stream_key(seed, layer, head, tag);
  auto next = [&state]() {
    state += 0x9E3779B97F4A7C15ULL;
    return mix64(state);
  };
  const double two_pi = 2.0 * M_PI;
  const double ulp53 = std::ldexp(1.0, -53);
  size_t i = 0;
  while (i < count) {
    const double u1 = static_cast<double>((next() >> 11) + 1) * ulp53;
    const double u2 = static_cast<double>(next() >> 11) * ulp53;
    const double r = std::sqrt(-2.0 * std::log(u1));
    const double theta = two_pi * u2;
    out[i++] = r * std::cos(theta);
    if (i < count) out[i++] = r * std::sin(theta);
  }
}

// Householder QR of A (d x d, row-major, overwritten).  Returns Q with the sign
// convention that makes diag(R) non-negative.
void haar_rotation(uint64_t seed, int layer, int head, int d, double* out) {
  std::vector<double> a(static_cast<size_t>(d) * d);
  gaussians(seed, static_cast<uint64_t>(layer), static_cast<uint64_t>(head), kTagRotation,
            a.size(), a.data());
  std::vector<std::vector<double>> vs(d);
  std::vector<double> rdiag(d);
  for (int k = 0; k < d; ++k) {
    double norm2 = 0.0;
    for (int i = k; i < d; ++i) norm2 += a[i * d + k] * a[i * d + k];
    const double norm = std::sqrt(norm2);
    const double x0 = a[k * d + k];
    const double alpha = (x0 >= 0.0) ? -norm : norm;  // reflect x onto alpha e1
    std::vector<double> v(d - k);
    for (int i = k; i < d; ++i) v[i - k] = a[i * d + k];
    v[0] -= alpha;
    double vn2 = 0.0;
    for (double x : v) vn2 += x * x;
    if (vn2 > 0.0) {
      const double inv = 1.0 / std::sqrt(vn2);
      for (double& x : v) x *= inv;
      for (int j = k; j < d; ++j) {
        double dot = 0.0;
        for (int i = k; i < d; ++i) dot += v[i - k] * a[i * d + j];
        for (int i = k; i < d; ++i) a[i * d + j] -= 2.0 * v[i - k] * dot;
      }
    } else {
      v.assign(d - k, 0.0);
    }
    rdiag[k] = a[k * d + k];
    vs[k] = std::move(v);
  }
  // Q = H_0 H_1 ... H_{d-1} I
  std::vector<double> q(static_cast<size_t>(d) * d, 0.0);
  for (int i = 0; i < d; ++i) q[i * d + i] = 1.0;
  for (int k = d - 1; k >= 0; --k) {
    const std::vector<double>& v = vs[k];
    for (int j = 0; j < d; ++j) {
      double dot = 0.0;
      for (int i = k; i < d; ++i) dot += v[i - k] * q[i * d + j];
      for (int i = k; i < d; ++i) q[i * d + j] -= 2.0 * v[i - k] * dot;
    }
  }
  for (int j = 0; j < d; ++j) {
    const double s = (rdiag[j] < 0.0) ? -1.0 : 1.0;
    for (int i = 0; i < d; ++i) out[i * d + j] = q[i * d + j] * s;
  }
}

// R = H D / sqrt(d): H[i][j] = (-1)^popcount(i & j) (Sylvester order), D[j] = +1
// when the top bit of the j-th output of the tag-3 SplitMix64 stream is 0, else -1.
void hadamard_rotation(uint64_t seed, int layer, int head, int d, double* out) {
  uint64_t state = stream_key(seed, static_cast<uint64_t>(layer), static_cast<uint64_t>(head), kTagSigns);
  std::vector<double> sgn(d);
  for (int j = 0; j < d; ++j) {
    state += 0x9E3779B97F4A7C15ULL;
    sgn[j] = (mix64(state) >> 63) == 0 ? 1.0 : -1.0;
  }
  const double inv = 1.0 / std::sqrt(static_cast<double>(d));
  for (int i = 0; i < d; ++i)
    for (int j = 0; j < d; ++j)
      out[i * d + j] = ((__builtin_popcount(static_cast<unsigned>(i & j)) & 1) ? -inv : inv) * sgn[j];
}

}  // namespace tq
