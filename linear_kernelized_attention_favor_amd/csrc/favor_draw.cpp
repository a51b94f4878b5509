// Host-side draw of the projection W [m, d]: positive orthogonal random
// features ("Rethinking Attention with Performers"; summary page "Key
// contributions" and "Limitations": orthogonality holds for at most d rows,
// features are periodically redrawn).  Blocks of at most d rows are exactly
// orthogonal; independent blocks are stacked to reach m; each row's norm is an
// independent chi(d) draw, so every row is marginally N(0, I_d).
//
// Random stream: counter-based SplitMix64 (Steele, Lea & Flood, "Fast
// splittable pseudorandom number generators", OOPSLA 2014): output i of seed s
// is the SplitMix64 finaliser applied to s + (i + 1) * gamma.  Uniforms take
// the top 53 bits plus one, times 2^-53, so they lie in (0, 1].  Normal n is
// the Box-Muller transform of uniforms 2*(n/2) and 2*(n/2)+1: the cosine
// branch for even n, the sine branch for odd n.
//
// Draw order per block b: d*d normals for G (row-major), then d normals for
// each of the block's rows (the norm vectors).  The block's directions are the
// Gram-Schmidt orthonormalisation of G's columns, in column order, each column
// orthogonalised twice against the earlier ones (fp64); row i of the block is
// direction i times |g_i|.
#include <cmath>
#include <cstdint>
#include <vector>

#include "favor.h"
#include "favor_internal.h"

namespace {

constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;

inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

inline double uniform_at(uint64_t seed, uint64_t i) {
  const uint64_t x = mix64(seed + (i + 1) * kGamma);
  return (static_cast<double>(x >> 11) + 1.0) * 0x1.0p-53;
}

// Normal number n of the stream.
inline double normal_at(uint64_t seed, uint64_t n) {
  const uint64_t p = n >> 1;
  const double u1 = uniform_at(seed, 2 * p);
  const double u2 = uniform_at(seed, 2 * p + 1);
  const double r = std::sqrt(-2.0 * std::log(u1));
  const double t = 2.0 * M_PI * u2;
  return (n & 1) ? r * std::sin(t) : r * std::cos(t);
}

}  // namespace

extern "C" int favor_draw_projection(uint64_t seed, int32_t m, int32_t d, float* W_host) {
  if (W_host == nullptr) return FAVOR_ERR_NULL;
  if (m < 1 || d < 1 || d > 1024) return FAVOR_ERR_SHAPE;
  std::vector<double> G(static_cast<size_t>(d) * d);
  std::vector<double> U(static_cast<size_t>(d) * d);  // U[j*d + a]: direction j
  uint64_t off = 0;
  for (int32_t row = 0; row < m;) {
    for (int64_t i = 0; i < static_cast<int64_t>(d) * d; ++i) G[i] = normal_at(seed, off + i);
    off += static_cast<uint64_t>(d) * d;
    // Gram-Schmidt on the columns of G, twice per column.
    for (int32_t j = 0; j < d; ++j) {
      double* u = &U[static_cast<size_t>(j) * d];
      for (int32_t a = 0; a < d; ++a) u[a] = G[static_cast<size_t>(a) * d + j];
      for (int pass = 0; pass < 2; ++pass) {
        for (int32_t k = 0; k < j; ++k) {
          const double* q = &U[static_cast<size_t>(k) * d];
          double dot = 0.0;
          for (int32_t a = 0; a < d; ++a) dot += q[a] * u[a];
          for (int32_t a = 0; a < d; ++a) u[a] -= dot * q[a];
        }
      }
      double nrm = 0.0;
      for (int32_t a = 0; a < d; ++a) nrm += u[a] * u[a];
      nrm = std::sqrt(nrm);
      for (int32_t a = 0; a < d; ++a) u[a] /= nrm;
    }
    const int32_t nb = (m - row < d) ? (m - row) : d;
    for (int32_t i = 0; i < nb; ++i) {
      double s2 = 0.0;
      for (int32_t a = 0; a < d; ++a) {
        const double g = normal_at(seed, off + a);
        s2 += g * g;
      }
      off += d;
      const double s = std::sqrt(s2);
      const double* u = &U[static_cast<size_t>(i) * d];
      float* w = W_host + static_cast<size_t>(row + i) * d;
      for (int32_t a = 0; a < d; ++a) w[a] = static_cast<float>(u[a] * s);
    }
    row += nb;
  }
  return FAVOR_OK;
}
