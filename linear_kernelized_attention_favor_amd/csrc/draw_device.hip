// On-device draw of the projection W [m, d] (positive orthogonal random
// features; summary page "Key contributions" and "Limitations": orthogonality
// for at most d rows, features periodically redrawn).  The same
// distribution, random stream and stream order as the host draw
// (favor_draw_projection): per block b of at most d rows, the d*d normals of a
// Gaussian matrix G (row-major) and then d normals per row for its chi(d)
// norm; counter-based SplitMix64 (Steele, Lea & Flood, OOPSLA 2014) through
// the Box-Muller transform.  The block's directions are the columns of G made
// orthonormal in column order in fp64; here by classical Gram-Schmidt applied
// twice per column (each pass projects the column on every earlier direction
// at once), where the host sweeps the earlier directions one at a time: the
// same directions in exact arithmetic, equal to fp64 rounding.
//
// One work-group per block, its directions in LDS (fp64 [d][d], d <= 128);
// columns of G are regenerated from the counter-based stream when needed.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "favor.h"
#include "favor_internal.h"

namespace favor {
namespace {

constexpr int kDrawThreads = 256;
constexpr int kDrawMaxD = 128;
constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;

__device__ inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// Uniform i of the stream, in (0, 1]: the top 53 bits plus one, times 2^-53.
__device__ inline double uniform_at(uint64_t seed, uint64_t i) {
  const uint64_t x = mix64(seed + (i + 1) * kGamma);
  return (static_cast<double>(x >> 11) + 1.0) * 0x1.0p-53;
}

// Normal n: Box-Muller of uniforms 2*(n/2) and 2*(n/2)+1, cosine branch for
// even n, sine branch for odd n.
__device__ inline double normal_at(uint64_t seed, uint64_t n) {
  const uint64_t p = n >> 1;
  const double u1 = uniform_at(seed, 2 * p);
  const double u2 = uniform_at(seed, 2 * p + 1);
  const double r = sqrt(-2.0 * log(u1));
  const double t = 2.0 * M_PI * u2;
  return (n & 1) ? r * sin(t) : r * cos(t);
}

// Sum of one double per thread over the work-group (result in every thread).
__device__ inline double block_sum(double x, double* red) {
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
  const int t = threadIdx.x;
  if ((t & 63) == 0) red[t >> 6] = x;
  __syncthreads();
  double s = 0.0;
  for (int i = 0; i < kDrawThreads / 64; ++i) s += red[i];
  __syncthreads();
  return s;
}

__global__ __launch_bounds__(kDrawThreads) void draw_block(uint64_t seed, int m, int d,
                                                           float* __restrict__ W) {
  const int b = blockIdx.x, t = threadIdx.x;
  __shared__ double Q[kDrawMaxD][kDrawMaxD + 1];   // directions, row j = direction j (padded)
  __shared__ double u[kDrawMaxD];
  __shared__ double cf[kDrawMaxD];
  __shared__ double red[kDrawThreads / 64];
  __shared__ double rn[kDrawMaxD];
  // Stream offset of block b: every earlier block is full (d*d + d*d normals).
  const uint64_t off = static_cast<uint64_t>(b) * 2ull * d * d;
  const int row0 = b * d;
  const int nb = min(d, m - row0);
  for (int j = 0; j < d; ++j) {
    if (t < d) u[t] = normal_at(seed, off + static_cast<uint64_t>(t) * d + j);
    __syncthreads();
    for (int pass = 0; pass < 2; ++pass) {
      if (t < j) {   // coefficients on the earlier directions
        double c = 0.0;
        for (int a = 0; a < d; ++a) c = fma(Q[t][a], u[a], c);
        cf[t] = c;
      }
      __syncthreads();
      double x = 0.0;
      if (t < d) {
        x = u[t];
        for (int k = 0; k < j; ++k) x = fma(-cf[k], Q[k][t], x);
      }
      __syncthreads();
      if (t < d) u[t] = x;
      __syncthreads();
    }
    const double x = (t < d) ? u[t] : 0.0;
    const double nrm = sqrt(block_sum(x * x, red));
    if (t < d) Q[j][t] = x / nrm;
    __syncthreads();
  }
  // Row norms: |g_i| over d further normals per row, then W row = q_i |g_i|.
  const uint64_t noff = off + static_cast<uint64_t>(d) * d;
  for (int i = 0; i < nb; ++i) {
    double g = 0.0;
    if (t < d) {
      g = normal_at(seed, noff + static_cast<uint64_t>(i) * d + t);
      g *= g;
    }
    const double s2 = block_sum(g, red);
    if (t == 0) rn[i] = sqrt(s2);
  }
  __syncthreads();
  for (int p = t; p < nb * d; p += kDrawThreads) {
    const int i = p / d, a = p - i * d;
    W[static_cast<size_t>(row0 + i) * d + a] = static_cast<float>(Q[i][a] * rn[i]);
  }
}

}  // namespace

hipError_t device_draw(uint64_t seed, int32_t m, int32_t d, float* W, hipStream_t stream) {
  const int nblk = (m + d - 1) / d;
  timing_before(stream);
  draw_block<<<nblk, kDrawThreads, 0, stream>>>(seed, m, d, W);
  const hipError_t e = hipGetLastError();
  timing_after(stream, "draw_block");
  return e;
}

}  // namespace favor
