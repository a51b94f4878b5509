// Helpers of the generic (fp32 FMA) kernels, forward and backward: tile
// constants, dtype loads and stores, row staging, norm terms, the feature
// function and the projection dot product.
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

namespace favor {
namespace generic_detail {

constexpr int kThreads = 256;
constexpr int kFB = 32;   // features per g_state block
constexpr int kTT = 8;    // tokens per tile
constexpr int kMaxD = 128;
constexpr int kMaxM = 1024;

__device__ inline float load_x(const float* p, size_t i) { return p[i]; }
__device__ inline float load_x(const uint16_t* p, size_t i) {
  return __uint_as_float(static_cast<uint32_t>(p[i]) << 16);
}

// fp32 -> bf16, round to nearest even; NaN stays NaN.
__device__ inline uint16_t to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}
__device__ inline void store_x(float* p, size_t i, float v) { p[i] = v; }
__device__ inline void store_x(uint16_t* p, size_t i, float v) { p[i] = to_bf16(v); }

// Loads kTT rows [j0, j0+kTT) of a [L, d] matrix into LDS (zero past L).
template <typename T>
__device__ inline void load_rows(const T* __restrict__ X, size_t base, int j0, int jend, int d,
                                 float (*dst)[kMaxD + 1]) {
  for (int i = threadIdx.x; i < kTT * d; i += kThreads) {
    const int j = i / d, a = i - j * d;
    dst[j][a] = (j0 + j < jend) ? load_x(X, base + static_cast<size_t>(j0 + j) * d + a) : 0.f;
  }
}

// Norm terms knorm |x|^2 of the kTT rows in `rows` (first kTT threads):
// knorm = 1/2 for the softmax kernel's features, 1 for the Gaussian's.
__device__ inline void norm_terms(const float (*rows)[kMaxD + 1], int d, float knorm, float* nrm) {
  if (threadIdx.x < kTT) {
    float acc = 0.f;
#pragma unroll 16
    for (int a = 0; a < d; ++a) acc = fmaf(rows[threadIdx.x][a], rows[threadIdx.x][a], acc);
    nrm[threadIdx.x] = knorm * acc;
  }
}

// The feature of exponent (or, for ReLU features, projection) e: exp(e), or
// max(e, 0) when relu is set.  ReLU features take no norm term and no
// reference (knorm = 0 and every reference 0).
__device__ inline float feat(float e, int relu) { return relu ? fmaxf(e, 0.f) : expf(e); }

// w . x over d coordinates, w from global memory (row of W), x from LDS.
__device__ inline float dot_w(const float* __restrict__ w, const float* x, int d) {
  float acc = 0.f;
#pragma unroll 8
  for (int a = 0; a < d; a += 4) {
    const float4 wv = *reinterpret_cast<const float4*>(w + a);
    acc = fmaf(wv.x, x[a], acc);
    acc = fmaf(wv.y, x[a + 1], acc);
    acc = fmaf(wv.z, x[a + 2], acc);
    acc = fmaf(wv.w, x[a + 3], acc);
  }
  return acc;
}

}  // namespace generic_detail
}  // namespace favor
