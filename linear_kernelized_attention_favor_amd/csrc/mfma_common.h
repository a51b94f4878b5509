// Device helpers shared by the MFMA kernels of libfavor.so (gfx950 / CDNA4).
//
// Matrix-core tiles are v_mfma_f32_16x16x32_{f16,bf16}: A is 16 x 32, B is
// 32 x 16, C/D is 16 x 16 fp32.  Lane l (0..63) of a wave holds
//   A[l % 16][8 (l / 16) + u],  B[8 (l / 16) + u][l % 16]   for u = 0..7,
//   D[4 (l / 16) + v][l % 16]                               for v = 0..3.
//
// A projection tile written by the MFMA has, per lane, 4 consecutive rows of
// one column; two such tiles stacked along the row axis therefore give each
// lane the 8 operand values of one column of the next MFMA's 32-long
// reduction axis, in the order
//   position p (0..31)  <->  row  perm_of(p) = 4 (p/8 % 4) + p % 4 + 16 [p % 8 >= 4].
// Both contraction operands are laid out in that order, which leaves the
// contraction unchanged (a sum does not depend on the order of its terms).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace favor {
namespace mfma {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

__device__ __host__ constexpr int perm_of(int p) {
  return 4 * ((p >> 3) & 3) + (p & 3) + ((p & 4) ? 16 : 0);
}
__device__ __host__ constexpr int perm_inv(int j) {
  return 8 * ((j & 15) >> 2) + (j & 3) + ((j & 16) ? 4 : 0);
}

__device__ inline f32x4 mma_f16(const f16x8& a, const f16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ inline f32x4 mma_bf16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ inline uint32_t pack_bf16(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Packed bf16 pair -> packed fp16 pair.  Exact for values inside fp16's
// normal range (bf16 carries 8 significant bits, fp16 11); magnitudes above
// 65504 saturate to the largest finite fp16 (round toward zero).
__device__ inline uint32_t bf16x2_to_f16x2(uint32_t x) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(__uint_as_float(x << 16),
                                                                 __uint_as_float(x & 0xffff0000u)));
}

__device__ inline float bf16_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ inline float bf16_hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// A feature from its (relative) projection s: 2^s for the exponential
// features of the softmax and Gaussian kernels, max(s, 0) for the ReLU
// features of generalized attention (no reference needed: they cannot
// overflow, and a constant factor on every feature cancels).
// max(s, 0) is taken on the bits as a signed integer maximum: every
// negative float (and -0, -inf) is a negative integer, every positive one a
// positive integer of the same order, so one v_max_i32 does it (fmaxf on a
// matrix-instruction result costs a canonicalising max as well).
template <bool RELU>
__device__ inline float feature(float s) {
  if constexpr (RELU) return __int_as_float(max(__float_as_int(s), 0));
  else return fast_exp2(s);
}

// fmaxf trees over values produced by ordinary arithmetic (already
// canonical) lower to v_max3_f32 without extra canonicalisation.
__device__ inline float max3(float a, float b, float c) { return fmaxf(a, fmaxf(b, c)); }

// Maximum over the four lanes {l, l^16, l^32, l^48} (one column of a 16x16
// tile): lane swaps across 16- and 32-lane rows (gfx950 v_permlane*_swap).
__device__ inline float colmax4(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Sum over aligned groups of N consecutive lanes (N = 8 or 16), with DPP.
template <int N>
__device__ inline float group_sum(float x) {
  static_assert(N == 8 || N == 16, "group of 8 or 16 lanes");
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false));
  if (N == 16)
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xF, 0xF, false));
  return x;
}

// Work-group barrier that orders LDS traffic only: outstanding global loads
// (prefetches of the next tile) stay in flight across it.
__device__ inline void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Work-group order across the chip's 8 accelerator dies (XCDs, each with its
// own L2): the dispatcher hands linear work-group i to XCD i % 8.  Mapping
// i to the work item (i % 8) (n / 8) + i / 8 gives every XCD a consecutive
// run of items, so items that read the same data (the query blocks of one
// head) share one L2.  Identity when n is not a multiple of 8.
__device__ inline int xcd_major(int i, int n) {
  return (n % 8) ? i : (i % 8) * (n / 8) + i / 8;
}

// Raw buffer access (gfx9 buffer resource: base, stride 0, size in bytes).
// A load whose byte offset (VGPR offset plus the instruction's immediate) is
// at or past `bytes` returns zeros without touching memory, which masks the
// tail of a token range with no per-lane branch.  The resource is built from
// wave-uniform values, so it lives in scalar registers.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
constexpr int kBufFlags = 0x00020000;   // 32-bit data format, as every gfx9 raw buffer uses
constexpr int kBufOff = 0x40000000;     // an offset past any valid size: always reads zero

__device__ inline __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, kBufFlags);
}
__device__ inline uint4 buffer_load16(__amdgpu_buffer_rsrc_t r, int off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ inline uint2 buffer_load8(__amdgpu_buffer_rsrc_t r, int off) {
  const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
  return make_uint2(v.x, v.y);
}

// 16 bytes per lane from global memory straight into LDS (gfx950
// global_load_lds_dwordx4): lane i's data lands at lds_dst + 16 i, where
// lds_dst is the same for the whole wave.  Completion is tracked by vmcnt.
__device__ inline void lds_dma16(const void* src, void* lds_dst) {
  __builtin_amdgcn_global_load_lds(src, lds_dst, 16, 0, 0);
}

// Compiler-only ordering point for LDS data exchanged between the lanes of
// one wave: a wave's LDS operations execute in issue order, so keeping the
// compiler from moving accesses across this point is all that is needed.
__device__ inline void wave_lds_fence() { asm volatile("" ::: "memory"); }

}  // namespace mfma
}  // namespace favor
