// Bidirectional FAVOR+ backward on the matrix cores (bf16 inputs, d = 64,
// m a multiple of 64 up to 256): the gradients of <dO, O> with respect to Q,
// K and V for an upstream gradient dO, W held fixed -- the chain rule through
// the features and the FA-part bracket of the "FAVOR+" method page.
//
// With the forward's stabilised quantities (log2 units, W' = W log2 e): key
// features K~_jr = exp2(w'_r . k_j - n_j - c_r), the state
// [S~ | z~] = sum_j K~_j [v_j | 1], query features Q~_ir = exp2(w'_r . q_i + c_r - M_i),
// den~_i = Q~_i . z~ and num~_i = Q~_i S~:
//
//   Ucat_i = [dO_i / den~_i | -(dO_i . num~_i) / den~_i^2]
//   query side:  T_ir = S~_r . U_i + z~_r u0_i,  P_ir = Q~_ir T_ir,
//                dq_i = sum_r P_ir w_r - 2 knorm (sum_r P_ir) q_i,
//                G_r += Q~_ir Ucat_i (per query block, summed in a fixed order)
//   key side:    H_jr = G_r . [v_j | 1],  R_jr = K~_jr H_jr,
//                dk_j = sum_r R_jr w_r - 2 knorm (sum_r R_jr) k_j,  dv_j = sum_r K~_jr G_r
//
// (ReLU features: Q~ = max(w' . q, 0), P = [Q~ > 0] T, R = [K~ > 0] H, no norm
// term; the factor log2 e of W' is put back into dq and dk.)  Every shift
// cancels as in the forward: P and R pair a query and a key factor whose
// references are opposite, and e^{-M_i} divides out through den~ in U.
//
// Launches: kpart (the forward's key partials), bprep (W' in fp16 and W^T in
// bf16), bcombine (the split partials summed into the operand layouts), bqr
// in three passes (1/den and u0; dq; the query blocks' G partials), gcombine
// (the blocks' G summed in block order), bkeyr in two passes (dk; dv).
//
// Matrix products run as 16x16x32 MFMAs, each wave on two 16-token column
// tiles; a work-group keeps the per-head operands it needs (W', W^T, the
// state, G) resident in LDS and walks a block of tokens.  A product's output
// tile feeds the next product's k-slice straight from registers where the
// other operand stores its features in the order feat_pos; Q~^T and Ucat^T
// for the query state go through LDS.
// Numerics: projections in fp16 (Q, K exact, W' rounded); features, P and R
// rounded to bf16 as operands; the state, U (with u0) and G, whose products
// cancel against a ones-column term (T = S~ U + z~ u0 and H = G v + G_z vanish
// when v_j = O_i), carried as bf16 hi + lo pairs (two MFMAs each), and dO
// (exact in bf16) used unscaled in T; all sums fp32.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "favor.h"
#include "favor_internal.h"
#include "mfma_common.h"

namespace favor {
namespace {

using namespace mfma;

constexpr int kD = 64;          // head dimension of this path

__device__ inline uint16_t bf16_bits(float x) {
  return static_cast<uint16_t>(pack_bf16(x, 0.f) & 0xffffu);
}

// Feature order of the operands contracted over features.  A product's
// 16x16 output tile holds, per lane (g, l16), rows 4g..4g+3 of one column;
// two such tiles (features 32p + [0, 16) and 32p + [16, 32)) give a lane the
// eight features {32p + 4g + j, 32p + 16 + 4g + j : j < 4} of its column,
// which serve directly as the lane's 8-value k-slice of the next product if
// the other operand stores its features in the same order: position
// 32p + 8g + j holds feature 32p + 4g + j (j < 4) or 32p + 16 + 4g + j - 4.
__device__ inline int feat_pos(int f) {
  const int p = f & ~31, i = f & 31;
  return p + 8 * ((i & 15) >> 2) + (i & 3) + (i >= 16 ? 4 : 0);
}
// Eight bf16 of column l16 from the output tiles ft = 2p and 2p + 1, in that order.
__device__ inline bf16x8 pack_k8(const f32x4& lo, const f32x4& hi) {
  return __builtin_bit_cast(bf16x8, make_uint4(pack_bf16(lo[0], lo[1]), pack_bf16(lo[2], lo[3]),
                                               pack_bf16(hi[0], hi[1]), pack_bf16(hi[2], hi[3])));
}

// ---------------------------------------------------------------------------
// bprep: W' = W log2 e as fp16 [m][64] and W^T as bf16 [64][m] (true W,
// features in the contraction order feat_pos).  grid (ceil(m*64/256)).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void bprep(const float* __restrict__ W,
                                             _Float16* __restrict__ W16,
                                             uint16_t* __restrict__ WT, int m) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= m * kD) return;
  const int r = i / kD, a = i - r * kD;
  const float w = W[i];
  W16[i] = static_cast<_Float16>(w * kLog2e);
  WT[static_cast<size_t>(a) * m + feat_pos(r)] = bf16_bits(w);
}

// ---------------------------------------------------------------------------
// bcombine: per head and feature, the splits' partial states rescaled to the
// largest reference and summed in split order.  Writes KzT [2][80][m] bf16
// (hi, lo; rows 0..63 S~^T, row 64 z~, rows 65..79 zero; features in the
// contraction order feat_pos), KzF [2][m][64] bf16
// (S~ hi, lo), zf [m] fp32 (z~) and cf [m] fp32 (the reference).  grid
// (ceil(m/64), BH), 256 threads: 64 features x 4 column groups.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void bcombine(const float* __restrict__ P,
                                                const float* __restrict__ cs,
                                                uint16_t* __restrict__ KzT,
                                                uint16_t* __restrict__ KzF,
                                                float* __restrict__ zf, float* __restrict__ cf,
                                                int m, int nseg) {
  const int bh = blockIdx.y;
  const int fl = threadIdx.x % 64, cg = threadIdx.x / 64;
  const int f = blockIdx.x * 64 + fl;
  if (f >= m) return;
  const size_t cb = static_cast<size_t>(bh) * nseg * m + f;
  float cm = -INFINITY;
  for (int s = 0; s < nseg; ++s) cm = fmaxf(cm, cs[cb + static_cast<size_t>(s) * m]);
  // columns cg, cg + 4, ... of [S~ | z~] (65 columns)
  for (int c = cg; c <= kD; c += 4) {
    float acc = 0.f;
    for (int s = 0; s < nseg; ++s) {
      const float sc = fast_exp2(cs[cb + static_cast<size_t>(s) * m] - cm);
      acc = fmaf(P[((static_cast<size_t>(bh) * nseg + s) * (kD + 1) + c) * m + f], sc, acc);
    }
    const uint16_t hi = bf16_bits(acc);
    const uint16_t lo = bf16_bits(acc - __uint_as_float(static_cast<uint32_t>(hi) << 16));
    KzT[(static_cast<size_t>(bh) * 160 + c) * m + feat_pos(f)] = hi;
    KzT[(static_cast<size_t>(bh) * 160 + 80 + c) * m + feat_pos(f)] = lo;
    if (c < kD) {
      KzF[(static_cast<size_t>(bh) * 2 * m + f) * kD + c] = hi;
      KzF[((static_cast<size_t>(bh) * 2 + 1) * m + f) * kD + c] = lo;
    } else {
      zf[static_cast<size_t>(bh) * m + f] = acc;
    }
  }
  for (int c = kD + 1 + cg; c < 80; c += 4) {
    KzT[(static_cast<size_t>(bh) * 160 + c) * m + feat_pos(f)] = 0;
    KzT[(static_cast<size_t>(bh) * 160 + 80 + c) * m + feat_pos(f)] = 0;
  }
  if (cg == 0) cf[static_cast<size_t>(bh) * m + f] = cm;
}

// Four bf16 values (8 bytes) at p, as floats.
__device__ inline void ld_bf16x4(const uint16_t* p, float (&x)[4]) {
  const uint2 u = *reinterpret_cast<const uint2*>(p);
  x[0] = bf16_lo(u.x);
  x[1] = bf16_hi(u.x);
  x[2] = bf16_lo(u.y);
  x[3] = bf16_hi(u.y);
}
__device__ inline void st_bf16x4(uint16_t* p, float a, float b, float c, float d) {
  *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16(a, b), pack_bf16(c, d));
}

// ---------------------------------------------------------------------------
// gcombine: G = sum over query blocks (block order) -> GF [2][m][64] bf16
// (hi, lo), GT [64][m] bf16 (features in the order feat_pos), Gz [m] fp32
// (the ones column).
// grid (ceil(m*65/256), BH).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void gcombine(const float* __restrict__ Gp,
                                                uint16_t* __restrict__ GF,
                                                uint16_t* __restrict__ GT,
                                                float* __restrict__ Gz, int m, int nqb) {
  const int bh = blockIdx.y;
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= m * (kD + 1)) return;
  const int f = e / (kD + 1), c = e - f * (kD + 1);
  float acc = 0.f;
  for (int b = 0; b < nqb; ++b) acc += Gp[(static_cast<size_t>(bh) * nqb + b) * m * (kD + 1) + e];
  if (c < kD) {
    const uint16_t x = bf16_bits(acc);
    GF[(static_cast<size_t>(bh) * 2 * m + f) * kD + c] = x;
    GF[((static_cast<size_t>(bh) * 2 + 1) * m + f) * kD + c] =
        bf16_bits(acc - __uint_as_float(static_cast<uint32_t>(x) << 16));
    GT[(static_cast<size_t>(bh) * kD + c) * m + feat_pos(f)] = x;
  } else {
    Gz[static_cast<size_t>(bh) * m + f] = acc;
  }
}

// ---------------------------------------------------------------------------
// bkeyr: the key side with its per-head operands resident in LDS.  grid
// (BH * nkb), 256 threads; work-group (bh, kb) takes keys [kb kblk,
// (kb+1) kblk) in steps of 128, wave w owning keys 32w..32w+31 of a step
// (two 16-key column tiles, so every operand fragment read from LDS feeds two
// products).  MODE 0: dk (operands W' [M][64] fp16, G hi/lo [2][M][64] bf16,
// W^T [64][M] bf16: 128 KB); MODE 1: dv (W', G^T [64][M]: 64 KB).  K and V
// fragments come straight from global memory as the products' B operands.
// LDS rows are XOR-swizzled in 16-byte chunks (chunk ^ (row & 7)).
// ---------------------------------------------------------------------------
template <int C>
__device__ inline int swz(int row, int col) {   // element offset in a [rows][C] tile
  return row * C + ((((col >> 3) ^ (row & 7))) << 3) + (col & 7);
}

// Copies a [rows][C] 16-bit matrix from global memory into a swizzled LDS tile.
template <int C>
__device__ inline void stage_swz(const uint16_t* __restrict__ src, uint16_t* dst, int rows) {
  const int nch = rows * (C / 8);
  for (int i = threadIdx.x; i < nch; i += 256) {
    const int r = i / (C / 8), c = (i % (C / 8)) * 8;
    *reinterpret_cast<uint4*>(dst + swz<C>(r, c)) =
        *reinterpret_cast<const uint4*>(src + static_cast<size_t>(r) * C + c);
  }
}

template <int M, bool RELU, int MODE>
__global__ __launch_bounds__(256, 1) void bkeyr(
    const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const _Float16* __restrict__ W16, const uint16_t* __restrict__ WT,
    const uint16_t* __restrict__ GF, const uint16_t* __restrict__ GT,
    const float* __restrict__ Gz, const float* __restrict__ cf, uint16_t* __restrict__ dK,
    uint16_t* __restrict__ dV, int L, int kblk, int nkb, float knorm) {
  constexpr int FT = M / 16;
  constexpr int KF = M / 32;
  const int bh = blockIdx.x / nkb, kb = blockIdx.x % nkb;
  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
  const int l16 = lane % 16, g = lane / 16;
  extern __shared__ __align__(16) uint16_t lds[];
  uint16_t* Wl = lds;                               // W' [M][64]
  uint16_t* Gl = lds + M * kD;                      // MODE 0: G hi, lo [2][M][64]
  uint16_t* Tl = lds + (MODE == 0 ? 3 : 1) * M * kD;   // W^T (MODE 0) or G^T (MODE 1) [64][M]

  stage_swz<kD>(reinterpret_cast<const uint16_t*>(W16), Wl, M);
  if constexpr (MODE == 0) {
    stage_swz<kD>(GF + static_cast<size_t>(bh) * 2 * M * kD, Gl, 2 * M);
    stage_swz<M>(WT, Tl, kD);
  } else {
    stage_swz<M>(GT + static_cast<size_t>(bh) * kD * M, Tl, kD);
  }
  __syncthreads();

  const size_t base = static_cast<size_t>(bh) * L * kD;
  const float* gz = Gz + static_cast<size_t>(bh) * M;
  const float* cfh = cf + static_cast<size_t>(bh) * M;
  const int j_beg = kb * kblk, j_end = min(L, j_beg + kblk);
  for (int t0 = j_beg + 32 * wave; t0 < j_end; t0 += 128) {
    // Key fragments of the two column tiles (B operands, k = d), as fp16;
    // norm terms n_j = knorm log2(e) |k_j|^2.
    f16x8 kf[2][2];
    float nrm[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int j = t0 + 16 * nt + l16;
      float ss = 0.f;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        uint4 u = make_uint4(0u, 0u, 0u, 0u);
        if (j < L) u = *reinterpret_cast<const uint4*>(K + base + static_cast<size_t>(j) * kD + 32 * ks + 8 * g);
        const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float lo = bf16_lo(w4[q]), hi = bf16_hi(w4[q]);
          ss = fmaf(lo, lo, ss);
          ss = fmaf(hi, hi, ss);
        }
        kf[nt][ks] = __builtin_bit_cast(f16x8, make_uint4(bf16x2_to_f16x2(u.x), bf16x2_to_f16x2(u.y),
                                                         bf16x2_to_f16x2(u.z), bf16x2_to_f16x2(u.w)));
      }
      ss += __shfl_xor(ss, 16);
      ss += __shfl_xor(ss, 32);
      nrm[nt] = knorm * kLog2e * ss;
    }
    // (1) E^T = W' K^T - n - c, K~ = exp2(E) (rows: features; columns: keys).
    f32x4 E[2][FT];
#pragma unroll
    for (int ft = 0; ft < FT; ++ft) {
      float c4[4] = {0.f, 0.f, 0.f, 0.f};
      if constexpr (!RELU) {
        const float4 cv = *reinterpret_cast<const float4*>(cfh + 16 * ft + 4 * g);
        c4[0] = cv.x; c4[1] = cv.y; c4[2] = cv.z; c4[3] = cv.w;
      }
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) E[nt][ft] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const f16x8 wa = *reinterpret_cast<const f16x8*>(Wl + swz<kD>(16 * ft + l16, 32 * ks + 8 * g));
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) E[nt][ft] = mma_f16(wa, kf[nt][ks], E[nt][ft]);
      }
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          E[nt][ft][v] = feature<RELU>(RELU ? E[nt][ft][v] : E[nt][ft][v] - nrm[nt] - c4[v]);
      __builtin_amdgcn_sched_barrier(0);   // bounded operand lookahead
    }
    if constexpr (MODE == 0) {
      // (2) H^T = G V^T + G_z (G hi + lo), R = K~ H in place of K~.
      bf16x8 vf[2][2];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int j = t0 + 16 * nt + l16;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          uint4 u = make_uint4(0u, 0u, 0u, 0u);
          if (j < L) u = *reinterpret_cast<const uint4*>(V + base + static_cast<size_t>(j) * kD + 32 * ks + 8 * g);
          vf[nt][ks] = __builtin_bit_cast(bf16x8, u);
        }
      }
      float rsum[2] = {0.f, 0.f};
#pragma unroll
      for (int ft = 0; ft < FT; ++ft) {
        f32x4 H[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const bf16x8 ghi = *reinterpret_cast<const bf16x8*>(Gl + swz<kD>(16 * ft + l16, 32 * ks + 8 * g));
          const bf16x8 glo = *reinterpret_cast<const bf16x8*>(Gl + swz<kD>(M + 16 * ft + l16, 32 * ks + 8 * g));
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) {
            H[nt] = mma_bf16(ghi, vf[nt][ks], H[nt]);
            H[nt] = mma_bf16(glo, vf[nt][ks], H[nt]);
          }
        }
        const float4 z4 = *reinterpret_cast<const float4*>(gz + 16 * ft + 4 * g);
        const float zz[4] = {z4.x, z4.y, z4.z, z4.w};
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const float hv = H[nt][v] + zz[v];
            const float r = RELU ? (E[nt][ft][v] > 0.f ? hv : 0.f) : E[nt][ft][v] * hv;
            E[nt][ft][v] = r;
            rsum[nt] += r;
          }
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        rsum[nt] += __shfl_xor(rsum[nt], 16);
        rsum[nt] += __shfl_xor(rsum[nt], 32);
      }
      // (3) dk^T = W^T R^T - 2 knorm (sum_r R) k.
#pragma unroll
      for (int at = 0; at < 4; ++at) {
        f32x4 Dk[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int ks = 0; ks < KF; ++ks) {
          const bf16x8 wa = *reinterpret_cast<const bf16x8*>(Tl + swz<M>(16 * at + l16, 32 * ks + 8 * g));
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) Dk[nt] = mma_bf16(wa, pack_k8(E[nt][2 * ks], E[nt][2 * ks + 1]), Dk[nt]);
        }
        const int a0 = 16 * at + 4 * g;
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          const int j = t0 + 16 * nt + l16;
          if (j < L) {
            float kv[4];
            ld_bf16x4(K + base + static_cast<size_t>(j) * kD + a0, kv);
            float o[4];
#pragma unroll
            for (int v = 0; v < 4; ++v)
              o[v] = RELU ? Dk[nt][v] * kLog2e : fmaf(-2.f * knorm * rsum[nt], kv[v], Dk[nt][v]);
            st_bf16x4(dK + base + static_cast<size_t>(j) * kD + a0, o[0], o[1], o[2], o[3]);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      // (4) dv^T = G^T K~^T.
#pragma unroll
      for (int at = 0; at < 4; ++at) {
        f32x4 Dv[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int ks = 0; ks < KF; ++ks) {
          const bf16x8 ga = *reinterpret_cast<const bf16x8*>(Tl + swz<M>(16 * at + l16, 32 * ks + 8 * g));
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) Dv[nt] = mma_bf16(ga, pack_k8(E[nt][2 * ks], E[nt][2 * ks + 1]), Dv[nt]);
        }
        const int a0 = 16 * at + 4 * g;
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          const int j = t0 + 16 * nt + l16;
          if (j < L) st_bf16x4(dV + base + static_cast<size_t>(j) * kD + a0, Dv[nt][0], Dv[nt][1], Dv[nt][2], Dv[nt][3]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// bqr: the query side with its per-head operands resident in LDS, in three
// passes that each rebuild the query features Q~ (cheaper than the operand
// traffic of one pass holding every operand).  grid (BH * nqb), 256 threads;
// work-group (bh, qb) takes queries [qb qblk, (qb+1) qblk) in steps of 128,
// wave w owning queries 32w..32w+31 of a step (two 16-query column tiles).
//   MODE 0: [num | den] = Q~ [S~ | z~] (state hi + lo) -> ru[i] = (1/den~_i, u0_i)
//           (operands W' and KzT: 112 KB)
//   MODE 1: T = S~ dO / den~ + z~ u0 (state hi + lo), P = Q~ T, dq = P W -
//           2 knorm (sum_r P) q (operands W', KzF, W^T: 128 KB)
//   MODE 2: G += Q~^T Ucat over the step's 128 queries (Ucat hi + lo), the
//           block's partial written at the end (operand W' and the step's
//           Q~^T / Ucat^T tiles: 144 KB at m = 256)
// ---------------------------------------------------------------------------
template <int M, bool RELU, int MODE>
__global__ __launch_bounds__(256, 1) void bqr(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ dO,
    const _Float16* __restrict__ W16, const uint16_t* __restrict__ WT,
    const uint16_t* __restrict__ KzT, const uint16_t* __restrict__ KzF,
    const float* __restrict__ zf, const float* __restrict__ cf, float* __restrict__ ru,
    uint16_t* __restrict__ dQ, float* __restrict__ Gp, int L, int qblk, int nqb, float knorm) {
  constexpr int FT = M / 16;
  constexpr int KF = M / 32;
  constexpr int GFT = M / 64;
  constexpr int kStep = 128;
  constexpr int kTRow = kStep + 8;
  const int bh = blockIdx.x / nqb, qb = blockIdx.x % nqb;
  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
  const int l16 = lane % 16, g = lane / 16;
  extern __shared__ __align__(16) uint16_t lds[];
  uint16_t* Wl = lds;                       // W' [M][64]
  uint16_t* Xl = lds + M * kD;              // MODE 0: KzT hi, lo [160][M]; MODE 1: KzF hi, lo
                                            // [2M][64] then W^T [64][M]; MODE 2: QT, UT
  stage_swz<kD>(reinterpret_cast<const uint16_t*>(W16), Wl, M);
  if constexpr (MODE == 0) {
    stage_swz<M>(KzT + static_cast<size_t>(bh) * 160 * M, Xl, 160);
  } else if constexpr (MODE == 1) {
    stage_swz<kD>(KzF + static_cast<size_t>(bh) * 2 * M * kD, Xl, 2 * M);
    stage_swz<M>(WT, Xl + 2 * M * kD, kD);
  } else {
    // rows 65..79 of both Ucat^T halves are zero
    uint16_t* UT = Xl + M * kTRow;
    for (int i = tid; i < 2 * 15 * kTRow; i += 256) {
      const int h = i / (15 * kTRow), r = i % (15 * kTRow);
      UT[(h * 80 + 65 + r / kTRow) * kTRow + r % kTRow] = 0;
    }
  }
  __syncthreads();

  const size_t base = static_cast<size_t>(bh) * L * kD;
  const float* cfh = cf + static_cast<size_t>(bh) * M;
  const float* zfh = zf + static_cast<size_t>(bh) * M;
  float* ruh = ru + static_cast<size_t>(bh) * L * 2;
  f32x4 G[MODE == 2 ? GFT : 1][5];
  if constexpr (MODE == 2) {
#pragma unroll
    for (int a = 0; a < GFT; ++a)
#pragma unroll
      for (int c = 0; c < 5; ++c) G[a][c] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const int i_beg = qb * qblk, i_end = min(L, i_beg + qblk);
  for (int s0 = i_beg; s0 < i_end; s0 += kStep) {
    const int t0 = s0 + 32 * wave;
    // Query fragments (B operands, k = d) as fp16.
    f16x8 qf[2][2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int i = t0 + 16 * nt + l16;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        uint4 u = make_uint4(0u, 0u, 0u, 0u);
        if (i < L) u = *reinterpret_cast<const uint4*>(Q + base + static_cast<size_t>(i) * kD + 32 * ks + 8 * g);
        qf[nt][ks] = __builtin_bit_cast(f16x8, make_uint4(bf16x2_to_f16x2(u.x), bf16x2_to_f16x2(u.y),
                                                         bf16x2_to_f16x2(u.z), bf16x2_to_f16x2(u.w)));
      }
    }
    // (1) S^T = W' Q^T + c; Q~ = exp2(S - M) with the row reference M (the
    // same arithmetic in every pass, so every pass rebuilds the same Q~).
    f32x4 S[2][FT];
#pragma unroll
    for (int ft = 0; ft < FT; ++ft) {
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) S[nt][ft] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const f16x8 wa = *reinterpret_cast<const f16x8*>(Wl + swz<kD>(16 * ft + l16, 32 * ks + 8 * g));
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) S[nt][ft] = mma_f16(wa, qf[nt][ks], S[nt][ft]);
      }
      if constexpr (!RELU) {
        const float4 c4 = *reinterpret_cast<const float4*>(cfh + 16 * ft + 4 * g);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          S[nt][ft][0] += c4.x; S[nt][ft][1] += c4.y; S[nt][ft][2] += c4.z; S[nt][ft][3] += c4.w;
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      float Mrow = 0.f;
      if constexpr (!RELU) {
        float mx = -INFINITY;
#pragma unroll
        for (int ft = 0; ft < FT; ++ft)
          mx = fmaxf(mx, max3(S[nt][ft][0], S[nt][ft][1], fmaxf(S[nt][ft][2], S[nt][ft][3])));
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        Mrow = mx;
      }
#pragma unroll
      for (int ft = 0; ft < FT; ++ft)
#pragma unroll
        for (int v = 0; v < 4; ++v) S[nt][ft][v] = feature<RELU>(S[nt][ft][v] - Mrow);
    }
    __builtin_amdgcn_sched_barrier(0);

    if constexpr (MODE == 0) {
      // (2) [num | den]^T = KzT Q~^T (hi + lo); den, dO . num -> (1/den, u0).
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int i = t0 + 16 * nt + l16;
        f32x4 N[5];
#pragma unroll
        for (int ct = 0; ct < 5; ++ct) {
          N[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < KF; ++ks) {
            const bf16x8 qb8 = pack_k8(S[nt][2 * ks], S[nt][2 * ks + 1]);
            N[ct] = mma_bf16(*reinterpret_cast<const bf16x8*>(Xl + swz<M>(16 * ct + l16, 32 * ks + 8 * g)), qb8, N[ct]);
            N[ct] = mma_bf16(*reinterpret_cast<const bf16x8*>(Xl + swz<M>(80 + 16 * ct + l16, 32 * ks + 8 * g)), qb8, N[ct]);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        const float den = __shfl(N[4][0], l16);
        float dot = 0.f;
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
          float dv[4] = {0.f, 0.f, 0.f, 0.f};
          if (i < L) ld_bf16x4(dO + base + static_cast<size_t>(i) * kD + 16 * ct + 4 * g, dv);
#pragma unroll
          for (int v = 0; v < 4; ++v) dot = fmaf(dv[v], N[ct][v], dot);
        }
        dot += __shfl_xor(dot, 16);
        dot += __shfl_xor(dot, 32);
        if (g == 0 && i < L) {
          const float rden = 1.f / den;
          *reinterpret_cast<float2*>(ruh + 2 * static_cast<size_t>(i)) = make_float2(rden, -dot * rden * rden);
        }
      }
    } else if constexpr (MODE == 1) {
      // (3) T^T = S~ dO^T / den + z~ u0 (hi + lo), P = Q~ T in place of Q~.
      const uint16_t* Kl = Xl;                 // KzF hi, lo [2M][64]
      const uint16_t* Tl = Xl + 2 * M * kD;    // W^T [64][M]
      bf16x8 df[2][2];
      float rden[2], u0[2], psum[2] = {0.f, 0.f};
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int i = t0 + 16 * nt + l16;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          uint4 u = make_uint4(0u, 0u, 0u, 0u);
          if (i < L) u = *reinterpret_cast<const uint4*>(dO + base + static_cast<size_t>(i) * kD + 32 * ks + 8 * g);
          df[nt][ks] = __builtin_bit_cast(bf16x8, u);
        }
        float2 r2 = make_float2(0.f, 0.f);
        if (i < L) r2 = *reinterpret_cast<const float2*>(ruh + 2 * static_cast<size_t>(i));
        rden[nt] = r2.x;
        u0[nt] = r2.y;
      }
#pragma unroll
      for (int ft = 0; ft < FT; ++ft) {
        f32x4 T[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const bf16x8 hi = *reinterpret_cast<const bf16x8*>(Kl + swz<kD>(16 * ft + l16, 32 * ks + 8 * g));
          const bf16x8 lo = *reinterpret_cast<const bf16x8*>(Kl + swz<kD>(M + 16 * ft + l16, 32 * ks + 8 * g));
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) {
            T[nt] = mma_bf16(hi, df[nt][ks], T[nt]);
            T[nt] = mma_bf16(lo, df[nt][ks], T[nt]);
          }
        }
        const float4 z4 = *reinterpret_cast<const float4*>(zfh + 16 * ft + 4 * g);
        const float zz[4] = {z4.x, z4.y, z4.z, z4.w};
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const float tv = fmaf(zz[v], u0[nt], T[nt][v] * rden[nt]);
            const float p = RELU ? (S[nt][ft][v] > 0.f ? tv : 0.f) : S[nt][ft][v] * tv;
            S[nt][ft][v] = p;
            psum[nt] += p;
          }
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        psum[nt] += __shfl_xor(psum[nt], 16);
        psum[nt] += __shfl_xor(psum[nt], 32);
      }
      // (4) dq^T = W^T P^T - 2 knorm (sum_r P) q.
#pragma unroll
      for (int at = 0; at < 4; ++at) {
        f32x4 Dq[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int ks = 0; ks < KF; ++ks) {
          const bf16x8 wa = *reinterpret_cast<const bf16x8*>(Tl + swz<M>(16 * at + l16, 32 * ks + 8 * g));
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) Dq[nt] = mma_bf16(wa, pack_k8(S[nt][2 * ks], S[nt][2 * ks + 1]), Dq[nt]);
        }
        const int a0 = 16 * at + 4 * g;
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          const int i = t0 + 16 * nt + l16;
          if (i < L) {
            float qv[4];
            ld_bf16x4(Q + base + static_cast<size_t>(i) * kD + a0, qv);
            float o[4];
#pragma unroll
            for (int v = 0; v < 4; ++v)
              o[v] = RELU ? Dq[nt][v] * kLog2e : fmaf(-2.f * knorm * psum[nt], qv[v], Dq[nt][v]);
            st_bf16x4(dQ + base + static_cast<size_t>(i) * kD + a0, o[0], o[1], o[2], o[3]);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      // (5) Q~^T and Ucat^T (hi, lo) of the step's 128 queries into LDS, then
      // G (this wave's feature rows) += Q~^T Ucat.
      uint16_t* QT = Xl;                    // [M][kTRow]
      uint16_t* UT = Xl + M * kTRow;        // [2][80][kTRow]
      __syncthreads();                      // the previous step's reads are done
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int il = 32 * wave + 16 * nt + l16, i = s0 + il;
#pragma unroll
        for (int ft = 0; ft < FT; ++ft)
#pragma unroll
          for (int v = 0; v < 4; ++v) QT[(16 * ft + 4 * g + v) * kTRow + il] = bf16_bits(S[nt][ft][v]);
        float2 r2 = make_float2(0.f, 0.f);
        if (i < L) r2 = *reinterpret_cast<const float2*>(ruh + 2 * static_cast<size_t>(i));
        auto put = [&](int row, float x) {
          const uint16_t hi = bf16_bits(x);
          UT[row * kTRow + il] = hi;
          UT[(80 + row) * kTRow + il] = bf16_bits(x - __uint_as_float(static_cast<uint32_t>(hi) << 16));
        };
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
          float dv[4] = {0.f, 0.f, 0.f, 0.f};
          if (i < L) ld_bf16x4(dO + base + static_cast<size_t>(i) * kD + 16 * ct + 4 * g, dv);
#pragma unroll
          for (int v = 0; v < 4; ++v) put(16 * ct + 4 * g + v, dv[v] * r2.x);
        }
        if (g == 0) put(64, r2.y);
      }
      __syncthreads();
#pragma unroll
      for (int a = 0; a < GFT; ++a) {
        const int f = wave * (M / 4) + 16 * a + l16;
#pragma unroll
        for (int ks = 0; ks < kStep / 32; ++ks) {
          const bf16x8 qa = *reinterpret_cast<const bf16x8*>(QT + f * kTRow + 32 * ks + 8 * g);
#pragma unroll
          for (int ct = 0; ct < 5; ++ct) {
            G[a][ct] = mma_bf16(qa, *reinterpret_cast<const bf16x8*>(UT + (16 * ct + l16) * kTRow + 32 * ks + 8 * g), G[a][ct]);
            G[a][ct] = mma_bf16(qa, *reinterpret_cast<const bf16x8*>(UT + (80 + 16 * ct + l16) * kTRow + 32 * ks + 8 * g), G[a][ct]);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  if constexpr (MODE == 2) {
    float* gp = Gp + (static_cast<size_t>(bh) * nqb + qb) * M * (kD + 1);
#pragma unroll
    for (int a = 0; a < GFT; ++a)
#pragma unroll
      for (int ct = 0; ct < 5; ++ct) {
        const int c = 16 * ct + l16;
        if (c > kD) continue;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int f = wave * (M / 4) + 16 * a + 4 * g + v;
          gp[static_cast<size_t>(f) * (kD + 1) + c] = G[a][ct][v];
        }
      }
  }
}

template <int M, bool RELU>
hipError_t launch_bwd(const Plan& p, const BwdPlan& b, const uint16_t* Q, const uint16_t* K,
                      const uint16_t* V, const float* W, const uint16_t* dO, uint16_t* dQ,
                      uint16_t* dK, uint16_t* dV, char* ws, hipStream_t st) {
  hipError_t e = mfma_bidir_key_partials(p, K, V, W, ws, st);
  if (e != hipSuccess) return e;
  const float* P = reinterpret_cast<const float*>(ws + p.off_T);
  const float* cs = reinterpret_cast<const float*>(ws + p.off_cseg);
  auto* W16 = reinterpret_cast<_Float16*>(ws + b.off_W16);
  auto* WT = reinterpret_cast<uint16_t*>(ws + b.off_WT);
  auto* KzT = reinterpret_cast<uint16_t*>(ws + b.off_KzT);
  auto* KzF = reinterpret_cast<uint16_t*>(ws + b.off_KzF);
  auto* zf = reinterpret_cast<float*>(ws + b.off_zf);
  auto* cf = reinterpret_cast<float*>(ws + b.off_cf);
  auto* Gp = reinterpret_cast<float*>(ws + b.off_G);
  auto* GF = reinterpret_cast<uint16_t*>(ws + b.off_GF);
  auto* GT = reinterpret_cast<uint16_t*>(ws + b.off_GT);
  auto* Gz = reinterpret_cast<float*>(ws + b.off_Gz);
  timing_before(st);
  bprep<<<dim3((M * kD + 255) / 256), 256, 0, st>>>(W, W16, WT, M);
  e = hipGetLastError();
  timing_after(st, "bprep");
  if (e != hipSuccess) return e;
  timing_before(st);
  bcombine<<<dim3(M / 64, p.BH), 256, 0, st>>>(P, cs, KzT, KzF, zf, cf, M, p.nseg);
  e = hipGetLastError();
  timing_after(st, "bcombine");
  if (e != hipSuccess) return e;
  auto* ru = reinterpret_cast<float*>(ws + b.off_ru);
  {
    constexpr int kq0 = (M * kD + 160 * M) * 2;
    constexpr int kq1 = (M * kD + 2 * M * kD + kD * M) * 2;
    constexpr int kq2 = (M * kD + M * 136 + 160 * 136) * 2;
    const void* fns[3] = {reinterpret_cast<const void*>(&bqr<M, RELU, 0>),
                          reinterpret_cast<const void*>(&bqr<M, RELU, 1>),
                          reinterpret_cast<const void*>(&bqr<M, RELU, 2>)};
    const int lds[3] = {kq0, kq1, kq2};
    for (int i = 0; i < 3; ++i) {
      e = hipFuncSetAttribute(fns[i], hipFuncAttributeMaxDynamicSharedMemorySize, lds[i]);
      if (e != hipSuccess) return e;
    }
    const dim3 grid(p.BH * b.nqb);
    timing_before(st);
    bqr<M, RELU, 0><<<grid, 256, kq0, st>>>(Q, dO, W16, WT, KzT, KzF, zf, cf, ru, dQ, Gp, p.L,
                                            b.qblk, b.nqb, p.knorm);
    e = hipGetLastError();
    timing_after(st, "bq_den");
    if (e != hipSuccess) return e;
    timing_before(st);
    bqr<M, RELU, 1><<<grid, 256, kq1, st>>>(Q, dO, W16, WT, KzT, KzF, zf, cf, ru, dQ, Gp, p.L,
                                            b.qblk, b.nqb, p.knorm);
    e = hipGetLastError();
    timing_after(st, "bq_dq");
    if (e != hipSuccess) return e;
    timing_before(st);
    bqr<M, RELU, 2><<<grid, 256, kq2, st>>>(Q, dO, W16, WT, KzT, KzF, zf, cf, ru, dQ, Gp, p.L,
                                            b.qblk, b.nqb, p.knorm);
    e = hipGetLastError();
    timing_after(st, "bq_g");
    if (e != hipSuccess) return e;
  }
  timing_before(st);
  gcombine<<<dim3((M * (kD + 1) + 255) / 256, p.BH), 256, 0, st>>>(Gp, GF, GT, Gz, M, b.nqb);
  e = hipGetLastError();
  timing_after(st, "gcombine");
  if (e != hipSuccess) return e;
  {
    auto* k0 = &bkeyr<M, RELU, 0>;
    auto* k1 = &bkeyr<M, RELU, 1>;
    const int lds0 = 4 * M * kD * 2, lds1 = 2 * M * kD * 2;
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(k0),
                            hipFuncAttributeMaxDynamicSharedMemorySize, lds0);
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(k1),
                            hipFuncAttributeMaxDynamicSharedMemorySize, lds1);
    if (e != hipSuccess) return e;
    timing_before(st);
    k0<<<dim3(p.BH * b.nkb), 256, lds0, st>>>(K, V, W16, WT, GF, GT, Gz, cf, dK, dV, p.L, b.kblk,
                                              b.nkb, p.knorm);
    e = hipGetLastError();
    timing_after(st, "bkey_dk");
    if (e != hipSuccess) return e;
    timing_before(st);
    k1<<<dim3(p.BH * b.nkb), 256, lds1, st>>>(K, V, W16, WT, GF, GT, Gz, cf, dK, dV, p.L, b.kblk,
                                              b.nkb, p.knorm);
    e = hipGetLastError();
    timing_after(st, "bkey_dv");
  }
  return e;
}

// ---------------------------------------------------------------------------
// sexport: the causal state after every key of the sequence -- the sum over
// all keys, i.e. the bidirectional key state -- from the splits' partials, in
// the exported layout [BH][m][d+4]: [S~ | z~ | c | 0 | 0] with c in natural-log
// units (the features here are exp2 of log2-unit exponents, the same values;
// ReLU features here are max(w' . k, 0) = log2(e) max(w . k, 0), so the state
// is scaled back by ln 2).  With an imported state Sin (same layout, not
// aliasing st) the result is Sin plus every key's contribution.
// grid (ceil(m/64), BH), 256 threads: 64 features x 4 column groups.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void sexport(const float* __restrict__ P,
                                               const float* __restrict__ cs,
                                               const float* __restrict__ Sin,
                                               float* __restrict__ st, int m, int nseg,
                                               int relu) {
  const int bh = blockIdx.y;
  const int fl = threadIdx.x % 64, cg = threadIdx.x / 64;
  const int f = blockIdx.x * 64 + fl;
  if (f >= m) return;
  const size_t cb = static_cast<size_t>(bh) * nseg * m + f;
  float cm = -INFINITY;
  for (int s = 0; s < nseg; ++s) cm = fmaxf(cm, cs[cb + static_cast<size_t>(s) * m]);
  const float* srow = Sin ? Sin + (static_cast<size_t>(bh) * m + f) * (kD + 4) : nullptr;
  // the imported state in the features' units: log2-unit reference, ReLU
  // values times log2(e)
  const float cin = srow ? srow[kD + 1] * kLog2e : -INFINITY;
  cm = fmaxf(cm, cin);
  const float sin_scale = srow ? (relu ? kLog2e : 1.f) * fast_exp2(cin - cm) : 0.f;
  float* row = st + (static_cast<size_t>(bh) * m + f) * (kD + 4);
  for (int c = cg; c <= kD; c += 4) {
    float acc = srow ? srow[c] * sin_scale : 0.f;
    for (int s = 0; s < nseg; ++s)
      acc = fmaf(P[((static_cast<size_t>(bh) * nseg + s) * (kD + 1) + c) * m + f],
                 fast_exp2(cs[cb + static_cast<size_t>(s) * m] - cm), acc);
    row[c] = relu ? acc * 0.6931471805599453f : acc;
  }
  if (cg == 0) {
    row[kD + 1] = cm * 0.6931471805599453f;
    row[kD + 2] = 0.f;
    row[kD + 3] = 0.f;
  }
}

}  // namespace

hipError_t mfma_state_export(const Plan& p, const void* ws, const float* state_in, float* state,
                             hipStream_t stream) {
  const char* w = static_cast<const char*>(ws);
  timing_before(stream);
  sexport<<<dim3((p.m + 63) / 64, p.BH), 256, 0, stream>>>(
      reinterpret_cast<const float*>(w + p.off_T), reinterpret_cast<const float*>(w + p.off_cseg),
      state_in, state, p.m, p.nseg, p.relu);
  const hipError_t e = hipGetLastError();
  timing_after(stream, "sexport");
  return e;
}

bool mfma_bwd_supported(int32_t d, int32_t m, int32_t dtype, int32_t causal) {
  const bool shape = dtype == FAVOR_BF16 && d == kD && (m == 64 || m == 128 || m == 192 || m == 256);
  return shape && (causal ? mfma_causal_supported(d, m, dtype) : mfma_bidir_supported(d, m, dtype));
}

hipError_t mfma_backward(const Plan& p, const BwdPlan& b, const void* Q, const void* K,
                         const void* V, const float* W, const void* dO, void* dQ, void* dK,
                         void* dV, void* ws, hipStream_t stream) {
  const auto* q = static_cast<const uint16_t*>(Q);
  const auto* k = static_cast<const uint16_t*>(K);
  const auto* v = static_cast<const uint16_t*>(V);
  const auto* g = static_cast<const uint16_t*>(dO);
  auto* dq = static_cast<uint16_t*>(dQ);
  auto* dk = static_cast<uint16_t*>(dK);
  auto* dv = static_cast<uint16_t*>(dV);
  char* w = static_cast<char*>(ws);
  if (p.causal) return mfma_causal_backward(p, b, Q, K, V, W, dO, dQ, dK, dV, ws, stream);
#define FAVOR_BCASE(M)                                                                   \
  if (p.m == M)                                                                          \
    return p.relu ? launch_bwd<M, true>(p, b, q, k, v, W, g, dq, dk, dv, w, stream)      \
                  : launch_bwd<M, false>(p, b, q, k, v, W, g, dq, dk, dv, w, stream);
  FAVOR_BCASE(64) FAVOR_BCASE(128) FAVOR_BCASE(192) FAVOR_BCASE(256)
#undef FAVOR_BCASE
  return hipErrorInvalidValue;
}

}  // namespace favor
