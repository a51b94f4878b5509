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
// bf16), bcombine (the split partials summed into the operand layouts),
// bquery (per query block: dq and the block's G partial), gcombine (the
// blocks' G summed in block order), bkey (per 64-key tile: dk, dv).
//
// Matrix products run as 16x16x32 MFMAs on 64-token tiles, one wave per 16
// tokens; every product reads its operands k-contiguous (from LDS for the
// per-tile values, from global memory -- L2-resident per head -- for W', W^T,
// the state and G).  Values change layout between products through LDS.
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
constexpr int kTok = 64;        // tokens per tile (4 waves x 16)
constexpr int kQRow = kD + 8;   // fp16 / bf16 per row of [token][d] LDS tiles
constexpr int kUTRow = kTok + 8;

__device__ inline uint16_t bf16_bits(float x) {
  return static_cast<uint16_t>(pack_bf16(x, 0.f) & 0xffffu);
}

// ---------------------------------------------------------------------------
// bprep: W' = W log2 e as fp16 [m][64] and W^T as bf16 [64][m] (true W).
// grid (ceil(m*64/256)).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void bprep(const float* __restrict__ W,
                                             _Float16* __restrict__ W16,
                                             uint16_t* __restrict__ WT, int m) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= m * kD) return;
  const int r = i / kD, a = i - r * kD;
  const float w = W[i];
  W16[i] = static_cast<_Float16>(w * kLog2e);
  WT[static_cast<size_t>(a) * m + r] = bf16_bits(w);
}

// ---------------------------------------------------------------------------
// bcombine: per head and feature, the splits' partial states rescaled to the
// largest reference and summed in split order.  Writes KzT [2][80][m] bf16
// (hi, lo; rows 0..63 S~^T, row 64 z~, rows 65..79 zero), KzF [2][m][64] bf16
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
    KzT[(static_cast<size_t>(bh) * 160 + c) * m + f] = hi;
    KzT[(static_cast<size_t>(bh) * 160 + 80 + c) * m + f] = lo;
    if (c < kD) {
      KzF[(static_cast<size_t>(bh) * 2 * m + f) * kD + c] = hi;
      KzF[((static_cast<size_t>(bh) * 2 + 1) * m + f) * kD + c] = lo;
    } else {
      zf[static_cast<size_t>(bh) * m + f] = acc;
    }
  }
  for (int c = kD + 1 + cg; c < 80; c += 4) {
    KzT[(static_cast<size_t>(bh) * 160 + c) * m + f] = 0;
    KzT[(static_cast<size_t>(bh) * 160 + 80 + c) * m + f] = 0;
  }
  if (cg == 0) cf[static_cast<size_t>(bh) * m + f] = cm;
}

// 16-byte operand loads.
__device__ inline f16x8 ld_f16x8(const _Float16* p) { return *reinterpret_cast<const f16x8*>(p); }
__device__ inline bf16x8 ld_bf16x8(const uint16_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
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

// Stages a 64-token tile of X [L][64] bf16 (rows past L zero) into an LDS
// tile [64][kQRow] as fp16 (exact for bf16 values in fp16's normal range);
// with nrm, also writes knorm log2(e) |x|^2 per token.  256 threads.
__device__ inline void stage_f16(const uint16_t* __restrict__ X, size_t base, int t0, int L,
                                 _Float16 (*dst)[kQRow], float* nrm, float ncoef) {
  const int t = threadIdx.x;
  // 64 tokens x 8 chunks of 8 values; thread t takes chunks t and t + 256
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int c = t + 256 * h;
    const int tok = c / 8, ch = c % 8;
    uint4 u = make_uint4(0u, 0u, 0u, 0u);
    if (t0 + tok < L) u = *reinterpret_cast<const uint4*>(X + base + static_cast<size_t>(t0 + tok) * kD + 8 * ch);
    float ss = 0.f;
    const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float lo = bf16_lo(w4[q]), hi = bf16_hi(w4[q]);
      ss = fmaf(lo, lo, ss);
      ss = fmaf(hi, hi, ss);
    }
    uint4 hv;
    hv.x = bf16x2_to_f16x2(u.x);
    hv.y = bf16x2_to_f16x2(u.y);
    hv.z = bf16x2_to_f16x2(u.z);
    hv.w = bf16x2_to_f16x2(u.w);
    *reinterpret_cast<uint4*>(&dst[tok][8 * ch]) = hv;
    if (nrm) {
      ss = group_sum<8>(ss);
      if (ch == 0) nrm[tok] = ncoef * ss;
    }
  }
}

// ---------------------------------------------------------------------------
// bquery: grid (BH * nqb), 256 threads.  Work-group (bh, qb) takes tokens
// [qb qblk, (qb+1) qblk) in 64-token tiles; wave w owns tokens 16w..16w+15 of
// a tile for the per-token products and features [w m/4, (w+1) m/4) for the
// block's G partial, written to Gp [BH][nqb][m][65] fp32 at the end.
// ---------------------------------------------------------------------------
template <int M, bool RELU>
__global__ __launch_bounds__(256, 1) void bquery(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ dO,
    const _Float16* __restrict__ W16, const uint16_t* __restrict__ WT,
    const uint16_t* __restrict__ KzT, const uint16_t* __restrict__ KzF,
    const float* __restrict__ zf, const float* __restrict__ cf, uint16_t* __restrict__ dQ,
    float* __restrict__ Gp, int L, int qblk, int nqb, float knorm) {
  constexpr int FT = M / 16;        // feature tiles (per token, all features)
  constexpr int KF = M / 32;        // k-steps over features
  constexpr int GFT = M / 64;       // feature tiles of this wave's G rows
  constexpr int QFRow = M + 8;
  const int bh = blockIdx.x / nqb, qb = blockIdx.x % nqb;
  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
  const int l16 = lane % 16, g = lane / 16;
  __shared__ _Float16 Qs[kTok][kQRow];
  __shared__ uint16_t QF[kTok][QFRow];     // Q~ [token][feature], then P
  __shared__ uint16_t QT[M][kUTRow];       // Q~^T [feature][token]
  __shared__ uint16_t Ds[kTok][kQRow];     // dO [token][column] (bf16, as given)
  __shared__ uint16_t UT[2][80][kUTRow];   // Ucat^T hi, lo [column][token] (row 64 = u0)

  const size_t base = static_cast<size_t>(bh) * L * kD;
  const uint16_t* kzt0 = KzT + static_cast<size_t>(bh) * 160 * M;       // hi; lo at + 80 M
  const uint16_t* kzf0 = KzF + static_cast<size_t>(bh) * 2 * M * kD;    // hi; lo at + M kD
  const float* zfh0 = zf + static_cast<size_t>(bh) * M;
  const float* cfh0 = cf + static_cast<size_t>(bh) * M;
  for (int i = tid; i < 2 * 15 * kUTRow; i += 256) {
    const int h = i / (15 * kUTRow), j = i % (15 * kUTRow);
    UT[h][65 + j / kUTRow][j % kUTRow] = 0;
  }

  f32x4 G[GFT][5];
#pragma unroll
  for (int a = 0; a < GFT; ++a)
#pragma unroll
    for (int c = 0; c < 5; ++c) G[a][c] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int i_beg = qb * qblk, i_end = min(L, i_beg + qblk);
  const int tl = 16 * wave + l16;            // this lane's token within the tile
  for (int t0 = i_beg; t0 < i_end; t0 += kTok) {
    // The per-head operands are re-read from memory (L2) every tile: made
    // opaque here so that the compiler does not hoist every one of their
    // loads out of the loop into registers.
    int z = 0;
    asm volatile("" : "+v"(z));
    const _Float16* w16 = W16 + z;
    const uint16_t* wt = WT + z;
    const uint16_t* kzt = kzt0 + z;
    const uint16_t* kzf = kzf0 + z;
    const float* zfh = zfh0 + z;
    const float* cfh = cfh0 + z;
    __syncthreads();                          // previous tile's QT / UT reads done
    stage_f16(Q, base, t0, L, Qs, nullptr, 0.f);
#pragma unroll
    for (int h = 0; h < 2; ++h) {            // dO rows as given (zero past L)
      const int c = tid + 256 * h;
      const int tok = c / 8, ch = c % 8;
      uint4 u = make_uint4(0u, 0u, 0u, 0u);
      if (t0 + tok < L) u = *reinterpret_cast<const uint4*>(dO + base + static_cast<size_t>(t0 + tok) * kD + 8 * ch);
      *reinterpret_cast<uint4*>(&Ds[tok][8 * ch]) = u;
    }
    __syncthreads();
    const bool live = t0 + tl < L;
    // (1) S^T = W' Q^T (rows: features 16 ft + 4 g + v; column: token tl).
    f32x4 S[FT];
#pragma unroll
    for (int ft = 0; ft < FT; ++ft) {
      S[ft] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        S[ft] = mma_f16(ld_f16x8(w16 + (16 * ft + l16) * kD + 32 * ks + 8 * g),
                        ld_f16x8(&Qs[tl][32 * ks + 8 * g]), S[ft]);
      if (ft % 4 == 3) __builtin_amdgcn_sched_barrier(0);   // bounded operand lookahead
    }
    // Query features: + c, row reference M (ReLU: none).
    float Mrow = 0.f;
    if constexpr (!RELU) {
      float mx = -INFINITY;
#pragma unroll
      for (int ft = 0; ft < FT; ++ft) {
        const float4 c4 = *reinterpret_cast<const float4*>(cfh + 16 * ft + 4 * g);
        S[ft][0] += c4.x; S[ft][1] += c4.y; S[ft][2] += c4.z; S[ft][3] += c4.w;
        mx = fmaxf(mx, max3(S[ft][0], S[ft][1], fmaxf(S[ft][2], S[ft][3])));
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      Mrow = mx;
    }
#pragma unroll
    for (int ft = 0; ft < FT; ++ft)
#pragma unroll
      for (int v = 0; v < 4; ++v) S[ft][v] = feature<RELU>(S[ft][v] - Mrow);
    // Q~ to QF [token][feature] (4 features per lane) and QT [feature][token].
#pragma unroll
    for (int ft = 0; ft < FT; ++ft) {
      st_bf16x4(&QF[tl][16 * ft + 4 * g], S[ft][0], S[ft][1], S[ft][2], S[ft][3]);
#pragma unroll
      for (int v = 0; v < 4; ++v) QT[16 * ft + 4 * g + v][tl] = bf16_bits(S[ft][v]);
    }
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    // (2) [num | den]^T = KzT Q~^T (rows: columns 16 ct + 4 g + v; column: token tl).
    f32x4 N[5];
#pragma unroll
    for (int ct = 0; ct < 5; ++ct) {
      N[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KF; ++ks) {
        const bf16x8 qb = ld_bf16x8(&QF[tl][32 * ks + 8 * g]);
        N[ct] = mma_bf16(ld_bf16x8(kzt + (16 * ct + l16) * M + 32 * ks + 8 * g), qb, N[ct]);
        N[ct] = mma_bf16(ld_bf16x8(kzt + (80 + 16 * ct + l16) * M + 32 * ks + 8 * g), qb, N[ct]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // den (column 64: ct 4, g 0, v 0) to every lane of the token
    const float den = __shfl(N[4][0], l16);
    // U = dO / den, u0 = -(dO . num) / den^2; dO rows past L are zero.
    float dov[4][4];
    float dot = 0.f;
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      ld_bf16x4(&Ds[tl][16 * ct + 4 * g], dov[ct]);
#pragma unroll
      for (int v = 0; v < 4; ++v) dot = fmaf(dov[ct][v], N[ct][v], dot);
    }
    dot += __shfl_xor(dot, 16);
    dot += __shfl_xor(dot, 32);
    const float rden = live ? 1.f / den : 0.f;
    const float u0 = -dot * rden * rden;
    // Ucat^T as bf16 hi + lo
    auto put = [&](int row, float x) {
      const uint16_t hi = bf16_bits(x);
      UT[0][row][tl] = hi;
      UT[1][row][tl] = bf16_bits(x - __uint_as_float(static_cast<uint32_t>(hi) << 16));
    };
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
#pragma unroll
      for (int v = 0; v < 4; ++v) put(16 * ct + 4 * g + v, dov[ct][v] * rden);
    if (g == 0) put(64, u0);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    // (3) T^T = S~ U^T + z~ u0 (rows: features; column: token tl), P = Q~ T
    // (Q~ read back from QF as the bf16 operand the products used, then P
    // written in its place).
    float psum = 0.f;
#pragma unroll
    for (int ft = 0; ft < FT; ++ft) {
      float qf[4];
      ld_bf16x4(&QF[tl][16 * ft + 4 * g], qf);
      f32x4 T = f32x4{0.f, 0.f, 0.f, 0.f};   // S~ . dO (hi + lo), scaled by 1/den below
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 db = ld_bf16x8(&Ds[tl][32 * ks + 8 * g]);
        T = mma_bf16(ld_bf16x8(kzf + (16 * ft + l16) * kD + 32 * ks + 8 * g), db, T);
        T = mma_bf16(ld_bf16x8(kzf + (M + 16 * ft + l16) * kD + 32 * ks + 8 * g), db, T);
      }
      const float4 z4 = *reinterpret_cast<const float4*>(zfh + 16 * ft + 4 * g);
      const float zz[4] = {z4.x, z4.y, z4.z, z4.w};
      float p[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float tv = fmaf(zz[v], u0, T[v] * rden);
        p[v] = RELU ? (qf[v] > 0.f ? tv : 0.f) : qf[v] * tv;
        psum += p[v];
      }
      st_bf16x4(&QF[tl][16 * ft + 4 * g], p[0], p[1], p[2], p[3]);
      if (ft % 4 == 3) __builtin_amdgcn_sched_barrier(0);
    }
    psum += __shfl_xor(psum, 16);
    psum += __shfl_xor(psum, 32);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    // (4) dq^T = W^T P^T (rows: d columns 16 at + 4 g + v; column: token tl).
    // (Every lane takes part in the products; only live tokens are stored.)
    {
#pragma unroll
      for (int at = 0; at < 4; ++at) {
        f32x4 Dq = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KF; ++ks)
          Dq = mma_bf16(ld_bf16x8(wt + (16 * at + l16) * M + 32 * ks + 8 * g),
                        ld_bf16x8(&QF[tl][32 * ks + 8 * g]), Dq);
        const int a0 = 16 * at + 4 * g;
        float o[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float qv = static_cast<float>(Qs[tl][a0 + v]);
          o[v] = RELU ? Dq[v] * kLog2e : fmaf(-2.f * knorm * psum, qv, Dq[v]);
        }
        if (live)
          st_bf16x4(dQ + base + static_cast<size_t>(t0 + tl) * kD + a0, o[0], o[1], o[2], o[3]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // (5) G (this wave's feature rows) += Q~^T Ucat over the tile's 64 tokens.
#pragma unroll
    for (int a = 0; a < GFT; ++a) {
      const int f = wave * (M / 4) + 16 * a + l16;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 qa = ld_bf16x8(&QT[f][32 * ks + 8 * g]);
#pragma unroll
        for (int ct = 0; ct < 5; ++ct) {
          G[a][ct] = mma_bf16(qa, ld_bf16x8(&UT[0][16 * ct + l16][32 * ks + 8 * g]), G[a][ct]);
          G[a][ct] = mma_bf16(qa, ld_bf16x8(&UT[1][16 * ct + l16][32 * ks + 8 * g]), G[a][ct]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // Block partial: Gp [bh][qb][f][c], rows f = wave m/4 + 16 a + 4 g + v, column 16 ct + l16.
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

// ---------------------------------------------------------------------------
// gcombine: G = sum over query blocks (block order) -> GF [2][m][64] bf16
// (hi, lo), GT [64][m] bf16, Gz [m] fp32 (the ones column).
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
    GT[(static_cast<size_t>(bh) * kD + c) * m + f] = x;
  } else {
    Gz[static_cast<size_t>(bh) * m + f] = acc;
  }
}

// ---------------------------------------------------------------------------
// bkey: grid (BH * ceil(L/64)), 256 threads, one 64-key tile per work-group,
// wave w owns keys 16w..16w+15.
// ---------------------------------------------------------------------------
template <int M, bool RELU>
__global__ __launch_bounds__(256, 1) void bkey(
    const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const _Float16* __restrict__ W16, const uint16_t* __restrict__ WT,
    const uint16_t* __restrict__ GF, const uint16_t* __restrict__ GT,
    const float* __restrict__ Gz, const float* __restrict__ cf, uint16_t* __restrict__ dK,
    uint16_t* __restrict__ dV, int L, int ntile, float knorm) {
  constexpr int FT = M / 16;
  constexpr int KF = M / 32;
  constexpr int FRow = M + 8;
  const int bh = blockIdx.x / ntile, t0 = (blockIdx.x % ntile) * kTok;
  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
  const int l16 = lane % 16, g = lane / 16;
  __shared__ _Float16 Ks[kTok][kQRow];
  __shared__ uint16_t Vs[kTok][kQRow];
  __shared__ uint16_t RF[kTok][FRow];     // R [key][feature]
  __shared__ uint16_t KF_[kTok][FRow];    // K~ [key][feature]
  __shared__ float nk[kTok];

  const size_t base = static_cast<size_t>(bh) * L * kD;
  const uint16_t* gf = GF + static_cast<size_t>(bh) * 2 * M * kD;   // hi; lo at + M kD
  const uint16_t* gt = GT + static_cast<size_t>(bh) * kD * M;
  const float* gz = Gz + static_cast<size_t>(bh) * M;
  const float* cfh = cf + static_cast<size_t>(bh) * M;
  stage_f16(K, base, t0, L, Ks, nk, knorm * kLog2e);
  {
    // V rows as bf16 (as stored)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = tid + 256 * h;
      const int tok = c / 8, ch = c % 8;
      uint4 u = make_uint4(0u, 0u, 0u, 0u);
      if (t0 + tok < L) u = *reinterpret_cast<const uint4*>(V + base + static_cast<size_t>(t0 + tok) * kD + 8 * ch);
      *reinterpret_cast<uint4*>(&Vs[tok][8 * ch]) = u;
    }
  }
  __syncthreads();
  const int tl = 16 * wave + l16;
  const bool live = t0 + tl < L;
  // (1) E^T = W' K^T - n - c (rows: features; column: key tl), K~ = exp2(E).
  f32x4 E[FT];
  const float ntok = nk[tl];
#pragma unroll
  for (int ft = 0; ft < FT; ++ft) {
    E[ft] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
      E[ft] = mma_f16(ld_f16x8(W16 + (16 * ft + l16) * kD + 32 * ks + 8 * g),
                      ld_f16x8(&Ks[tl][32 * ks + 8 * g]), E[ft]);
    if constexpr (!RELU) {
      const float4 c4 = *reinterpret_cast<const float4*>(cfh + 16 * ft + 4 * g);
      E[ft][0] -= ntok + c4.x; E[ft][1] -= ntok + c4.y;
      E[ft][2] -= ntok + c4.z; E[ft][3] -= ntok + c4.w;
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) E[ft][v] = feature<RELU>(E[ft][v]);
    st_bf16x4(&KF_[tl][16 * ft + 4 * g], E[ft][0], E[ft][1], E[ft][2], E[ft][3]);
  }
  // (2) H^T = G V^T + Gz (rows: features; column: key tl), R = K~ H.
  float rsum = 0.f;
#pragma unroll
  for (int ft = 0; ft < FT; ++ft) {
    f32x4 H = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const bf16x8 vb = ld_bf16x8(&Vs[tl][32 * ks + 8 * g]);
      H = mma_bf16(ld_bf16x8(gf + (16 * ft + l16) * kD + 32 * ks + 8 * g), vb, H);
      H = mma_bf16(ld_bf16x8(gf + (M + 16 * ft + l16) * kD + 32 * ks + 8 * g), vb, H);
    }
    const float4 z4 = *reinterpret_cast<const float4*>(gz + 16 * ft + 4 * g);
    const float zz[4] = {z4.x, z4.y, z4.z, z4.w};
    float r[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const float hv = H[v] + zz[v];
      r[v] = RELU ? (E[ft][v] > 0.f ? hv : 0.f) : E[ft][v] * hv;
      rsum += r[v];
    }
    st_bf16x4(&RF[tl][16 * ft + 4 * g], r[0], r[1], r[2], r[3]);
  }
  rsum += __shfl_xor(rsum, 16);
  rsum += __shfl_xor(rsum, 32);
  __syncthreads();
  // (3) dk^T = W^T R^T - 2 knorm (sum_r R) k; (4) dv^T = G^T K~^T (every lane
  // takes part in the products; only live keys are stored).
#pragma unroll
  for (int at = 0; at < 4; ++at) {
    f32x4 Dk = f32x4{0.f, 0.f, 0.f, 0.f}, Dv = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KF; ++ks) {
      Dk = mma_bf16(ld_bf16x8(WT + (16 * at + l16) * M + 32 * ks + 8 * g),
                    ld_bf16x8(&RF[tl][32 * ks + 8 * g]), Dk);
      Dv = mma_bf16(ld_bf16x8(gt + (16 * at + l16) * M + 32 * ks + 8 * g),
                    ld_bf16x8(&KF_[tl][32 * ks + 8 * g]), Dv);
    }
    const int a0 = 16 * at + 4 * g;
    float o[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const float kv = static_cast<float>(Ks[tl][a0 + v]);
      o[v] = RELU ? Dk[v] * kLog2e : fmaf(-2.f * knorm * rsum, kv, Dk[v]);
    }
    if (live) {
      const size_t row = base + static_cast<size_t>(t0 + tl) * kD + a0;
      st_bf16x4(dK + row, o[0], o[1], o[2], o[3]);
      st_bf16x4(dV + row, Dv[0], Dv[1], Dv[2], Dv[3]);
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
  timing_before(st);
  bquery<M, RELU><<<dim3(p.BH * b.nqb), 256, 0, st>>>(Q, dO, W16, WT, KzT, KzF, zf, cf, dQ, Gp,
                                                       p.L, b.qblk, b.nqb, p.knorm);
  e = hipGetLastError();
  timing_after(st, "bquery");
  if (e != hipSuccess) return e;
  timing_before(st);
  gcombine<<<dim3((M * (kD + 1) + 255) / 256, p.BH), 256, 0, st>>>(Gp, GF, GT, Gz, M, b.nqb);
  e = hipGetLastError();
  timing_after(st, "gcombine");
  if (e != hipSuccess) return e;
  const int ntile = (p.L + kTok - 1) / kTok;
  timing_before(st);
  bkey<M, RELU><<<dim3(p.BH * ntile), 256, 0, st>>>(K, V, W16, WT, GF, GT, Gz, cf, dK, dV, p.L,
                                                     ntile, p.knorm);
  e = hipGetLastError();
  timing_after(st, "bkey");
  return e;
}

}  // namespace

bool mfma_bwd_supported(int32_t d, int32_t m, int32_t dtype, int32_t causal) {
  return dtype == FAVOR_BF16 && !causal && d == kD && (m == 64 || m == 128 || m == 192 ||
                                                       m == 256) &&
         mfma_bidir_supported(d, m, dtype);
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
#define FAVOR_BCASE(M)                                                                   \
  if (p.m == M)                                                                          \
    return p.relu ? launch_bwd<M, true>(p, b, q, k, v, W, g, dq, dk, dv, w, stream)      \
                  : launch_bwd<M, false>(p, b, q, k, v, W, g, dq, dk, dv, w, stream);
  FAVOR_BCASE(64) FAVOR_BCASE(128) FAVOR_BCASE(192) FAVOR_BCASE(256)
#undef FAVOR_BCASE
  return hipErrorInvalidValue;
}

}  // namespace favor
