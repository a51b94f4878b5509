// Bidirectional FAVOR+ on the matrix cores (bf16 inputs, d in {64, 128}).
//
// FA-part of the "FAVOR+" method page: O = D^-1 (Q' ((K')^T V)),
// D = diag(Q' ((K')^T 1_L)), with phi(x) = exp(w . x - |x|^2/2)/sqrt(m).
// Three launches:
//
//   kpart    per (head, sequence split): for each 32-token tile the feature
//            exponents S = K W'^T - |k|^2/2 (fp16 MFMA; W' = W log2 e so the
//            exponentials are exp2), a per-feature running reference c_r (the
//            maximum exponent seen so far, raised only when a tile exceeds it
//            by more than kTau), K~ = exp2(S - c_r) in bf16, and the
//            contraction [V | 1]^T K~ accumulated in fp32 (bf16 MFMA).  Each
//            wave owns a slice of features; the 32-token tile is staged once
//            per work-group in LDS (K in fp16, V transposed).
//   kcombine per head: the splits' partial states, rescaled to the largest
//            per-feature reference, summed in split order; written as the
//            bf16 operand of the query side.
//   qapply   per (head, query block): query exponents with the key references
//            added (s_ir + c_r), a per-row reference over 64-feature chunks
//            (set by the first chunk, raised lazily), Q~ = exp2(. - M_i) in
//            bf16, the product [KV | z]^T Q~^T in fp32 on the matrix cores, and
//            O = num / den.
//
// The shifts cancel exactly: sum_r e^{s_ir + c_r - M_i} sum_j e^{e_jr - c_r}
// [v_j | 1] = e^{-M_i} sum_r e^{s_ir} sum_j e^{e_jr} [v_j | 1].
//
// Numerics: Q and K are converted to fp16 for the projection (exact for
// |x| < 65504 outside fp16's subnormal range), W' is rounded to fp16, the
// features and [KV | z] are rounded to bf16 (full fp32 exponent range), all
// sums are fp32.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "favor.h"
#include "favor_internal.h"
#include "mfma_common.h"

namespace favor {
namespace {

using namespace mfma;

// A reference (per key feature, or per query row) is set by the first tile or
// chunk and raised only when a later one exceeds it by more than kTau (log2
// units): features then stay below 2^kTau, far inside bf16/fp32 range, and
// raises (which rescale the accumulators) are rare.
constexpr float kTau = 20.0f;

#ifndef FAVOR_QAPPLY_NTQ
#define FAVOR_QAPPLY_NTQ 2      // 16-token tiles per query-side wave iteration
#endif
constexpr int kTT = 32;        // tokens per key tile

template <int D>
struct KCfg {
  static constexpr int FPW = (D == 64) ? 64 : 32;  // features per wave
  static constexpr int NT = FPW / 16;               // feature tiles per wave
  static constexpr int KS = D / 32;                 // projection k-steps
  static constexpr int MV = D / 16;                 // value-column tiles
  static constexpr int KROW = D + 8;                // fp16 per K row in LDS
  static constexpr int VROW = kTT + 8;              // bf16 per V^T row in LDS
  static constexpr int CPR = D / 8;                 // 16-byte chunks per row
  static constexpr int CH = kTT * CPR;              // chunks per tile and tensor
};

// ---------------------------------------------------------------------------
// kpart: grid (nsplit, BH), NW waves of 64 threads, wave w owns features
// [w FPW, (w+1) FPW).  Output: P [BH][nsplit][D+1][m] fp32 (row D = z) and
// cs [BH][nsplit][m] fp32 (per-feature references, log2 units).
// ---------------------------------------------------------------------------
template <int D, int NW>
__global__ __launch_bounds__(NW * 64, 2) void kpart(const uint16_t* __restrict__ K,
                                                 const uint16_t* __restrict__ V,
                                                 const float* __restrict__ W,
                                                 float* __restrict__ P, float* __restrict__ cs,
                                                 int L, int m, int SL, int nsplit) {
  using C = KCfg<D>;
  constexpr int NTH = NW * 64;
  constexpr int CPT = (C::CH + NTH - 1) / NTH;
  const int s = blockIdx.x, bh = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int f0 = wave * C::FPW;

  __shared__ __align__(16) _Float16 Ks[2][kTT][C::KROW];
  __shared__ __align__(16) uint16_t Vt[2][D][C::VROW];
  __shared__ __align__(16) float Ns[2][kTT];   // -|k|^2 log2(e) / 2 per token

  // Projection B operands, kept in registers: W'[f][32 ks + 8 g + u].
  f16x8 wb[C::NT][C::KS];
#pragma unroll
  for (int nt = 0; nt < C::NT; ++nt) {
    const float* wr = W + static_cast<size_t>(f0 + 16 * nt + l16) * D + 8 * g;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      const float4 a = *reinterpret_cast<const float4*>(wr + 32 * ks);
      const float4 b = *reinterpret_cast<const float4*>(wr + 32 * ks + 4);
      f16x8 v;
      v[0] = static_cast<_Float16>(a.x * kLog2e); v[1] = static_cast<_Float16>(a.y * kLog2e);
      v[2] = static_cast<_Float16>(a.z * kLog2e); v[3] = static_cast<_Float16>(a.w * kLog2e);
      v[4] = static_cast<_Float16>(b.x * kLog2e); v[5] = static_cast<_Float16>(b.y * kLog2e);
      v[6] = static_cast<_Float16>(b.z * kLog2e); v[7] = static_cast<_Float16>(b.w * kLog2e);
      wb[nt][ks] = v;
    }
  }

  f32x4 acc[C::MV + 1][C::NT];
#pragma unroll
  for (int i = 0; i <= C::MV; ++i)
#pragma unroll
    for (int nt = 0; nt < C::NT; ++nt) acc[i][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float cref[C::NT];   // per-feature reference (log2 units)
#pragma unroll
  for (int nt = 0; nt < C::NT; ++nt) cref[nt] = 0.f;
  bool fresh = true;   // no tile seen yet: the first tile sets the references

  const int j0 = s * SL, j1 = min(L, j0 + SL);
  const int ntiles = (j1 - j0 + kTT - 1) / kTT;
  const size_t base = static_cast<size_t>(bh) * L * D;

  // Global loads of tile t+1 are in flight while tile t is computed.
  uint4 kA[CPT], vA[CPT];
  auto gload = [&](int t, uint4 (&kreg)[CPT], uint4 (&vreg)[CPT]) {
    const int jt = j0 + t * kTT;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + i * NTH;
      const int j = c / C::CPR, ch = c % C::CPR;
      const int tok = jt + j;
      if (c < C::CH && tok < j1) {
        const size_t off = base + static_cast<size_t>(tok) * D + ch * 8;
        kreg[i] = *reinterpret_cast<const uint4*>(K + off);
        vreg[i] = *reinterpret_cast<const uint4*>(V + off);
      } else {
        kreg[i] = make_uint4(0, 0, 0, 0);
        vreg[i] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto lstore = [&](int buf, int t, const uint4 (&kreg)[CPT], const uint4 (&vreg)[CPT]) {
    const int jt = j0 + t * kTT;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + i * NTH;
      const int j = (c / C::CPR) % kTT, ch = c % C::CPR;
      const uint4 kv = kreg[i];
      float ss = 0.f;
      {
        const uint32_t w4[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float lo = bf16_lo(w4[q]), hi = bf16_hi(w4[q]);
          ss = fmaf(lo, lo, ss);
          ss = fmaf(hi, hi, ss);
        }
      }
      // Sum of squares over the CPR threads holding one token (consecutive lanes).
      ss = group_sum<C::CPR>(ss);
      if (c < C::CH) {
        uint4 h;
        h.x = bf16x2_to_f16x2(kv.x); h.y = bf16x2_to_f16x2(kv.y);
        h.z = bf16x2_to_f16x2(kv.z); h.w = bf16x2_to_f16x2(kv.w);
        *reinterpret_cast<uint4*>(&Ks[buf][j][ch * 8]) = h;
        const uint32_t v4[4] = {vreg[i].x, vreg[i].y, vreg[i].z, vreg[i].w};
        const int pj = perm_inv(j);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          Vt[buf][ch * 8 + 2 * q][pj] = static_cast<uint16_t>(v4[q] & 0xffffu);
          Vt[buf][ch * 8 + 2 * q + 1][pj] = static_cast<uint16_t>(v4[q] >> 16);
        }
        if (ch == 0) Ns[buf][j] = (jt + j < j1) ? -0.5f * kLog2e * ss : -INFINITY;
      }
    }
  };

  bf16x8 ones;
#pragma unroll
  for (int u = 0; u < 8; ++u) ones[u] = static_cast<__bf16>(1.0f);

  auto compute = [&](const int buf) {
    // S = K W'^T - n'  (rows: tokens 16 mt + 4 g + v; column: feature f0 + 16 nt + l16)
    f32x4 S[2][C::NT];
    {
      f32x4 cinit[2];
      f16x8 ka[2][C::KS];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        cinit[mt] = *reinterpret_cast<const f32x4*>(&Ns[buf][16 * mt + 4 * g]);
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks)
          ka[mt][ks] = *reinterpret_cast<const f16x8*>(&Ks[buf][16 * mt + l16][32 * ks + 8 * g]);
      }
      // k-step outermost: consecutive MFMAs are independent.
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int nt = 0; nt < C::NT; ++nt)
            S[mt][nt] = mma_f16(ka[mt][ks], wb[nt][ks], ks == 0 ? cinit[mt] : S[mt][nt]);
    }

    // Exponents relative to the per-feature reference, their tile maximum,
    // and the lazy reference update (always on the work-group's first tile).
    float e[C::NT][8];
    bool raise = false;
    float tm[C::NT];
#pragma unroll
    for (int nt = 0; nt < C::NT; ++nt) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        e[nt][v] = S[0][nt][v] - cref[nt];
        e[nt][4 + v] = S[1][nt][v] - cref[nt];
      }
      const float a = max3(e[nt][0], e[nt][1], e[nt][2]);
      const float b = max3(e[nt][3], e[nt][4], e[nt][5]);
      tm[nt] = max3(a, b, fmaxf(e[nt][6], e[nt][7]));   // this lane's 8 tokens
      raise |= tm[nt] > kTau;
    }
    // Only the first tile, or a lane above the headroom, needs the exact
    // per-feature maximum (a column reduction) and a reference update.
    if (__builtin_expect(fresh || __ballot(raise) != 0, 0)) {
#pragma unroll
      for (int nt = 0; nt < C::NT; ++nt) {
        tm[nt] = colmax4(tm[nt]);
        const float dlt = (fresh || tm[nt] > kTau) ? tm[nt] : 0.f;
        if (!fresh) {   // accumulators are still zero on the first tile
          const float f = fast_exp2(-dlt);
#pragma unroll
          for (int i = 0; i <= C::MV; ++i) acc[i][nt] *= f;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) e[nt][u] -= dlt;
        cref[nt] += dlt;
      }
    }
    fresh = false;

    // K~ = exp2(e) as the contraction's B operand (positions perm_of).
    bf16x8 kb[C::NT];
#pragma unroll
    for (int nt = 0; nt < C::NT; ++nt) {
      uint32_t p[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) p[q] = pack_bf16(fast_exp2(e[nt][2 * q]), fast_exp2(e[nt][2 * q + 1]));
      kb[nt] = __builtin_bit_cast(bf16x8, make_uint4(p[0], p[1], p[2], p[3]));
    }

    // [V | 1]^T K~ : rows = value columns, columns = features.
#pragma unroll
    for (int mv = 0; mv < C::MV; ++mv) {
      const bf16x8 va = *reinterpret_cast<const bf16x8*>(&Vt[buf][16 * mv + l16][8 * g]);
#pragma unroll
      for (int nt = 0; nt < C::NT; ++nt) acc[mv][nt] = mma_bf16(va, kb[nt], acc[mv][nt]);
    }
#pragma unroll
    for (int nt = 0; nt < C::NT; ++nt) acc[C::MV][nt] = mma_bf16(ones, kb[nt], acc[C::MV][nt]);

  };

  gload(0, kA, vA);
  lstore(0, 0, kA, vA);
  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < ntiles) gload(t + 1, kA, vA);
    lds_barrier();
    compute(buf);
    if (t + 1 < ntiles) lstore(buf ^ 1, t + 1, kA, vA);
  }

  // Partial state out: P[bh][s][row][f].
  const size_t pb = (static_cast<size_t>(bh) * nsplit + s) * (D + 1);
#pragma unroll
  for (int nt = 0; nt < C::NT; ++nt) {
    const int f = f0 + 16 * nt + l16;
#pragma unroll
    for (int mv = 0; mv < C::MV; ++mv)
#pragma unroll
      for (int v = 0; v < 4; ++v) P[(pb + 16 * mv + 4 * g + v) * m + f] = acc[mv][nt][v];
    if (g == 0) {
      P[(pb + D) * m + f] = acc[C::MV][nt][0];
      cs[(static_cast<size_t>(bh) * nsplit + s) * m + f] = cref[nt];
    }
  }
}

// ---------------------------------------------------------------------------
// kcombine: grid (ceil((D+16) * m / 256), BH), 256 threads, one thread per
// (row, feature) entry of the combined state.  The splits are summed in split
// order after rescaling to the largest per-feature reference.  Output Kz
// [BH][D+16][m+8] bf16 in the query side's operand order (features permuted
// within 32-blocks; row D = z, rows above D zero) and cfin [BH][m].  Head 0's
// work-groups also write W16 [m][D+8]: W log2(e) in fp16, the query side's
// projection operand.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void kcombine(const float* __restrict__ P,
                                                const float* __restrict__ cs,
                                                const float* __restrict__ W,
                                                uint16_t* __restrict__ Kz,
                                                float* __restrict__ cfin,
                                                _Float16* __restrict__ W16, int m, int nsplit) {
  const int bh = blockIdx.y;
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (bh == 0) {
    for (int i = e; i < m * D; i += gridDim.x * 256) {
      const int f = i / D, a = i - f * D;
      W16[static_cast<size_t>(f) * (D + 8) + a] = static_cast<_Float16>(W[i] * kLog2e);
    }
  }
  if (e >= (D + 16) * m) return;
  const int row = e / m, f = e - row * m;
  const size_t cb = static_cast<size_t>(bh) * nsplit * m + f;
  float cmax = -INFINITY;
  for (int s = 0; s < nsplit; ++s) cmax = fmaxf(cmax, cs[cb + static_cast<size_t>(s) * m]);
  float a = 0.f;
  if (row <= D) {
    for (int s = 0; s < nsplit; ++s) {
      const float sc = fast_exp2(cs[cb + static_cast<size_t>(s) * m] - cmax);
      a = fmaf(P[((static_cast<size_t>(bh) * nsplit + s) * (D + 1) + row) * m + f], sc, a);
    }
  }
  const int kzrow = m + 8;
  const int pos = (f & ~31) + perm_inv(f & 31);
  Kz[(static_cast<size_t>(bh) * (D + 16) + row) * kzrow + pos] =
      static_cast<uint16_t>(pack_bf16(a, 0.f) & 0xffffu);
  if (row == 0) cfin[static_cast<size_t>(bh) * m + f] = cmax;
}

// ---------------------------------------------------------------------------
// qapply: grid (nqb, BH), NW waves; each wave takes 16*NTQ-token tiles of the
// block [qb QL, (qb+1) QL).  LDS: W' fp16 [m][D+8], Kz bf16 [D+16][m+8],
// c [m] fp32 (dynamic).
// ---------------------------------------------------------------------------
template <int D, int NTQ_>
struct QCfg {
  static constexpr int NTQ = NTQ_;                // token tiles per wave tile
  static constexpr int TQ = 16 * NTQ;
  static constexpr int KS = D / 32;
  static constexpr int MV = D / 16;
  static constexpr int WROW = D + 8;
};

template <int D>
size_t qapply_lds_bytes(int m) {
  return static_cast<size_t>(m) * (D + 8) * 2 + static_cast<size_t>(D + 16) * (m + 8) * 2 +
         static_cast<size_t>(m) * 4;
}

template <int D, int NW, int NTQ>
__global__ __launch_bounds__(NW * 64, 2) void qapply(const uint16_t* __restrict__ Q,
                                                  const _Float16* __restrict__ W16,
                                                  const uint16_t* __restrict__ Kz,
                                                  const float* __restrict__ cfin,
                                                  uint16_t* __restrict__ O, int L, int m, int QL) {
  using C = QCfg<D, NTQ>;
  constexpr int NTH = NW * 64;
  extern __shared__ __align__(16) unsigned char smem[];
  _Float16* Wl = reinterpret_cast<_Float16*>(smem);
  uint16_t* Kzl = reinterpret_cast<uint16_t*>(smem + static_cast<size_t>(m) * C::WROW * 2);
  float* cl = reinterpret_cast<float*>(smem + static_cast<size_t>(m) * C::WROW * 2 +
                                       static_cast<size_t>(D + 16) * (m + 8) * 2);
  const int qb = blockIdx.x, bh = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int kzrow = m + 8;

  // Stage W' (fp16), Kz and c for this head.
  {
    const uint4* src = reinterpret_cast<const uint4*>(W16);
    uint4* dst = reinterpret_cast<uint4*>(Wl);
    const int n16 = m * C::WROW / 8;
    for (int i = tid; i < n16; i += NTH) dst[i] = src[i];
  }
  {
    const uint4* src = reinterpret_cast<const uint4*>(Kz + static_cast<size_t>(bh) * (D + 16) * kzrow);
    uint4* dst = reinterpret_cast<uint4*>(Kzl);
    const int n16 = (D + 16) * kzrow / 8;
    for (int i = tid; i < n16; i += NTH) dst[i] = src[i];
  }
  for (int i = tid; i < m; i += NTH) cl[i] = cfin[static_cast<size_t>(bh) * m + i];
  __syncthreads();

  const size_t base = static_cast<size_t>(bh) * L * D;
  const int q0 = qb * QL, q1 = min(L, q0 + QL);
  const int nch = m / 64;

  // Q tiles: raw bf16 loads one tile ahead of their use, two register sets.
  using Raw = uint4[C::NTQ][C::KS];
  auto qload = [&](int tt, Raw& raw) {
#pragma unroll
    for (int nt = 0; nt < C::NTQ; ++nt) {
      const int tok = tt + 16 * nt + l16;
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks)
        raw[nt][ks] = (tok < q1) ? *reinterpret_cast<const uint4*>(
                                       Q + base + static_cast<size_t>(tok) * D + 32 * ks + 8 * g)
                                 : make_uint4(0, 0, 0, 0);
    }
  };
  // Q^T operands: token tt + 16 nt + l16, dims 32 ks + 8 g .. +7, in fp16.
  auto convert = [&](const Raw& raw, f16x8 (&qb_)[C::NTQ][C::KS]) {
#pragma unroll
    for (int nt = 0; nt < C::NTQ; ++nt)
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        const uint4 x = raw[nt][ks];
        uint4 h;
        h.x = bf16x2_to_f16x2(x.x); h.y = bf16x2_to_f16x2(x.y);
        h.z = bf16x2_to_f16x2(x.z); h.w = bf16x2_to_f16x2(x.w);
        qb_[nt][ks] = __builtin_bit_cast(f16x8, h);
      }
  };
  auto tile = [&](const int tt, const f16x8 (&qb_)[C::NTQ][C::KS]) {
    f32x4 acc[C::MV + 1][C::NTQ];
#pragma unroll
    for (int i = 0; i <= C::MV; ++i)
#pragma unroll
      for (int nt = 0; nt < C::NTQ; ++nt) acc[i][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float M[C::NTQ];   // per-row reference (log2 units), set by the first chunk
#pragma unroll
    for (int nt = 0; nt < C::NTQ; ++nt) M[nt] = 0.f;

    for (int ch = 0; ch < nch; ++ch) {
      // S^T = W' Q^T + c  (rows: features 64 ch + 16 mt + 4 g + v; column: token)
      f32x4 S[4][C::NTQ];
      {
        f32x4 cb[4];
        f16x8 wa[4][C::KS];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          const int fr = 64 * ch + 16 * mt;
          cb[mt] = *reinterpret_cast<const f32x4*>(&cl[fr + 4 * g]);
#pragma unroll
          for (int ks = 0; ks < C::KS; ++ks)
            wa[mt][ks] = *reinterpret_cast<const f16x8*>(
                &Wl[static_cast<size_t>(fr + l16) * C::WROW + 32 * ks + 8 * g]);
        }
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
          for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int nt = 0; nt < C::NTQ; ++nt)
              S[mt][nt] = mma_f16(wa[mt][ks], qb_[nt][ks], ks == 0 ? cb[mt] : S[mt][nt]);
      }
      // Exponents relative to the row reference; the first chunk sets the
      // reference to the chunk's row maximum, later chunks raise it lazily.
      float e[4][C::NTQ][4];
      bool raise = false;
      float cm[C::NTQ];
#pragma unroll
      for (int nt = 0; nt < C::NTQ; ++nt) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int v = 0; v < 4; ++v) e[mt][nt][v] = S[mt][nt][v] - M[nt];
        const float a = max3(e[0][nt][0], e[0][nt][1], e[0][nt][2]);
        const float b = max3(e[0][nt][3], e[1][nt][0], e[1][nt][1]);
        const float c = max3(e[1][nt][2], e[1][nt][3], e[2][nt][0]);
        const float d = max3(e[2][nt][1], e[2][nt][2], e[2][nt][3]);
        const float f = max3(e[3][nt][0], e[3][nt][1], e[3][nt][2]);
        cm[nt] = max3(max3(a, b, c), max3(d, f, e[3][nt][3]), a);   // this lane's 16 features
        raise |= cm[nt] > kTau;
      }
      // Only the first chunk, or a lane above the headroom, needs the exact
      // row maximum (a column reduction) and a reference update.
      if (__builtin_expect(ch == 0 || __ballot(raise) != 0, 0)) {
#pragma unroll
        for (int nt = 0; nt < C::NTQ; ++nt) {
          cm[nt] = colmax4(cm[nt]);
          const float dlt = (ch == 0 || cm[nt] > kTau) ? cm[nt] : 0.f;
          if (ch != 0) {   // accumulators are still zero on the first chunk
            const float f = fast_exp2(-dlt);
#pragma unroll
            for (int i = 0; i <= C::MV; ++i) acc[i][nt] *= f;
          }
#pragma unroll
          for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int v = 0; v < 4; ++v) e[mt][nt][v] -= dlt;
          M[nt] += dlt;
        }
      }
      // Q~^T operands (features at positions perm_of within each 32-block).
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        bf16x8 qt[C::NTQ];
#pragma unroll
        for (int nt = 0; nt < C::NTQ; ++nt) {
          uint32_t p[4];
          p[0] = pack_bf16(fast_exp2(e[2 * kb][nt][0]), fast_exp2(e[2 * kb][nt][1]));
          p[1] = pack_bf16(fast_exp2(e[2 * kb][nt][2]), fast_exp2(e[2 * kb][nt][3]));
          p[2] = pack_bf16(fast_exp2(e[2 * kb + 1][nt][0]), fast_exp2(e[2 * kb + 1][nt][1]));
          p[3] = pack_bf16(fast_exp2(e[2 * kb + 1][nt][2]), fast_exp2(e[2 * kb + 1][nt][3]));
          qt[nt] = __builtin_bit_cast(bf16x8, make_uint4(p[0], p[1], p[2], p[3]));
        }
        const int kcol = 64 * ch + 32 * kb + 8 * g;
#pragma unroll
        for (int mv = 0; mv <= C::MV; ++mv) {
          const bf16x8 ka = *reinterpret_cast<const bf16x8*>(&Kzl[static_cast<size_t>(16 * mv + l16) * kzrow + kcol]);
#pragma unroll
          for (int nt = 0; nt < C::NTQ; ++nt) acc[mv][nt] = mma_bf16(ka, qt[nt], acc[mv][nt]);
        }
      }
    }

    // O = num / den; den is row 0 of the last tile (lanes with g = 0, v = 0).
#pragma unroll
    for (int nt = 0; nt < C::NTQ; ++nt) {
      const float den = __shfl(acc[C::MV][nt][0], l16, 64);
      const float inv = 1.0f / den;
      const int tok = tt + 16 * nt + l16;
      if (tok < q1) {
        uint16_t* orow = O + base + static_cast<size_t>(tok) * D + 4 * g;
#pragma unroll
        for (int mv = 0; mv < C::MV; ++mv) {
          uint2 o;
          o.x = pack_bf16(acc[mv][nt][0] * inv, acc[mv][nt][1] * inv);
          o.y = pack_bf16(acc[mv][nt][2] * inv, acc[mv][nt][3] * inv);
          *reinterpret_cast<uint2*>(orow + 16 * mv) = o;
        }
      }
    }
  };

  const int step = NW * C::TQ;
  Raw rA, rB;
  int tt = q0 + wave * C::TQ;
  if (tt < q1) qload(tt, rA);
  if (tt + step < q1) qload(tt + step, rB);
  for (; tt < q1; tt += 2 * step) {
    f16x8 qa[C::NTQ][C::KS];
    convert(rA, qa);
    if (tt + 2 * step < q1) qload(tt + 2 * step, rA);
    tile(tt, qa);
    if (tt + step >= q1) break;
    convert(rB, qa);
    if (tt + 3 * step < q1) qload(tt + 3 * step, rB);
    tile(tt + step, qa);
  }
}

template <int D, int NW>
hipError_t launch_d(const Plan& p, const uint16_t* Q, const uint16_t* K, const uint16_t* V,
                    const float* W, uint16_t* O, char* ws, hipStream_t st) {
  float* P = reinterpret_cast<float*>(ws + p.off_T);
  float* cs = reinterpret_cast<float*>(ws + p.off_cseg);
  uint16_t* Kz = reinterpret_cast<uint16_t*>(ws + p.off_KV);
  float* cfin = reinterpret_cast<float*>(ws + p.off_cfin);
  _Float16* W16 = reinterpret_cast<_Float16*>(ws + p.off_cP);
  kpart<D, NW><<<dim3(p.nseg, p.BH), NW * 64, 0, st>>>(K, V, W, P, cs, p.L, p.m, p.seg, p.nseg);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  kcombine<D><<<dim3(((D + 16) * p.m + 255) / 256, p.BH), 256, 0, st>>>(P, cs, W, Kz, cfin, W16,
                                                                        p.m, p.nseg);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t lds = qapply_lds_bytes<D>(p.m);
  constexpr int NTQ = FAVOR_QAPPLY_NTQ;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(&qapply<D, 4, NTQ>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
  if (e != hipSuccess) return e;
  const int nqb = (p.L + p.qblk - 1) / p.qblk;
  qapply<D, 4, NTQ><<<dim3(nqb, p.BH), 256, lds, st>>>(Q, W16, Kz, cfin, O, p.L, p.m, p.qblk);
  return hipGetLastError();
}

}  // namespace

bool mfma_bidir_supported(int32_t d, int32_t m, int32_t dtype) {
  if (dtype != FAVOR_BF16) return false;
  if (m % 64 != 0) return false;
  if (d == 64) return m <= 1024 && qapply_lds_bytes<64>(m) <= 160 * 1024;
  if (d == 128) return m <= 512 && qapply_lds_bytes<128>(m) <= 160 * 1024;
  return false;
}

size_t mfma_bidir_lds_bytes(int32_t d, int32_t m) {
  return d == 64 ? qapply_lds_bytes<64>(m) : qapply_lds_bytes<128>(m);
}

hipError_t mfma_bidir_forward(const Plan& p, const void* Q, const void* K, const void* V,
                              const float* W, void* O, void* ws, hipStream_t stream) {
  const auto* q = static_cast<const uint16_t*>(Q);
  const auto* k = static_cast<const uint16_t*>(K);
  const auto* v = static_cast<const uint16_t*>(V);
  auto* o = static_cast<uint16_t*>(O);
  char* w = static_cast<char*>(ws);
  if (p.d == 64) {
    switch (p.m / 64) {
      case 1: return launch_d<64, 1>(p, q, k, v, W, o, w, stream);
      case 2: return launch_d<64, 2>(p, q, k, v, W, o, w, stream);
      case 3: return launch_d<64, 3>(p, q, k, v, W, o, w, stream);
      case 4: return launch_d<64, 4>(p, q, k, v, W, o, w, stream);
      case 5: return launch_d<64, 5>(p, q, k, v, W, o, w, stream);
      case 6: return launch_d<64, 6>(p, q, k, v, W, o, w, stream);
      case 7: return launch_d<64, 7>(p, q, k, v, W, o, w, stream);
      case 8: return launch_d<64, 8>(p, q, k, v, W, o, w, stream);
      default: break;
    }
  } else if (p.d == 128) {
    switch (p.m / 32) {
      case 2: return launch_d<128, 2>(p, q, k, v, W, o, w, stream);
      case 4: return launch_d<128, 4>(p, q, k, v, W, o, w, stream);
      case 6: return launch_d<128, 6>(p, q, k, v, W, o, w, stream);
      case 8: return launch_d<128, 8>(p, q, k, v, W, o, w, stream);
      default: break;
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace favor
