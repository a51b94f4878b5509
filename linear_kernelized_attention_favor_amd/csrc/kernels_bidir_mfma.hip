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
#ifndef FAVOR_QAPPLY_WPE
#define FAVOR_QAPPLY_WPE 2      // query-side waves per SIMD the register budget targets
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
  constexpr int KCH = kTT * D / 8;           // 16-byte K chunks per tile
  constexpr int KPT = (KCH + NTH - 1) / NTH;
  constexpr int VUN = (kTT / 2) * (D / 4);   // (token pair, 4-column group) units per tile
  constexpr int VPT = (VUN + NTH - 1) / NTH;
  const int s = blockIdx.x, bh = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int f0 = wave * C::FPW;

  // Three-stage ring: tile t's V^T, tile t+1's K (projection running ahead)
  // and tile t+2 being written.
  __shared__ __align__(16) _Float16 Ks[3][kTT][C::KROW];
  __shared__ __align__(16) uint32_t Vt[3][D][C::VROW / 2];   // bf16 pairs, token order perm_of
  __shared__ __align__(16) float Ns[3][kTT];                 // -|k|^2 log2(e) / 2 per token

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
  float cref[C::NT];   // per-feature reference (log2 units), set by the first tile
#pragma unroll
  for (int nt = 0; nt < C::NT; ++nt) cref[nt] = 0.f;

  const int j0 = s * SL, j1 = min(L, j0 + SL);
  const int ntiles = (j1 - j0 + kTT - 1) / kTT;
  const size_t base = static_cast<size_t>(bh) * L * D;

  // Global loads of tile t+3 are in flight while tile t is consumed.  Loads
  // past the split read nothing and stage zeros.
  uint4 kreg[KPT];
  uint2 vreg[VPT][2];
  auto gload = [&](int t) {
    const int jt = j0 + t * kTT;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int c = tid + i * NTH;
      const int tok = jt + c / C::CPR;
      kreg[i] = make_uint4(0, 0, 0, 0);
      if (c < KCH && tok < j1)
        kreg[i] = *reinterpret_cast<const uint4*>(K + base + static_cast<size_t>(tok) * D +
                                                  (c % C::CPR) * 8);
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int u = tid + i * NTH;
      const int tok = jt + 2 * (u % 16);
      const size_t off = base + static_cast<size_t>(tok) * D + 4 * (u / 16);
      vreg[i][0] = make_uint2(0, 0);
      vreg[i][1] = make_uint2(0, 0);
      if (u < VUN && tok < j1) vreg[i][0] = *reinterpret_cast<const uint2*>(V + off);
      if (u < VUN && tok + 1 < j1) vreg[i][1] = *reinterpret_cast<const uint2*>(V + off + D);
    }
  };
  auto lstore = [&](int buf, int t) {
    const int jt = j0 + t * kTT;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
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
      if (c < KCH) {
        uint4 h;
        h.x = bf16x2_to_f16x2(kv.x); h.y = bf16x2_to_f16x2(kv.y);
        h.z = bf16x2_to_f16x2(kv.z); h.w = bf16x2_to_f16x2(kv.w);
        *reinterpret_cast<uint4*>(&Ks[buf][j][ch * 8]) = h;
        if (ch == 0) Ns[buf][j] = (jt + j < j1) ? -0.5f * kLog2e * ss : -INFINITY;
      }
    }
    // V^T: two consecutive tokens share one 32-bit word (positions perm_of
    // keep token pairs 2p, 2p+1 adjacent), four columns per unit.
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int u = tid + i * NTH;
      if (u < VUN) {
        const int col = 4 * (u / 16);
        const int w = perm_inv(2 * (u % 16)) >> 1;
        const uint2 a = vreg[i][0], b = vreg[i][1];
        Vt[buf][col + 0][w] = __builtin_amdgcn_perm(b.x, a.x, 0x05040100u);
        Vt[buf][col + 1][w] = __builtin_amdgcn_perm(b.x, a.x, 0x07060302u);
        Vt[buf][col + 2][w] = __builtin_amdgcn_perm(b.y, a.y, 0x05040100u);
        Vt[buf][col + 3][w] = __builtin_amdgcn_perm(b.y, a.y, 0x07060302u);
      }
    }
  };

  bf16x8 ones;
#pragma unroll
  for (int u = 0; u < 8; ++u) ones[u] = static_cast<__bf16>(1.0f);

  using SArr = f32x4[2][C::NT];
  // S = K W'^T - n'  (rows: tokens 16 mt + 4 g + v; column: feature f0 + 16 nt + l16)
  auto proj = [&](int buf, SArr& S) {
    f32x4 cinit[2];
    f16x8 ka[2][C::KS];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      cinit[mt] = *reinterpret_cast<const f32x4*>(&Ns[buf][16 * mt + 4 * g]);
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks)
        ka[mt][ks] = *reinterpret_cast<const f16x8*>(&Ks[buf][16 * mt + l16][32 * ks + 8 * g]);
    }
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < C::NT; ++nt)
          S[mt][nt] = mma_f16(ka[mt][ks], wb[nt][ks], ks == 0 ? cinit[mt] : S[mt][nt]);
  };
  // Exponents relative to the references, in place; true if any lane of the
  // wave exceeds the headroom.
  auto relative = [&](SArr& S, float (&lm)[C::NT]) {
    bool raise = false;
#pragma unroll
    for (int nt = 0; nt < C::NT; ++nt) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int v = 0; v < 4; ++v) S[mt][nt][v] -= cref[nt];
      const float a = max3(S[0][nt][0], S[0][nt][1], S[0][nt][2]);
      const float b = max3(S[0][nt][3], S[1][nt][0], S[1][nt][1]);
      lm[nt] = max3(a, b, fmaxf(S[1][nt][2], S[1][nt][3]));   // this lane's 8 tokens
      raise |= lm[nt] > kTau;
    }
    return __ballot(raise) != 0;
  };
  // Reference update: exact per-feature maximum (column reduction); always
  // on the first tile, otherwise only where a lane exceeded the headroom.
  auto rebase = [&](SArr& S, float (&lm)[C::NT], bool first) {
#pragma unroll
    for (int nt = 0; nt < C::NT; ++nt) {
      const float tm = colmax4(lm[nt]);
      const float dlt = (first || tm > kTau) ? tm : 0.f;
      if (!first) {   // accumulators are still zero on the first tile
        const float f = fast_exp2(-dlt);
#pragma unroll
        for (int i = 0; i <= C::MV; ++i) acc[i][nt] *= f;
      }
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int v = 0; v < 4; ++v) S[mt][nt][v] -= dlt;
      cref[nt] += dlt;
    }
  };
  // K~ = exp2(S) as the contraction's B operand (token positions perm_of).
  auto features = [&](const SArr& S, bf16x8 (&kb)[C::NT]) {
#pragma unroll
    for (int nt = 0; nt < C::NT; ++nt) {
      uint32_t p[4];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        p[q] = pack_bf16(fast_exp2(S[0][nt][2 * q]), fast_exp2(S[0][nt][2 * q + 1]));
        p[2 + q] = pack_bf16(fast_exp2(S[1][nt][2 * q]), fast_exp2(S[1][nt][2 * q + 1]));
      }
      kb[nt] = __builtin_bit_cast(bf16x8, make_uint4(p[0], p[1], p[2], p[3]));
    }
  };
  // [V | 1]^T K~ : rows = value columns, columns = features.
  auto contract = [&](int buf, const bf16x8 (&kb)[C::NT]) {
#pragma unroll
    for (int mv = 0; mv < C::MV; ++mv) {
      const bf16x8 va = *reinterpret_cast<const bf16x8*>(&Vt[buf][16 * mv + l16][4 * g]);
#pragma unroll
      for (int nt = 0; nt < C::NT; ++nt) acc[mv][nt] = mma_bf16(va, kb[nt], acc[mv][nt]);
    }
#pragma unroll
    for (int nt = 0; nt < C::NT; ++nt) acc[C::MV][nt] = mma_bf16(ones, kb[nt], acc[C::MV][nt]);
  };

  // Prologue: tiles 0 and 1 staged, tile 2 in flight, tile 0 projected.
  gload(0);
  lstore(0, 0);
  gload(1);
  lstore(1, 1);
  gload(2);
  lds_barrier();
  SArr SA, SB;
  float lm[C::NT];
  proj(0, SA);
  relative(SA, lm);
  rebase(SA, lm, true);

  // Iteration t: project tile t+1 while tile t's features are formed, then
  // contract tile t, stage tile t+2, load tile t+3, and check tile t+1.
  auto step = [&](int t, SArr& Scur, SArr& Snext) {
    bf16x8 kb[C::NT];
    proj((t + 1) % 3, Snext);
    features(Scur, kb);
    contract(t % 3, kb);
    lstore((t + 2) % 3, t + 2);
    gload(t + 3);
    if (__builtin_expect(relative(Snext, lm), 0)) rebase(Snext, lm, false);
    lds_barrier();
  };
  for (int t = 0; t < ntiles; t += 2) {
    step(t, SA, SB);
    if (t + 1 >= ntiles) break;
    step(t + 1, SB, SA);
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
// kcombine: grid (ceil((D+16) * m / 1024), BH), 256 threads; each thread owns
// four consecutive features of one row of the combined state.  The splits are
// summed in split order after rescaling to the largest per-feature reference.
// Output Kz [BH][D+16][m+8] bf16 in the query side's operand order (features
// permuted within 32-blocks; row D = z, rows above D zero) and cfin [BH][m].
// Head 0's work-groups also write W16 [m][D+8]: W log2(e) in fp16, the query
// side's projection operand.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void kcombine(const float* __restrict__ P,
                                                const float* __restrict__ cs,
                                                const float* __restrict__ W,
                                                uint16_t* __restrict__ Kz,
                                                float* __restrict__ cfin,
                                                _Float16* __restrict__ W16, int m, int nsplit) {
  const int bh = blockIdx.y;
  const int e = blockIdx.x * 256 + threadIdx.x;   // (row, feature quad)
  if (bh == 0) {
    for (int i = e; i < m * D; i += gridDim.x * 256) {
      const int f = i / D, a = i - f * D;
      W16[static_cast<size_t>(f) * (D + 8) + a] = static_cast<_Float16>(W[i] * kLog2e);
    }
  }
  const int mq = m / 4;
  if (e >= (D + 16) * mq) return;
  const int row = e / mq, f = 4 * (e - row * mq);
  const float4* csq = reinterpret_cast<const float4*>(cs + static_cast<size_t>(bh) * nsplit * m + f);
  float4 cmax = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
  for (int s = 0; s < nsplit; ++s) {
    const float4 c = csq[static_cast<size_t>(s) * mq];
    cmax.x = fmaxf(cmax.x, c.x); cmax.y = fmaxf(cmax.y, c.y);
    cmax.z = fmaxf(cmax.z, c.z); cmax.w = fmaxf(cmax.w, c.w);
  }
  float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
  if (row <= D) {
    const float4* pq = reinterpret_cast<const float4*>(
        P + (static_cast<size_t>(bh) * nsplit * (D + 1) + row) * m + f);
    const size_t sstride = static_cast<size_t>(D + 1) * mq;
    for (int s = 0; s < nsplit; ++s) {
      const float4 c = csq[static_cast<size_t>(s) * mq];
      const float4 v = pq[s * sstride];
      a.x = fmaf(v.x, fast_exp2(c.x - cmax.x), a.x);
      a.y = fmaf(v.y, fast_exp2(c.y - cmax.y), a.y);
      a.z = fmaf(v.z, fast_exp2(c.z - cmax.z), a.z);
      a.w = fmaf(v.w, fast_exp2(c.w - cmax.w), a.w);
    }
  }
  // Four features stay inside one 32-block; their permuted positions are
  // scattered within it.
  uint16_t* kzr = Kz + (static_cast<size_t>(bh) * (D + 16) + row) * (m + 8) + (f & ~31);
  const float av[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
  for (int q = 0; q < 4; ++q)
    kzr[perm_inv((f & 31) + q)] = static_cast<uint16_t>(pack_bf16(av[q], 0.f) & 0xffffu);
  if (row == 0) *reinterpret_cast<float4*>(cfin + static_cast<size_t>(bh) * m + f) = cmax;
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

template <int D, int NW, int NTQ, int NCH>
__global__ __launch_bounds__(NW * 64, FAVOR_QAPPLY_WPE) void qapply(const uint16_t* __restrict__ Q,
                                                  const _Float16* __restrict__ W16,
                                                  const uint16_t* __restrict__ Kz,
                                                  const float* __restrict__ cfin,
                                                  uint16_t* __restrict__ O, int L, int QL) {
  using C = QCfg<D, NTQ>;
  constexpr int NTH = NW * 64;
  constexpr int m = 64 * NCH;
  constexpr int kzrow = m + 8;
  extern __shared__ __align__(16) unsigned char smem[];
  _Float16* Wl = reinterpret_cast<_Float16*>(smem);
  uint16_t* Kzl = reinterpret_cast<uint16_t*>(smem + static_cast<size_t>(m) * C::WROW * 2);
  float* cl = reinterpret_cast<float*>(smem + static_cast<size_t>(m) * C::WROW * 2 +
                                       static_cast<size_t>(D + 16) * kzrow * 2);
  const int qb = blockIdx.x, bh = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;

  // Stage W' (fp16), Kz and c for this head.
  {
    const uint4* src = reinterpret_cast<const uint4*>(W16);
    uint4* dst = reinterpret_cast<uint4*>(Wl);
    constexpr int n16 = m * C::WROW / 8;
    for (int i = tid; i < n16; i += NTH) dst[i] = src[i];
  }
  {
    const uint4* src = reinterpret_cast<const uint4*>(Kz + static_cast<size_t>(bh) * (D + 16) * kzrow);
    uint4* dst = reinterpret_cast<uint4*>(Kzl);
    constexpr int n16 = (D + 16) * kzrow / 8;
    for (int i = tid; i < n16; i += NTH) dst[i] = src[i];
  }
  for (int i = tid; i < m; i += NTH) cl[i] = cfin[static_cast<size_t>(bh) * m + i];
  __syncthreads();   // the only barrier: LDS is read-only from here on

  const size_t base = static_cast<size_t>(bh) * L * D;
  const int q0 = qb * QL, q1 = min(L, q0 + QL);
  const int step = NW * C::TQ;
  const int tt0 = q0 + wave * C::TQ;
  if (tt0 >= q1) return;
  const int ntile = (q1 - tt0 + step - 1) / step;

  // Q tiles: raw bf16 loads one tile ahead of their use.
  using Raw = uint4[C::NTQ][C::KS];
  using Qop = f16x8[C::NTQ][C::KS];
  auto qload = [&](int tt, Raw& raw) {
#pragma unroll
    for (int nt = 0; nt < C::NTQ; ++nt) {
      const int tok = tt + 16 * nt + l16;
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        raw[nt][ks] = make_uint4(0, 0, 0, 0);
        if (tok < q1)
          raw[nt][ks] = *reinterpret_cast<const uint4*>(Q + base + static_cast<size_t>(tok) * D +
                                                        32 * ks + 8 * g);
      }
    }
  };
  // Q^T operands: token tt + 16 nt + l16, dims 32 ks + 8 g .. +7, in fp16.
  auto convert = [&](const Raw& raw, Qop& qop) {
#pragma unroll
    for (int nt = 0; nt < C::NTQ; ++nt)
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        const uint4 x = raw[nt][ks];
        uint4 h;
        h.x = bf16x2_to_f16x2(x.x); h.y = bf16x2_to_f16x2(x.y);
        h.z = bf16x2_to_f16x2(x.z); h.w = bf16x2_to_f16x2(x.w);
        qop[nt][ks] = __builtin_bit_cast(f16x8, h);
      }
  };

  f32x4 acc[C::MV + 1][C::NTQ];
  float M[C::NTQ];   // per-row reference (log2 units), set by each tile's first chunk
  using SArr = f32x4[4][C::NTQ];
  // S^T = W' Q^T + c  (rows: features 64 ch + 16 mt + 4 g + v; column: token)
  auto proj = [&](int ch, const Qop& qop, SArr& S) {
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
          S[mt][nt] = mma_f16(wa[mt][ks], qop[nt][ks], ks == 0 ? cb[mt] : S[mt][nt]);
  };
  // Exponents relative to the row references, in place; true if any lane of
  // the wave exceeds the headroom.
  float lm[C::NTQ];
  auto relative = [&](SArr& S) {
    bool raise = false;
#pragma unroll
    for (int nt = 0; nt < C::NTQ; ++nt) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int v = 0; v < 4; ++v) S[mt][nt][v] -= M[nt];
      const float a = max3(S[0][nt][0], S[0][nt][1], S[0][nt][2]);
      const float b = max3(S[0][nt][3], S[1][nt][0], S[1][nt][1]);
      const float c = max3(S[1][nt][2], S[1][nt][3], S[2][nt][0]);
      const float d = max3(S[2][nt][1], S[2][nt][2], S[2][nt][3]);
      const float e = max3(S[3][nt][0], S[3][nt][1], S[3][nt][2]);
      lm[nt] = max3(max3(a, b, c), max3(d, e, S[3][nt][3]), a);   // this lane's 16 features
      raise |= lm[nt] > kTau;
    }
    return __ballot(raise) != 0;
  };
  // Row reference update: exact row maximum (column reduction); always on a
  // tile's first chunk, otherwise only where a lane exceeded the headroom.
  auto rebase = [&](SArr& S, bool first) {
#pragma unroll
    for (int nt = 0; nt < C::NTQ; ++nt) {
      const float cm = colmax4(lm[nt]);
      const float dlt = (first || cm > kTau) ? cm : 0.f;
      if (!first) {   // accumulators are still zero on the first chunk
        const float f = fast_exp2(-dlt);
#pragma unroll
        for (int i = 0; i <= C::MV; ++i) acc[i][nt] *= f;
      }
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int v = 0; v < 4; ++v) S[mt][nt][v] -= dlt;
      M[nt] += dlt;
    }
  };
  // Q~^T = exp2(S) (features at positions perm_of) times [KV | z]^T.
  auto apply = [&](int ch, const SArr& S) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      bf16x8 qt[C::NTQ];
#pragma unroll
      for (int nt = 0; nt < C::NTQ; ++nt) {
        uint32_t p[4];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          p[q] = pack_bf16(fast_exp2(S[2 * kb][nt][2 * q]), fast_exp2(S[2 * kb][nt][2 * q + 1]));
          p[2 + q] = pack_bf16(fast_exp2(S[2 * kb + 1][nt][2 * q]),
                               fast_exp2(S[2 * kb + 1][nt][2 * q + 1]));
        }
        qt[nt] = __builtin_bit_cast(bf16x8, make_uint4(p[0], p[1], p[2], p[3]));
      }
      const int kcol = 64 * ch + 32 * kb + 8 * g;
#pragma unroll
      for (int mv = 0; mv <= C::MV; ++mv) {
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(&Kzl[(16 * mv + l16) * kzrow + kcol]);
#pragma unroll
        for (int nt = 0; nt < C::NTQ; ++nt) acc[mv][nt] = mma_bf16(ka, qt[nt], acc[mv][nt]);
      }
    }
  };
  // O = num / den for one tile; den is row 0 of the last tile (g = 0, v = 0).
  auto finish = [&](int tt) {
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
  auto reset = [&]() {
#pragma unroll
    for (int i = 0; i <= C::MV; ++i)
#pragma unroll
      for (int nt = 0; nt < C::NTQ; ++nt) acc[i][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int nt = 0; nt < C::NTQ; ++nt) M[nt] = 0.f;
  };

  // Software pipeline over (tile, chunk): chunk k+1 is projected on the
  // matrix cores while chunk k's features are formed and applied; a tile's
  // last step projects the next tile's first chunk.
  Raw raw;
  Qop qcur;
  qload(tt0, raw);
  convert(raw, qcur);
  if (ntile > 1) qload(tt0 + step, raw);
  reset();
  SArr SA, SB;
  proj(0, qcur, SA);
  relative(SA);
  rebase(SA, true);
  for (int ti = 0; ti < ntile; ++ti) {
    const int tt = tt0 + ti * step;
    const bool more = ti + 1 < ntile;
    // Regular step: project chunk ch+1, apply chunk ch, check chunk ch+1.
    auto regular = [&](const int ch, SArr& Scur, SArr& Snext) {
      __builtin_amdgcn_sched_barrier(0);
      proj(ch + 1, qcur, Snext);
      apply(ch, Scur);
      if (__builtin_expect(relative(Snext), 0)) rebase(Snext, false);
    };
    // Last step of a tile: project the next tile's first chunk, apply the
    // last chunk, write the tile, start the next one.
    auto last = [&](const int ch, SArr& Scur, SArr& Snext) {
      __builtin_amdgcn_sched_barrier(0);
      if (more) convert(raw, qcur);   // the current tile's operands are done
      proj(0, qcur, Snext);           // unused after the wave's last tile
      apply(ch, Scur);
      finish(tt);
      reset();
      if (more) {
        if (ti + 2 < ntile) qload(tt + 2 * step, raw);
        relative(Snext);
        rebase(Snext, true);
      }
    };
    int ch = 0;
#pragma unroll 1
    for (; ch + 2 < NCH; ch += 2) {
      regular(ch, SA, SB);
      regular(ch + 1, SB, SA);
    }
    if constexpr ((NCH % 2) == 0) {
      regular(NCH - 2, SA, SB);
      last(NCH - 1, SB, SA);
    } else {
      last(NCH - 1, SA, SB);   // the next tile's first chunk landed in SB
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < C::NTQ; ++nt) SA[mt][nt] = SB[mt][nt];
    }
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
  kcombine<D><<<dim3(((D + 16) * p.m / 4 + 255) / 256, p.BH), 256, 0, st>>>(P, cs, W, Kz, cfin,
                                                                            W16, p.m, p.nseg);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t lds = qapply_lds_bytes<D>(p.m);
  const int nqb = (p.L + p.qblk - 1) / p.qblk;
  constexpr int NTQ = FAVOR_QAPPLY_NTQ;
  // m = 64 NCH; the key side runs m / FPW waves, so NCH follows from NW.
  constexpr int NCH = NW * KCfg<D>::FPW / 64;
  auto* kern = &qapply<D, 4, NTQ, NCH>;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                          hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
  if (e != hipSuccess) return e;
  kern<<<dim3(nqb, p.BH), 256, lds, st>>>(Q, W16, Kz, cfin, O, p.L, p.qblk);
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
