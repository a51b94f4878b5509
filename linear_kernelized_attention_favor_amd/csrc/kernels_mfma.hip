// Bidirectional FAVOR+ on the matrix cores (bf16 inputs, d in {64, 128}).
//
// FA-part of the "FAVOR+" method page: O = D^-1 (Q' ((K')^T V)),
// D = diag(Q' ((K')^T 1_L)), with phi(x) = exp(w . x - |x|^2/2)/sqrt(m).
// Three launches:
//
//   kpart    per (head, sequence split): for each 32-token tile the relative
//            feature exponents S = K W'^T - knorm |k|^2 - c_r (knorm = 1/2
//            for the softmax kernel's features, 1 for the Gaussian kernel's;
//            the query side's norm term cancels per row) (fp16 MFMA; W' =
//            W log2 e so the exponentials are exp2; the norm and the
//            per-feature reference c_r enter through one extra MFMA k-step
//            whose operands hold them as fp16 hi/lo pairs), K~ = exp2(S) in
//            bf16, and the contraction [V | 1]^T K~ accumulated in fp32 (bf16
//            MFMA).  c_r sits kKeyBias above the largest exponent seen when it
//            was set and is raised only when some K~ reaches 2 (the top bit of
//            a bf16 exponent, tested on the packed features).  Each wave owns
//            a slice of features; the 32-token tile is staged once per
//            work-group in LDS (K in fp16, V transposed).
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
// ReLU features (generalized attention, template flag RELU): the same
// kernels with max(s, 0) in place of exp2(s), no norm term, every reference
// 0 and no row reference.  s is then w . x log2 e; the common factor
// (log2 e)^2 of numerator and denominator cancels in the division.
//
// Numerics: Q and K are converted to fp16 for the projection (exact for
// |x| < 65504 outside fp16's subnormal range), W' is rounded to fp16, the
// features and [KV | z] are rounded to bf16 (full fp32 exponent range), all
// sums are fp32.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <type_traits>

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

// Key-side reference placement: after a (re)set, a feature's largest
// exponent sits kKeyBias below its reference, so K~ <= 2^-kKeyBias; a tile is
// re-referenced only when some K~ >= 2 (kKeyBias + 1 log2 units of headroom),
// and values more than 126 - kKeyBias below the maximum flush to zero (bf16
// normal range), where they are far below fp32 resolution of the sums.
constexpr float kKeyBias = 40.0f;
// The same for the query side's per-row reference (the products of query and
// key features stay above 2^-(kKeyBias + kQBias), far inside fp32).
constexpr float kQBias = 20.0f;

#ifndef FAVOR_QAPPLY_NTQ
#define FAVOR_QAPPLY_NTQ 2      // 16-token tiles per query-side wave iteration
#endif
#ifndef FAVOR_QAPPLY_WPE
#define FAVOR_QAPPLY_WPE 2      // query-side waves per SIMD the register budget targets
#endif
#ifndef FAVOR_QAPPLY_NW
#define FAVOR_QAPPLY_NW 4       // waves per query-side work-group
#endif
#ifndef FAVOR_QAPPLY_WGS
#define FAVOR_QAPPLY_WGS 512    // query-side work-groups per call the plan aims for
#endif
#ifndef FAVOR_QSTREAM_NW
#define FAVOR_QSTREAM_NW 12     // waves per streamed query-side work-group
#endif
#ifndef FAVOR_QSTREAM_NTQ
#define FAVOR_QSTREAM_NTQ 2     // 16-token tiles per streamed query-side wave
#endif
#ifndef FAVOR_QSTREAM_WPE
#define FAVOR_QSTREAM_WPE 3     // streamed query-side waves per SIMD
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
// kpart: grid (BH x nsplit_run x m / (NW FPW)) items, TG x NW waves of 64
// threads; wave w of feature block z owns features [(z NW + w) FPW,
// (z NW + w + 1) FPW).  nsplit_run <= nsplit splits are computed (the causal
// form skips the last segment); the layout keeps nsplit slots per head.
// Output: P [BH][nsplit][D+1][m] fp32 (row D = z) and cs [BH][nsplit][m]
// fp32 (per-feature references, log2 units).
// ---------------------------------------------------------------------------
// TG token groups of NW waves each: group gi takes the split's tiles gi,
// gi + TG, ... (every group runs the same number of steps; tiles past the
// split are masked), and the groups' states are merged through LDS at the
// end.  More groups per work-group mean fewer, longer splits for the same
// number of waves, hence fewer partial states to write and combine.
template <int D, int NW, int TG>
struct KLds {
  using C = KCfg<D>;
  static constexpr int KS_BYTES = 3 * kTT * C::KROW * 2;
  static constexpr int VT_BYTES = 3 * D * (C::VROW / 2) * 4;
  static constexpr int NAROW = 40;                    // halves per token row (32 + pad)
  static constexpr int NA_BYTES = 3 * kTT * NAROW * 2;   // per token: 1, 1, n_hi, n_lo, 0 ...
  static constexpr int RING = KS_BYTES + VT_BYTES + NA_BYTES;
  static constexpr int M = NW * C::FPW;                          // features
  static constexpr int BYTES = TG * RING;
};

template <int D, int NW, int TG, bool RELU>
__global__ __launch_bounds__(TG * NW * 64, 2) void kpart(const uint16_t* __restrict__ K,
                                                 const uint16_t* __restrict__ V,
                                                 const float* __restrict__ W,
                                                 float* __restrict__ P, float* __restrict__ cs,
                                                 int L, int m, int SL, int nsplit,
                                                 int nsplit_run, float knorm) {
  using C = KCfg<D>;
  using LD = KLds<D, NW, TG>;
  constexpr int NTH = NW * 64;               // threads per token group
  constexpr int KCH = kTT * D / 8;           // 16-byte K chunks per tile
  constexpr int KPT = (KCH + NTH - 1) / NTH;
  constexpr int VUN = (kTT / 2) * (D / 4);   // (token pair, 4-column group) units per tile
  constexpr int VPT = (VUN + NTH - 1) / NTH;
  // 1-D grid of (head, split, feature block) items in XCD-major order, the
  // feature block fastest: the blocks of one split read the same K and V
  // tiles on one XCD at about the same time (one HBM read, L2 hits after).
  const int nfb = m / LD::M;
  const int item = xcd_major(blockIdx.x, gridDim.x);
  const int fb = item % nfb, s = (item / nfb) % nsplit_run, bh = item / (nfb * nsplit_run);
  // (wave-uniform: tells the compiler that per-group values are scalar)
  const int grp = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / NTH);
  const int tid = threadIdx.x % NTH, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  // Feature block fb: features [fb NW FPW, (fb+1) NW FPW) (several blocks
  // when m needs more than 8 waves); f0 is global, fl0 block-local.
  const int fl0 = wave * C::FPW;
  const int f0 = fb * LD::M + fl0;

  // Per group, a three-stage ring: tile t's V^T, tile t+1's K (projection
  // running ahead) and tile t+2 being written.
  __shared__ __align__(16) unsigned char kp_smem[LD::BYTES];
  unsigned char* const ring = kp_smem + grp * LD::RING;
  auto Ks = reinterpret_cast<_Float16(*)[kTT][C::KROW]>(ring);
  auto Vt = reinterpret_cast<uint32_t(*)[D][C::VROW / 2]>(ring + LD::KS_BYTES);   // bf16 pairs
  // Per token the A operand of the extra k-step: [1, 1, n_hi, n_lo, 0 x 28]
  // with n = knorm |k|^2 log2(e) (lanes of the upper k rows read the zeros).
  // (A full k=32 step: chaining a k=16 product into a k=32 accumulation was
  // seen to read the accumulator too early on this part.)
  auto Na = reinterpret_cast<_Float16(*)[kTT][LD::NAROW]>(ring + LD::KS_BYTES + LD::VT_BYTES);
  for (int i = tid; i < LD::NA_BYTES / 16; i += NTH)
    reinterpret_cast<uint4*>(Na)[i] = make_uint4(0, 0, 0, 0);
  lds_barrier();

  // Projection B operands, kept in registers: W'[f][32 ks + 8 g + u]
  // (loaded in the prologue, together with the first tiles).
  f16x8 wb[C::NT][C::KS];
  auto load_w = [&]() {
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
  };

  f32x4 acc[C::MV + 1][C::NT];
#pragma unroll
  for (int i = 0; i <= C::MV; ++i)
#pragma unroll
    for (int nt = 0; nt < C::NT; ++nt) acc[i][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float cref[C::NT];   // per-feature reference (log2 units), set by the first tile
  f16x8 baug[C::NT];   // B operand of the extra step: [-c_hi, -c_lo, -1, -1] on k rows 0..3
  auto set_baug = [&](int nt) {
    const _Float16 hi = static_cast<_Float16>(cref[nt]);
    const _Float16 lo = static_cast<_Float16>(cref[nt] - static_cast<float>(hi));
    const _Float16 z = static_cast<_Float16>(0.f), m1 = static_cast<_Float16>(-1.f);
    baug[nt] = (g == 0) ? f16x8{-hi, -lo, m1, m1, z, z, z, z} : f16x8{z, z, z, z, z, z, z, z};
  };
#pragma unroll
  for (int nt = 0; nt < C::NT; ++nt) {
    cref[nt] = 0.f;
    set_baug(nt);
  }

  const int j0 = s * SL, j1 = min(L, j0 + SL);
  // Steps per group (the group's tile t is the split's tile t TG + grp).
  const int ntiles = ((j1 - j0 + kTT - 1) / kTT + TG - 1) / TG;
  const size_t base = static_cast<size_t>(bh) * L * D;
  auto tile0 = [&](int t) { return j0 + (t * TG + grp) * kTT; };

  // Global loads of tile t+3 are issued at the start of step t and consumed
  // at the start of step t+1.  Buffer loads past the split's end return
  // zeros (the tail needs no per-lane branch); per-thread byte offsets
  // within a tile are fixed.
  using KRegs = uint4[KPT];
  using VRegs = uint2[VPT][2];
  KRegs kreg;
  VRegs vreg;
  int kvo[KPT], vvo[VPT];
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const int c = tid + i * NTH;
    kvo[i] = (c < KCH) ? ((c / C::CPR) * D + (c % C::CPR) * 8) * 2 : kBufOff;
  }
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const int u = tid + i * NTH;
    vvo[i] = (u < VUN) ? (2 * (u % 16) * D + 4 * (u / 16)) * 2 : kBufOff;
  }
  auto gload_to = [&](int t, KRegs& kr, VRegs& vr) {
    const int jt = tile0(t);
    const int bytes = max(0, j1 - jt) * D * 2;
    const __amdgpu_buffer_rsrc_t rk = buffer_rsrc(K + base + static_cast<size_t>(jt) * D, bytes);
    const __amdgpu_buffer_rsrc_t rv = buffer_rsrc(V + base + static_cast<size_t>(jt) * D, bytes);
#pragma unroll
    for (int i = 0; i < KPT; ++i) kr[i] = buffer_load16(rk, kvo[i]);
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      vr[i][0] = buffer_load8(rv, vvo[i]);
      vr[i][1] = buffer_load8(rv, vvo[i] + D * 2);
    }
  };
  auto gload = [&](int t) { gload_to(t, kreg, vreg); };
  auto lstore_from = [&](int buf, int t, const KRegs& kr, const VRegs& vr) {
    const int jt = tile0(t);
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int c = tid + i * NTH;
      const int j = (c / C::CPR) % kTT, ch = c % C::CPR;
      const uint4 kv = kr[i];
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
        if (ch == 0) {
          // n as an fp16 hi/lo pair (clamped: a larger norm underflows K~ anyway);
          // a token past the split gets n = +inf, i.e. K~ = 0.
          const float n = fminf(knorm * kLog2e * ss, 65504.f);
          const _Float16 nh = static_cast<_Float16>(n);
          const _Float16 nl = static_cast<_Float16>(n - static_cast<float>(nh));
          const _Float16 one = static_cast<_Float16>(1.f);
          const bool live = jt + j < j1;
          *reinterpret_cast<f16x4*>(&Na[buf][j][0]) =
              f16x4{one, one, live ? nh : static_cast<_Float16>(INFINITY),
                    live ? nl : static_cast<_Float16>(0.f)};
        }
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
        const uint2 a = vr[i][0], b = vr[i][1];
        Vt[buf][col + 0][w] = __builtin_amdgcn_perm(b.x, a.x, 0x05040100u);
        Vt[buf][col + 1][w] = __builtin_amdgcn_perm(b.x, a.x, 0x07060302u);
        Vt[buf][col + 2][w] = __builtin_amdgcn_perm(b.y, a.y, 0x05040100u);
        Vt[buf][col + 3][w] = __builtin_amdgcn_perm(b.y, a.y, 0x07060302u);
      }
    }
  };
  auto lstore = [&](int buf, int t) { lstore_from(buf, t, kreg, vreg); };

  bf16x8 ones;
#pragma unroll
  for (int u = 0; u < 8; ++u) ones[u] = static_cast<__bf16>(1.0f);

  using SArr = f32x4[2][C::NT];
  // S = K W'^T - n - c  (rows: tokens 16 mt + 4 g + v; column: feature f0 + 16 nt + l16)
  auto proj = [&](int buf, SArr& S) {
    f16x8 aa[2];
    f16x8 ka[2][C::KS];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      aa[mt] = *reinterpret_cast<const f16x8*>(&Na[buf][16 * mt + l16][8 * g]);
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks)
        ka[mt][ks] = *reinterpret_cast<const f16x8*>(&Ks[buf][16 * mt + l16][32 * ks + 8 * g]);
    }
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nt = 0; nt < C::NT; ++nt) {
        // ReLU: no norm term and no reference.  The extra step is kept where
        // TG = 1 (it adds exact zeros there: knorm = 0 and the reference stays
        // 0), again for the register allocation.
        if constexpr (RELU && TG > 1)
          S[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
        else
          S[mt][nt] = mma_f16(aa[mt], baug[nt], f32x4{0.f, 0.f, 0.f, 0.f});
      }
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < C::NT; ++nt) S[mt][nt] = mma_f16(ka[mt][ks], wb[nt][ks], S[mt][nt]);
  };
  // True if some feature of the tile reached 2 (or is not finite): the top
  // exponent bit of a packed bf16 value, ORed over the wave's features.
  auto overflow = [&](const bf16x8 (&kb)[C::NT]) {
    uint32_t o = 0;
#pragma unroll
    for (int nt = 0; nt < C::NT; ++nt) {
      const uint4 w = __builtin_bit_cast(uint4, kb[nt]);
      o |= w.x | w.y | w.z | w.w;
    }
    return __ballot((o & 0x40004000u) != 0) != 0;
  };
  // Reference update from the exact per-feature maximum tm of S (relative to
  // the current reference): raise by tm + kKeyBias where that is positive
  // (always reset on the first tile, whose accumulators are still zero).
  // S and any tile already projected with the old reference move along.
  auto rebase = [&](SArr& S, bool first, float (&dl)[C::NT]) {
#pragma unroll
    for (int nt = 0; nt < C::NT; ++nt) {
      const float a = max3(S[0][nt][0], S[0][nt][1], S[0][nt][2]);
      const float b = max3(S[0][nt][3], S[1][nt][0], S[1][nt][1]);
      const float tm = colmax4(max3(a, b, fmaxf(S[1][nt][2], S[1][nt][3])));
      // (a group whose first tile lies past the split keeps a finite reference)
      const float dlt = (tm == -INFINITY) ? 0.f : (first ? tm + kKeyBias : fmaxf(tm + kKeyBias, 0.f));
      if (!first) {
        const float f = fast_exp2(-dlt);
#pragma unroll
        for (int i = 0; i <= C::MV; ++i) acc[i][nt] *= f;
      }
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int v = 0; v < 4; ++v) S[mt][nt][v] -= dlt;
      cref[nt] += dlt;
      set_baug(nt);
      dl[nt] = dlt;
    }
  };
  // K~ = exp2(S) as the contraction's B operand (token positions perm_of).
  auto features = [&](const SArr& S, bf16x8 (&kb)[C::NT]) {
#pragma unroll
    for (int nt = 0; nt < C::NT; ++nt) {
      uint32_t p[4];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        p[q] = pack_bf16(feature<RELU>(S[0][nt][2 * q]), feature<RELU>(S[0][nt][2 * q + 1]));
        p[2 + q] = pack_bf16(feature<RELU>(S[1][nt][2 * q]), feature<RELU>(S[1][nt][2 * q + 1]));
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

  // Prologue: tiles 0 and 1 staged, tile 2 in flight, tile 0's features
  // formed (its reference set from the exact maximum).  The loads of tiles
  // 0..2 and of W' are all issued before the first wait (when a thread's
  // share of a tile is one load of each kind: the registers are there).
  if constexpr (KPT == 1 && VPT == 1) {
    KRegs k0, k1;
    VRegs v0, v1;
    gload_to(0, k0, v0);
    gload_to(1, k1, v1);
    gload(2);
    load_w();
    lstore_from(0, 0, k0, v0);
    lstore_from(1, 1, k1, v1);
  } else {
    load_w();
    gload(0);
    lstore(0, 0);
    gload(1);
    lstore(1, 1);
    gload(2);
  }
  lds_barrier();
  bf16x8 kbA[C::NT], kbB[C::NT];
  {
    SArr S;
    float dl[C::NT];
    proj(0, S);
    if constexpr (!RELU) rebase(S, true, dl);
    features(S, kbA);
  }

  // Step t: stage tile t+2 (loaded during step t-1), load tile t+3, project
  // tile t+1 on the matrix cores while tile t is contracted, then form and
  // check tile t+1's features (so every projection is consumed in its own
  // step).  The loop body holds six steps (the ring's period 3 times the
  // feature double buffer's period 2), so every ring slot is a compile-time
  // constant and LDS addresses fold into the instructions' offsets.
  auto step = [&](auto R, int t, const bf16x8 (&kcur)[C::NT], bf16x8 (&knext)[C::NT]) {
    constexpr int r = decltype(R)::value;
    __builtin_amdgcn_sched_barrier(0);   // keep the scheduler within one step
    lstore((r + 2) % 3, t + 2);
    gload(t + 3);
    SArr S;
    proj((r + 1) % 3, S);
    contract(r % 3, kcur);
    features(S, knext);
    // ReLU features take no reference: for them the check below is compiled
    // but never taken (knorm is 0), because the branch keeps the register
    // allocation of the exponential features (without it the compiler spills
    // the accumulators).
    if (__builtin_expect((RELU ? knorm < 0.f : true) && overflow(knext), 0)) {
      float dl[C::NT];
      rebase(S, false, dl);
      features(S, knext);
    }
    lds_barrier();
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  for (int t = 0; t < ntiles; t += 6) {
    step(I0{}, t, kbA, kbB);
    if (t + 1 >= ntiles) break;
    step(I1{}, t + 1, kbB, kbA);
    if (t + 2 >= ntiles) break;
    step(I2{}, t + 2, kbA, kbB);
    if (t + 3 >= ntiles) break;
    step(I0{}, t + 3, kbB, kbA);
    if (t + 4 >= ntiles) break;
    step(I1{}, t + 4, kbA, kbB);
    if (t + 5 >= ntiles) break;
    step(I2{}, t + 5, kbB, kbA);
  }

  if constexpr (TG > 1) {
    // Merge the groups' states into group 0's registers through LDS, one
    // group at a time, each rescaled to the larger of the two references.
    // Each lane moves its own registers (16-byte slots, lane-major, one
    // slot row per accumulator tile, then z and the references): wave w of
    // every group holds the same features in the same lanes.
    constexpr int SL = NW * 64;
    constexpr int NSLOT = C::MV * C::NT + 2;
    static_assert(C::NT <= 4, "z and the references of a lane fit one slot each");
    static_assert(NSLOT * SL * 16 <= LD::BYTES, "merge slots fit in the block's LDS");
    f32x4* const xv = reinterpret_cast<f32x4*>(kp_smem) + wave * 64 + lane;
    for (int src = 1; src < TG; ++src) {
      __syncthreads();
      if (grp == src) {
        const bool empty = tile0(0) >= j1;   // the group saw no token of the split
        f32x4 z4 = f32x4{0.f, 0.f, 0.f, 0.f}, c4 = z4;
#pragma unroll
        for (int nt = 0; nt < C::NT; ++nt) {
#pragma unroll
          for (int mv = 0; mv < C::MV; ++mv) xv[(mv * C::NT + nt) * SL] = acc[mv][nt];
          z4[nt] = acc[C::MV][nt][0];
          c4[nt] = empty ? -INFINITY : cref[nt];
        }
        xv[(C::MV * C::NT) * SL] = z4;
        xv[(C::MV * C::NT + 1) * SL] = c4;
      }
      __syncthreads();
      if (grp == 0) {
        const f32x4 z4 = xv[(C::MV * C::NT) * SL], c4 = xv[(C::MV * C::NT + 1) * SL];
#pragma unroll
        for (int nt = 0; nt < C::NT; ++nt) {
          const float co = c4[nt];
          const float cn = fmaxf(cref[nt], co);
          const float a = fast_exp2(cref[nt] - cn), b = fast_exp2(co - cn);
#pragma unroll
          for (int mv = 0; mv < C::MV; ++mv) acc[mv][nt] = acc[mv][nt] * a + xv[(mv * C::NT + nt) * SL] * b;
          acc[C::MV][nt][0] = acc[C::MV][nt][0] * a + z4[nt] * b;
          cref[nt] = cn;
        }
      }
    }
    if (grp != 0) return;
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
  const float4* pq = reinterpret_cast<const float4*>(
      P + (static_cast<size_t>(bh) * nsplit * (D + 1) + (row <= D ? row : 0)) * m + f);
  const size_t sstride = static_cast<size_t>(D + 1) * mq;
  // Splits in batches of KB, every load of a batch issued before the first
  // use (one memory round trip per batch); the running sum is rescaled when
  // a later batch raises the reference.
  constexpr int KB = 8;
  float4 cmax = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
  float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s0 = 0; s0 < nsplit; s0 += KB) {
    float4 c[KB], v[KB];
#pragma unroll
    for (int j = 0; j < KB; ++j) {
      const bool in = s0 + j < nsplit;
      c[j] = in ? csq[static_cast<size_t>(s0 + j) * mq]
                : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
      v[j] = (in && row <= D) ? pq[(s0 + j) * sstride] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    float4 nm = cmax;
#pragma unroll
    for (int j = 0; j < KB; ++j) {
      nm.x = fmaxf(nm.x, c[j].x); nm.y = fmaxf(nm.y, c[j].y);
      nm.z = fmaxf(nm.z, c[j].z); nm.w = fmaxf(nm.w, c[j].w);
    }
    // (a reference still at -inf means no split so far: its sum is zero)
    a.x *= (cmax.x == -INFINITY) ? 0.f : fast_exp2(cmax.x - nm.x);
    a.y *= (cmax.y == -INFINITY) ? 0.f : fast_exp2(cmax.y - nm.y);
    a.z *= (cmax.z == -INFINITY) ? 0.f : fast_exp2(cmax.z - nm.z);
    a.w *= (cmax.w == -INFINITY) ? 0.f : fast_exp2(cmax.w - nm.w);
#pragma unroll
    for (int j = 0; j < KB; ++j) {
      if (s0 + j < nsplit) {
        a.x = fmaf(v[j].x, fast_exp2(c[j].x - nm.x), a.x);
        a.y = fmaf(v[j].y, fast_exp2(c[j].y - nm.y), a.y);
        a.z = fmaf(v[j].z, fast_exp2(c[j].z - nm.z), a.z);
        a.w = fmaf(v[j].w, fast_exp2(c[j].w - nm.w), a.w);
      }
    }
    cmax = nm;
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
// qapply: grid (nqb * BH) in XCD-major item order, NW waves; each wave takes
// 16*NTQ-token tiles of the block [qb QL, (qb+1) QL).  LDS (dynamic): W'
// fp16 [m][D+8], Kz bf16 [D+16][m+8], c [m] as fp16 hi/lo pairs.  The query
// exponents relative to the row reference, S^T = W' Q^T + c - M, come out of
// the matrix cores directly: an extra k-step multiplies [c_hi, c_lo, 1, 1]
// per feature by [1, 1, -M_hi, -M_lo] per token.  M sits kQBias above the
// row's largest exponent when set (first chunk of a tile) and is raised only
// when some feature reaches 2 (the bf16 exponent's top bit).
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

template <int D, int NW, int NTQ, int NCH, bool RELU>
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
  uint32_t* chl = reinterpret_cast<uint32_t*>(smem + static_cast<size_t>(m) * C::WROW * 2 +
                                              static_cast<size_t>(D + 16) * kzrow * 2);
  // 1-D grid of (head, query block) items, one head's blocks on one XCD.
  const int nqb = (L + QL - 1) / QL;
  const int item = xcd_major(blockIdx.x, gridDim.x);
  const int qb = item % nqb, bh = item / nqb;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;

  // Stage W' (fp16), Kz and c (as fp16 hi/lo pairs) for this head.  W' and
  // Kz go global -> LDS directly (each wave instruction moves 64 16-byte
  // units), all issued before the first wait: one memory round trip.
  {
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    auto copy = [&](const uint4* src, uint4* dst, int n16) {
      for (int j = wv; 64 * j < n16; j += NW)
        if (64 * j + lane < n16) lds_dma16(src + 64 * j + lane, dst + 64 * j);
    };
    copy(reinterpret_cast<const uint4*>(W16), reinterpret_cast<uint4*>(Wl), m * C::WROW / 8);
    copy(reinterpret_cast<const uint4*>(Kz + static_cast<size_t>(bh) * (D + 16) * kzrow),
         reinterpret_cast<uint4*>(Kzl), (D + 16) * kzrow / 8);
  }
  const size_t base = static_cast<size_t>(bh) * L * D;
  const int q0 = qb * QL, q1 = min(L, q0 + QL);
  const int step = NW * C::TQ;
  const int tt0 = q0 + wave * C::TQ;
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
  // The wave's first tile is loaded while the staging is in flight.
  Raw raw;
  qload(tt0, raw);

  for (int i = tid; i < m; i += NTH) {
    const float c = cfin[static_cast<size_t>(bh) * m + i];
    const _Float16 hi = static_cast<_Float16>(c);
    const _Float16 lo = static_cast<_Float16>(c - static_cast<float>(hi));
    chl[i] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, hi)) |
             (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, lo)) << 16);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wave's staging has landed
  __syncthreads();   // the only barrier: LDS is read-only from here on
  if (tt0 >= q1) return;

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
  float M[C::NTQ];     // per-row reference (log2 units)
  f16x8 baug[C::NTQ];  // B operand of the extra step: [1, 1, -M_hi, -M_lo] on k rows 0..3
  auto set_baug = [&](int nt) {
    const _Float16 hi = static_cast<_Float16>(M[nt]);
    const _Float16 lo = static_cast<_Float16>(M[nt] - static_cast<float>(hi));
    const _Float16 z = static_cast<_Float16>(0.f), one = static_cast<_Float16>(1.f);
    baug[nt] = (g == 0) ? f16x8{one, one, -hi, -lo, z, z, z, z} : f16x8{z, z, z, z, z, z, z, z};
  };
  using SArr = f32x4[4][C::NTQ];
  using Feat = bf16x8[2][C::NTQ];   // [kb][nt]: lane = token, 8 features (perm_of)
  // S^T = W' Q^T + c - M  (rows: features 64 ch + 16 mt + 4 g + v; column: token)
  auto proj = [&](int ch, const Qop& qop, SArr& S) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const uint32_t cw = chl[64 * ch + 16 * mt + l16];
      const f16x8 aa = __builtin_bit_cast(
          f16x8, (g == 0) ? make_uint4(cw, 0x3C003C00u, 0u, 0u) : make_uint4(0u, 0u, 0u, 0u));
#pragma unroll
      for (int nt = 0; nt < C::NTQ; ++nt) {
        if constexpr (RELU)   // (no reference on either side)
          S[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
        else
          S[mt][nt] = mma_f16(aa, baug[nt], f32x4{0.f, 0.f, 0.f, 0.f});
      }
    }
    // (W' operands one k-step at a time: bounded registers at d = 128)
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      f16x8 wa[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        wa[mt] = *reinterpret_cast<const f16x8*>(
            &Wl[static_cast<size_t>(64 * ch + 16 * mt + l16) * C::WROW + 32 * ks + 8 * g]);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < C::NTQ; ++nt) S[mt][nt] = mma_f16(wa[mt], qop[nt][ks], S[mt][nt]);
    }
  };
  // Q~^T = exp2(S) in bf16 as the contraction's B operand.
  auto features = [&](const SArr& S, Feat& qt) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int nt = 0; nt < C::NTQ; ++nt) {
        uint32_t p[4];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          p[q] = pack_bf16(feature<RELU>(S[2 * kb][nt][2 * q]),
                           feature<RELU>(S[2 * kb][nt][2 * q + 1]));
          p[2 + q] = pack_bf16(feature<RELU>(S[2 * kb + 1][nt][2 * q]),
                               feature<RELU>(S[2 * kb + 1][nt][2 * q + 1]));
        }
        qt[kb][nt] = __builtin_bit_cast(bf16x8, make_uint4(p[0], p[1], p[2], p[3]));
      }
  };
  // True if some feature reached 2 (or is not finite), as in the key kernel.
  auto overflow = [&](const Feat& qt) {
    uint32_t o = 0;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int nt = 0; nt < C::NTQ; ++nt) {
        const uint4 w = __builtin_bit_cast(uint4, qt[kb][nt]);
        o |= w.x | w.y | w.z | w.w;
      }
    return __ballot((o & 0x40004000u) != 0) != 0;
  };
  // Row reference update from the exact row maximum of S (over the chunk's
  // features): reset on a tile's first chunk, otherwise raised where
  // positive, with the accumulators rescaled.
  auto rebase = [&](SArr& S, bool first) {
#pragma unroll
    for (int nt = 0; nt < C::NTQ; ++nt) {
      const float a = max3(S[0][nt][0], S[0][nt][1], S[0][nt][2]);
      const float b = max3(S[0][nt][3], S[1][nt][0], S[1][nt][1]);
      const float c = max3(S[1][nt][2], S[1][nt][3], S[2][nt][0]);
      const float d = max3(S[2][nt][1], S[2][nt][2], S[2][nt][3]);
      const float e = max3(S[3][nt][0], S[3][nt][1], S[3][nt][2]);
      const float tm = colmax4(max3(max3(a, b, c), max3(d, e, S[3][nt][3]), a));
      const float dlt = first ? tm + kQBias : fmaxf(tm + kQBias, 0.f);
      if (!first) {
        const float f = fast_exp2(-dlt);
#pragma unroll
        for (int i = 0; i <= C::MV; ++i) acc[i][nt] *= f;
      }
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int v = 0; v < 4; ++v) S[mt][nt][v] -= dlt;
      M[nt] += dlt;
      set_baug(nt);
    }
  };
  // [KV | z]^T Q~^T accumulated over the chunk's features.
  auto apply = [&](int ch, const Feat& qt) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int kcol = 64 * ch + 32 * kb + 8 * g;
#pragma unroll
      for (int mv = 0; mv <= C::MV; ++mv) {
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(&Kzl[(16 * mv + l16) * kzrow + kcol]);
#pragma unroll
        for (int nt = 0; nt < C::NTQ; ++nt) acc[mv][nt] = mma_bf16(ka, qt[kb][nt], acc[mv][nt]);
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
    for (int nt = 0; nt < C::NTQ; ++nt) {
      M[nt] = 0.f;
      set_baug(nt);
    }
  };

  // Software pipeline over (tile, chunk): chunk k+1 is projected on the
  // matrix cores while chunk k is applied, then its features are formed and
  // checked in the same step; a tile's last step projects the next tile's
  // first chunk.
  Qop qcur;
  convert(raw, qcur);
  if (ntile > 1) qload(tt0 + step, raw);
  reset();
  Feat FA, FB;
  {
    SArr S;
    proj(0, qcur, S);
    if constexpr (!RELU) rebase(S, true);
    features(S, FA);
  }
  for (int ti = 0; ti < ntile; ++ti) {
    const int tt = tt0 + ti * step;
    const bool more = ti + 1 < ntile;
    // Regular step: project chunk ch+1, apply chunk ch, form chunk ch+1.
    auto regular = [&](const int ch, const Feat& Fcur, Feat& Fnext) {
      __builtin_amdgcn_sched_barrier(0);
      SArr S;
      proj(ch + 1, qcur, S);
      apply(ch, Fcur);
      features(S, Fnext);
      if constexpr (!RELU) {
        if (__builtin_expect(overflow(Fnext), 0)) {
          rebase(S, false);
          features(S, Fnext);
        }
      }
    };
    // Last step of a tile: apply the last chunk, write the tile, then project
    // and form the next tile's first chunk.
    auto last = [&](const int ch, const Feat& Fcur, Feat& Fnext) {
      __builtin_amdgcn_sched_barrier(0);
      if (more) convert(raw, qcur);   // the current tile's operands are done
      apply(ch, Fcur);
      finish(tt);
      reset();
      if (more) {
        if (ti + 2 < ntile) qload(tt + 2 * step, raw);
        SArr S;
        proj(0, qcur, S);
        if constexpr (!RELU) rebase(S, true);
        features(S, Fnext);
      }
    };
    int ch = 0;
#pragma unroll 1
    for (; ch + 2 < NCH; ch += 2) {
      regular(ch, FA, FB);
      regular(ch + 1, FB, FA);
    }
    if constexpr ((NCH % 2) == 0) {
      regular(NCH - 2, FA, FB);
      last(NCH - 1, FB, FA);
    } else {
      last(NCH - 1, FA, FB);   // the next tile's first chunk landed in FB
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int nt = 0; nt < C::NTQ; ++nt) FA[kb][nt] = FB[kb][nt];
    }
  }
}

// ---------------------------------------------------------------------------
// qstream: the query side when W' and [KV | z] do not fit in LDS together
// (m (d+8) + (d+16)(m+8) halves over 160 KB, e.g. d = 128 with m = 512).
// Grid as qapply.  The NW waves take their 16*NTQ-token tiles in lockstep
// rounds, and each round streams the features through LDS in 64-feature
// chunks, in a ring of three buffers: chunks k+1 and k+2 travel from global
// memory straight into LDS (global_load_lds, no registers) while chunk k is
// used, and a step waits only for chunk k+1 (the barriers order LDS only,
// so chunk k+2's loads stay in flight across them).  A wave's Q tile for the
// next round is fetched at the start of the current one.  Per chunk
// buffer: W' rows [64][D+8] fp16 (as laid out in the workspace), [KV | z]
// columns [D+16][64] bf16 with the 16-byte units of row r XOR-swizzled by
// (r >> 1) & 7 (conflict-free operand reads without padding), c [64] fp32.
// A chunk is used in two 32-feature halves (projection, features,
// application), so that only one half's S is live (no spill at d = 128).
// Every LDS operand read feeds NTQ matrix instructions, so the operand
// traffic per token falls as 1/NTQ; NTQ = 4 needs one wave per SIMD
// (WPE = 1, accumulators in the AGPRs), which at d = 128, m = 512 measured
// slower than eight waves of NTQ = 2 (1128 against 922 us): a lone wave
// leaves the latency of its exponentials and LDS reads exposed.  The other
// way pays: twelve waves of NTQ = 2, three per SIMD (at most 168 registers,
// so a wave fetches its Q tile at the start of the round instead of one
// round ahead), measured 3% faster than eight.  Q and O
// pass with the non-temporal hint (once each; the chunks, re-read every
// round, stay in L2), O in 64-byte row pieces (finish): stored 8 bytes per
// lane, plainly the lines cost a fill read each (fetch up by the output's
// size), with the hint the written bytes doubled.
// ---------------------------------------------------------------------------
template <int D>
struct QsLds {
  static constexpr int WROW = D + 8;
  static constexpr int KROWS = D + 16;
  static constexpr int W_BYTES = 64 * WROW * 2;
  static constexpr int K_BYTES = KROWS * 64 * 2;
  static constexpr int BUF = W_BYTES + K_BYTES + 64 * 4;
  static constexpr int W16 = 64 * WROW / 8;     // 16-byte units per chunk
  static constexpr int K16 = KROWS * 8;
  static constexpr int WJOBS = W16 / 64;        // one wave instruction moves 64 units
  static constexpr int KJOBS = K16 / 64;
  static constexpr int JOBS = WJOBS + KJOBS + 1;   // + c (16 units)
  static_assert(W16 % 64 == 0 && K16 % 64 == 0, "whole waves per staging job");
};

template <int D, int NW, int NTQ, int NCH, bool RELU, int WPE>
__global__ __launch_bounds__(NW * 64, WPE) void qstream(const uint16_t* __restrict__ Q,
                                                     const _Float16* __restrict__ W16,
                                                     const uint16_t* __restrict__ Kz,
                                                     const float* __restrict__ cfin,
                                                     uint16_t* __restrict__ O, int L, int QL) {
  using C = QCfg<D, NTQ>;
  using LS = QsLds<D>;
  constexpr int m = 64 * NCH;
  constexpr int kzrow = m + 8;
  constexpr int NBUF = 3;
  __shared__ __align__(16) unsigned char qs_smem[NBUF * LS::BUF];
  const int nqb = (L + QL - 1) / QL;
  const int item = xcd_major(blockIdx.x, gridDim.x);
  const int qb = item % nqb, bh = item / nqb;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  const size_t base = static_cast<size_t>(bh) * L * D;
  const int q0 = qb * QL, q1 = min(L, q0 + QL);
  const int nround = (q1 - q0 + NW * C::TQ - 1) / (NW * C::TQ);
  if constexpr (WPE == 1) {
    // (an AGPR operand: the compiler then gives the matrix instructions'
    // accumulators the AGPRs, beside the 256 VGPRs)
    asm volatile("; accumulators in AGPRs %0" ::"a"(0.f));
  }

  auto Wl = [&](int b) { return reinterpret_cast<_Float16*>(qs_smem + b * LS::BUF); };
  auto Kzl = [&](int b) {
    return reinterpret_cast<uint16_t*>(qs_smem + b * LS::BUF + LS::W_BYTES);
  };
  auto cl = [&](int b) {
    return reinterpret_cast<float*>(qs_smem + b * LS::BUF + LS::W_BYTES + LS::K_BYTES);
  };

  // Chunk staging: job j (one wave instruction, 64 units of 16 bytes, lane i
  // landing at unit i) goes to wave j % NW.
  const uint4* const wsrc = reinterpret_cast<const uint4*>(W16);
  const uint4* const ksrc =
      reinterpret_cast<const uint4*>(Kz + static_cast<size_t>(bh) * (D + 16) * kzrow);
  const uint4* const csrc = reinterpret_cast<const uint4*>(cfin + static_cast<size_t>(bh) * m);
  auto stage = [&](int ch, int b) {
#pragma unroll
    for (int i = 0; i < (LS::JOBS + NW - 1) / NW; ++i) {
      const int j = wave + NW * i;
      if (j < LS::WJOBS) {
        lds_dma16(wsrc + ch * LS::W16 + 64 * j + lane, reinterpret_cast<uint4*>(Wl(b)) + 64 * j);
      } else if (j < LS::WJOBS + LS::KJOBS) {
        const int u = 64 * (j - LS::WJOBS) + lane;      // destination unit
        const int row = u >> 3, c8 = (u & 7) ^ ((row >> 1) & 7);
        lds_dma16(ksrc + (row * kzrow + 64 * ch) / 8 + c8,
                  reinterpret_cast<uint4*>(Kzl(b)) + 64 * (j - LS::WJOBS));
      } else if (j < LS::JOBS && lane < 16) {
        lds_dma16(csrc + 16 * ch + lane, cl(b));
      }
    }
  };
  // This wave's staging loads have landed in LDS (then a barrier publishes).
  auto staged = [&]() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };
  // ... all but this wave's staging loads of the newest chunk
  const int myjobs = (LS::JOBS - wave + NW - 1) / NW;
  auto staged_but_newest = [&]() {
    constexpr int lo = LS::JOBS / NW;
    if (myjobs > lo) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(lo + 1) : "memory");
    else asm volatile("s_waitcnt vmcnt(%0)" ::"n"(lo) : "memory");
  };

  using Qop = f16x8[C::NTQ][C::KS];
  using Qraw = u32x4[C::NTQ][C::KS];
  // Q rows of the tile at tt (zeros past the block), fetched a round ahead
  auto qfetch = [&](int tt, Qraw& x) {
#pragma unroll
    for (int nt = 0; nt < C::NTQ; ++nt) {
      const int tok = tt + 16 * nt + l16;
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        x[nt][ks] = u32x4{0u, 0u, 0u, 0u};
        if (tok < q1)
          x[nt][ks] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
              Q + base + static_cast<size_t>(tok) * D + 32 * ks + 8 * g));
      }
    }
  };
  auto qconv = [&](const Qraw& x, Qop& qop) {
#pragma unroll
    for (int nt = 0; nt < C::NTQ; ++nt)
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks)
        qop[nt][ks] = __builtin_bit_cast(
            f16x8, u32x4{bf16x2_to_f16x2(x[nt][ks].x), bf16x2_to_f16x2(x[nt][ks].y),
                         bf16x2_to_f16x2(x[nt][ks].z), bf16x2_to_f16x2(x[nt][ks].w)});
  };

  f32x4 acc[C::MV + 1][C::NTQ];
  float M[C::NTQ];
  using SArr = f32x4[2][C::NTQ];
  // S^T = W' Q^T + c for half kb of the chunk in buffer b (rows: features
  // 32 kb + 16 mh + 4 g + v of the chunk).
  auto proj = [&](int b, int kb, const Qop& qop, SArr& S) {
    const _Float16* w = Wl(b);
    const float* c = cl(b);
#pragma unroll
    for (int mh = 0; mh < 2; ++mh) {
      const int mt = 2 * kb + mh;
      f16x8 wa[C::KS];
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks)
        wa[ks] = *reinterpret_cast<const f16x8*>(&w[(16 * mt + l16) * LS::WROW + 32 * ks + 8 * g]);
      const f32x4 cb = *reinterpret_cast<const f32x4*>(&c[16 * mt + 4 * g]);
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
        for (int nt = 0; nt < C::NTQ; ++nt)
          S[mh][nt] = mma_f16(wa[ks], qop[nt][ks], ks == 0 ? cb : S[mh][nt]);
    }
  };
  // The per-token reference M: the exact maximum of the first half, raised
  // only when a later half exceeds it by more than kTau (the accumulators
  // are then rescaled by 2^-raise).
  auto stabilise = [&](SArr& S, bool first) {
    float lm[C::NTQ];
    bool raise = false;
#pragma unroll
    for (int nt = 0; nt < C::NTQ; ++nt) {
#pragma unroll
      for (int mh = 0; mh < 2; ++mh)
#pragma unroll
        for (int v = 0; v < 4; ++v) S[mh][nt][v] -= M[nt];
      const float a = max3(S[0][nt][0], S[0][nt][1], S[0][nt][2]);
      const float b = max3(S[0][nt][3], S[1][nt][0], S[1][nt][1]);
      lm[nt] = max3(a, b, fmaxf(S[1][nt][2], S[1][nt][3]));
      raise |= lm[nt] > kTau;
    }
    if (first || __builtin_expect(__ballot(raise) != 0, 0)) {
#pragma unroll
      for (int nt = 0; nt < C::NTQ; ++nt) {
        const float cm = colmax4(lm[nt]);
        const float dlt = (first || cm > kTau) ? cm : 0.f;
        if (!first) {
          const float f = fast_exp2(-dlt);
#pragma unroll
          for (int i = 0; i <= C::MV; ++i) acc[i][nt] *= f;
        }
#pragma unroll
        for (int mh = 0; mh < 2; ++mh)
#pragma unroll
          for (int v = 0; v < 4; ++v) S[mh][nt][v] -= dlt;
        M[nt] += dlt;
      }
    }
  };
  auto apply = [&](int b, int kb, const SArr& S) {
    const uint16_t* kz = Kzl(b);
    bf16x8 qt[C::NTQ];
#pragma unroll
    for (int nt = 0; nt < C::NTQ; ++nt) {
      uint32_t p[4];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        p[q] = pack_bf16(feature<RELU>(S[0][nt][2 * q]), feature<RELU>(S[0][nt][2 * q + 1]));
        p[2 + q] = pack_bf16(feature<RELU>(S[1][nt][2 * q]), feature<RELU>(S[1][nt][2 * q + 1]));
      }
      qt[nt] = __builtin_bit_cast(bf16x8, make_uint4(p[0], p[1], p[2], p[3]));
    }
#pragma unroll
    for (int mv = 0; mv <= C::MV; ++mv) {
      const int row = 16 * mv + l16, c8 = (4 * kb + g) ^ ((row >> 1) & 7);
      const bf16x8 ka = *reinterpret_cast<const bf16x8*>(&kz[row * 64 + 8 * c8]);
#pragma unroll
      for (int nt = 0; nt < C::NTQ; ++nt) acc[mv][nt] = mma_bf16(ka, qt[nt], acc[mv][nt]);
    }
  };
  // O rows: lanes g and g ^ 1 trade a quarter of two 16-value blocks, so
  // that each lane stores 16 contiguous bytes and the four lanes of a token
  // 64 (two blocks); streamed past L2 with the non-temporal hint.
  const __amdgpu_buffer_rsrc_t ro = buffer_rsrc(O + base, q1 * D * 2);
  auto finish = [&](int tt) {
    // (the lane's group, read here: its column offsets are not worth a
    // register through the round)
    int ln;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
    const int gq = (ln >> 4) & 3;
    const bool odd = (gq & 1) != 0;
#pragma unroll
    for (int nt = 0; nt < C::NTQ; ++nt) {
      const float den = __shfl(acc[C::MV][nt][0], l16, 64);
      const float inv = 1.0f / den;
      const int tok = tt + 16 * nt + l16;
#pragma unroll
      for (int pr = 0; pr < C::MV / 2; ++pr) {
        const f32x4 x0 = acc[2 * pr][nt], x1 = acc[2 * pr + 1][nt];
        const u32x2 a0 = u32x2{pack_bf16(x0[0] * inv, x0[1] * inv), pack_bf16(x0[2] * inv, x0[3] * inv)};
        const u32x2 a1 = u32x2{pack_bf16(x1[0] * inv, x1[1] * inv), pack_bf16(x1[2] * inv, x1[3] * inv)};
        // even g keeps block 2 pr (values 4 g .. 4 g + 7), odd g block
        // 2 pr + 1 (values 4 (g - 1) .. 4 g + 3)
        const u32x2 give = odd ? a0 : a1;
        const u32x2 got = u32x2{static_cast<uint32_t>(__shfl_xor(static_cast<int>(give.x), 16, 64)),
                                static_cast<uint32_t>(__shfl_xor(static_cast<int>(give.y), 16, 64))};
        const u32x4 out = odd ? u32x4{got.x, got.y, a1.x, a1.y} : u32x4{a0.x, a0.y, got.x, got.y};
        const int col = odd ? 16 * (2 * pr + 1) + 4 * (gq - 1) : 16 * (2 * pr) + 4 * gq;
        // (a buffer store past the head's last token is dropped; cache
        // policy 2: non-temporal)
        __builtin_amdgcn_raw_buffer_store_b128(out, ro, (tok * D + col) * 2, 0, 2);
      }
    }
  };

  // Every wave runs every round and chunk (tiles past the block compute on
  // zeros and store nothing), so the work-group barriers always match.
  const int T = nround * NCH;
  stage(0, 0);
  if (T > 1) {
    stage(1 % NCH, 1);
    staged_but_newest();
  } else {
    staged();
  }
  lds_barrier();
  int t = 0;
  Qop qcur;
  // (with three waves per SIMD the registers do not hold a second tile:
  // the round's tile is fetched at its start)
  constexpr bool QPF = WPE <= 2;
  Qraw qraw;
  if constexpr (QPF) qfetch(q0 + wave * C::TQ, qraw);
  for (int r = 0; r < nround; ++r) {
    const int tt = q0 + (r * NW + wave) * C::TQ;
    if constexpr (QPF) {
      qconv(qraw, qcur);
      if (r + 1 < nround) qfetch(tt + NW * C::TQ, qraw);
    } else {
      qfetch(tt, qraw);
      qconv(qraw, qcur);
    }
#pragma unroll
    for (int i = 0; i <= C::MV; ++i)
#pragma unroll
      for (int nt = 0; nt < C::NTQ; ++nt) acc[i][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int nt = 0; nt < C::NTQ; ++nt) M[nt] = 0.f;
#pragma unroll 1
    for (int ch = 0; ch < NCH; ++ch, ++t) {
      // (buffer (t + 2) % 3 was last read in step t - 1, before its barrier)
      if (t + 2 < T) stage((t + 2) % NCH, (t + 2) % NBUF);
      const int b = t % NBUF;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        SArr S;
        proj(b, kb, qcur, S);
        if constexpr (!RELU) stabilise(S, ch == 0 && kb == 0);
        apply(b, kb, S);
      }
      if (t + 2 < T) staged_but_newest();
      else staged();
      lds_barrier();
    }
    finish(tt);
  }
}

// ---------------------------------------------------------------------------
// Causal (masked) form, three launches:
//   kpart    per (head, segment): the segment's key state, as above;
//   kprefix  per head: exclusive prefix of the segment states in segment
//            order (rescaled to a running per-feature reference), in place;
//   cscan    per (head, segment): 32-token chunks in order, carrying the
//            state [S | z] in registers from the prefix, with the masked
//            in-chunk term on the matrix cores.
// ---------------------------------------------------------------------------

// kprefix: grid (ceil((D+1) m / 1024), BH), 256 threads; a thread owns four
// features of one row.  P[bh][s] becomes the sum of segments before s and
// cP[bh][s] its per-feature reference, for s >= 1 (the scan starts the first
// segment from a zero state and reads neither).  The last segment's own
// state is not needed for the scan, so the state kernels leave it out,
// unless Sout is given: then P[bh][nseg-1] holds it too and the total (the
// state after the last token) goes to Sout in the exported layout (values
// in units of e^c, c in natural-log units, zero pads; softmax and Gaussian
// features only).  With an imported state Sin (the exported layout
// [BH][m][D+4], reference in natural-log units) the sum starts from it, and
// every segment, the first included, gets a carry.
template <int D>
__global__ __launch_bounds__(256) void kprefix(float* __restrict__ P, const float* __restrict__ cs,
                                               float* __restrict__ cP, const float* __restrict__ Sin,
                                               int m, int nseg, float sin_scale,
                                               float* __restrict__ Sout = nullptr) {
  const int bh = blockIdx.y;
  const int e = blockIdx.x * 256 + threadIdx.x;
  const int mq = m / 4;
  if (e >= (D + 1) * mq) return;
  const int row = e / mq, f = 4 * (e - row * mq);
  float4 run = make_float4(0.f, 0.f, 0.f, 0.f);
  float4 rc = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
  const bool carry = Sin != nullptr;
  if (carry) {
    // exported values: log2-unit reference c log2(e); ReLU states in the
    // features' log2(e) scale (sin_scale)
    const float* sr = Sin + (static_cast<size_t>(bh) * m + f) * (D + 4);
    run = make_float4(sr[row] * sin_scale, sr[(D + 4) + row] * sin_scale,
                      sr[2 * (D + 4) + row] * sin_scale, sr[3 * (D + 4) + row] * sin_scale);
    rc = make_float4(sr[D + 1] * kLog2e, sr[(D + 4) + D + 1] * kLog2e,
                     sr[2 * (D + 4) + D + 1] * kLog2e, sr[3 * (D + 4) + D + 1] * kLog2e);
  }
  // Segments in batches of KB: the batch's loads are issued together (the
  // sum is a chain; its latency is paid once per batch, not per segment).
  constexpr int KB = 8;
  auto slot = [&](int s) {
    return reinterpret_cast<float4*>(P + ((static_cast<size_t>(bh) * nseg + s) * (D + 1) + row) * m + f);
  };
  auto cidx = [&](int s) { return (static_cast<size_t>(bh) * nseg + s) * m + f; };
  for (int s0 = 0; s0 < nseg; s0 += KB) {
    float4 ts[KB], c[KB];
#pragma unroll
    for (int k = 0; k < KB; ++k) {
      // (the last segment's own state is read only for the total)
      if (s0 + k + 1 < nseg || (Sout && s0 + k < nseg)) {
        ts[k] = *slot(s0 + k);
        c[k] = *reinterpret_cast<const float4*>(cs + cidx(s0 + k));
      }
    }
#pragma unroll
    for (int k = 0; k < KB; ++k) {
      const int s = s0 + k;
      if (s >= nseg) break;
      const bool put = s > 0 || carry;
      if (row == 0 && put) *reinterpret_cast<float4*>(cP + cidx(s)) = rc;
      if (put) *slot(s) = run;
      if (s + 1 == nseg && !Sout) break;
      float4 nc;
      nc.x = fmaxf(rc.x, c[k].x); nc.y = fmaxf(rc.y, c[k].y);
      nc.z = fmaxf(rc.z, c[k].z); nc.w = fmaxf(rc.w, c[k].w);
      run.x = run.x * fast_exp2(rc.x - nc.x) + ts[k].x * fast_exp2(c[k].x - nc.x);
      run.y = run.y * fast_exp2(rc.y - nc.y) + ts[k].y * fast_exp2(c[k].y - nc.y);
      run.z = run.z * fast_exp2(rc.z - nc.z) + ts[k].z * fast_exp2(c[k].z - nc.z);
      run.w = run.w * fast_exp2(rc.w - nc.w) + ts[k].w * fast_exp2(c[k].w - nc.w);
      rc = nc;
      if (s + 1 == nseg) break;
    }
  }
  if (Sout) {
    float* o = Sout + (static_cast<size_t>(bh) * m + f) * (D + 4);
    o[row] = run.x;
    o[(D + 4) + row] = run.y;
    o[2 * (D + 4) + row] = run.z;
    o[3 * (D + 4) + row] = run.w;
    if (row == 0) {
      const float rcn[4] = {rc.x, rc.y, rc.z, rc.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        o[j * (D + 4) + D + 1] = rcn[j] * 0.6931471805599453f;
        o[j * (D + 4) + D + 2] = 0.f;
        o[j * (D + 4) + D + 3] = 0.f;
      }
    }
  }
}

// cscan: grid (nseg, BH), NW waves (d = 64; wave w owns features
// [64 w, 64 w + 64)).  State per wave, in registers: st[mt][tv] with lane =
// value column 16 tv + l16 (tv = 4: the ones column, z) and rows = features
// 16 mt + 4 g + v; its per-feature references cref (log2 units).
//
// BWD: the same scan for the backward pass; instead of O it writes, per
// query, lp[i] = (L_i, p_i) with L_i = log2 of the denominator taken with no
// reference (log2 sum_{j <= i} sum_r 2^(s_ir + e_jr), the same in every
// frame of references) and p_i = dO_i . O_i in fp32.
template <int NW, bool RELU, bool BWD = false>
__global__ __launch_bounds__(NW * 64, 2) void cscan(const uint16_t* __restrict__ Q,
                                                  const uint16_t* __restrict__ K,
                                                  const uint16_t* __restrict__ V,
                                                  const float* __restrict__ W,
                                                  const float* __restrict__ P,
                                                  const float* __restrict__ cP,
                                                  uint16_t* __restrict__ O, int L, int m, int SEG,
                                                  int nseg, float knorm, int carry0,
                                                  const uint16_t* __restrict__ dO = nullptr,
                                                  float2* __restrict__ lp = nullptr) {
  constexpr int D = 64;
  constexpr int NTH = NW * 64;
  constexpr int KS = 2, NT = 4, TV = 5;
  constexpr int CPR = D / 8;                 // 16-byte chunks per row
  constexpr int KCH = kTT * CPR;             // per tile and tensor
  constexpr int KPT = (KCH + NTH - 1) / NTH;
  constexpr int VUN = (kTT / 2) * (D / 4);
  constexpr int VPT = (VUN + NTH - 1) / NTH;
  constexpr int KROW = D + 8;
  constexpr int CROW = D + 4;                // floats per (wave, query) row of partial outputs
  const int s = blockIdx.x, bh = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int f0 = wave * 64;

  __shared__ __align__(16) _Float16 Ks[2][kTT][KROW];
  __shared__ __align__(16) _Float16 Qs[2][kTT][KROW];
  __shared__ __align__(16) uint32_t Vt[2][D][kTT / 2 + 4];
  __shared__ __align__(16) float Ns[2][kTT];
  __shared__ __align__(16) float Nq[2][kTT];   // fast pass: -|q|^2 log2(e) / 2 per query
  __shared__ unsigned vote;
  // Per wave, one region holds first this chunk's K~ over the wave's features
  // (key rows; read only by the wave itself) and then the wave's partial
  // outputs [query][column], columns 0..D-1 the numerator, D the
  // denominator (read by all after a barrier).
  static_assert(kTT * CROW * 4 >= kTT * KROW * 2, "K~ tile fits the partial-output region");
  __shared__ __align__(16) float ured[NW][kTT * CROW];
  __shared__ __align__(16) float cb[NW][64];                // per-feature references
  __shared__ __align__(16) float mq[NW][kTT];               // per-wave row references
  uint16_t* const Kt = reinterpret_cast<uint16_t*>(&ured[wave][0]);

  // W' (fp16) operands of both projections: W'[f0 + 16 nt + l16][32 ks + 8 g + u].
  f16x8 wreg[NT][KS];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const float* wr = W + static_cast<size_t>(f0 + 16 * nt + l16) * D + 8 * g;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const float4 a = *reinterpret_cast<const float4*>(wr + 32 * ks);
      const float4 b = *reinterpret_cast<const float4*>(wr + 32 * ks + 4);
      f16x8 v;
      v[0] = static_cast<_Float16>(a.x * kLog2e); v[1] = static_cast<_Float16>(a.y * kLog2e);
      v[2] = static_cast<_Float16>(a.z * kLog2e); v[3] = static_cast<_Float16>(a.w * kLog2e);
      v[4] = static_cast<_Float16>(b.x * kLog2e); v[5] = static_cast<_Float16>(b.y * kLog2e);
      v[6] = static_cast<_Float16>(b.z * kLog2e); v[7] = static_cast<_Float16>(b.w * kLog2e);
      wreg[nt][ks] = v;
    }
  }

  // Carry-in: the prefix state of the segments before this one (none for
  // the first segment unless a state was imported: zero state, no reference
  // yet).
  f32x4 st[NT][TV];
  float cref[NT];
  auto carry_in = [&]() {
#pragma unroll
    for (int mt = 0; mt < NT; ++mt) {
      cref[mt] = -INFINITY;
#pragma unroll
      for (int tv = 0; tv < TV; ++tv) st[mt][tv] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    if (s > 0 || carry0) {
      const size_t pbase = (static_cast<size_t>(bh) * nseg + s) * (D + 1);
      const size_t cbase = (static_cast<size_t>(bh) * nseg + s) * m;
#pragma unroll
      for (int mt = 0; mt < NT; ++mt) {
        const int f = f0 + 16 * mt + 4 * g;
#pragma unroll
        for (int tv = 0; tv < TV; ++tv) {
          const int col = 16 * tv + l16;
          if (col <= D) st[mt][tv] = *reinterpret_cast<const f32x4*>(P + (pbase + col) * m + f);
        }
        cref[mt] = cP[cbase + f0 + 16 * mt + l16];   // this lane's feature (S layout)
      }
    }
  };
  carry_in();

  const int j0 = s * SEG, j1 = min(L, j0 + SEG);
  const int nch = (j1 - j0 + kTT - 1) / kTT;
  const size_t base = static_cast<size_t>(bh) * L * D;

  uint4 kreg[KPT], qreg[KPT];
  uint2 vreg[VPT][2];
  auto gload = [&](int t) {
    const int jt = j0 + t * kTT;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int c = tid + i * NTH;
      const int tok = jt + c / CPR;
      kreg[i] = make_uint4(0, 0, 0, 0);
      qreg[i] = make_uint4(0, 0, 0, 0);
      if (c < KCH && tok < j1) {
        const size_t off = base + static_cast<size_t>(tok) * D + (c % CPR) * 8;
        kreg[i] = *reinterpret_cast<const uint4*>(K + off);
        qreg[i] = *reinterpret_cast<const uint4*>(Q + off);
      }
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
  // -knorm log2(e), kept in a scalar register
  const float nk2 = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(-knorm * kLog2e)));
  auto lstore = [&](auto FASTC, int buf, int t) {
    constexpr bool F = decltype(FASTC)::value;
    const int jt = j0 + t * kTT;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int c = tid + i * NTH;
      const int j = (c / CPR) % kTT, ch = c % CPR;
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
      ss = group_sum<CPR>(ss);
      float sq = 0.f;
      if constexpr (F) {
        const uint32_t w4[4] = {qreg[i].x, qreg[i].y, qreg[i].z, qreg[i].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float lo = bf16_lo(w4[q]), hi = bf16_hi(w4[q]);
          sq = fmaf(lo, lo, sq);
          sq = fmaf(hi, hi, sq);
        }
        sq = group_sum<CPR>(sq);
      }
      if (c < KCH) {
        uint4 h;
        h.x = bf16x2_to_f16x2(kv.x); h.y = bf16x2_to_f16x2(kv.y);
        h.z = bf16x2_to_f16x2(kv.z); h.w = bf16x2_to_f16x2(kv.w);
        *reinterpret_cast<uint4*>(&Ks[buf][j][ch * 8]) = h;
        if constexpr (F) {
          if (ch == 0) Nq[buf][j] = -0.5f * kLog2e * sq;
        }
        const uint4 qv = qreg[i];
        h.x = bf16x2_to_f16x2(qv.x); h.y = bf16x2_to_f16x2(qv.y);
        h.z = bf16x2_to_f16x2(qv.z); h.w = bf16x2_to_f16x2(qv.w);
        *reinterpret_cast<uint4*>(&Qs[buf][j][ch * 8]) = h;
        if (ch == 0) Ns[buf][j] = (jt + j < j1) ? nk2 * ss : -INFINITY;
      }
    }
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

  bf16x8 ones, onecol;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    ones[u] = static_cast<__bf16>(1.0f);
    onecol[u] = static_cast<__bf16>(l16 == 0 ? 1.0f : 0.0f);   // [V | 1]'s last column
  }
  // B operand [V | 1] (tokens x value columns) for value-column tile tv.
  auto vop = [&](int buf, int tv) -> bf16x8 {
    if (tv < 4) return *reinterpret_cast<const bf16x8*>(&Vt[buf][16 * tv + l16][4 * g]);
    return onecol;
  };

  // FASTC true: the fast pass (softmax and Gaussian features, no carried
  // reference): no per-feature key reference (the key exponent is at most
  // |w|^2 log2(e) / 2 whatever k is) and the query's norm term as its row
  // shift (it cancels in D^-1 and bounds the query exponent the same way),
  // so the waves' partial outputs share one reference; a query whose
  // denominator leaves [2^-100, 2^100] (or is not finite) sets `bad`.
  bool bad = false;
  auto chunk = [&](auto FASTC, const int buf, const int jt) {
    constexpr bool F = decltype(FASTC)::value;
    // (1) Key exponents S = K W'^T - n' (lane = feature, rows = tokens).
    f32x4 SK[2][NT];
    {
      f32x4 cinit[2];
      f16x8 ka[2][KS];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        cinit[mt] = *reinterpret_cast<const f32x4*>(&Ns[buf][16 * mt + 4 * g]);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          ka[mt][ks] = *reinterpret_cast<const f16x8*>(&Ks[buf][16 * mt + l16][32 * ks + 8 * g]);
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
            SK[mt][nt] = mma_f16(ka[mt][ks], wreg[nt][ks], ks == 0 ? cinit[mt] : SK[mt][nt]);
    }
    // Per-feature references: lazy raise, always on a segment with no carry
    // (none for ReLU features).
    bool raise = false;
    float lm[NT];
#pragma unroll
    for (int nt = 0; nt < NT && !RELU && !F; ++nt) {
      const float c = cref[nt] == -INFINITY ? 0.f : cref[nt];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int v = 0; v < 4; ++v) SK[mt][nt][v] -= c;
      const float a = max3(SK[0][nt][0], SK[0][nt][1], SK[0][nt][2]);
      const float b = max3(SK[0][nt][3], SK[1][nt][0], SK[1][nt][1]);
      lm[nt] = max3(a, b, fmaxf(SK[1][nt][2], SK[1][nt][3]));
      raise |= (cref[nt] == -INFINITY) || lm[nt] > kTau;
    }
    if (!RELU && !F && __builtin_expect(__ballot(raise) != 0, 0)) {
      float fk[NT];   // rescale factor of feature 16 nt + l16 (every g)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const float tm = colmax4(lm[nt]);
        const bool empty = cref[nt] == -INFINITY;
        const float base_c = empty ? 0.f : cref[nt];
        const float dlt = (empty || tm > kTau) ? tm : 0.f;
        fk[nt] = empty ? 1.f : fast_exp2(-dlt);
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int v = 0; v < 4; ++v) SK[mt][nt][v] -= dlt;
        cref[nt] = base_c + dlt;
      }
      // The state's rows are features 16 mt + 4 g + v: their factors sit in
      // lanes 4 g + v.  (The lane index is read here, in this rare branch,
      // so that no register carries it through the scan.)
      int ln;
      asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
      const int src = 16 * ((ln >> 4) & 3);   // byte address of lane 4 g
      auto from = [&](float x, int v) {
        return __int_as_float(__builtin_amdgcn_ds_bpermute(src + 4 * v, __float_as_int(x)));
      };
#pragma unroll
      for (int mt = 0; mt < NT; ++mt) {
        const f32x4 fv = f32x4{from(fk[mt], 0), from(fk[mt], 1), from(fk[mt], 2), from(fk[mt], 3)};
#pragma unroll
        for (int tv = 0; tv < TV; ++tv) st[mt][tv] *= fv;
      }
    }
    if constexpr (!F) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        if (g == 0) cb[wave][16 * nt + l16] = RELU ? 0.f : cref[nt];
    }
    // K~ (lane = feature, 8 tokens at positions perm_of), and its transpose
    // into Kt (key rows; features permuted within 32-blocks for the MFMA).
    bf16x8 kb[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      uint32_t p[4];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        p[q] = pack_bf16(feature<RELU>(SK[0][nt][2 * q]), feature<RELU>(SK[0][nt][2 * q + 1]));
        p[2 + q] = pack_bf16(feature<RELU>(SK[1][nt][2 * q]), feature<RELU>(SK[1][nt][2 * q + 1]));
      }
      kb[nt] = __builtin_bit_cast(bf16x8, make_uint4(p[0], p[1], p[2], p[3]));
      const int fl = 16 * nt + l16;                               // local feature
      const int fc = (fl & ~31) + perm_inv(fl & 31);              // its column in Kt
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const uint32_t w = p[u >> 1];
        Kt[perm_of(8 * g + u) * KROW + fc] = static_cast<uint16_t>((u & 1) ? (w >> 16) : (w & 0xffffu));
      }
    }

    wave_lds_fence();   // cb and K~ written above, read below by other lanes

    // (2) Query exponents S^T = W' Q^T + c (lane = query, rows = features),
    // with the wave's own row maximum as reference.
    f32x4 SQ[NT][2];
    {
      f32x4 cq[NT];
      f32x4 cn[2];   // (fast pass) the query's norm term, lane = query
      f16x8 qa[2][KS];
      if constexpr (F) {
#pragma unroll
        for (int nq = 0; nq < 2; ++nq) {
          const float x = Nq[buf][16 * nq + l16];
          cn[nq] = f32x4{x, x, x, x};
        }
      } else {
#pragma unroll
        for (int mt = 0; mt < NT; ++mt) cq[mt] = *reinterpret_cast<const f32x4*>(&cb[wave][16 * mt + 4 * g]);
      }
#pragma unroll
      for (int nq = 0; nq < 2; ++nq)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          qa[nq][ks] = *reinterpret_cast<const f16x8*>(&Qs[buf][16 * nq + l16][32 * ks + 8 * g]);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int mt = 0; mt < NT; ++mt)
#pragma unroll
          for (int nq = 0; nq < 2; ++nq)
            SQ[mt][nq] = mma_f16(wreg[mt][ks], qa[nq][ks],
                                 ks == 0 ? (F ? cn[nq] : cq[mt]) : SQ[mt][nq]);
    }
    bf16x8 qt[2][2];   // [kb][nq]: lane = query, 8 features (perm_of within 32-block kb)
#pragma unroll
    for (int nq = 0; nq < 2; ++nq) {
      float M = 0.f;
      if constexpr (!RELU && !F) {
        const float a = max3(SQ[0][nq][0], SQ[0][nq][1], SQ[0][nq][2]);
        const float b = max3(SQ[0][nq][3], SQ[1][nq][0], SQ[1][nq][1]);
        const float c = max3(SQ[1][nq][2], SQ[1][nq][3], SQ[2][nq][0]);
        const float d = max3(SQ[2][nq][1], SQ[2][nq][2], SQ[2][nq][3]);
        const float e = max3(SQ[3][nq][0], SQ[3][nq][1], SQ[3][nq][2]);
        M = colmax4(max3(max3(a, b, c), max3(d, e, SQ[3][nq][3]), a));
      }
      if (!F && g == 0) mq[wave][16 * nq + l16] = M;
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
        uint32_t p[4];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          p[q] = pack_bf16(feature<RELU>(SQ[2 * kb2][nq][2 * q] - M),
                           feature<RELU>(SQ[2 * kb2][nq][2 * q + 1] - M));
          p[2 + q] = pack_bf16(feature<RELU>(SQ[2 * kb2 + 1][nq][2 * q] - M),
                               feature<RELU>(SQ[2 * kb2 + 1][nq][2 * q + 1] - M));
        }
        qt[kb2][nq] = __builtin_bit_cast(bf16x8, make_uint4(p[0], p[1], p[2], p[3]));
      }
    }

    // (3) Partial output over the wave's features, transposed:
    // num^T = [S|z]^T Q~^T + [V|1]^T A^T (lane = query, rows = value columns
    // 16 tv + 4 g + v); first the carried state, as bf16 operands (the same
    // registers serve as the A operand [column][feature]).
    f32x4 num[TV][2];
#pragma unroll
    for (int tv = 0; tv < TV; ++tv)
#pragma unroll
      for (int nq = 0; nq < 2; ++nq) num[tv][nq] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int tv = 0; tv < TV; ++tv) {
        const f32x4 lo = st[2 * kb2][tv], hi = st[2 * kb2 + 1][tv];
        const bf16x8 sb = __builtin_bit_cast(
            bf16x8, make_uint4(pack_bf16(lo[0], lo[1]), pack_bf16(lo[2], lo[3]),
                               pack_bf16(hi[0], hi[1]), pack_bf16(hi[2], hi[3])));
#pragma unroll
        for (int nq = 0; nq < 2; ++nq) num[tv][nq] = mma_bf16(sb, qt[kb2][nq], num[tv][nq]);
      }
    // (4) State update with this chunk's keys: [S|z] += K~^T [V|1].
#pragma unroll
    for (int tv = 0; tv < TV; ++tv) {
      const bf16x8 vb = vop(buf, tv);
#pragma unroll
      for (int mt = 0; mt < NT; ++mt) st[mt][tv] = mma_bf16(kb[mt], vb, st[mt][tv]);
    }

    // (5) In-chunk term A^T = K~ Q~^T over the wave's features (keys x
    // queries), lower triangle only; masked, to bf16 as [key] operands.
    bf16x8 ab[2];
    {
      f32x4 At[2][2];
#pragma unroll
      for (int mk = 0; mk < 2; ++mk)
#pragma unroll
        for (int nq = 0; nq < 2; ++nq) At[mk][nq] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
        for (int mk = 0; mk < 2; ++mk) {
          const bf16x8 ka = *reinterpret_cast<const bf16x8*>(&Kt[(16 * mk + l16) * KROW + 32 * kb2 + 8 * g]);
#pragma unroll
          for (int nq = mk; nq < 2; ++nq) At[mk][nq] = mma_bf16(ka, qt[kb2][nq], At[mk][nq]);
        }
      }
#pragma unroll
      for (int nq = 0; nq < 2; ++nq) {
        float x[8];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          // key 16 mk + 4 g + v against query 16 nq + l16 (the diagonal counts)
          x[v] = (nq > 0 || 4 * g + v <= l16) ? At[0][nq][v] : 0.f;
          x[4 + v] = (nq == 1 && 16 + 4 * g + v <= 16 + l16) ? At[1][nq][v] : 0.f;
        }
        ab[nq] = __builtin_bit_cast(bf16x8, make_uint4(pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3]),
                                                       pack_bf16(x[4], x[5]), pack_bf16(x[6], x[7])));
      }
    }

    // ... and the in-chunk term ([V|1]^T as the A operand: same registers).
#pragma unroll
    for (int tv = 0; tv < TV; ++tv) {
      const bf16x8 vb = vop(buf, tv);
#pragma unroll
      for (int nq = 0; nq < 2; ++nq) num[tv][nq] = mma_bf16(vb, ab[nq], num[tv][nq]);
    }

    wave_lds_fence();   // K~ tile read above; its region is overwritten next

    // (6) Partial outputs to LDS, [wave][query][column], over the K~ tile
    // (the wave's own step (3) is done with it); of the last column tile only
    // the denominator's quad (g = 0: columns D..D+3).
#pragma unroll
    for (int tv = 0; tv < TV; ++tv)
#pragma unroll
      for (int nq = 0; nq < 2; ++nq)
        if (tv < TV - 1 || g == 0)
          *reinterpret_cast<f32x4*>(&ured[wave][(16 * nq + l16) * CROW + 16 * tv + 4 * g]) = num[tv][nq];
    lds_barrier();
    // Combine the waves' partials (row references differ per wave) and
    // write O: thread -> (query, 8 columns); eight threads cover one row.
    for (int o = tid; o < kTT * (D / 8); o += NTH) {
      const int i = o / (D / 8), c0 = 8 * (o % (D / 8));
      float mw[NW], mx = F ? 0.f : -INFINITY;
      if constexpr (!F) {
#pragma unroll
        for (int w = 0; w < NW; ++w) { mw[w] = mq[w][i]; mx = fmaxf(mx, mw[w]); }
      }
      float acc8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      float den = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float sc = F ? 1.f : fast_exp2(mw[w] - mx);
        const float* row = &ured[w][i * CROW];
        den = fmaf(sc, row[D], den);
        const f32x4 a = *reinterpret_cast<const f32x4*>(row + c0);
        const f32x4 b = *reinterpret_cast<const f32x4*>(row + c0 + 4);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          acc8[c] = fmaf(sc, a[c], acc8[c]);
          acc8[4 + c] = fmaf(sc, b[c], acc8[4 + c]);
        }
      }
      const float inv = 1.0f / den;
      if constexpr (F) bad |= (jt + i < j1) && !(den >= 0x1p-100f && den <= 0x1p100f);
      if constexpr (BWD) {
        // (the eight threads of a row are consecutive lanes of one wave)
        float pd = 0.f;
        if (jt + i < j1) {
          const uint4 gv = *reinterpret_cast<const uint4*>(dO + base + static_cast<size_t>(jt + i) * D + c0);
          const uint32_t g4[4] = {gv.x, gv.y, gv.z, gv.w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            pd = fmaf(bf16_lo(g4[q]), acc8[2 * q] * inv, pd);
            pd = fmaf(bf16_hi(g4[q]), acc8[2 * q + 1] * inv, pd);
          }
        }
        pd = group_sum<8>(pd);
        if (c0 == 0 && jt + i < j1)
          lp[static_cast<size_t>(bh) * L + jt + i] = make_float2(log2f(den) + mx, pd);
      } else if (jt + i < j1) {
        uint4 ov;
        ov.x = pack_bf16(acc8[0] * inv, acc8[1] * inv);
        ov.y = pack_bf16(acc8[2] * inv, acc8[3] * inv);
        ov.z = pack_bf16(acc8[4] * inv, acc8[5] * inv);
        ov.w = pack_bf16(acc8[6] * inv, acc8[7] * inv);
        *reinterpret_cast<uint4*>(O + base + static_cast<size_t>(jt + i) * D + c0) = ov;
      }
    }
  };

  auto scan = [&](auto FASTC) {
    gload(0);
    lstore(FASTC, 0, 0);
    for (int t = 0; t < nch; ++t) {
      const int buf = t & 1;
      if (t + 1 < nch) gload(t + 1);
      lds_barrier();
      chunk(FASTC, buf, j0 + t * kTT);
      if (t + 1 < nch) lstore(FASTC, buf ^ 1, t + 1);
    }
  };
  if constexpr (!RELU && !BWD) {
    // The fast pass when the carried state has no reference (every earlier
    // segment's keys were summed without one); the referenced pass again
    // from the carry-in when any query's denominator came out of range.
    bool refd = false;
#pragma unroll
    for (int mt = 0; mt < NT; ++mt) refd |= cref[mt] != -INFINITY && cref[mt] != 0.f;
    if (tid == 0) vote = 0u;
    lds_barrier();
    if (refd) vote = 1u;
    lds_barrier();
    if (vote == 0u) {
#pragma unroll
      for (int mt = 0; mt < NT; ++mt) cref[mt] = 0.f;
      scan(std::true_type{});
      lds_barrier();   // (every wave is done with the LDS tiles and the vote word)
      if (tid == 0) vote = 0u;
      lds_barrier();
      if (bad) vote = 1u;
      lds_barrier();
      if (vote == 0u) return;
      carry_in();
    }
  }
  scan(std::false_type{});
}

// The bidirectional path for m = NFB NW FPW features: kpart in NFB feature
// blocks of NW waves, kcombine, then qapply (W', [KV | z] and c resident in
// LDS) or, when they do not fit, qstream.
template <int D, int NW, int NFB, bool RELU>
hipError_t launch_d(const Plan& p, const uint16_t* Q, const uint16_t* K, const uint16_t* V,
                    const float* W, uint16_t* O, char* ws, hipStream_t st) {
  float* P = reinterpret_cast<float*>(ws + p.off_T);
  float* cs = reinterpret_cast<float*>(ws + p.off_cseg);
  uint16_t* Kz = reinterpret_cast<uint16_t*>(ws + p.off_KV);
  float* cfin = reinterpret_cast<float*>(ws + p.off_cfin);
  _Float16* W16 = reinterpret_cast<_Float16*>(ws + p.off_cP);
  // Two token groups while a work-group stays within 8 waves (two per SIMD).
  constexpr int TG = (NW <= 4) ? 2 : 1;
  timing_before(st);
  kpart<D, NW, TG, RELU><<<dim3(p.nseg * p.BH * NFB), TG * NW * 64, 0, st>>>(K, V, W, P, cs, p.L, p.m,
                                                                       p.seg, p.nseg, p.nseg,
                                                                       p.knorm);
  hipError_t e = hipGetLastError();
  timing_after(st, "kpart");
  if (e != hipSuccess) return e;
  timing_before(st);
  kcombine<D><<<dim3(((D + 16) * p.m / 4 + 255) / 256, p.BH), 256, 0, st>>>(P, cs, W, Kz, cfin,
                                                                            W16, p.m, p.nseg);
  e = hipGetLastError();
  timing_after(st, "kcombine");
  if (e != hipSuccess) return e;
  const int nqb = (p.L + p.qblk - 1) / p.qblk;
  constexpr int NTQ = FAVOR_QAPPLY_NTQ;
  constexpr int NCH = NFB * NW * KCfg<D>::FPW / 64;   // m / 64
  const size_t lds = qapply_lds_bytes<D>(p.m);
  if (lds <= 160 * 1024) {
    constexpr int QNW = FAVOR_QAPPLY_NW;
    auto* kern = &qapply<D, QNW, NTQ, NCH, RELU>;
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                            hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
    timing_before(st);
    kern<<<dim3(nqb * p.BH), QNW * 64, lds, st>>>(Q, W16, Kz, cfin, O, p.L, p.qblk);
    e = hipGetLastError();
    timing_after(st, "qapply");
  } else {
    timing_before(st);
    constexpr int SNW = FAVOR_QSTREAM_NW, SNTQ = FAVOR_QSTREAM_NTQ;
    qstream<D, SNW, SNTQ, NCH, RELU, FAVOR_QSTREAM_WPE><<<dim3(nqb * p.BH), SNW * 64, 0, st>>>(
        Q, W16, Kz, cfin, O, p.L, p.qblk);
    e = hipGetLastError();
    timing_after(st, "qstream");
  }
  return e;
}

template <int NW, bool RELU>
hipError_t launch_causal(const Plan& p, const uint16_t* Q, const uint16_t* K, const uint16_t* V,
                         const float* W, uint16_t* O, char* ws, const float* Sin,
                         hipStream_t st, float* Sout, bool* exported) {
  // The state after the last token comes out of the prefix pass when the
  // segment states come from ckey (every segment's state, the last one's
  // included).
  const bool ckey_path = !RELU && NW == 4;
  if (!ckey_path) Sout = nullptr;
  float* P = reinterpret_cast<float*>(ws + p.off_T);
  float* cs = reinterpret_cast<float*>(ws + p.off_cseg);
  float* cP = reinterpret_cast<float*>(ws + p.off_cP);
  hipError_t e;
  if (ckey_path && (p.nseg > 1 || Sout)) {
    // Key states of every segment but the last (with Sout: every segment),
    // two segments per work-group (m = 256, softmax and Gaussian features).
    e = fused_causal_key_states(p, K, V, W, P, cs, st, Sout != nullptr);
    if (e != hipSuccess) return e;
  } else if (p.nseg > 1) {
    // Key states of every segment but the last (grid nseg - 1; the layout
    // keeps nseg slots per head).
    timing_before(st);
    kpart<64, NW, 1, RELU><<<dim3((p.nseg - 1) * p.BH), NW * 64, 0, st>>>(K, V, W, P, cs, p.L, p.m,
                                                                    p.seg, p.nseg, p.nseg - 1,
                                                                    p.knorm);
    e = hipGetLastError();
    timing_after(st, "kpart");
    if (e != hipSuccess) return e;
  }
  if (p.nseg > 1 || Sin || Sout) {
    timing_before(st);
    kprefix<64><<<dim3((65 * p.m / 4 + 255) / 256, p.BH), 256, 0, st>>>(
        P, cs, cP, Sin, p.m, p.nseg, RELU ? kLog2e : 1.f, Sout);
    e = hipGetLastError();
    timing_after(st, "kprefix");
    if (e != hipSuccess) return e;
    if (Sout && exported) *exported = true;
  }
  timing_before(st);
  cscan<NW, RELU><<<dim3(p.nseg, p.BH), NW * 64, 0, st>>>(Q, K, V, W, P, cP, O, p.L, p.m, p.seg, p.nseg,
                                                     p.knorm, Sin ? 1 : 0);
  e = hipGetLastError();
  timing_after(st, "cscan");
  return e;
}

// The backward's first launches: every segment's key state (the last one's
// reference is needed too), the exclusive prefix, and the scan's per-query
// (L_i, p_i).
template <int NW, bool RELU>
hipError_t launch_rowstats(const Plan& p, const uint16_t* Q, const uint16_t* K, const uint16_t* V,
                           const float* W, const uint16_t* dO, float2* lp, char* ws,
                           hipStream_t st) {
  float* P = reinterpret_cast<float*>(ws + p.off_T);
  float* cs = reinterpret_cast<float*>(ws + p.off_cseg);
  float* cP = reinterpret_cast<float*>(ws + p.off_cP);
  hipError_t e;
  if (!RELU && NW == 4) {
    // every segment's state, two segments per work-group (m = 256, softmax
    // and Gaussian features)
    e = fused_causal_key_states(p, K, V, W, P, cs, st, true);
  } else {
    timing_before(st);
    kpart<64, NW, 1, RELU><<<dim3(p.nseg * p.BH), NW * 64, 0, st>>>(K, V, W, P, cs, p.L, p.m, p.seg,
                                                                    p.nseg, p.nseg, p.knorm);
    e = hipGetLastError();
    timing_after(st, "kpart");
  }
  if (e != hipSuccess) return e;
  if (p.nseg > 1) {
    timing_before(st);
    kprefix<64><<<dim3((65 * p.m / 4 + 255) / 256, p.BH), 256, 0, st>>>(P, cs, cP, nullptr, p.m,
                                                                         p.nseg, 1.f);
    e = hipGetLastError();
    timing_after(st, "kprefix");
    if (e != hipSuccess) return e;
  }
  timing_before(st);
  cscan<NW, RELU, true><<<dim3(p.nseg, p.BH), NW * 64, 0, st>>>(
      Q, K, V, W, P, cP, nullptr, p.L, p.m, p.seg, p.nseg, p.knorm, 0, dO, lp);
  e = hipGetLastError();
  timing_after(st, "cscan_lp");
  return e;
}

}  // namespace

hipError_t mfma_causal_rowstats(const Plan& p, const void* Q, const void* K, const void* V,
                                const float* W, const void* dO, float* lp, void* ws,
                                hipStream_t stream) {
  const auto* q = static_cast<const uint16_t*>(Q);
  const auto* k = static_cast<const uint16_t*>(K);
  const auto* v = static_cast<const uint16_t*>(V);
  const auto* g = static_cast<const uint16_t*>(dO);
  auto* l2 = reinterpret_cast<float2*>(lp);
  char* w = static_cast<char*>(ws);
#define FAVOR_RCASE(NW)                                                                   \
  case NW:                                                                                \
    return p.relu ? launch_rowstats<NW, true>(p, q, k, v, W, g, l2, w, stream)            \
                  : launch_rowstats<NW, false>(p, q, k, v, W, g, l2, w, stream);
  switch (p.d == 64 ? p.m / 64 : 0) {
    FAVOR_RCASE(1) FAVOR_RCASE(2) FAVOR_RCASE(3) FAVOR_RCASE(4)
    default: break;
  }
#undef FAVOR_RCASE
  return hipErrorInvalidValue;
}

bool mfma_causal_supported(int32_t d, int32_t m, int32_t dtype) {
  return dtype == FAVOR_BF16 && d == 64 && m % 64 == 0 && m <= 256;
}

hipError_t mfma_causal_forward(const Plan& p, const void* Q, const void* K, const void* V,
                               const float* W, void* O, void* ws, hipStream_t stream,
                               const float* state_in, float* state_out, bool* exported) {
  if (exported) *exported = false;
  const auto* q = static_cast<const uint16_t*>(Q);
  const auto* k = static_cast<const uint16_t*>(K);
  const auto* v = static_cast<const uint16_t*>(V);
  auto* o = static_cast<uint16_t*>(O);
  char* w = static_cast<char*>(ws);
  if (p.d == 64) {
#define FAVOR_CCASE(NW)                                                            \
  case NW:                                                                         \
    return p.relu ? launch_causal<NW, true>(p, q, k, v, W, o, w, state_in, stream, state_out, exported) \
                  : launch_causal<NW, false>(p, q, k, v, W, o, w, state_in, stream, state_out, exported);
    switch (p.m / 64) {
      FAVOR_CCASE(1) FAVOR_CCASE(2) FAVOR_CCASE(3) FAVOR_CCASE(4)
      default: break;
    }
#undef FAVOR_CCASE
  }
  return hipErrorInvalidValue;
}

namespace {
// Waves of the key side per feature block, and feature blocks, for (d, m);
// 0 waves when the MFMA path does not take the shape.
void bidir_blocks(int32_t d, int32_t m, int* nw, int* nfb) {
  *nw = 0;
  *nfb = 1;
  if (m % 64 != 0 || m > 1024 || (d != 64 && d != 128)) return;
  const int total = m / (d == 64 ? KCfg<64>::FPW : KCfg<128>::FPW);
  if (total <= 8) {
    *nw = total;
  } else if (total % 2 == 0 && total <= 16) {
    *nw = total / 2;
    *nfb = 2;
  }
}
}  // namespace

int mfma_bidir_token_groups(int32_t d, int32_t m) {
  int nw, nfb;
  bidir_blocks(d, m, &nw, &nfb);
  return (nw > 0 && nw <= 4) ? 2 : 1;
}

int mfma_bidir_feature_blocks(int32_t d, int32_t m) {
  int nw, nfb;
  bidir_blocks(d, m, &nw, &nfb);
  return nfb;
}

bool mfma_bidir_supported(int32_t d, int32_t m, int32_t dtype) {
  int nw, nfb;
  bidir_blocks(d, m, &nw, &nfb);
  return dtype == FAVOR_BF16 && nw > 0;
}

int mfma_bidir_query_workgroups() { return FAVOR_QAPPLY_WGS; }

int mfma_bidir_stream_round() { return FAVOR_QSTREAM_NW * 16 * FAVOR_QSTREAM_NTQ; }

bool mfma_bidir_streams_queries(int32_t d, int32_t m) {
  return (d == 64 ? qapply_lds_bytes<64>(m) : qapply_lds_bytes<128>(m)) > 160 * 1024;
}

namespace {
// kpart alone, with the bidirectional plan's configuration.
template <int D, int NW, int NFB, bool RELU>
hipError_t launch_kpart(const Plan& p, const uint16_t* K, const uint16_t* V, const float* W,
                        char* ws, hipStream_t st) {
  float* P = reinterpret_cast<float*>(ws + p.off_T);
  float* cs = reinterpret_cast<float*>(ws + p.off_cseg);
  constexpr int TG = (NW <= 4) ? 2 : 1;
  timing_before(st);
  kpart<D, NW, TG, RELU><<<dim3(p.nseg * p.BH * NFB), TG * NW * 64, 0, st>>>(
      K, V, W, P, cs, p.L, p.m, p.seg, p.nseg, p.nseg, p.knorm);
  const hipError_t e = hipGetLastError();
  timing_after(st, "kpart");
  return e;
}
}  // namespace

hipError_t mfma_bidir_key_partials(const Plan& p, const void* K, const void* V, const float* W,
                                   void* ws, hipStream_t stream) {
  const auto* k = static_cast<const uint16_t*>(K);
  const auto* v = static_cast<const uint16_t*>(V);
  char* w = static_cast<char*>(ws);
  int nw, nfb;
  bidir_blocks(p.d, p.m, &nw, &nfb);
#define FAVOR_CASE(D, NW, NFB)                                                       \
  if (p.d == D && nw == NW && nfb == NFB)                                            \
    return p.relu ? launch_kpart<D, NW, NFB, true>(p, k, v, W, w, stream)            \
                  : launch_kpart<D, NW, NFB, false>(p, k, v, W, w, stream);
  FAVOR_CASE(64, 1, 1) FAVOR_CASE(64, 2, 1) FAVOR_CASE(64, 3, 1) FAVOR_CASE(64, 4, 1)
#undef FAVOR_CASE
  return hipErrorInvalidValue;
}

hipError_t mfma_bidir_forward(const Plan& p, const void* Q, const void* K, const void* V,
                              const float* W, void* O, void* ws, hipStream_t stream) {
  const auto* q = static_cast<const uint16_t*>(Q);
  const auto* k = static_cast<const uint16_t*>(K);
  const auto* v = static_cast<const uint16_t*>(V);
  auto* o = static_cast<uint16_t*>(O);
  char* w = static_cast<char*>(ws);
  int nw, nfb;
  bidir_blocks(p.d, p.m, &nw, &nfb);
#define FAVOR_CASE(D, NW, NFB)                                                       \
  if (p.d == D && nw == NW && nfb == NFB)                                            \
    return p.relu ? launch_d<D, NW, NFB, true>(p, q, k, v, W, o, w, stream)          \
                  : launch_d<D, NW, NFB, false>(p, q, k, v, W, o, w, stream);
  FAVOR_CASE(64, 1, 1) FAVOR_CASE(64, 2, 1) FAVOR_CASE(64, 3, 1) FAVOR_CASE(64, 4, 1)
  FAVOR_CASE(64, 5, 1) FAVOR_CASE(64, 6, 1) FAVOR_CASE(64, 7, 1) FAVOR_CASE(64, 8, 1)
  FAVOR_CASE(64, 5, 2) FAVOR_CASE(64, 6, 2) FAVOR_CASE(64, 7, 2) FAVOR_CASE(64, 8, 2)
  FAVOR_CASE(128, 2, 1) FAVOR_CASE(128, 4, 1) FAVOR_CASE(128, 6, 1) FAVOR_CASE(128, 8, 1)
  FAVOR_CASE(128, 5, 2) FAVOR_CASE(128, 6, 2) FAVOR_CASE(128, 7, 2) FAVOR_CASE(128, 8, 2)
#undef FAVOR_CASE
  return hipErrorInvalidValue;
}

}  // namespace favor
