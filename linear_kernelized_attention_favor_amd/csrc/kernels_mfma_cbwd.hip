// Causal FAVOR+ backward on the matrix cores (bf16 inputs, d = 64, m a
// multiple of 64 up to 256): the gradients of <dO, O> with respect to Q, K
// and V for the masked (prefix-sum) form of the "FAVOR+" method page, W held
// fixed.  The chain rule is the bidirectional one with every sum over keys
// restricted to j <= i and every sum over queries to i >= j:
//
//   T_ir = sum_{j <= i} K~_jr (v_j . dO_i - p_i),   p_i = dO_i . O_i
//   dq_i = sum_r P_ir w_r - 2 knorm (sum_r P_ir) q_i,  P_ir = Q'_ir T_ir
//   G_r(j) = sum_{i >= j} Q'_ir [dO_i | -p_i]
//   dk_j = sum_r R_jr w_r - 2 knorm (sum_r R_jr) k_j,  R_jr = K~_jr G_r(j) . [v_j | 1]
//   dv_j = sum_r K~_jr G_r(j)[0:d]
//
// with log2-unit exponents s_ir = w'_r . q_i and e_jr = w'_r . k_j - n_j
// (W' = W log2 e, n_j = knorm log2(e) |k_j|^2), key features
// K~_jr = 2^(e_jr - c_r) in a frame of per-feature references c, and query
// factors Q'_ir = 2^(s_ir + c_r - L_i), where
// L_i = log2 sum_{j <= i} sum_r 2^(s_ir + e_jr) is the log of the
// denominator taken with no reference.  Q' holds the 1 / den of U = dO / den,
// and every product of a Q' and a K~ is 2^(s_ir + e_jr - L_i) <= 1 whatever
// the frame, so each kernel may pick its own: here each segment s works at
// c*(s) = max of the references of the segments up to s (its own included),
// fixed for the segment.  ReLU features (generalized attention):
// K~ = max(e, 0), Q' = max(s, 0) 2^(-L), gates [s > 0] and [e > 0] in P and
// R, no norm term, and the factor log2 e of W' put back into dq and dk.
//
// Launches (segments and references of the causal forward's plan):
//   kpart + kprefix   every segment's key state and reference; the prefix
//                     states (the causal forward's first launches)
//   cscan (BWD)       the forward scan, writing (L_i, p_i) per query
//   cbq               per (head, segment): 32-token chunks in order, the
//                     prefix state carried in registers as S^T tiles; dq
//   cbg               per (head, segment >= 1): the segment's query state
//                     G^T = sum_i [dO_i | -p_i]^T Q'_i
//   cbsuffix          per head: the exclusive suffix of those states over
//                     later segments, each carried down to the earlier
//                     segment's frame (factors 2^(c*(s) - c*(t)) <= 1)
//   cbk (MODE 0, 1)   per (head, segment): chunks in reverse order, the
//                     suffix G carried in registers; dk (G^T tiles) and dv
//                     (G tiles)
// Within a chunk the masked terms pair the chunk's keys and queries
// directly (32 x 32 products); every reduction over features is split across
// the waves (wave w owns features [16 FT w, 16 FT (w + 1)), FT = 2 or 4
// feature tiles of 16) and summed through LDS in wave order, so results are
// bitwise reproducible.
//
// Numerics as the bidirectional backward: projections in fp16 (Q, K exact,
// W' rounded); features rounded to bf16 as operands; the carried states and
// the masked (v . dO - p) factors, whose sums cancel, as bf16 hi + lo pairs;
// -p as a hi + lo pair in two columns of [dO | -p] (the states' ones column
// is doubled to match); dO exact; all sums fp32.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "favor.h"
#include "favor_internal.h"
#include "mfma_common.h"

namespace favor {
namespace {

using namespace mfma;

constexpr int kD = 64;               // head dimension of this path
constexpr int kC = 32;               // tokens per chunk
constexpr int kRow = kD + 8;         // 16-bit values per staged token row
constexpr int kTRow = kC / 2 + 4;    // token pairs (uint32) per transposed row
constexpr int kGRows = kD + 2;       // rows of a stored query state: dO part, -p hi, -p lo
constexpr int kRedRow = kD + 4;      // floats per token of the cross-wave sums

__device__ inline uint16_t bf16_bits(float x) {
  return static_cast<uint16_t>(pack_bf16(x, 0.f) & 0xffffu);
}
__device__ inline float bf16_val(uint16_t b) { return __uint_as_float(static_cast<uint32_t>(b) << 16); }

// Eight values (two output tiles stacked along the k axis: positions 0..3
// from a, 4..7 from b) as a bf16 hi operand and the lo operand of the
// remainders.
__device__ inline void split8(const f32x4& a, const f32x4& b, bf16x8& hi, bf16x8& lo) {
  float x[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  uint32_t h[4], l[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    h[q] = pack_bf16(x[2 * q], x[2 * q + 1]);
    l[q] = pack_bf16(x[2 * q] - bf16_lo(h[q]), x[2 * q + 1] - bf16_hi(h[q]));
  }
  hi = __builtin_bit_cast(bf16x8, make_uint4(h[0], h[1], h[2], h[3]));
  lo = __builtin_bit_cast(bf16x8, make_uint4(l[0], l[1], l[2], l[3]));
}
__device__ inline bf16x8 pack8(const f32x4& a, const f32x4& b) {
  return __builtin_bit_cast(bf16x8, make_uint4(pack_bf16(a[0], a[1]), pack_bf16(a[2], a[3]),
                                               pack_bf16(b[0], b[1]), pack_bf16(b[2], b[3])));
}

// The reference frame of segment s for feature f.
__device__ inline float seg_ref(const float* __restrict__ cs, const float* __restrict__ cP, int bh,
                                int s, int nseg, int m, int f) {
  const size_t i = (static_cast<size_t>(bh) * nseg + s) * m + f;
  return s > 0 ? fmaxf(cP[i], cs[i]) : cs[i];
}

// One chunk's operands in LDS.
struct __align__(16) Stage {
  _Float16 Kh[kC][kRow];     // K rows (fp16, exact from bf16)
  _Float16 Qh[kC][kRow];     // Q rows
  uint16_t Vr[kC][kRow];     // V rows (bf16)
  uint16_t Gr[kC][kRow];     // dO rows (bf16)
  uint32_t Vt[kD][kTRow];    // V^T: column, token pairs in position order
  uint32_t Gt[kD][kTRow];    // dO^T likewise
  float nk[kC];              // -n_j (-inf past the end)
  float Lq[kC];              // L_i (+inf past the end)
  float pq[kC];              // p_i (0 past the end)
  uint16_t pn[2][kC];        // -p_i as bf16 hi, lo, in position order
};

// Loads chunk [jt, jt + 32) (tokens from j1 on read as zero) into st.
// Every thread of the work-group (NTH) takes part.
template <int NTH>
__device__ inline void stage_chunk(Stage& st, const uint16_t* __restrict__ Q,
                                   const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
                                   const uint16_t* __restrict__ dO, const float2* __restrict__ lp,
                                   size_t base, size_t lbase, int jt, int j1, float knorm) {
  const int tid = threadIdx.x;
  // rows: 32 tokens x 8 chunks of 8 values; the eight threads of a row are
  // consecutive lanes (the key norm sums over them)
  for (int u = tid; u < kC * 8; u += NTH) {
    const int t = u / 8, ch = u % 8;
    const bool ok = jt + t < j1;
    const size_t off = base + static_cast<size_t>(jt + t) * kD + 8 * ch;
    uint4 kv = make_uint4(0, 0, 0, 0), qv = kv, vv = kv, gv = kv;
    if (ok) {
      kv = *reinterpret_cast<const uint4*>(K + off);
      qv = *reinterpret_cast<const uint4*>(Q + off);
      vv = *reinterpret_cast<const uint4*>(V + off);
      gv = *reinterpret_cast<const uint4*>(dO + off);
    }
    float ss = 0.f;
    const uint32_t w4[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      ss = fmaf(bf16_lo(w4[q]), bf16_lo(w4[q]), ss);
      ss = fmaf(bf16_hi(w4[q]), bf16_hi(w4[q]), ss);
    }
    ss = group_sum<8>(ss);
    *reinterpret_cast<uint4*>(&st.Kh[t][8 * ch]) =
        make_uint4(bf16x2_to_f16x2(kv.x), bf16x2_to_f16x2(kv.y), bf16x2_to_f16x2(kv.z),
                   bf16x2_to_f16x2(kv.w));
    *reinterpret_cast<uint4*>(&st.Qh[t][8 * ch]) =
        make_uint4(bf16x2_to_f16x2(qv.x), bf16x2_to_f16x2(qv.y), bf16x2_to_f16x2(qv.z),
                   bf16x2_to_f16x2(qv.w));
    *reinterpret_cast<uint4*>(&st.Vr[t][8 * ch]) = vv;
    *reinterpret_cast<uint4*>(&st.Gr[t][8 * ch]) = gv;
    if (ch == 0) st.nk[t] = ok ? -knorm * kLog2e * ss : -INFINITY;
  }
  // transposes: (token pair, 4 columns) units
  for (int u = tid; u < (kC / 2) * (kD / 4); u += NTH) {
    const int t = 2 * (u % (kC / 2)), col = 4 * (u / (kC / 2));
    const int w = perm_inv(t) >> 1;
    const size_t off = base + static_cast<size_t>(jt + t) * kD + col;
    uint2 va = make_uint2(0, 0), vb = va, ga = va, gb = va;
    if (jt + t < j1) {
      va = *reinterpret_cast<const uint2*>(V + off);
      ga = *reinterpret_cast<const uint2*>(dO + off);
    }
    if (jt + t + 1 < j1) {
      vb = *reinterpret_cast<const uint2*>(V + off + kD);
      gb = *reinterpret_cast<const uint2*>(dO + off + kD);
    }
    st.Vt[col + 0][w] = __builtin_amdgcn_perm(vb.x, va.x, 0x05040100u);
    st.Vt[col + 1][w] = __builtin_amdgcn_perm(vb.x, va.x, 0x07060302u);
    st.Vt[col + 2][w] = __builtin_amdgcn_perm(vb.y, va.y, 0x05040100u);
    st.Vt[col + 3][w] = __builtin_amdgcn_perm(vb.y, va.y, 0x07060302u);
    st.Gt[col + 0][w] = __builtin_amdgcn_perm(gb.x, ga.x, 0x05040100u);
    st.Gt[col + 1][w] = __builtin_amdgcn_perm(gb.x, ga.x, 0x07060302u);
    st.Gt[col + 2][w] = __builtin_amdgcn_perm(gb.y, ga.y, 0x05040100u);
    st.Gt[col + 3][w] = __builtin_amdgcn_perm(gb.y, ga.y, 0x07060302u);
  }
  if (tid < kC) {
    float2 v = make_float2(INFINITY, 0.f);
    if (jt + tid < j1) v = lp[lbase + jt + tid];
    st.Lq[tid] = v.x;
    st.pq[tid] = v.y;
    const uint16_t hi = bf16_bits(-v.y);
    st.pn[0][perm_inv(tid)] = hi;
    st.pn[1][perm_inv(tid)] = bf16_bits(-v.y - bf16_val(hi));
  }
}

// The same chunk load split in two for a work-group of 256 threads (one row
// unit and one transpose unit per thread): the global loads into registers,
// issued a chunk ahead, and the LDS stores.
struct ChunkRegs {
  uint4 k, q, v, g;        // row unit (token tid / 8, values 8 (tid % 8) ..)
  uint2 va, vb, ga, gb;    // transpose unit: tokens t, t + 1, columns col ..
  float2 l;                // (L, p) of token tid (tid < 32)
};
__device__ inline void gload_chunk(ChunkRegs& r, const uint16_t* __restrict__ Q,
                                   const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
                                   const uint16_t* __restrict__ dO, const float2* __restrict__ lp,
                                   size_t base, size_t lbase, int jt, int j1) {
  const int tid = threadIdx.x;
  {
    const int t = tid / 8, ch = tid % 8;
    const size_t off = base + static_cast<size_t>(jt + t) * kD + 8 * ch;
    r.k = r.q = r.v = r.g = make_uint4(0, 0, 0, 0);
    if (jt + t < j1) {
      r.k = *reinterpret_cast<const uint4*>(K + off);
      r.q = *reinterpret_cast<const uint4*>(Q + off);
      r.v = *reinterpret_cast<const uint4*>(V + off);
      r.g = *reinterpret_cast<const uint4*>(dO + off);
    }
  }
  {
    const int t = 2 * (tid % (kC / 2)), col = 4 * (tid / (kC / 2));
    const size_t off = base + static_cast<size_t>(jt + t) * kD + col;
    r.va = r.vb = r.ga = r.gb = make_uint2(0, 0);
    if (jt + t < j1) {
      r.va = *reinterpret_cast<const uint2*>(V + off);
      r.ga = *reinterpret_cast<const uint2*>(dO + off);
    }
    if (jt + t + 1 < j1) {
      r.vb = *reinterpret_cast<const uint2*>(V + off + kD);
      r.gb = *reinterpret_cast<const uint2*>(dO + off + kD);
    }
  }
  r.l = make_float2(INFINITY, 0.f);
  if (tid < kC && jt + tid < j1) r.l = lp[lbase + jt + tid];
}
__device__ inline void lstore_chunk(Stage& st, const ChunkRegs& r, int jt, int j1, float knorm) {
  const int tid = threadIdx.x;
  {
    const int t = tid / 8, ch = tid % 8;
    float ss = 0.f;
    const uint32_t w4[4] = {r.k.x, r.k.y, r.k.z, r.k.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      ss = fmaf(bf16_lo(w4[q]), bf16_lo(w4[q]), ss);
      ss = fmaf(bf16_hi(w4[q]), bf16_hi(w4[q]), ss);
    }
    ss = group_sum<8>(ss);
    *reinterpret_cast<uint4*>(&st.Kh[t][8 * ch]) =
        make_uint4(bf16x2_to_f16x2(r.k.x), bf16x2_to_f16x2(r.k.y), bf16x2_to_f16x2(r.k.z),
                   bf16x2_to_f16x2(r.k.w));
    *reinterpret_cast<uint4*>(&st.Qh[t][8 * ch]) =
        make_uint4(bf16x2_to_f16x2(r.q.x), bf16x2_to_f16x2(r.q.y), bf16x2_to_f16x2(r.q.z),
                   bf16x2_to_f16x2(r.q.w));
    *reinterpret_cast<uint4*>(&st.Vr[t][8 * ch]) = r.v;
    *reinterpret_cast<uint4*>(&st.Gr[t][8 * ch]) = r.g;
    if (ch == 0) st.nk[t] = (jt + t < j1) ? -knorm * kLog2e * ss : -INFINITY;
  }
  {
    const int t = 2 * (tid % (kC / 2)), col = 4 * (tid / (kC / 2));
    const int w = perm_inv(t) >> 1;
    st.Vt[col + 0][w] = __builtin_amdgcn_perm(r.vb.x, r.va.x, 0x05040100u);
    st.Vt[col + 1][w] = __builtin_amdgcn_perm(r.vb.x, r.va.x, 0x07060302u);
    st.Vt[col + 2][w] = __builtin_amdgcn_perm(r.vb.y, r.va.y, 0x05040100u);
    st.Vt[col + 3][w] = __builtin_amdgcn_perm(r.vb.y, r.va.y, 0x07060302u);
    st.Gt[col + 0][w] = __builtin_amdgcn_perm(r.gb.x, r.ga.x, 0x05040100u);
    st.Gt[col + 1][w] = __builtin_amdgcn_perm(r.gb.x, r.ga.x, 0x07060302u);
    st.Gt[col + 2][w] = __builtin_amdgcn_perm(r.gb.y, r.ga.y, 0x05040100u);
    st.Gt[col + 3][w] = __builtin_amdgcn_perm(r.gb.y, r.ga.y, 0x07060302u);
  }
  if (tid < kC) {
    st.Lq[tid] = r.l.x;
    st.pq[tid] = r.l.y;
    const uint16_t hi = bf16_bits(-r.l.y);
    st.pn[0][perm_inv(tid)] = hi;
    st.pn[1][perm_inv(tid)] = bf16_bits(-r.l.y - bf16_val(hi));
  }
}

// Chunk loads of a sweep: with at least 256 threads, each chunk's global
// loads are issued one chunk ahead by the first 256 (next()) and stored to
// LDS at the start of its turn (put()); otherwise loaded and stored at once.
template <int NTH>
struct ChunkLoader {
  ChunkRegs r;
  const uint16_t *Q, *K, *V, *dO;
  const float2* lp;
  size_t base, lbase;
  int j1;
  float knorm;
  __device__ void next(int jt) {
    if constexpr (NTH >= 256)
      if (threadIdx.x < 256) gload_chunk(r, Q, K, V, dO, lp, base, lbase, jt, j1);
  }
  __device__ void put(Stage& st, int jt) {
    if constexpr (NTH >= 256) {
      if (threadIdx.x < 256) lstore_chunk(st, r, jt, j1, knorm);
    } else {
      stage_chunk<NTH>(st, Q, K, V, dO, lp, base, lbase, jt, j1, knorm);
    }
  }
};

// W' (fp16) of the wave's features as the projections' operand:
// W'[f0 + 16 nt + l16][32 ks + 8 g + u].
template <int FT = 4>
__device__ inline void load_wreg(const float* __restrict__ W, int f0, int l16, int g,
                                 f16x8 (&wreg)[FT][2]) {
#pragma unroll
  for (int nt = 0; nt < FT; ++nt) {
    const float* wr = W + static_cast<size_t>(f0 + 16 * nt + l16) * kD + 8 * g;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
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
}

// W^T (true W, bf16) [64][M + 8] in LDS, features in the contraction order
// feat_pos: position 32p + 8g + j holds feature 32p + 4g + j (j < 4) or
// 32p + 16 + 4g + j - 4.
__device__ inline int feat_pos(int f) {
  const int p = f & ~31, i = f & 31;
  return p + 8 * ((i & 15) >> 2) + (i & 3) + (i >= 16 ? 4 : 0);
}
template <int NTH>
__device__ inline void load_wt(const float* __restrict__ W, int m, uint16_t* wt) {
  for (int i = threadIdx.x; i < m * kD; i += NTH) {
    const int r = i / kD, a = i - r * kD;
    wt[a * (m + 8) + feat_pos(r)] = bf16_bits(W[i]);
  }
}

// Projections of the chunk's rows X (fp16 in LDS) on the wave's features.
// E orientation (lane = feature 16 nt + l16, rows = tokens 16 mt + 4 g + v):
template <int FT = 4>
__device__ inline void proj_e(const _Float16 (*X)[kRow], const f16x8 (&wreg)[FT][2], int l16,
                              int g, const f32x4 (&init)[2], f32x4 (&E)[2][FT]) {
  f16x8 xa[2][2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) xa[mt][ks] = *reinterpret_cast<const f16x8*>(&X[16 * mt + l16][32 * ks + 8 * g]);
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nt = 0; nt < FT; ++nt) E[mt][nt] = mma_f16(xa[mt][ks], wreg[nt][ks], ks == 0 ? init[mt] : E[mt][nt]);
}
// E^T orientation (lane = token 16 nt + l16, rows = features 16 mt + 4 g + v):
template <int FT = 4>
__device__ inline void proj_et(const _Float16 (*X)[kRow], const f16x8 (&wreg)[FT][2], int l16,
                               int g, const f32x4 (&init)[FT], f32x4 (&E)[FT][2]) {
  f16x8 xb[2][2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) xb[nt][ks] = *reinterpret_cast<const f16x8*>(&X[16 * nt + l16][32 * ks + 8 * g]);
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int mt = 0; mt < FT; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) E[mt][nt] = mma_f16(wreg[mt][ks], xb[nt][ks], ks == 0 ? init[mt] : E[mt][nt]);
}

// The cross-wave sum of per-wave partials D[at][n] (lane = token 16 n + l16,
// rows = columns 16 at + 4 g + v) and of a per-token scalar, then
// out_t = scale (sum D) - 2 knorm (sum x) X_t (X_t the token's row in fp16),
// stored as bf16 for tokens below j1.
template <int NW, bool RELU>
__device__ inline void reduce_store(float (*red)[kC][kRedRow], const f32x4 (&D)[4][2],
                                    const float (&xs)[2], const _Float16 (*X)[kRow], int wave,
                                    int l16, int g, float knorm, uint16_t* __restrict__ out,
                                    size_t base, int jt, int j1, bool norm_term) {
#pragma unroll
  for (int at = 0; at < 4; ++at)
#pragma unroll
    for (int n = 0; n < 2; ++n)
      *reinterpret_cast<f32x4*>(&red[wave][16 * n + l16][16 * at + 4 * g]) = D[at][n];
  if (g == 0) {
    red[wave][l16][kD] = xs[0];
    red[wave][16 + l16][kD] = xs[1];
  }
  lds_barrier();
  for (int o = threadIdx.x; o < kC * (kD / 8); o += NW * 64) {
    const int t = o / (kD / 8), c0 = 8 * (o % (kD / 8));
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float ps = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(&red[w][t][c0]);
      const f32x4 b = *reinterpret_cast<const f32x4*>(&red[w][t][c0 + 4]);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        acc[c] += a[c];
        acc[4 + c] += b[c];
      }
      ps += red[w][t][kD];
    }
    if (jt + t < j1) {
      float o8[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        if (RELU) o8[c] = norm_term ? acc[c] * kLog2e : acc[c];
        else o8[c] = norm_term ? fmaf(-2.f * knorm * ps, static_cast<float>(X[t][c0 + c]), acc[c]) : acc[c];
      }
      *reinterpret_cast<uint4*>(out + base + static_cast<size_t>(jt + t) * kD + c0) =
          make_uint4(pack_bf16(o8[0], o8[1]), pack_bf16(o8[2], o8[3]), pack_bf16(o8[4], o8[5]),
                     pack_bf16(o8[6], o8[7]));
    }
  }
}

// The A operand [dO | -p_hi | -p_lo]^T (lane = column 16 ct + l16, k = the
// chunk's 8 queries at positions 8 g ..) from the staged transposes.
__device__ inline bf16x8 dop_t(const Stage& st, int ct, int l16, int g) {
  if (ct < 4) return *reinterpret_cast<const bf16x8*>(&st.Gt[16 * ct + l16][4 * g]);
  if (l16 < 2) return *reinterpret_cast<const bf16x8*>(&st.pn[l16][8 * g]);
  return __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
}

// ---------------------------------------------------------------------------
// cbq: grid (ceil(nseg / spw), BH), NW = m / (16 FT) waves.  dq of the
// queries of spw consecutive segments, in order.  State per wave: stT[ct][ft],
// S^T tiles (lane = feature f0 + 16 ft + l16, rows = columns 16 ct + 4 g + v
// of [S~ | z~ | z~]), in the frame c*(s) of the segment being swept (moved to
// the next segment's frame at its start, factors 2^(c*(s) - c*(s+1)) <= 1).
// ---------------------------------------------------------------------------
template <int NW, bool RELU, int FT>
__global__ __launch_bounds__(NW * 64, 1) void cbq(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ W, const float* __restrict__ P,
    const float* __restrict__ cs, const float* __restrict__ cP, const float2* __restrict__ lp,
    uint16_t* __restrict__ dQ, int L, int SEG, int nseg, int spw, float knorm) {
  constexpr int NTH = NW * 64;
  constexpr int M = NW * 16 * FT;   // FT feature tiles of 16 per wave
  const int sA = blockIdx.x * spw, sB = min(nseg, sA + spw), bh = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int f0 = 16 * FT * wave;
  __shared__ Stage st;
  __shared__ __align__(16) uint16_t wt[kD * (M + 8)];
  __shared__ __align__(16) float red[NW][kC][kRedRow];
  __shared__ __align__(16) float cst[M];

  for (int r = tid; r < M; r += NTH) cst[r] = RELU ? 0.f : seg_ref(cs, cP, bh, sA, nseg, M, r);
  load_wt<NTH>(W, M, wt);
  f16x8 wreg[FT][2];
  load_wreg<FT>(W, f0, l16, g, wreg);

  // Carry-in: the prefix state (at cP) moved to c*(s); column 65 repeats z~.
  f32x4 stT[5][FT];
#pragma unroll
  for (int ct = 0; ct < 5; ++ct)
#pragma unroll
    for (int ft = 0; ft < FT; ++ft) stT[ct][ft] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (sA > 0) {
    const size_t pb = (static_cast<size_t>(bh) * nseg + sA) * (kD + 1);
#pragma unroll
    for (int ft = 0; ft < FT; ++ft) {
      const int f = f0 + 16 * ft + l16;
      const size_t ci = (static_cast<size_t>(bh) * nseg + sA) * M + f;
      const float sc = RELU ? 1.f : fast_exp2(cP[ci] - fmaxf(cP[ci], cs[ci]));
#pragma unroll
      for (int ct = 0; ct < 5; ++ct)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          int col = 16 * ct + 4 * g + v;
          if (col == kD + 1) col = kD;
          if (col <= kD) stT[ct][ft][v] = P[(pb + col) * M + f] * sc;
        }
    }
  }
  const f32x4 zero4 = f32x4{0.f, 0.f, 0.f, 0.f};
  // rows 64 and 65 of [V | 1 | 1]^T (every key position)
  const bf16x8 ones = (l16 < 2) ? __builtin_bit_cast(bf16x8, make_uint4(0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u))
                                : __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));

  const size_t base = static_cast<size_t>(bh) * L * kD;
  const size_t lbase = static_cast<size_t>(bh) * L;
  __syncthreads();

  ChunkLoader<NTH> ld{ChunkRegs{}, Q, K, V, dO, lp, base, lbase, 0, RELU ? 0.f : knorm};
  for (int s = sA; s < sB; ++s) {
    if (!RELU && s > sA) {
      // the carried state into segment s's frame
      float fac[FT];
#pragma unroll
      for (int ft = 0; ft < FT; ++ft) {
        const int f = f0 + 16 * ft + l16;
        fac[ft] = fast_exp2(cst[f] - seg_ref(cs, cP, bh, s, nseg, M, f));
      }
      lds_barrier();   // every wave has read the previous frame
      for (int r = tid; r < M; r += NTH) cst[r] = seg_ref(cs, cP, bh, s, nseg, M, r);
#pragma unroll
      for (int ct = 0; ct < 5; ++ct)
#pragma unroll
        for (int ft = 0; ft < FT; ++ft) stT[ct][ft] *= fac[ft];
      lds_barrier();
    }
    const int j0 = s * SEG, j1 = min(L, j0 + SEG);
    ld.j1 = j1;
    ld.next(j0);
    for (int jt = j0; jt < j1; jt += kC) {
      ld.put(st, jt);
      lds_barrier();
      if (jt + kC < j1) ld.next(jt + kC);

      // (1) key features K~ (E orientation) -> kb[nt]: lane = feature, the
      // chunk's 8 keys at positions 8 g ..
      bf16x8 kb[FT];
      {
        f32x4 SK[2][FT];
        const f32x4 init[2] = {*reinterpret_cast<const f32x4*>(&st.nk[4 * g]),
                               *reinterpret_cast<const f32x4*>(&st.nk[16 + 4 * g])};
        proj_e<FT>(st.Kh, wreg, l16, g, init, SK);
#pragma unroll
        for (int nt = 0; nt < FT; ++nt) {
          const float c = cst[f0 + 16 * nt + l16];
#pragma unroll
          for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int v = 0; v < 4; ++v) SK[mt][nt][v] = feature<RELU>(SK[mt][nt][v] - c);
          kb[nt] = pack8(SK[0][nt], SK[1][nt]);
        }
      }
      // (2) query factors Q' (E^T orientation: lane = query 16 nq + l16, rows
      // = features 16 mt + 4 g + v).
      f32x4 SQ[FT][2];
      float rl[2];
      {
        f32x4 init[FT];
#pragma unroll
        for (int mt = 0; mt < FT; ++mt) init[mt] = *reinterpret_cast<const f32x4*>(&cst[f0 + 16 * mt + 4 * g]);
        proj_et<FT>(st.Qh, wreg, l16, g, init, SQ);
#pragma unroll
        for (int nq = 0; nq < 2; ++nq) {
          const float Lq = st.Lq[16 * nq + l16];
          rl[nq] = fast_exp2(-Lq);
#pragma unroll
          for (int mt = 0; mt < FT; ++mt)
#pragma unroll
            for (int v = 0; v < 4; ++v)
              SQ[mt][nq][v] = RELU ? SQ[mt][nq][v] : fast_exp2(SQ[mt][nq][v] - Lq);
        }
      }
      // (3) T^T = S [dO | -p]^T from the carried state (hi + lo), then (4) the
      // masked in-chunk term K~^T a, a_ji = v_j . dO_i - p_i for j <= i.
      f32x4 T[FT][2];
#pragma unroll
      for (int ft = 0; ft < FT; ++ft)
#pragma unroll
        for (int nq = 0; nq < 2; ++nq) T[ft][nq] = zero4;
#pragma unroll
      for (int p = 0; p < 3; ++p) {
        bf16x8 db[2];
#pragma unroll
        for (int nq = 0; nq < 2; ++nq) {
          const int q = 16 * nq + l16;
          if (p < 2) {
            const uint2 a = *reinterpret_cast<const uint2*>(&st.Gr[q][32 * p + 4 * g]);
            const uint2 b = *reinterpret_cast<const uint2*>(&st.Gr[q][32 * p + 16 + 4 * g]);
            db[nq] = __builtin_bit_cast(bf16x8, make_uint4(a.x, a.y, b.x, b.y));
          } else {
            const float pv = -st.pq[q];
            const uint16_t hi = bf16_bits(pv);
            const uint16_t lo = bf16_bits(pv - bf16_val(hi));
            db[nq] = __builtin_bit_cast(
                bf16x8, make_uint4(g == 0 ? (static_cast<uint32_t>(lo) << 16) | hi : 0u, 0u, 0u, 0u));
          }
        }
#pragma unroll
        for (int ft = 0; ft < FT; ++ft) {
          bf16x8 ah, al;
          split8(stT[2 * p][ft], p < 2 ? stT[2 * p + 1][ft] : zero4, ah, al);
#pragma unroll
          for (int nq = 0; nq < 2; ++nq) {
            T[ft][nq] = mma_bf16(ah, db[nq], T[ft][nq]);
            T[ft][nq] = mma_bf16(al, db[nq], T[ft][nq]);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      {
        f32x4 A[2][2];   // [mk][nq]: lane = query 16 nq + l16, rows = keys 16 mk + 4 g + v
#pragma unroll
        for (int mk = 0; mk < 2; ++mk)
#pragma unroll
          for (int nq = 0; nq < 2; ++nq) A[mk][nq] = zero4;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          bf16x8 va[2], ga[2];
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            va[i] = *reinterpret_cast<const bf16x8*>(&st.Vr[16 * i + l16][32 * ks + 8 * g]);
            ga[i] = *reinterpret_cast<const bf16x8*>(&st.Gr[16 * i + l16][32 * ks + 8 * g]);
          }
#pragma unroll
          for (int mk = 0; mk < 2; ++mk)
#pragma unroll
            for (int nq = 0; nq < 2; ++nq) A[mk][nq] = mma_bf16(va[mk], ga[nq], A[mk][nq]);
        }
#pragma unroll
        for (int nq = 0; nq < 2; ++nq) {
          const int q = 16 * nq + l16;
          const float pv = st.pq[q];
#pragma unroll
          for (int mk = 0; mk < 2; ++mk)
#pragma unroll
            for (int v = 0; v < 4; ++v) A[mk][nq][v] = (16 * mk + 4 * g + v <= q) ? A[mk][nq][v] - pv : 0.f;
          bf16x8 ah, al;
          split8(A[0][nq], A[1][nq], ah, al);
#pragma unroll
          for (int ft = 0; ft < FT; ++ft) {
            T[ft][nq] = mma_bf16(kb[ft], ah, T[ft][nq]);
            T[ft][nq] = mma_bf16(kb[ft], al, T[ft][nq]);
          }
        }
      }
      // (5) P = Q' T (ReLU: [s > 0] T 2^-L), in place of Q'; per-query sums.
      float ps[2] = {0.f, 0.f};
#pragma unroll
      for (int ft = 0; ft < FT; ++ft)
#pragma unroll
        for (int nq = 0; nq < 2; ++nq)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const float x = RELU ? (SQ[ft][nq][v] > 0.f ? T[ft][nq][v] * rl[nq] : 0.f)
                                 : SQ[ft][nq][v] * T[ft][nq][v];
            SQ[ft][nq][v] = x;
            ps[nq] += x;
          }
#pragma unroll
      for (int nq = 0; nq < 2; ++nq) {
        ps[nq] += __shfl_xor(ps[nq], 16);
        ps[nq] += __shfl_xor(ps[nq], 32);
      }
      // (6) dq^T partial = W^T P^T over the wave's features.
      f32x4 Dq[4][2];
#pragma unroll
      for (int at = 0; at < 4; ++at) {
        Dq[at][0] = zero4;
        Dq[at][1] = zero4;
#pragma unroll
        for (int kf = 0; kf < FT / 2; ++kf) {
          const bf16x8 wa = *reinterpret_cast<const bf16x8*>(&wt[(16 * at + l16) * (M + 8) + f0 + 32 * kf + 8 * g]);
#pragma unroll
          for (int nq = 0; nq < 2; ++nq) Dq[at][nq] = mma_bf16(wa, pack8(SQ[2 * kf][nq], SQ[2 * kf + 1][nq]), Dq[at][nq]);
        }
      }
      // (8) state update with the chunk's keys: S^T += [V | 1 | 1]^T K~.
#pragma unroll
      for (int ct = 0; ct < 5; ++ct) {
        const bf16x8 va = ct < 4 ? *reinterpret_cast<const bf16x8*>(&st.Vt[16 * ct + l16][4 * g]) : ones;
#pragma unroll
        for (int ft = 0; ft < FT; ++ft) stT[ct][ft] = mma_bf16(va, kb[ft], stT[ct][ft]);
      }
      // (7) sum over the waves, norm term, store.
      reduce_store<NW, RELU>(red, Dq, ps, st.Qh, wave, l16, g, knorm, dQ, base, jt, j1, true);
      lds_barrier();   // (LDS only: the next chunk's loads stay in flight)
    }
  }
}

// ---------------------------------------------------------------------------
// cbg: grid (nseg - 1, BH), segments 1.. : the segment's query state
// G^T = sum_i [dO_i | -p_hi,i | -p_lo,i]^T Q'_i in the frame c*(s), written
// as Gs[bh][s][66][m] fp32 (row = column of [dO | -p_hi | -p_lo]).
// ---------------------------------------------------------------------------
template <bool RELU, int FT = 4>
__device__ inline void query_factors_e(const Stage& st, const f16x8 (&wreg)[FT][2], const float* cst,
                                       int f0, int l16, int g, bf16x8 (&qb)[FT]) {
  f32x4 E[2][FT];
  const f32x4 init[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
  proj_e<FT>(st.Qh, wreg, l16, g, init, E);
  const f32x4 L0 = *reinterpret_cast<const f32x4*>(&st.Lq[4 * g]);
  const f32x4 L1 = *reinterpret_cast<const f32x4*>(&st.Lq[16 + 4 * g]);
#pragma unroll
  for (int nt = 0; nt < FT; ++nt) {
    const float c = cst[f0 + 16 * nt + l16];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      if (RELU) {
        E[0][nt][v] = fmaxf(E[0][nt][v], 0.f) * fast_exp2(-L0[v]);
        E[1][nt][v] = fmaxf(E[1][nt][v], 0.f) * fast_exp2(-L1[v]);
      } else {
        E[0][nt][v] = fast_exp2(E[0][nt][v] + c - L0[v]);
        E[1][nt][v] = fast_exp2(E[1][nt][v] + c - L1[v]);
      }
    }
    qb[nt] = pack8(E[0][nt], E[1][nt]);
  }
}

template <int NW, bool RELU, int FT>
__global__ __launch_bounds__(NW * 64, 2) void cbg(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ W, const float* __restrict__ cs,
    const float* __restrict__ cP, const float2* __restrict__ lp, float* __restrict__ Gs, int L,
    int SEG, int nseg) {
  constexpr int NTH = NW * 64;
  constexpr int M = NW * 16 * FT;
  const int s = blockIdx.x + 1, bh = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int f0 = 16 * FT * wave;
  __shared__ Stage st;
  __shared__ __align__(16) float cst[M];
  for (int r = tid; r < M; r += NTH) cst[r] = RELU ? 0.f : seg_ref(cs, cP, bh, s, nseg, M, r);
  f16x8 wreg[FT][2];
  load_wreg<FT>(W, f0, l16, g, wreg);
  f32x4 gT[5][FT];
#pragma unroll
  for (int ct = 0; ct < 5; ++ct)
#pragma unroll
    for (int ft = 0; ft < FT; ++ft) gT[ct][ft] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int j0 = s * SEG, j1 = min(L, j0 + SEG);
  const size_t base = static_cast<size_t>(bh) * L * kD;
  const size_t lbase = static_cast<size_t>(bh) * L;
  __syncthreads();
  ChunkLoader<NTH> ld{ChunkRegs{}, Q, K, V, dO, lp, base, lbase, j1, 0.f};
  ld.next(j0);
  for (int jt = j0; jt < j1; jt += kC) {
    ld.put(st, jt);
    lds_barrier();
    if (jt + kC < j1) ld.next(jt + kC);
    bf16x8 qb[FT];
    query_factors_e<RELU, FT>(st, wreg, cst, f0, l16, g, qb);
#pragma unroll
    for (int ct = 0; ct < 5; ++ct) {
      const bf16x8 a = dop_t(st, ct, l16, g);
#pragma unroll
      for (int ft = 0; ft < FT; ++ft) gT[ct][ft] = mma_bf16(a, qb[ft], gT[ct][ft]);
    }
    lds_barrier();
  }
  float* gs = Gs + (static_cast<size_t>(bh) * nseg + s) * kGRows * M;
#pragma unroll
  for (int ct = 0; ct < 5; ++ct)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int col = 16 * ct + 4 * g + v;
      if (col < kGRows) {
#pragma unroll
        for (int ft = 0; ft < FT; ++ft) gs[static_cast<size_t>(col) * M + f0 + 16 * ft + l16] = gT[ct][ft][v];
      }
    }
}

// ---------------------------------------------------------------------------
// cbsuffix: grid (ceil(66 m / 256), BH).  In place: Gs[bh][s] becomes the
// sum of the states of the segments after s, in the frame c*(s).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void cbsuffix(float* __restrict__ Gs, const float* __restrict__ cs,
                                                const float* __restrict__ cP, int m, int nseg,
                                                int relu) {
  const int bh = blockIdx.y;
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= kGRows * m) return;
  const int f = e % m;
  float run = 0.f;
  for (int s = nseg - 1; s >= 0; --s) {
    float* gp = Gs + (static_cast<size_t>(bh) * nseg + s) * kGRows * m + e;
    const float gsv = s > 0 ? *gp : 0.f;
    *gp = run;
    if (s > 0) {
      const float sc = relu ? 1.f : fast_exp2(seg_ref(cs, cP, bh, s - 1, nseg, m, f) -
                                              seg_ref(cs, cP, bh, s, nseg, m, f));
      run = (run + gsv) * sc;
    }
  }
}

// ---------------------------------------------------------------------------
// cbk: grid (ceil(nseg / SPW), BH), NW = m / (16 FT) waves; the chunks of SPW
// consecutive segments in reverse order (the state moved to each earlier
// segment's frame, factors 2^(c*(s) - c*(s+1)) <= 1) with
// the suffix query state carried in registers (queries of later chunks and
// segments), in the frame c*(s).
//   MODE 0: dk.  G^T tiles gT[ct][ft] (lane = feature, rows = columns of
//           [dO | -p_hi | -p_lo]); H^T = G [v | 1 | 1]^T plus the masked
//           term Q'^T b, b_ij = v_j . dO_i - p_i for i >= j; R = K~ H.
//   MODE 1: dv.  G tiles gF[ft][at] (lane = column at of dO, rows =
//           features); dv^T = G^T K~^T plus the masked term dO^T sc,
//           sc_ij = Q'_i . K~_j for i >= j (over the wave's features).
// ---------------------------------------------------------------------------
template <int NW, bool RELU, int MODE, int FT, int SPW>
__global__ __launch_bounds__(NW * 64, 1) void cbk(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ W, const float* __restrict__ cs,
    const float* __restrict__ cP, const float2* __restrict__ lp, const float* __restrict__ Gs,
    uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, int L, int SEG, int nseg,
    float knorm) {
  constexpr int NTH = NW * 64;
  constexpr int M = NW * 16 * FT;   // FT feature tiles of 16 per wave
  const int sA = blockIdx.x * SPW, sB = min(nseg, sA + SPW), bh = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int f0 = 16 * FT * wave;
  __shared__ Stage st;
  __shared__ __align__(16) uint16_t wt[MODE == 0 ? kD * (M + 8) : 8];
  __shared__ __align__(16) float red[NW][kC][kRedRow];
  __shared__ __align__(16) float cst[M];

  for (int r = tid; r < M; r += NTH) cst[r] = RELU ? 0.f : seg_ref(cs, cP, bh, sB - 1, nseg, M, r);
  if constexpr (MODE == 0) load_wt<NTH>(W, M, wt);
  f16x8 wreg[FT][2];
  load_wreg<FT>(W, f0, l16, g, wreg);
  const f32x4 zero4 = f32x4{0.f, 0.f, 0.f, 0.f};

  // Carry-in: the suffix state of the segments after the last one swept.
  const float* gs = Gs + (static_cast<size_t>(bh) * nseg + sB - 1) * kGRows * M;
  f32x4 gT[MODE == 0 ? 5 : 1][FT];
  f32x4 gF[MODE == 1 ? FT : 1][4];
  if constexpr (MODE == 0) {
#pragma unroll
    for (int ct = 0; ct < 5; ++ct)
#pragma unroll
      for (int ft = 0; ft < FT; ++ft)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int col = 16 * ct + 4 * g + v;
          gT[ct][ft][v] = col < kGRows ? gs[static_cast<size_t>(col) * M + f0 + 16 * ft + l16] : 0.f;
        }
  } else {
#pragma unroll
    for (int ft = 0; ft < FT; ++ft)
#pragma unroll
      for (int at = 0; at < 4; ++at) {
        const int col = 16 * at + l16;
        gF[ft][at] = *reinterpret_cast<const f32x4*>(gs + static_cast<size_t>(col) * M + f0 + 16 * ft + 4 * g);
      }
  }
  const bf16x8 ones = (g == 0) ? __builtin_bit_cast(bf16x8, make_uint4(0x3f803f80u, 0u, 0u, 0u))
                               : __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));

  const size_t base = static_cast<size_t>(bh) * L * kD;
  const size_t lbase = static_cast<size_t>(bh) * L;
  __syncthreads();

  ChunkLoader<NTH> ld{ChunkRegs{}, Q, K, V, dO, lp, base, lbase, 0, RELU ? 0.f : knorm};
  for (int s = sB - 1; s >= sA; --s) {
    if (!RELU && SPW > 1 && s < sB - 1) {
      // the carried state into segment s's frame (factors 2^(c*(s) - c*(s+1)) <= 1)
      float fac[FT][4];
#pragma unroll
      for (int ft = 0; ft < FT; ++ft)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          // MODE 0: the lane's feature; MODE 1: the tile rows' features
          const int f = MODE == 0 ? f0 + 16 * ft + l16 : f0 + 16 * ft + 4 * g + v;
          fac[ft][v] = fast_exp2(seg_ref(cs, cP, bh, s, nseg, M, f) - cst[f]);
        }
      lds_barrier();   // every wave has read the previous frame
      for (int r = tid; r < M; r += NTH) cst[r] = seg_ref(cs, cP, bh, s, nseg, M, r);
      if constexpr (MODE == 0) {
#pragma unroll
        for (int ct = 0; ct < 5; ++ct)
#pragma unroll
          for (int ft = 0; ft < FT; ++ft) gT[ct][ft] *= fac[ft][0];
      } else {
#pragma unroll
        for (int ft = 0; ft < FT; ++ft)
#pragma unroll
          for (int at = 0; at < 4; ++at)
#pragma unroll
            for (int v = 0; v < 4; ++v) gF[ft][at][v] *= fac[ft][v];
      }
      lds_barrier();
    }
    const int j0 = s * SEG, j1 = min(L, j0 + SEG);
    const int nch = (j1 - j0 + kC - 1) / kC;
    ld.j1 = j1;
    ld.next(j0 + kC * (nch - 1));
    for (int t = nch - 1; t >= 0; --t) {
      const int jt = j0 + kC * t;
      ld.put(st, jt);
      lds_barrier();
      if (t > 0) ld.next(jt - kC);

      // (1) key features K~^T (E^T orientation: lane = key 16 nk + l16, rows =
      // features 16 ft + 4 g + v).
      f32x4 EK[FT][2];
      {
        f32x4 init[FT];
#pragma unroll
        for (int ft = 0; ft < FT; ++ft) {
          const f32x4 c = *reinterpret_cast<const f32x4*>(&cst[f0 + 16 * ft + 4 * g]);
          init[ft] = -c;
        }
        proj_et<FT>(st.Kh, wreg, l16, g, init, EK);
#pragma unroll
        for (int nk = 0; nk < 2; ++nk) {
          const float n = st.nk[16 * nk + l16];
#pragma unroll
          for (int ft = 0; ft < FT; ++ft)
#pragma unroll
            for (int v = 0; v < 4; ++v) EK[ft][nk][v] = feature<RELU>(EK[ft][nk][v] + n);
        }
      }
      // Query factors Q' (E orientation, lane = feature): the state update's
      // operand and, for dk, the masked term's.
      bf16x8 qb[FT];
      query_factors_e<RELU, FT>(st, wreg, cst, f0, l16, g, qb);

      if constexpr (MODE == 0) {
        // (2) H^T = G [v | 1 | 1]^T (G hi + lo).
        f32x4 H[FT][2];
#pragma unroll
        for (int ft = 0; ft < FT; ++ft) H[ft][0] = H[ft][1] = zero4;
#pragma unroll
        for (int p = 0; p < 3; ++p) {
          bf16x8 vb[2];
#pragma unroll
          for (int nk = 0; nk < 2; ++nk) {
            const int k = 16 * nk + l16;
            if (p < 2) {
              const uint2 a = *reinterpret_cast<const uint2*>(&st.Vr[k][32 * p + 4 * g]);
              const uint2 b = *reinterpret_cast<const uint2*>(&st.Vr[k][32 * p + 16 + 4 * g]);
              vb[nk] = __builtin_bit_cast(bf16x8, make_uint4(a.x, a.y, b.x, b.y));
            } else {
              vb[nk] = ones;
            }
          }
#pragma unroll
          for (int ft = 0; ft < FT; ++ft) {
            bf16x8 ah, al;
            split8(gT[2 * p][ft], p < 2 ? gT[2 * p + 1][ft] : zero4, ah, al);
#pragma unroll
            for (int nk = 0; nk < 2; ++nk) {
              H[ft][nk] = mma_bf16(ah, vb[nk], H[ft][nk]);
              H[ft][nk] = mma_bf16(al, vb[nk], H[ft][nk]);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        // (3) masked term: b (queries x keys) = dO V^T - p, i >= j.
        {
          f32x4 Bm[2][2];   // [mi][nk]: lane = key 16 nk + l16, rows = queries 16 mi + 4 g + v
#pragma unroll
          for (int mi = 0; mi < 2; ++mi) Bm[mi][0] = Bm[mi][1] = zero4;
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            bf16x8 ga[2], vbk[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
              ga[i] = *reinterpret_cast<const bf16x8*>(&st.Gr[16 * i + l16][32 * ks + 8 * g]);
              vbk[i] = *reinterpret_cast<const bf16x8*>(&st.Vr[16 * i + l16][32 * ks + 8 * g]);
            }
#pragma unroll
            for (int mi = 0; mi < 2; ++mi)
#pragma unroll
              for (int nk = 0; nk < 2; ++nk) Bm[mi][nk] = mma_bf16(ga[mi], vbk[nk], Bm[mi][nk]);
          }
          const f32x4 p0 = *reinterpret_cast<const f32x4*>(&st.pq[4 * g]);
          const f32x4 p1 = *reinterpret_cast<const f32x4*>(&st.pq[16 + 4 * g]);
#pragma unroll
          for (int nk = 0; nk < 2; ++nk) {
            const int k = 16 * nk + l16;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              Bm[0][nk][v] = (4 * g + v >= k) ? Bm[0][nk][v] - p0[v] : 0.f;
              Bm[1][nk][v] = (16 + 4 * g + v >= k) ? Bm[1][nk][v] - p1[v] : 0.f;
            }
            bf16x8 bh_, bl_;
            split8(Bm[0][nk], Bm[1][nk], bh_, bl_);
#pragma unroll
            for (int ft = 0; ft < FT; ++ft) {
              H[ft][nk] = mma_bf16(qb[ft], bh_, H[ft][nk]);
              H[ft][nk] = mma_bf16(qb[ft], bl_, H[ft][nk]);
            }
          }
        }
        // (4) R = K~ H (ReLU: [e > 0] H), per-key sums.
        float rs[2] = {0.f, 0.f};
#pragma unroll
        for (int ft = 0; ft < FT; ++ft)
#pragma unroll
          for (int nk = 0; nk < 2; ++nk)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              const float x = RELU ? (EK[ft][nk][v] > 0.f ? H[ft][nk][v] : 0.f) : EK[ft][nk][v] * H[ft][nk][v];
              EK[ft][nk][v] = x;
              rs[nk] += x;
            }
#pragma unroll
        for (int nk = 0; nk < 2; ++nk) {
          rs[nk] += __shfl_xor(rs[nk], 16);
          rs[nk] += __shfl_xor(rs[nk], 32);
        }
        // (5) dk^T partial = W^T R^T.
        f32x4 Dk[4][2];
#pragma unroll
        for (int at = 0; at < 4; ++at) {
          Dk[at][0] = Dk[at][1] = zero4;
#pragma unroll
          for (int kf = 0; kf < FT / 2; ++kf) {
            const bf16x8 wa = *reinterpret_cast<const bf16x8*>(&wt[(16 * at + l16) * (M + 8) + f0 + 32 * kf + 8 * g]);
#pragma unroll
            for (int nk = 0; nk < 2; ++nk) Dk[at][nk] = mma_bf16(wa, pack8(EK[2 * kf][nk], EK[2 * kf + 1][nk]), Dk[at][nk]);
          }
        }
        // (6) state update with the chunk's queries: G^T += [dO | -p]^T Q'.
#pragma unroll
        for (int ct = 0; ct < 5; ++ct) {
          const bf16x8 a = dop_t(st, ct, l16, g);
#pragma unroll
          for (int ft = 0; ft < FT; ++ft) gT[ct][ft] = mma_bf16(a, qb[ft], gT[ct][ft]);
        }
        reduce_store<NW, RELU>(red, Dk, rs, st.Kh, wave, l16, g, knorm, dK, base, jt, j1, true);
      } else {
        // (2) dv^T = G^T K~^T from the carried state.
        f32x4 Dv[4][2];
#pragma unroll
        for (int at = 0; at < 4; ++at) {
          Dv[at][0] = Dv[at][1] = zero4;
#pragma unroll
          for (int kf = 0; kf < FT / 2; ++kf) {
            const bf16x8 ga = pack8(gF[2 * kf][at], gF[2 * kf + 1][at]);
#pragma unroll
            for (int nk = 0; nk < 2; ++nk) Dv[at][nk] = mma_bf16(ga, pack8(EK[2 * kf][nk], EK[2 * kf + 1][nk]), Dv[at][nk]);
          }
        }
        // (3) masked term: sc (queries x keys) = Q' K~^T over the wave's
        // features for i >= j, then dv^T += dO^T sc.
        {
          f32x4 SQ[FT][2];   // Q' in the E^T orientation (lane = query)
          f32x4 init[FT];
#pragma unroll
          for (int mt = 0; mt < FT; ++mt) init[mt] = *reinterpret_cast<const f32x4*>(&cst[f0 + 16 * mt + 4 * g]);
          proj_et<FT>(st.Qh, wreg, l16, g, init, SQ);
#pragma unroll
          for (int nq = 0; nq < 2; ++nq) {
            const float Lq = st.Lq[16 * nq + l16];
#pragma unroll
            for (int mt = 0; mt < FT; ++mt)
#pragma unroll
              for (int v = 0; v < 4; ++v)
                SQ[mt][nq][v] = RELU ? fmaxf(SQ[mt][nq][v], 0.f) * fast_exp2(-Lq) : fast_exp2(SQ[mt][nq][v] - Lq);
          }
          f32x4 Sc[2][2];   // [mi][nk]: lane = key, rows = queries 16 mi + 4 g + v
#pragma unroll
          for (int mi = 0; mi < 2; ++mi) Sc[mi][0] = Sc[mi][1] = zero4;
#pragma unroll
          for (int kf = 0; kf < FT / 2; ++kf)
#pragma unroll
            for (int mi = 0; mi < 2; ++mi) {
              const bf16x8 qa = pack8(SQ[2 * kf][mi], SQ[2 * kf + 1][mi]);
#pragma unroll
              for (int nk = 0; nk < 2; ++nk) Sc[mi][nk] = mma_bf16(qa, pack8(EK[2 * kf][nk], EK[2 * kf + 1][nk]), Sc[mi][nk]);
            }
#pragma unroll
          for (int nk = 0; nk < 2; ++nk) {
            const int k = 16 * nk + l16;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              if (4 * g + v < k) Sc[0][nk][v] = 0.f;
              if (16 + 4 * g + v < k) Sc[1][nk][v] = 0.f;
            }
            const bf16x8 sb = pack8(Sc[0][nk], Sc[1][nk]);
#pragma unroll
            for (int at = 0; at < 4; ++at)
              Dv[at][nk] = mma_bf16(*reinterpret_cast<const bf16x8*>(&st.Gt[16 * at + l16][4 * g]), sb, Dv[at][nk]);
          }
        }
        // (4) state update with the chunk's queries: G += Q'^T dO.
#pragma unroll
        for (int at = 0; at < 4; ++at) {
          const bf16x8 b = *reinterpret_cast<const bf16x8*>(&st.Gt[16 * at + l16][4 * g]);
#pragma unroll
          for (int ft = 0; ft < FT; ++ft) gF[ft][at] = mma_bf16(qb[ft], b, gF[ft][at]);
        }
        const float zs[2] = {0.f, 0.f};
        reduce_store<NW, RELU>(red, Dv, zs, st.Kh, wave, l16, g, knorm, dV, base, jt, j1, false);
      }
      lds_barrier();
    }
  }
}

template <int NW, bool RELU>
hipError_t launch_cbwd(const Plan& p, const BwdPlan& b, const uint16_t* Q, const uint16_t* K,
                       const uint16_t* V, const float* W, const uint16_t* dO, uint16_t* dQ,
                       uint16_t* dK, uint16_t* dV, char* ws, hipStream_t st) {
  float* lpf = reinterpret_cast<float*>(ws + b.off_ru);
  hipError_t e = mfma_causal_rowstats(p, Q, K, V, W, dO, lpf, ws, st);
  if (e != hipSuccess) return e;
  const float* P = reinterpret_cast<const float*>(ws + p.off_T);
  const float* cs = reinterpret_cast<const float*>(ws + p.off_cseg);
  const float* cP = reinterpret_cast<const float*>(ws + p.off_cP);
  const auto* lp = reinterpret_cast<const float2*>(lpf);
  float* Gs = reinterpret_cast<float*>(ws + b.off_G);
  timing_before(st);
  // dq: 32 features per wave (twice the waves, half the registers each)
  // (two segments per work-group: 8-wave work-groups, one per compute unit)
  constexpr int kSpw = 2;
  const dim3 grid2((p.nseg + kSpw - 1) / kSpw, p.BH);
  cbq<2 * NW, RELU, 2><<<grid2, 2 * NW * 64, 0, st>>>(Q, K, V, dO, W, P, cs, cP, lp, dQ, p.L, p.seg,
                                                      p.nseg, kSpw, p.knorm);
  e = hipGetLastError();
  timing_after(st, "cbq");
  if (e != hipSuccess) return e;
  if (p.nseg > 1) {
    timing_before(st);
    cbg<NW, RELU, 4><<<dim3(p.nseg - 1, p.BH), NW * 64, 0, st>>>(Q, K, V, dO, W, cs, cP, lp, Gs, p.L,
                                                              p.seg, p.nseg);
    e = hipGetLastError();
    timing_after(st, "cbg");
    if (e != hipSuccess) return e;
  }
  timing_before(st);
  cbsuffix<<<dim3((kGRows * p.m + 255) / 256, p.BH), 256, 0, st>>>(Gs, cs, cP, p.m, p.nseg, p.relu);
  e = hipGetLastError();
  timing_after(st, "cbsuffix");
  if (e != hipSuccess) return e;
  // dk and dv: 32 features per wave and two segments per work-group, as dq
  timing_before(st);
  cbk<2 * NW, RELU, 0, 2, kSpw><<<grid2, 2 * NW * 64, 0, st>>>(Q, K, V, dO, W, cs, cP, lp, Gs, dK,
                                                               dV, p.L, p.seg, p.nseg, p.knorm);
  e = hipGetLastError();
  timing_after(st, "cbk_dk");
  if (e != hipSuccess) return e;
  timing_before(st);
  cbk<2 * NW, RELU, 1, 2, kSpw><<<grid2, 2 * NW * 64, 0, st>>>(Q, K, V, dO, W, cs, cP, lp, Gs, dK,
                                                               dV, p.L, p.seg, p.nseg, p.knorm);
  e = hipGetLastError();
  timing_after(st, "cbk_dv");
  return e;
}

}  // namespace

hipError_t mfma_causal_backward(const Plan& p, const BwdPlan& b, const void* Q, const void* K,
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
#define FAVOR_CBCASE(NW)                                                                   \
  case NW:                                                                                 \
    return p.relu ? launch_cbwd<NW, true>(p, b, q, k, v, W, g, dq, dk, dv, w, stream)      \
                  : launch_cbwd<NW, false>(p, b, q, k, v, W, g, dq, dk, dv, w, stream);
  switch (p.d == kD ? p.m / 64 : 0) {
    FAVOR_CBCASE(1) FAVOR_CBCASE(2) FAVOR_CBCASE(3) FAVOR_CBCASE(4)
    default: break;
  }
#undef FAVOR_CBCASE
  return hipErrorInvalidValue;
}

}  // namespace favor
