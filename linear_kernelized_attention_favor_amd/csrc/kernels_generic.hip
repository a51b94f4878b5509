// Generic FAVOR+ kernels: plain fp32 FMA arithmetic for every supported shape
// and both input dtypes.  They are the path for fp32 inputs and for shapes the
// MFMA path does not cover, and they are organised the same way:
//
//   1. g_state    per (head, segment, 32-feature block): the key state of the
//                 segment, T = sum_j exp(e_jr - c_r) [v_j | 1], where
//                 e_jr = w_r . k_j - |k_j|^2 / 2 and c_r = max_j e_jr over the
//                 segment (a per-feature exponent reference);
//   2. g_combine  per (head, state entry): bidirectional -- the total over
//                 segments, rescaled to the largest reference, in segment
//                 order; causal -- the exclusive prefix over earlier segments;
//   3. g_apply    per (head, 8-query tile): query features with the key
//                 references added, a per-row reference (row max), the carry
//                 term q~ . [KV | z], the masked in-segment term (causal), and
//                 the division by the last column.
//
// Correctness of the shifts: with key references c_r and row references M_i,
//   sum_r e^{s_ir + c_r - M_i} sum_j e^{e_jr - c_r} [v_j | 1]
//     = e^{-M_i} sum_r e^{s_ir} sum_j e^{e_jr} [v_j | 1],
// and e^{-M_i}, e^{-|q_i|^2/2} and 1/sqrt(m) cancel in the final division, so
// the result is the FA-part equation of the "FAVOR+" method page (bidirectional)
// or its masked prefix-sum form.  Reductions run in a fixed order, so results
// are bitwise reproducible.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <type_traits>

#include "favor.h"
#include "favor_internal.h"
#include "generic_common.h"

namespace favor {
namespace {

using namespace generic_detail;

// ---------------------------------------------------------------------------
// 1. Per-segment key state.  grid (nseg, ceil(m / kFB), BH).
// ---------------------------------------------------------------------------
// (D: the head dimension, a template argument so that every loop over it
// is unrolled and its loads issued together.)
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void g_state(const T* __restrict__ K,
                                                    const T* __restrict__ V,
                                                    const float* __restrict__ W,
                                                    float* __restrict__ Tout,
                                                    float* __restrict__ cseg, int L, int m,
                                                    int seg, int nseg, float knorm, int relu) {
  constexpr int d = D;
  const int s = blockIdx.x, fb = blockIdx.y, bh = blockIdx.z;
  const int t = threadIdx.x;
  const int r = t % kFB, jj = t / kFB;  // this thread's feature and tile row
  const int ncol = d + 1;
  const int nfb = min(kFB, m - fb * kFB);  // features in this block (m % 16 == 0)
  const bool rv = r < nfb;
  __shared__ float Kt[kTT][kMaxD + 1];
  __shared__ float Vt[kTT][kMaxD + 1];
  __shared__ float nrm[kTT];
  __shared__ float E[kTT][kFB];
  __shared__ float cref[kFB];

  const size_t base = static_cast<size_t>(bh) * L * d;
  const int j0 = s * seg, j1 = min(L, j0 + seg);
  const float* wrow = W + static_cast<size_t>(fb * kFB + (rv ? r : 0)) * d;

  // Pass 1: per-feature maximum exponent over the segment (0 for ReLU).
  float mx = relu ? 0.f : -INFINITY;
  for (int jt = j0; jt < j1 && !relu; jt += kTT) {
    __syncthreads();
    load_rows(K, base, jt, j1, d, Kt);
    __syncthreads();
    norm_terms(Kt, d, knorm, nrm);
    __syncthreads();
    if (rv && jt + jj < j1) mx = fmaxf(mx, dot_w(wrow, Kt[jj], d) - nrm[jj]);
  }
  E[jj][r] = mx;
  __syncthreads();
  if (jj == 0) {
    float c = E[0][r];
    for (int k = 1; k < kTT; ++k) c = fmaxf(c, E[k][r]);
    cref[r] = c;
  }
  __syncthreads();

  // Pass 2: T[r][c] = sum_j exp(e_jr - c_r) * [v_j | 1][c].
  constexpr int kAcc = (kFB * (kMaxD + 1) + kThreads - 1) / kThreads;
  float acc[kAcc];
#pragma unroll
  for (int u = 0; u < kAcc; ++u) acc[u] = 0.f;
  const int nent = nfb * ncol;
  for (int jt = j0; jt < j1; jt += kTT) {
    __syncthreads();
    load_rows(K, base, jt, j1, d, Kt);
    for (int i = t; i < kTT * ncol; i += kThreads) {
      const int j = i / ncol, c = i - j * ncol;
      float v = 0.f;
      if (jt + j < j1) v = (c < d) ? load_x(V, base + static_cast<size_t>(jt + j) * d + c) : 1.f;
      Vt[j][c] = v;
    }
    __syncthreads();
    norm_terms(Kt, d, knorm, nrm);
    __syncthreads();
    E[jj][r] = (rv && jt + jj < j1) ? feat(dot_w(wrow, Kt[jj], d) - nrm[jj] - cref[r], relu) : 0.f;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kAcc; ++u) {
      const int e = t + u * kThreads;
      if (e < nent) {
        const int rr = e / ncol, c = e - rr * ncol;
        float a = acc[u];
        for (int j = 0; j < kTT; ++j) a = fmaf(E[j][rr], Vt[j][c], a);
        acc[u] = a;
      }
    }
  }
  const size_t sb = static_cast<size_t>(bh) * nseg + s;
#pragma unroll
  for (int u = 0; u < kAcc; ++u) {
    const int e = t + u * kThreads;
    if (e < nent) {
      const int rr = e / ncol, c = e - rr * ncol;
      Tout[(sb * m + fb * kFB + rr) * ncol + c] = acc[u];
    }
  }
  if (jj == 0 && rv) cseg[sb * m + fb * kFB + r] = cref[r];
}

// ---------------------------------------------------------------------------
// 2. Combine segment states in segment order.  grid (ceil(m*(d+1)/256), BH).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void g_combine(float* __restrict__ Tst,
                                                      const float* __restrict__ cseg,
                                                      float* __restrict__ cP,
                                                      float* __restrict__ KV,
                                                      float* __restrict__ cfin, int nseg, int m,
                                                      int d, int causal,
                                                      const float* __restrict__ st_in,
                                                      float* __restrict__ st_out) {
  const int bh = blockIdx.y;
  const int ncol = d + 1;
  const int e = blockIdx.x * kThreads + threadIdx.x;
  if (e >= m * ncol) return;
  const int r = e / ncol, c = e - r * ncol;
  const size_t cb = static_cast<size_t>(bh) * nseg * m + r;            // + s*m
  const size_t tb = static_cast<size_t>(bh) * nseg * m * ncol + e;     // + s*m*ncol
  if (!causal) {
    float cm = -INFINITY;
    for (int s = 0; s < nseg; ++s) cm = fmaxf(cm, cseg[cb + static_cast<size_t>(s) * m]);
    float acc = 0.f;
    for (int s = 0; s < nseg; ++s)
      acc = fmaf(Tst[tb + static_cast<size_t>(s) * m * ncol],
                 expf(cseg[cb + static_cast<size_t>(s) * m] - cm), acc);
    KV[(static_cast<size_t>(bh) * m + r) * ncol + c] = acc;
    if (c == 0) cfin[static_cast<size_t>(bh) * m + r] = cm;
  } else {
    // (st_in: a carried state [S~ | z~ | c] per head and feature row, the
    // prefix before the first segment; st_out: the total after the last)
    const size_t sr = (static_cast<size_t>(bh) * m + r) * (d + 4);
    float rc = -INFINITY, run = 0.f;
    if (st_in) {
      run = st_in[sr + c];
      rc = st_in[sr + d + 1];
    }
    for (int s = 0; s < nseg; ++s) {
      const size_t ti = tb + static_cast<size_t>(s) * m * ncol;
      const float ts = Tst[ti];
      const float cs = cseg[cb + static_cast<size_t>(s) * m];
      Tst[ti] = run;  // exclusive prefix of the segments before s
      if (c == 0) cP[cb + static_cast<size_t>(s) * m] = rc;
      const float nc = fmaxf(rc, cs);
      run = run * expf(rc - nc) + ts * expf(cs - nc);
      rc = nc;
    }
    if (st_out) {
      st_out[sr + c] = run;
      if (c == 0) {
        st_out[sr + d + 1] = rc;
        st_out[sr + d + 2] = 0.f;
        st_out[sr + d + 3] = 0.f;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// 3. Query side.  grid (ceil(L/kTT), BH).
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void g_apply(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const float* __restrict__ W, const float* __restrict__ KVst, const float* __restrict__ cst,
    const float* __restrict__ csg, T* __restrict__ O, int L, int m, int seg, int nseg,
    int causal, float knorm, int relu) {
  constexpr int d = D;
  const int tile = blockIdx.x, bh = blockIdx.y;
  const int t = threadIdx.x;
  const int i0 = tile * kTT;
  const int ncol = d + 1;
  __shared__ float Qe[kTT][kMaxM];
  __shared__ float Ke[kTT][kMaxM];
  __shared__ float Xt[kTT][kMaxD + 1];
  __shared__ float Vt[kTT][kMaxD + 1];
  __shared__ float cstar[kMaxM];
  __shared__ float cscale[kMaxM];
  __shared__ float nrm[kTT];
  __shared__ float Mrow[kTT];
  __shared__ float Sij[kTT][kTT];
  __shared__ float Num[kTT][kMaxD + 1];

  const size_t base = static_cast<size_t>(bh) * L * d;
  const int s = causal ? (i0 / seg) : 0;
  const float* KVs;  // state rows [m][ncol]
  if (causal) {
    const size_t sb = static_cast<size_t>(bh) * nseg + s;
    KVs = KVst + sb * m * ncol;
    for (int r = t; r < m; r += kThreads) {
      const float cp = cst[sb * m + r], cg = csg[sb * m + r];
      const float cs = fmaxf(cp, cg);
      cstar[r] = cs;
      cscale[r] = expf(cp - cs);  // 0 for the first segment (cp = -inf)
    }
  } else {
    KVs = KVst + static_cast<size_t>(bh) * m * ncol;
    for (int r = t; r < m; r += kThreads) {
      cstar[r] = cst[static_cast<size_t>(bh) * m + r];
      cscale[r] = 1.f;
    }
  }
  load_rows(Q, base, i0, L, d, Xt);
  __syncthreads();

  // Query exponents with the key references added; per-row maximum.
  for (int r = t; r < m; r += kThreads) {
    const float* w = W + static_cast<size_t>(r) * d;
    float e[kTT];
#pragma unroll
    for (int i = 0; i < kTT; ++i) e[i] = 0.f;
    for (int a = 0; a < d; ++a) {
      const float wa = w[a];
#pragma unroll
      for (int i = 0; i < kTT; ++i) e[i] = fmaf(wa, Xt[i][a], e[i]);
    }
#pragma unroll
    for (int i = 0; i < kTT; ++i) Qe[i][r] = e[i] + cstar[r];
  }
  __syncthreads();
  {
    // 32 lanes per row: lane k scans features k, k+32, ...; then a shuffle tree.
    const int i = t / 32, k = t % 32;
    float mx = -INFINITY;
    for (int r = k; r < m; r += 32) mx = fmaxf(mx, Qe[i][r]);
    for (int off = 16; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 32));
    if (k == 0) Mrow[i] = relu ? 0.f : mx;
  }
  __syncthreads();
  for (int p = t; p < kTT * m; p += kThreads) {
    const int i = p / m, r = p - i * m;
    Qe[i][r] = feat(Qe[i][r] - Mrow[i], relu);
  }
  __syncthreads();

  // Carry / total term: num[i][c] = sum_r q~_ir * scale_r * KV[r][c].
  constexpr int kAcc = (kTT * (kMaxD + 1) + kThreads - 1) / kThreads;
  float acc[kAcc];
#pragma unroll
  for (int u = 0; u < kAcc; ++u) {
    acc[u] = 0.f;
    const int p = t + u * kThreads;
    if (p < kTT * ncol) {
      const int i = p / ncol, c = p - i * ncol;
      float a = 0.f;
      for (int r = 0; r < m; ++r) a = fmaf(Qe[i][r] * cscale[r], KVs[static_cast<size_t>(r) * ncol + c], a);
      acc[u] = a;
    }
  }

  if (causal) {
    // Masked term over this segment's keys up to the end of the tile.
    const int js = s * seg;
    for (int jc = js; jc <= i0; jc += kTT) {
      __syncthreads();
      load_rows(K, base, jc, L, d, Xt);
      for (int i = t; i < kTT * ncol; i += kThreads) {
        const int j = i / ncol, c = i - j * ncol;
        float v = 0.f;
        if (jc + j < L) v = (c < d) ? load_x(V, base + static_cast<size_t>(jc + j) * d + c) : 1.f;
        Vt[j][c] = v;
      }
      __syncthreads();
      norm_terms(Xt, d, knorm, nrm);
      __syncthreads();
      for (int r = t; r < m; r += kThreads) {
        const float* w = W + static_cast<size_t>(r) * d;
        float e[kTT];
#pragma unroll
        for (int j = 0; j < kTT; ++j) e[j] = 0.f;
        for (int a = 0; a < d; ++a) {
          const float wa = w[a];
#pragma unroll
          for (int j = 0; j < kTT; ++j) e[j] = fmaf(wa, Xt[j][a], e[j]);
        }
#pragma unroll
        for (int j = 0; j < kTT; ++j) Ke[j][r] = feat(e[j] - nrm[j] - cstar[r], relu);
      }
      __syncthreads();
      if (t < kTT * kTT * 4) {
        const int pr = t / 4, part = t % 4;
        const int i = pr / kTT, j = pr % kTT;
        float a = 0.f;
        for (int r = part; r < m; r += 4) a = fmaf(Qe[i][r], Ke[j][r], a);
        a += __shfl_xor(a, 1, 4);
        a += __shfl_xor(a, 2, 4);
        const bool keep = (jc + j <= i0 + i) && (jc + j < L);
        if (part == 0) Sij[i][j] = keep ? a : 0.f;
      }
      __syncthreads();
#pragma unroll
      for (int u = 0; u < kAcc; ++u) {
        const int p = t + u * kThreads;
        if (p < kTT * ncol) {
          const int i = p / ncol, c = p - i * ncol;
          float a = acc[u];
          for (int j = 0; j < kTT; ++j) a = fmaf(Sij[i][j], Vt[j][c], a);
          acc[u] = a;
        }
      }
    }
  }

#pragma unroll
  for (int u = 0; u < kAcc; ++u) {
    const int p = t + u * kThreads;
    if (p < kTT * ncol) Num[p / ncol][p % ncol] = acc[u];
  }
  __syncthreads();
  for (int p = t; p < kTT * d; p += kThreads) {
    const int i = p / d, c = p - i * d;
    if (i0 + i < L) store_x(O, base + static_cast<size_t>(i0 + i) * d + c, Num[i][c] / Num[i][d]);
  }
}

// ---------------------------------------------------------------------------
// Feature map test kernel: Xp = exp(w . x - knorm |x|^2) / sqrt(m), no shift,
// or max(w . x, 0) / sqrt(m) when relu is set.
// grid (ceil(L/kTT), BH).
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(kThreads) void g_feature_map(const T* __restrict__ X,
                                                          const float* __restrict__ W,
                                                          float* __restrict__ Xp, int L, int d,
                                                          int m, float knorm, int relu) {
  const int tile = blockIdx.x, bh = blockIdx.y;
  const int i0 = tile * kTT;
  __shared__ float Xt[kTT][kMaxD + 1];
  __shared__ float nrm[kTT];
  const size_t base = static_cast<size_t>(bh) * L * d;
  load_rows(X, base, i0, L, d, Xt);
  __syncthreads();
  norm_terms(Xt, d, knorm, nrm);
  __syncthreads();
  const float inv_sqrt_m = 1.0f / sqrtf(static_cast<float>(m));
  for (int r = threadIdx.x; r < m; r += kThreads) {
    const float* w = W + static_cast<size_t>(r) * d;
    for (int i = 0; i < kTT && i0 + i < L; ++i) {
      const float e = dot_w(w, Xt[i], d) - nrm[i];
      Xp[(static_cast<size_t>(bh) * L + i0 + i) * m + r] = feat(e, relu) * inv_sqrt_m;
    }
  }
}

// Steps 1 and 2: the key state (bidirectional: KV and cfin; causal: the
// exclusive prefixes in T with references cP, and the segment references).
template <typename T>
hipError_t key_state_t(const Plan& p, const T* K, const T* V, const float* W, char* ws,
                       hipStream_t st, const float* st_in = nullptr, float* st_out = nullptr) {
  float* Tst = reinterpret_cast<float*>(ws + p.off_T);
  float* cseg = reinterpret_cast<float*>(ws + p.off_cseg);
  float* cP = reinterpret_cast<float*>(ws + p.off_cP);
  float* KV = reinterpret_cast<float*>(ws + p.off_KV);
  float* cfin = reinterpret_cast<float*>(ws + p.off_cfin);
  timing_before(st);
  const dim3 gs(p.nseg, (p.m + kFB - 1) / kFB, p.BH);
  switch (p.d) {
    case 16: g_state<T, 16><<<gs, kThreads, 0, st>>>(K, V, W, Tst, cseg, p.L, p.m, p.seg, p.nseg, p.knorm, p.relu); break;
    case 32: g_state<T, 32><<<gs, kThreads, 0, st>>>(K, V, W, Tst, cseg, p.L, p.m, p.seg, p.nseg, p.knorm, p.relu); break;
    case 64: g_state<T, 64><<<gs, kThreads, 0, st>>>(K, V, W, Tst, cseg, p.L, p.m, p.seg, p.nseg, p.knorm, p.relu); break;
    case 128: g_state<T, 128><<<gs, kThreads, 0, st>>>(K, V, W, Tst, cseg, p.L, p.m, p.seg, p.nseg, p.knorm, p.relu); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  timing_after(st, "g_state");
  if (e != hipSuccess) return e;
  const int nent = p.m * (p.d + 1);
  timing_before(st);
  g_combine<<<dim3((nent + kThreads - 1) / kThreads, p.BH), kThreads, 0, st>>>(
      Tst, cseg, cP, KV, cfin, p.nseg, p.m, p.d, p.causal, st_in, st_out);
  e = hipGetLastError();
  timing_after(st, "g_combine");
  return e;
}

template <typename T>
hipError_t forward_t(const Plan& p, const T* Q, const T* K, const T* V, const float* W, T* O,
                     char* ws, hipStream_t st, const float* st_in = nullptr,
                     float* st_out = nullptr) {
  hipError_t e = key_state_t(p, K, V, W, ws, st, st_in, st_out);
  if (e != hipSuccess) return e;
  float* Tst = reinterpret_cast<float*>(ws + p.off_T);
  float* cseg = reinterpret_cast<float*>(ws + p.off_cseg);
  float* cP = reinterpret_cast<float*>(ws + p.off_cP);
  float* KV = reinterpret_cast<float*>(ws + p.off_KV);
  float* cfin = reinterpret_cast<float*>(ws + p.off_cfin);
  const dim3 ga((p.L + kTT - 1) / kTT, p.BH);
  timing_before(st);
  const float* kvs = p.causal ? Tst : KV;
  const float* cst = p.causal ? cP : cfin;
  const float* csg = p.causal ? cseg : nullptr;
  auto apply = [&](auto DC) {
    constexpr int D = decltype(DC)::value;
    g_apply<T, D><<<ga, kThreads, 0, st>>>(Q, K, V, W, kvs, cst, csg, O, p.L, p.m, p.seg, p.nseg,
                                           p.causal ? 1 : 0, p.knorm, p.relu);
  };
  switch (p.d) {
    case 16: apply(std::integral_constant<int, 16>{}); break;
    case 32: apply(std::integral_constant<int, 32>{}); break;
    case 64: apply(std::integral_constant<int, 64>{}); break;
    case 128: apply(std::integral_constant<int, 128>{}); break;
    default: return hipErrorInvalidValue;
  }
  e = hipGetLastError();
  timing_after(st, "g_apply");
  return e;
}

// ---------------------------------------------------------------------------
// Incremental causal state.  A head's state is fp32 [m][d+4]: row r holds
// [S~_r | z~_r | c_r | 0 | 0] (16-byte rows) with the true state [S | z]_r = e^{c_r} [S~_r | z~_r]
// (the features' 1/sqrt(m) left out, as everywhere on this path; ReLU: c_r is
// 0 once a token has been added).  Empty: S~ = z~ = 0, c = -inf.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void g_state_reset(float* __restrict__ st, size_t rows,
                                                          int d) {
  const int sw = d + 4;
  const size_t n = rows * sw;
  for (size_t i = static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x; i < n;
       i += static_cast<size_t>(gridDim.x) * kThreads)
    st[i] = (static_cast<int>(i % sw) == d + 1) ? -INFINITY : 0.f;
}

// One token per head: add (k, v) to the state (the reference of each feature
// raised to cover the new key), then o = q~ [S | z] -> num / den with the
// query's own row reference.  grid (BH), one work-group per head; the state
// rows move as float4 quads, a quad column per thread and the rows split
// over groups of threads.  The step is a chain of dependent memory round
// trips, so every load a thread needs is issued before its first use: the
// head dimension D is a template argument (a row of W is D / 4 float4 loads
// issued at once), and the state rows go in batches of RB whose loads all
// precede their stores.
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void g_decode(const T* __restrict__ q,
                                                     const T* __restrict__ k,
                                                     const T* __restrict__ v,
                                                     const float* __restrict__ W,
                                                     T* __restrict__ o, float* __restrict__ st,
                                                     int m, float knorm, int relu) {
  constexpr int d = D;
  const int bh = blockIdx.x, t = threadIdx.x;
  const int sw = d + 4, nq = sw / 4;
  const int ng = kThreads / nq;                  // row groups
  __shared__ float xq[kMaxD], xk[kMaxD], xv[kMaxD + 4];
  __shared__ float kt[kMaxM], sc[kMaxM], qt[kMaxM];
  __shared__ float part[kThreads / 5][kMaxD + 4];  // (nq >= 5)
  __shared__ float wred[kThreads / 64];
  __shared__ float nk;
  const size_t base = static_cast<size_t>(bh) * d;
  for (int a = t; a < d; a += kThreads) {
    xq[a] = load_x(q, base + a);
    xk[a] = load_x(k, base + a);
    xv[a] = load_x(v, base + a);
  }
  if (t < 4) xv[d + t] = (t == 0) ? 1.f : 0.f;
  __syncthreads();
  if (t < 64) {
    float acc = 0.f;
    for (int a = t; a < d; a += 64) acc = fmaf(xk[a], xk[a], acc);
    for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    if (t == 0) nk = knorm * acc;
  }
  __syncthreads();
  float* S = st + static_cast<size_t>(bh) * m * sw;
  float mx = -INFINITY;
  for (int r = t; r < m; r += kThreads) {
    const float4* w4 = reinterpret_cast<const float4*>(W + static_cast<size_t>(r) * d);
    float4 wr[D / 4];
#pragma unroll
    for (int a = 0; a < D / 4; ++a) wr[a] = w4[a];
    const float c = S[static_cast<size_t>(r) * sw + d + 1];
    float e0 = 0.f, e1 = 0.f, s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int a = 0; a < D / 4; ++a) {
      e0 = fmaf(wr[a].x, xk[4 * a], e0); e1 = fmaf(wr[a].y, xk[4 * a + 1], e1);
      e0 = fmaf(wr[a].z, xk[4 * a + 2], e0); e1 = fmaf(wr[a].w, xk[4 * a + 3], e1);
      s0 = fmaf(wr[a].x, xq[4 * a], s0); s1 = fmaf(wr[a].y, xq[4 * a + 1], s1);
      s0 = fmaf(wr[a].z, xq[4 * a + 2], s0); s1 = fmaf(wr[a].w, xq[4 * a + 3], s1);
    }
    const float e = (e0 + e1) - nk;
    float cn;
    if (relu) {
      cn = 0.f;
      sc[r] = 1.f;
      kt[r] = fmaxf(e, 0.f);
    } else {
      cn = fmaxf(c, e);
      sc[r] = expf(c - cn);     // 0 for an empty row (c = -inf)
      kt[r] = expf(e - cn);
    }
    S[static_cast<size_t>(r) * sw + d + 1] = cn;
    const float s = s0 + s1;
    qt[r] = relu ? fmaxf(s, 0.f) : s + cn;
    mx = fmaxf(mx, qt[r]);
  }
  // row reference of the query (ReLU: none)
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  if ((t & 63) == 0) wred[t >> 6] = mx;
  __syncthreads();
  if (!relu) {
    float M = wred[0];
    for (int i = 1; i < kThreads / 64; ++i) M = fmaxf(M, wred[i]);
    for (int r = t; r < m; r += kThreads) qt[r] = expf(qt[r] - M);
  }
  __syncthreads();
  // State update and the query's contraction: thread (quad j, group g) owns
  // columns 4j..4j+3 of rows g, g+ng, ...  Columns above d (the reference
  // and the padding) pass through unchanged.
  const int j = t % nq, g = t / nq;
  if (g < ng) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    const int c0 = 4 * j;
    const float v0 = xv[c0], v1 = xv[c0 + 1], v2 = xv[c0 + 2], v3 = xv[c0 + 3];
    const bool up1 = c0 + 1 <= d, up2 = c0 + 2 <= d, up3 = c0 + 3 <= d;
    float4* S4 = reinterpret_cast<float4*>(S);
    constexpr int RB = 24;   // (m = 256, d = 64: one batch)
    for (int r0 = g; r0 < m; r0 += RB * ng) {
      float4 xs[RB];
#pragma unroll
      for (int u = 0; u < RB; ++u) {
        const int r = r0 + u * ng;
        if (r < m) xs[u] = S4[static_cast<size_t>(r) * nq + j];
      }
#pragma unroll
      for (int u = 0; u < RB; ++u) {
        const int r = r0 + u * ng;
        if (r < m) {
          float4 x = xs[u];
          const float a = sc[r], b = kt[r], qr = qt[r];
          x.x = fmaf(x.x, a, b * v0);
          if (up1) x.y = fmaf(x.y, a, b * v1);
          if (up2) x.z = fmaf(x.z, a, b * v2);
          if (up3) x.w = fmaf(x.w, a, b * v3);
          S4[static_cast<size_t>(r) * nq + j] = x;
          acc.x = fmaf(qr, x.x, acc.x);
          acc.y = fmaf(qr, x.y, acc.y);
          acc.z = fmaf(qr, x.z, acc.z);
          acc.w = fmaf(qr, x.w, acc.w);
        }
      }
    }
    part[g][c0] = acc.x;
    part[g][c0 + 1] = acc.y;
    part[g][c0 + 2] = acc.z;
    part[g][c0 + 3] = acc.w;
  }
  __syncthreads();
  if (t <= d) {
    float a = 0.f;
    for (int i = 0; i < ng; ++i) a += part[i][t];
    xv[t] = a;     // (xv no longer needed: reused for [num | den])
  }
  __syncthreads();
  for (int c = t; c < d; c += kThreads) store_x(o, base + c, xv[c] / xv[d]);
}

}  // namespace

hipError_t generic_state_reset(int32_t BH, int32_t d, int32_t m, float* state,
                               hipStream_t stream) {
  const size_t rows = static_cast<size_t>(BH) * m;
  const size_t n = rows * (d + 4);
  const int blocks = static_cast<int>(std::min<size_t>((n + kThreads - 1) / kThreads, 4096));
  g_state_reset<<<blocks, kThreads, 0, stream>>>(state, rows, d);
  return hipGetLastError();
}

hipError_t generic_decode(int32_t BH, int32_t d, int32_t m, int32_t dtype, float knorm,
                          int32_t relu, const void* q, const void* k, const void* v,
                          const float* W, void* o, float* state, hipStream_t stream) {
  timing_before(stream);
  auto launch = [&](auto DC) {
    constexpr int D = decltype(DC)::value;
    if (dtype == FAVOR_F32)
      g_decode<float, D><<<BH, kThreads, 0, stream>>>(
          static_cast<const float*>(q), static_cast<const float*>(k), static_cast<const float*>(v),
          W, static_cast<float*>(o), state, m, knorm, relu);
    else
      g_decode<uint16_t, D><<<BH, kThreads, 0, stream>>>(
          static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
          static_cast<const uint16_t*>(v), W, static_cast<uint16_t*>(o), state, m, knorm, relu);
  };
  switch (d) {
    case 16: launch(std::integral_constant<int, 16>{}); break;
    case 32: launch(std::integral_constant<int, 32>{}); break;
    case 64: launch(std::integral_constant<int, 64>{}); break;
    case 128: launch(std::integral_constant<int, 128>{}); break;
    default: return hipErrorInvalidValue;
  }
  const hipError_t e = hipGetLastError();
  timing_after(stream, "g_decode");
  return e;
}

hipError_t generic_prefill(const Plan& p, const void* Q, const void* K, const void* V,
                           const float* W, void* O, const float* st_in, float* st_out, void* ws,
                           hipStream_t stream) {
  char* w = static_cast<char*>(ws);
  if (p.dtype == FAVOR_F32)
    return forward_t<float>(p, static_cast<const float*>(Q), static_cast<const float*>(K),
                            static_cast<const float*>(V), W, static_cast<float*>(O), w, stream,
                            st_in, st_out);
  return forward_t<uint16_t>(p, static_cast<const uint16_t*>(Q), static_cast<const uint16_t*>(K),
                             static_cast<const uint16_t*>(V), W, static_cast<uint16_t*>(O), w,
                             stream, st_in, st_out);
}

hipError_t generic_forward(const Plan& p, const void* Q, const void* K, const void* V,
                           const float* W, void* O, void* ws, hipStream_t stream) {
  char* w = static_cast<char*>(ws);
  if (p.dtype == FAVOR_F32)
    return forward_t<float>(p, static_cast<const float*>(Q), static_cast<const float*>(K),
                            static_cast<const float*>(V), W, static_cast<float*>(O), w, stream);
  return forward_t<uint16_t>(p, static_cast<const uint16_t*>(Q), static_cast<const uint16_t*>(K),
                             static_cast<const uint16_t*>(V), W, static_cast<uint16_t*>(O), w,
                             stream);
}

hipError_t generic_key_state(const Plan& p, const void* K, const void* V, const float* W,
                             void* ws, hipStream_t stream) {
  char* w = static_cast<char*>(ws);
  if (p.dtype == FAVOR_F32)
    return key_state_t<float>(p, static_cast<const float*>(K), static_cast<const float*>(V), W, w,
                              stream);
  return key_state_t<uint16_t>(p, static_cast<const uint16_t*>(K), static_cast<const uint16_t*>(V),
                               W, w, stream);
}

hipError_t generic_feature_map(int32_t BH, int32_t L, int32_t d, int32_t m, int32_t dtype,
                               float knorm, int32_t relu, const void* X, const float* W, float* Xp,
                               hipStream_t stream) {
  const dim3 g((L + kTT - 1) / kTT, BH);
  if (dtype == FAVOR_F32)
    g_feature_map<float><<<g, kThreads, 0, stream>>>(static_cast<const float*>(X), W, Xp, L, d, m,
                                                     knorm, relu);
  else
    g_feature_map<uint16_t><<<g, kThreads, 0, stream>>>(static_cast<const uint16_t*>(X), W, Xp,
                                                        L, d, m, knorm, relu);
  return hipGetLastError();
}

}  // namespace favor
