// Generic FAVOR+ backward kernels: plain fp32 FMA arithmetic for every
// supported shape, both input dtypes, both forms and every kernel of
// attention.  They give the gradients of <dO, O> with respect to Q, K and V
// for an upstream gradient dO, W held fixed: the chain rule through the
// features and the FA-part bracket of the "FAVOR+" method page (bidirectional)
// or its masked prefix-sum form (causal).
//
// The forward's stabilised quantities are rebuilt first (g_state and
// g_combine): key features K~_jr = exp(e_jr - c_r), the state
// [S~ | z~] = sum_j K~_j [v_j | 1] and, per query, Q~_ir = exp(s_ir + c_r - M_i)
// and den~_i = Q~_i . z~.  Then, per query i,
//
//   Ucat_i = [U_i | u0_i],  U_i = dO_i / den~_i,  u0_i = -(dO_i . O_i) / den~_i,
//
// and
//   query side  T_ir = [S~_r | z~_r] . Ucat_i,  P_ir = Q~_ir T_ir,
//               dq_i = sum_r P_ir w_r - 2 knorm (sum_r P_ir) q_i
//   key side    G_r = sum_i Q~_ir Ucat_i (bidirectional: every query; causal:
//               the queries i >= j, as an exclusive suffix over later
//               segments plus a masked term inside the key's segment),
//               H_jr = G_r . [v_j | 1],  R_jr = K~_jr H_jr,
//               dk_j = sum_r R_jr w_r - 2 knorm (sum_r R_jr) k_j,
//               dv_j = sum_r K~_jr G_r[0:d].
// ReLU features: P_ir = [s_ir > 0] T_ir and R_jr = [e_jr > 0] H_jr, no norm
// term (knorm = 0).  Every shift cancels: P and R are products of a query
// factor and a key factor whose references are opposite, and the row factor
// e^{-M_i} of Q~ is divided out through den~ in U.  The query features' own
// norm term is a per-row factor that cancels in D^-1, so the forward leaves it
// out; its gradient term, -2 knorm (sum_r P_ir) q_i, is zero up to rounding
// and is kept for fidelity to the chain rule.
//
// Causal references: segment s works at c*(s) = max over segments u <= s of
// their per-feature references (non-decreasing in s), the forward's own.  The
// suffix over later segments t > s is carried down at c*(s) with factors
// exp(c*(s) - c*(t)) <= 1.  Reductions run in a fixed order: results are
// bitwise reproducible.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "favor.h"
#include "favor_internal.h"
#include "generic_common.h"

namespace favor {
namespace {

using namespace generic_detail;

constexpr int kTc = kTT * kMaxD / kThreads;   // (token, column) entries per thread

// Per-feature references of a head's segment: c*(s) and, for the carried
// state, the factor exp(cP - c*) (0 for the first causal segment).
__device__ inline void segment_refs(const float* __restrict__ cst, const float* __restrict__ csg,
                                    int bh, int s, int m, int nseg, int causal, float* cstar,
                                    float* cscale) {
  for (int r = threadIdx.x; r < m; r += kThreads) {
    if (causal) {
      const size_t sb = static_cast<size_t>(bh) * nseg + s;
      const float cp = cst[sb * m + r], cg = csg[sb * m + r];
      const float cs = fmaxf(cp, cg);
      cstar[r] = cs;
      if (cscale) cscale[r] = expf(cp - cs);
    } else {
      cstar[r] = cst[static_cast<size_t>(bh) * m + r];
      if (cscale) cscale[r] = 1.f;
    }
  }
}

// Loads kTT rows of [V | 1] (zero rows, the ones column included, past jend).
template <typename T>
__device__ inline void load_vcat(const T* __restrict__ V, size_t base, int j0, int jend, int d,
                                 float (*dst)[kMaxD + 1]) {
  const int ncol = d + 1;
  for (int i = threadIdx.x; i < kTT * ncol; i += kThreads) {
    const int j = i / ncol, c = i - j * ncol;
    float v = 0.f;
    if (j0 + j < jend) v = (c < d) ? load_x(V, base + static_cast<size_t>(j0 + j) * d + c) : 1.f;
    dst[j][c] = v;
  }
}

// Features of kTT rows in `rows` for every feature r < m:
// out[i][r] = feat(w_r . x_i + add_r - sub_i), zero for rows i >= nvalid.
__device__ inline void features_of(const float* __restrict__ W, const float (*rows)[kMaxD + 1],
                                   int d, int m, const float* add, const float* sub, int nvalid,
                                   int relu, float (*out)[kMaxM]) {
  for (int r = threadIdx.x; r < m; r += kThreads) {
    const float* w = W + static_cast<size_t>(r) * d;
    float e[kTT];
#pragma unroll
    for (int i = 0; i < kTT; ++i) e[i] = 0.f;
    for (int a = 0; a < d; ++a) {
      const float wa = w[a];
#pragma unroll
      for (int i = 0; i < kTT; ++i) e[i] = fmaf(wa, rows[i][a], e[i]);
    }
#pragma unroll
    for (int i = 0; i < kTT; ++i) out[i][r] = (i < nvalid) ? feat(e[i] + add[r] - sub[i], relu) : 0.f;
  }
}

// 8x8 dot products over n entries, four threads per pair:
// out[i][j] = keep(i, j) ? sum_k a[i][k] b[j][k] : 0.
template <int N, typename Keep>
__device__ inline void pair_dots(const float (*a)[N], const float (*b)[N], int n, Keep keep,
                                 float (*out)[kTT]) {
  const int t = threadIdx.x;
  if (t < kTT * kTT * 4) {
    const int pr = t / 4, part = t % 4;
    const int i = pr / kTT, j = pr % kTT;
    float acc = 0.f;
    for (int k = part; k < n; k += 4) acc = fmaf(a[i][k], b[j][k], acc);
    acc += __shfl_xor(acc, 1, 4);
    acc += __shfl_xor(acc, 2, 4);
    if (part == 0) out[i][j] = keep(i, j) ? acc : 0.f;
  }
}

// Row sums of an [kTT][m] LDS array (32 lanes per row) into out[kTT].
__device__ inline void row_sums(const float (*x)[kMaxM], int m, float* out) {
  const int i = threadIdx.x / 32, k = threadIdx.x % 32;
  float acc = 0.f;
  for (int r = k; r < m; r += 32) acc += x[i][r];
  for (int off = 16; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 32);
  if (k == 0) out[i] = acc;
}

// ---------------------------------------------------------------------------
// Query side.  grid (ceil(L/kTT), BH).  Rebuilds num and den as the forward
// does, forms Ucat (written to the workspace with the row reference M), and
// dq = P W - 2 knorm (sum_r P) q.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(kThreads) void gb_query(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const T* __restrict__ dO, const float* __restrict__ W, const float* __restrict__ KVst,
    const float* __restrict__ cst, const float* __restrict__ csg, float* __restrict__ Ucat,
    float* __restrict__ Mst, T* __restrict__ dQ, int L, int d, int m, int seg, int nseg,
    int causal, float knorm, int relu) {
  const int tile = blockIdx.x, bh = blockIdx.y;
  const int t = threadIdx.x;
  const int i0 = tile * kTT;
  const int ncol = d + 1;
  __shared__ float Qe[kTT][kMaxM];
  __shared__ float Ke[kTT][kMaxM];
  __shared__ float Tq[kTT][kMaxM];
  __shared__ float Xt[kTT][kMaxD + 1];   // Q rows
  __shared__ float Kt[kTT][kMaxD + 1];   // K rows of the masked term
  __shared__ float Vt[kTT][kMaxD + 1];   // [V | 1] rows of the masked term
  __shared__ float Dt[kTT][kMaxD + 1];   // dO rows
  __shared__ float Uc[kTT][kMaxD + 1];   // [num | den], then Ucat
  __shared__ float cstar[kMaxM];
  __shared__ float cscale[kMaxM];
  __shared__ float negc[kMaxM];   // -c*: key features exp(e - n - c*)
  __shared__ float nrm[kTT];
  __shared__ float Mrow[kTT];
  __shared__ float den[kTT];
  __shared__ float red[kTT];
  __shared__ float Sij[kTT][kTT];

  const size_t base = static_cast<size_t>(bh) * L * d;
  const int s = causal ? (i0 / seg) : 0;
  const float* KVs = KVst + (causal ? (static_cast<size_t>(bh) * nseg + s) : static_cast<size_t>(bh)) *
                                m * ncol;
  segment_refs(cst, csg, bh, s, m, nseg, causal, cstar, cscale);
  load_rows(Q, base, i0, L, d, Xt);
  load_rows(dO, base, i0, L, d, Dt);
  __syncthreads();
  for (int r = t; r < m; r += kThreads) negc[r] = -cstar[r];

  // Query exponents with the key references added; the row reference M_i.
  for (int r = t; r < m; r += kThreads) {
    const float* w = W + static_cast<size_t>(r) * d;
    for (int i = 0; i < kTT; ++i) Qe[i][r] = dot_w(w, Xt[i], d) + cstar[r];
  }
  __syncthreads();
  {
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

  // [num | den] = Q~ . (carried state) + masked in-segment term (causal).
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
  const int js = s * seg;
  if (causal) {
    for (int jc = js; jc <= i0; jc += kTT) {
      __syncthreads();
      load_rows(K, base, jc, L, d, Kt);
      load_vcat(V, base, jc, L, d, Vt);
      __syncthreads();
      norm_terms(Kt, d, knorm, nrm);
      __syncthreads();
      features_of(W, Kt, d, m, negc, nrm, kTT, relu, Ke);
      __syncthreads();
      pair_dots<kMaxM>(Qe, Ke, m, [&](int i, int j) { return jc + j <= i0 + i && jc + j < L; }, Sij);
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
    if (p < kTT * ncol) Uc[p / ncol][p % ncol] = acc[u];
  }
  __syncthreads();

  // Ucat = [dO / den | -(dO . num) / den^2].
  {
    const int i = t / 32, k = t % 32;
    float dn = 0.f;
    for (int c = k; c < d; c += 32) dn = fmaf(Dt[i][c], Uc[i][c], dn);
    for (int off = 16; off > 0; off >>= 1) dn += __shfl_xor(dn, off, 32);
    if (k == 0) {
      den[i] = Uc[i][d];
      red[i] = dn;
    }
  }
  __syncthreads();
  for (int p = t; p < kTT * ncol; p += kThreads) {
    const int i = p / ncol, c = p - i * ncol;
    const float dv = den[i];
    const float u = (c < d) ? Dt[i][c] / dv : -red[i] / (dv * dv);
    Uc[i][c] = u;
    if (i0 + i < L) Ucat[(static_cast<size_t>(bh) * L + i0 + i) * ncol + c] = u;
  }
  if (t < kTT && i0 + t < L) Mst[static_cast<size_t>(bh) * L + i0 + t] = Mrow[t];
  __syncthreads();

  // T = (carried state) . Ucat + masked term, per (token, feature).
  for (int p = t; p < kTT * m; p += kThreads) {
    const int i = p / m, r = p - i * m;
    const float* kv = KVs + static_cast<size_t>(r) * ncol;
    float a = 0.f;
    for (int c = 0; c < ncol; ++c) a = fmaf(kv[c], Uc[i][c], a);
    Tq[i][r] = a * cscale[r];
  }
  if (causal) {
    for (int jc = js; jc <= i0; jc += kTT) {
      __syncthreads();
      load_rows(K, base, jc, L, d, Kt);
      load_vcat(V, base, jc, L, d, Vt);
      __syncthreads();
      norm_terms(Kt, d, knorm, nrm);
      __syncthreads();
      features_of(W, Kt, d, m, negc, nrm, kTT, relu, Ke);
      __syncthreads();
      // C[i][j] = Ucat_i . [v_j | 1] for keys j <= i
      pair_dots<kMaxD + 1>(Uc, Vt, ncol, [&](int i, int j) { return jc + j <= i0 + i && jc + j < L; },
                           Sij);
      __syncthreads();
      for (int p = t; p < kTT * m; p += kThreads) {
        const int i = p / m, r = p - i * m;
        float a = Tq[i][r];
        for (int j = 0; j < kTT; ++j) a = fmaf(Ke[j][r], Sij[i][j], a);
        Tq[i][r] = a;
      }
    }
  }
  __syncthreads();
  // P = Q~ T (ReLU: the gate of the query's projection), in place of Q~.
  for (int p = t; p < kTT * m; p += kThreads) {
    const int i = p / m, r = p - i * m;
    const float q = Qe[i][r];
    Qe[i][r] = relu ? (q > 0.f ? Tq[i][r] : 0.f) : q * Tq[i][r];
  }
  __syncthreads();
  row_sums(Qe, m, red);
  __syncthreads();
  const float cq = 2.f * knorm;
  for (int p = t; p < kTT * d; p += kThreads) {
    const int i = p / d, a = p - i * d;
    float g = 0.f;
    for (int r = 0; r < m; ++r) g = fmaf(Qe[i][r], W[static_cast<size_t>(r) * d + a], g);
    g = fmaf(-cq * red[i], Xt[i][a], g);
    if (i0 + i < L) store_x(dQ, base + static_cast<size_t>(i0 + i) * d + a, g);
  }
}

// ---------------------------------------------------------------------------
// Per-segment query state G_s = sum_{i in s} Q~_ir Ucat_i.
// grid (nseg, ceil(m / kFB), BH).
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(kThreads) void gb_gstate(
    const T* __restrict__ Q, const float* __restrict__ W, const float* __restrict__ Ucat,
    const float* __restrict__ Mst, const float* __restrict__ cst, const float* __restrict__ csg,
    float* __restrict__ Gst, int L, int d, int m, int seg, int nseg, int causal, int relu) {
  const int s = blockIdx.x, fb = blockIdx.y, bh = blockIdx.z;
  const int t = threadIdx.x;
  const int r = t % kFB, jj = t / kFB;
  const int ncol = d + 1;
  const int nfb = min(kFB, m - fb * kFB);
  const bool rv = r < nfb;
  const int f = fb * kFB + (rv ? r : 0);
  __shared__ float Qt[kTT][kMaxD + 1];
  __shared__ float Ut[kTT][kMaxD + 1];
  __shared__ float Mq[kTT];
  __shared__ float E[kTT][kFB];

  float cref;
  if (causal) {
    const size_t sb = static_cast<size_t>(bh) * nseg + s;
    cref = fmaxf(cst[sb * m + f], csg[sb * m + f]);
  } else {
    cref = cst[static_cast<size_t>(bh) * m + f];
  }
  const size_t base = static_cast<size_t>(bh) * L * d;
  const size_t ub = static_cast<size_t>(bh) * L;
  const int i0 = s * seg, i1 = min(L, i0 + seg);
  const float* wrow = W + static_cast<size_t>(f) * d;
  constexpr int kAcc = (kFB * (kMaxD + 1) + kThreads - 1) / kThreads;
  float acc[kAcc];
#pragma unroll
  for (int u = 0; u < kAcc; ++u) acc[u] = 0.f;
  const int nent = nfb * ncol;
  for (int it = i0; it < i1; it += kTT) {
    __syncthreads();
    load_rows(Q, base, it, i1, d, Qt);
    for (int p = t; p < kTT * ncol; p += kThreads) {
      const int i = p / ncol, c = p - i * ncol;
      Ut[i][c] = (it + i < i1) ? Ucat[(ub + it + i) * ncol + c] : 0.f;
    }
    if (t < kTT) Mq[t] = (it + t < i1) ? Mst[ub + it + t] : 0.f;
    __syncthreads();
    E[jj][r] = (rv && it + jj < i1) ? feat(dot_w(wrow, Qt[jj], d) + cref - Mq[jj], relu) : 0.f;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kAcc; ++u) {
      const int e = t + u * kThreads;
      if (e < nent) {
        const int rr = e / ncol, c = e - rr * ncol;
        float a = acc[u];
        for (int i = 0; i < kTT; ++i) a = fmaf(E[i][rr], Ut[i][c], a);
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
      Gst[(sb * m + fb * kFB + rr) * ncol + c] = acc[u];
    }
  }
}

// ---------------------------------------------------------------------------
// Combine the segments' query states.  Bidirectional: the total, in segment
// order.  Causal: in place, the exclusive suffix over later segments, each
// carried down to the earlier segment's references.
// grid (ceil(m*(d+1)/256), BH).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void gb_gcombine(float* __restrict__ Gst,
                                                        const float* __restrict__ cst,
                                                        const float* __restrict__ csg,
                                                        float* __restrict__ Gfin, int nseg, int m,
                                                        int d, int causal) {
  const int bh = blockIdx.y;
  const int ncol = d + 1;
  const int e = blockIdx.x * kThreads + threadIdx.x;
  if (e >= m * ncol) return;
  const int r = e / ncol;
  const size_t gb = static_cast<size_t>(bh) * nseg * m * ncol + e;    // + s*m*ncol
  if (!causal) {
    float acc = 0.f;
    for (int s = 0; s < nseg; ++s) acc += Gst[gb + static_cast<size_t>(s) * m * ncol];
    Gfin[static_cast<size_t>(bh) * m * ncol + e] = acc;
    return;
  }
  const size_t cb = static_cast<size_t>(bh) * nseg * m + r;            // + s*m
  auto cstar = [&](int s) {
    return fmaxf(cst[cb + static_cast<size_t>(s) * m], csg[cb + static_cast<size_t>(s) * m]);
  };
  float run = 0.f;   // suffix of the segments after s, at c*(s)
  float cs = cstar(nseg - 1);
  for (int s = nseg - 1; s >= 0; --s) {
    const size_t gi = gb + static_cast<size_t>(s) * m * ncol;
    const float gs = Gst[gi];
    Gst[gi] = run;
    if (s > 0) {
      const float cprev = cstar(s - 1);
      run = (run + gs) * expf(cprev - cs);
      cs = cprev;
    }
  }
}

// ---------------------------------------------------------------------------
// Key side.  grid (ceil(L/kTT), BH).  H = G . [v | 1] (causal: the suffix
// state plus the masked term over the segment's later queries), dv = K~ G,
// dk = R W - 2 knorm (sum_r R) k.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(kThreads) void gb_key(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const float* __restrict__ W, const float* __restrict__ Ucat, const float* __restrict__ Mst,
    const float* __restrict__ Gs, const float* __restrict__ cst, const float* __restrict__ csg,
    T* __restrict__ dK, T* __restrict__ dV, int L, int d, int m, int seg, int nseg, int causal,
    float knorm, int relu) {
  const int tile = blockIdx.x, bh = blockIdx.y;
  const int t = threadIdx.x;
  const int j0 = tile * kTT;
  const int ncol = d + 1;
  __shared__ float Ke[kTT][kMaxM];   // K~, then R
  __shared__ float Qe[kTT][kMaxM];   // Q~ of the masked term
  __shared__ float Hk[kTT][kMaxM];   // H = G . [v | 1]
  __shared__ float Kt[kTT][kMaxD + 1];
  __shared__ float Vt[kTT][kMaxD + 1];   // [V | 1]
  __shared__ float Qt[kTT][kMaxD + 1];
  __shared__ float Ut[kTT][kMaxD + 1];
  __shared__ float cstar[kMaxM];
  __shared__ float negc[kMaxM];
  __shared__ float nrm[kTT];
  __shared__ float Mq[kTT];
  __shared__ float red[kTT];
  __shared__ float Cm[kTT][kTT];   // Ucat_i . [v_j | 1], as [j][i]
  __shared__ float Bm[kTT][kTT];   // K~_j . Q~_i, as [j][i]

  const size_t base = static_cast<size_t>(bh) * L * d;
  const size_t ub = static_cast<size_t>(bh) * L;
  const int s = causal ? (j0 / seg) : 0;
  const float* G = Gs + (causal ? (static_cast<size_t>(bh) * nseg + s) : static_cast<size_t>(bh)) *
                            m * ncol;
  segment_refs(cst, csg, bh, s, m, nseg, causal, cstar, nullptr);
  load_rows(K, base, j0, L, d, Kt);
  load_vcat(V, base, j0, L, d, Vt);
  __syncthreads();
  for (int r = t; r < m; r += kThreads) negc[r] = -cstar[r];
  norm_terms(Kt, d, knorm, nrm);
  __syncthreads();
  features_of(W, Kt, d, m, negc, nrm, kTT, relu, Ke);
  __syncthreads();

  // H = G . [v | 1] per (token, feature); dv = K~ G[:, 0:d] per (token, column).
  for (int p = t; p < kTT * m; p += kThreads) {
    const int j = p / m, r = p - j * m;
    const float* g = G + static_cast<size_t>(r) * ncol;
    float a = 0.f;
    for (int c = 0; c < ncol; ++c) a = fmaf(g[c], Vt[j][c], a);
    Hk[j][r] = a;
  }
  float dv[kTc];
#pragma unroll
  for (int u = 0; u < kTc; ++u) {
    dv[u] = 0.f;
    const int p = t + u * kThreads;
    if (p < kTT * d) {
      const int j = p / d, c = p - j * d;
      float a = 0.f;
      for (int r = 0; r < m; ++r) a = fmaf(Ke[j][r], G[static_cast<size_t>(r) * ncol + c], a);
      dv[u] = a;
    }
  }

  if (causal) {
    // Masked term over the segment's queries i >= j.
    const int ie = min(L, (s + 1) * seg);
    for (int ic = j0; ic < ie; ic += kTT) {
      __syncthreads();
      load_rows(Q, base, ic, ie, d, Qt);
      for (int p = t; p < kTT * ncol; p += kThreads) {
        const int i = p / ncol, c = p - i * ncol;
        Ut[i][c] = (ic + i < ie) ? Ucat[(ub + ic + i) * ncol + c] : 0.f;
      }
      if (t < kTT) Mq[t] = (ic + t < ie) ? Mst[ub + ic + t] : 0.f;
      __syncthreads();
      features_of(W, Qt, d, m, cstar, Mq, min(kTT, ie - ic), relu, Qe);
      __syncthreads();
      auto keep = [&](int j, int i) { return ic + i >= j0 + j && ic + i < ie && j0 + j < L; };
      pair_dots<kMaxD + 1>(Vt, Ut, ncol, keep, Cm);
      __syncthreads();
      pair_dots<kMaxM>(Ke, Qe, m, keep, Bm);
      __syncthreads();
      for (int p = t; p < kTT * m; p += kThreads) {
        const int j = p / m, r = p - j * m;
        float a = Hk[j][r];
        for (int i = 0; i < kTT; ++i) a = fmaf(Qe[i][r], Cm[j][i], a);
        Hk[j][r] = a;
      }
#pragma unroll
      for (int u = 0; u < kTc; ++u) {
        const int p = t + u * kThreads;
        if (p < kTT * d) {
          const int j = p / d, c = p - j * d;
          float a = dv[u];
          for (int i = 0; i < kTT; ++i) a = fmaf(Bm[j][i], Ut[i][c], a);
          dv[u] = a;
        }
      }
    }
  }
  __syncthreads();
  // R = K~ H (ReLU: the gate of the key's projection), in place of K~.
  for (int p = t; p < kTT * m; p += kThreads) {
    const int j = p / m, r = p - j * m;
    const float k = Ke[j][r];
    Ke[j][r] = relu ? (k > 0.f ? Hk[j][r] : 0.f) : k * Hk[j][r];
  }
  __syncthreads();
  row_sums(Ke, m, red);
  __syncthreads();
  const float ck = 2.f * knorm;
  for (int p = t; p < kTT * d; p += kThreads) {
    const int j = p / d, a = p - j * d;
    float g = 0.f;
    for (int r = 0; r < m; ++r) g = fmaf(Ke[j][r], W[static_cast<size_t>(r) * d + a], g);
    g = fmaf(-ck * red[j], Kt[j][a], g);
    if (j0 + j < L) store_x(dK, base + static_cast<size_t>(j0 + j) * d + a, g);
  }
#pragma unroll
  for (int u = 0; u < kTc; ++u) {
    const int p = t + u * kThreads;
    if (p < kTT * d) {
      const int j = p / d, c = p - j * d;
      if (j0 + j < L) store_x(dV, base + static_cast<size_t>(j0 + j) * d + c, dv[u]);
    }
  }
}

template <typename T>
hipError_t backward_t(const Plan& p, const BwdPlan& b, const T* Q, const T* K, const T* V,
                      const float* W, const T* dO, T* dQ, T* dK, T* dV, char* ws,
                      hipStream_t st) {
  hipError_t e = generic_key_state(p, K, V, W, ws, st);
  if (e != hipSuccess) return e;
  float* Tst = reinterpret_cast<float*>(ws + p.off_T);
  float* cseg = reinterpret_cast<float*>(ws + p.off_cseg);
  float* cP = reinterpret_cast<float*>(ws + p.off_cP);
  float* KV = reinterpret_cast<float*>(ws + p.off_KV);
  float* cfin = reinterpret_cast<float*>(ws + p.off_cfin);
  float* U = reinterpret_cast<float*>(ws + b.off_U);
  float* M = reinterpret_cast<float*>(ws + b.off_M);
  float* Gst = reinterpret_cast<float*>(ws + b.off_G);
  float* Gfin = reinterpret_cast<float*>(ws + b.off_Gfin);
  const float* cst = p.causal ? cP : cfin;
  const float* csg = p.causal ? cseg : nullptr;
  const dim3 gt((p.L + kTT - 1) / kTT, p.BH);
  timing_before(st);
  gb_query<T><<<gt, kThreads, 0, st>>>(Q, K, V, dO, W, p.causal ? Tst : KV, cst, csg, U, M, dQ,
                                       p.L, p.d, p.m, p.seg, p.nseg, p.causal, p.knorm, p.relu);
  e = hipGetLastError();
  timing_after(st, "gb_query");
  if (e != hipSuccess) return e;
  timing_before(st);
  gb_gstate<T><<<dim3(p.nseg, (p.m + kFB - 1) / kFB, p.BH), kThreads, 0, st>>>(
      Q, W, U, M, cst, csg, Gst, p.L, p.d, p.m, p.seg, p.nseg, p.causal, p.relu);
  e = hipGetLastError();
  timing_after(st, "gb_gstate");
  if (e != hipSuccess) return e;
  const int nent = p.m * (p.d + 1);
  timing_before(st);
  gb_gcombine<<<dim3((nent + kThreads - 1) / kThreads, p.BH), kThreads, 0, st>>>(
      Gst, cst, csg, Gfin, p.nseg, p.m, p.d, p.causal);
  e = hipGetLastError();
  timing_after(st, "gb_gcombine");
  if (e != hipSuccess) return e;
  timing_before(st);
  gb_key<T><<<gt, kThreads, 0, st>>>(Q, K, V, W, U, M, p.causal ? Gst : Gfin, cst, csg, dK, dV,
                                     p.L, p.d, p.m, p.seg, p.nseg, p.causal, p.knorm, p.relu);
  e = hipGetLastError();
  timing_after(st, "gb_key");
  return e;
}

}  // namespace

hipError_t generic_backward(const Plan& p, const BwdPlan& b, const void* Q, const void* K,
                            const void* V, const float* W, const void* dO, void* dQ, void* dK,
                            void* dV, void* ws, hipStream_t stream) {
  char* w = static_cast<char*>(ws);
  if (p.dtype == FAVOR_F32)
    return backward_t<float>(p, b, static_cast<const float*>(Q), static_cast<const float*>(K),
                             static_cast<const float*>(V), W, static_cast<const float*>(dO),
                             static_cast<float*>(dQ), static_cast<float*>(dK),
                             static_cast<float*>(dV), w, stream);
  return backward_t<uint16_t>(p, b, static_cast<const uint16_t*>(Q),
                              static_cast<const uint16_t*>(K), static_cast<const uint16_t*>(V), W,
                              static_cast<const uint16_t*>(dO), static_cast<uint16_t*>(dQ),
                              static_cast<uint16_t*>(dK), static_cast<uint16_t*>(dV), w, stream);
}

}  // namespace favor
