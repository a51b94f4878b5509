// C-ABI layer of libfavor.so: argument validation (pure host code, before any
// HIP call), workspace planning, path selection and error mapping.
#include <cstdint>
#include <cstring>

#include <hip/hip_runtime.h>

#include "favor.h"
#include "favor_internal.h"

namespace favor {
namespace {

thread_local int g_last_hip_error = 0;

constexpr size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

bool is_aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Shape checks shared by every entry point.
int check_shape(int32_t B, int32_t H, int32_t L, int32_t d, int32_t m, int32_t dtype) {
  if (B < 1 || H < 1 || L < 1) return FAVOR_ERR_SHAPE;
  if (!(d == 16 || d == 32 || d == 64 || d == 128)) return FAVOR_ERR_UNSUPPORTED;
  if (m < 16 || m > 1024 || (m % 16) != 0) return FAVOR_ERR_UNSUPPORTED;
  if (dtype != FAVOR_F32 && dtype != FAVOR_BF16) return FAVOR_ERR_UNSUPPORTED;
  const int64_t n = static_cast<int64_t>(B) * H * L * d;
  if (n >= (static_cast<int64_t>(1) << 31)) return FAVOR_ERR_SHAPE;
  const int64_t nf = static_cast<int64_t>(B) * H * L * m;  // feature-map output size
  if (nf >= (static_cast<int64_t>(1) << 40)) return FAVOR_ERR_SHAPE;
  return FAVOR_OK;
}

int fail_hip(hipError_t e) { return record_hip_error(e); }

// Norm coefficient of the features of an attention kernel (0 for the ReLU
// features, which have no norm term), or a negative value for an unknown
// kernel.
float norm_coefficient(int32_t attn_kernel) {
  switch (attn_kernel) {
    case FAVOR_SOFTMAX: return 0.5f;
    case FAVOR_GAUSSIAN: return 1.0f;
    case FAVOR_RELU: return 0.0f;
    default: return -1.0f;
  }
}

int backward(int32_t B, int32_t H, int32_t L, int32_t d, int32_t m, int32_t dtype, int32_t causal,
             int32_t attn_kernel, const void* Q, const void* K, const void* V, const float* W,
             const void* dO, void* dQ, void* dK, void* dV, void* ws, size_t ws_bytes,
             void* stream) {
  const int status = check_shape(B, H, L, d, m, dtype);
  if (status != FAVOR_OK) return status;
  const float knorm = norm_coefficient(attn_kernel);
  if (knorm < 0.f) return FAVOR_ERR_UNSUPPORTED;
  if (!Q || !K || !V || !W || !dO || !dQ || !dK || !dV || !ws) return FAVOR_ERR_NULL;
  for (const void* x : {Q, K, V, static_cast<const void*>(W), dO,
                        static_cast<const void*>(dQ), static_cast<const void*>(dK),
                        static_cast<const void*>(dV)})
    if (!is_aligned(x, 16)) return FAVOR_ERR_ALIGN;
  if (!is_aligned(ws, 256)) return FAVOR_ERR_ALIGN;
  Plan p;
  BwdPlan b;
  make_bwd_plan(B, H, L, d, m, dtype, causal, &p, &b);
  if (ws_bytes < b.bytes) return FAVOR_ERR_WORKSPACE;
  p.knorm = knorm;
  p.relu = attn_kernel == FAVOR_RELU ? 1 : 0;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const hipError_t e = b.path == kPathMfma
                           ? mfma_backward(p, b, Q, K, V, W, dO, dQ, dK, dV, ws, st)
                           : generic_backward(p, b, Q, K, V, W, dO, dQ, dK, dV, ws, st);
  if (e != hipSuccess) return fail_hip(e);
  return FAVOR_OK;
}

// Prefill segments: 64 tokens (the masked in-segment term of the generic
// causal kernels costs O(segment) per token).
constexpr int32_t kPrefillSeg = 64;

// A prefill on the matrix cores: the causal forward's plan (a carried state
// enters as the first segment's carry), then the bidirectional key partials
// (the final state is the carried state plus the sum over every key) at the
// next 256-byte boundary.  False when the shape is not covered (the generic
// kernels run it).
bool mfma_prefill_plans(int32_t B, int32_t H, int32_t L, int32_t d, int32_t m, int32_t dtype,
                        Plan* pc, Plan* pb, size_t* off_b, size_t* bytes) {
  if (!mfma_causal_supported(d, m, dtype) || !mfma_bidir_supported(d, m, dtype) || d != 64 ||
      m > 256)
    return false;
  make_plan(B, H, L, d, m, dtype, 1, pc);
  make_plan(B, H, L, d, m, dtype, 0, pb);
  if (pc->path != kPathMfma || pb->path != kPathMfma) return false;
  *off_b = align256(pc->bytes);
  *bytes = *off_b + pb->bytes;
  return true;
}

// Incremental causal state: shape checks shared by its entry points.
int check_state(int32_t B, int32_t H, int32_t d, int32_t m, int32_t attn_kernel) {
  const int st = check_shape(B, H, 1, d, m, FAVOR_F32);
  if (st != FAVOR_OK) return st;
  return norm_coefficient(attn_kernel) < 0.f ? FAVOR_ERR_UNSUPPORTED : FAVOR_OK;
}

}  // namespace

int forward_call(int32_t B, int32_t H, int32_t L, int32_t d, int32_t m, int32_t dtype, int32_t causal,
            int32_t attn_kernel, const void* Q, const void* K, const void* V, const float* W,
            void* O, void* ws, size_t ws_bytes, void* stream) {
  const int status = check_shape(B, H, L, d, m, dtype);
  if (status != FAVOR_OK) return status;
  const float knorm = norm_coefficient(attn_kernel);
  if (knorm < 0.f) return FAVOR_ERR_UNSUPPORTED;
  if (!Q || !K || !V || !W || !O || !ws) return FAVOR_ERR_NULL;
  if (!is_aligned(Q, 16) || !is_aligned(K, 16) || !is_aligned(V, 16) || !is_aligned(W, 16) ||
      !is_aligned(O, 16) || !is_aligned(ws, 256))
    return FAVOR_ERR_ALIGN;
  // The ReLU features take the three-kernel matrix-core path where the
  // persistent kernel would otherwise run: its ReLU form needs more
  // registers than a wave has in the key loop.
  Plan p;
  make_plan(B, H, L, d, m, dtype, causal, &p, true, attn_kernel != FAVOR_RELU);
  if (ws_bytes < p.bytes) return FAVOR_ERR_WORKSPACE;
  p.knorm = knorm;
  p.relu = attn_kernel == FAVOR_RELU ? 1 : 0;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (p.path == kPathFused)
    e = fused_bidir_forward(p, Q, K, V, W, O, ws, st);
  else if (p.path == kPathMfma)
    e = causal ? mfma_causal_forward(p, Q, K, V, W, O, ws, st)
               : mfma_bidir_forward(p, Q, K, V, W, O, ws, st);
  else
    e = generic_forward(p, Q, K, V, W, O, ws, st);
  if (e != hipSuccess) return fail_hip(e);
  return FAVOR_OK;
}


void make_generic_plan(Plan* p);

void make_generic_only_plan(int32_t B, int32_t H, int32_t L, int32_t d, int32_t m, int32_t dtype,
                            int32_t causal, int32_t seg, Plan* p) {
  std::memset(p, 0, sizeof(*p));
  p->B = B; p->H = H; p->L = L; p->d = d; p->m = m; p->dtype = dtype; p->causal = causal;
  p->BH = B * H;
  p->seg = seg;
  make_generic_plan(p);
}

int record_hip_error(hipError_t e) {
  g_last_hip_error = static_cast<int>(e);
  return FAVOR_ERR_HIP;
}

void make_plan(int32_t B, int32_t H, int32_t L, int32_t d, int32_t m, int32_t dtype,
               int32_t causal, Plan* p, bool forward, bool allow_fused) {
  std::memset(p, 0, sizeof(*p));
  p->B = B; p->H = H; p->L = L; p->d = d; p->m = m; p->dtype = dtype; p->causal = causal;
  p->BH = B * H;
  const size_t ncol = static_cast<size_t>(d) + 1;
  const size_t BH = static_cast<size_t>(p->BH);
  size_t off = 0;
  if (forward && !causal && allow_fused && fused_bidir_supported(B, H, L, d, m, dtype)) {
    p->path = kPathFused;
    fused_bidir_layout(p, kPlanCUs);
    const size_t ns = static_cast<size_t>(p->nseg);
    p->off_cP = off;   off = align256(off + static_cast<size_t>(m) * (d + 8) * 2);
    p->off_T = off;    off = align256(off + BH * ns * ncol * m * sizeof(float));
    p->off_cseg = off; off = align256(off + BH * ns * m * sizeof(float));
    p->off_KV = off;
    p->off_cfin = off;
    p->off_ctrl = off; off = align256(off + fused_ctrl_words(p->BH) * 4);
    p->bytes = off;
    return;
  }
  if (!causal && mfma_bidir_supported(d, m, dtype)) {
    p->path = kPathMfma;
    // Splits: about 512 key-side token groups in total (one or two per
    // work-group, times the feature blocks), at least 128 tokens per group.
    const int tg = mfma_bidir_token_groups(d, m);
    const int nfb = mfma_bidir_feature_blocks(d, m);
    int ns = (512 / (tg * nfb) + p->BH - 1) / p->BH;
    const int maxs = (L + 128 * tg - 1) / (128 * tg);
    ns = ns < 1 ? 1 : (ns > maxs ? maxs : ns);
    p->seg = ((L + ns - 1) / ns + 31) / 32 * 32;
    p->nseg = (L + p->seg - 1) / p->seg;
    // Query blocks: about 512 work-groups of 4 waves (qapply) or 256, one
    // per compute unit (qstream); a multiple of 64 tokens (qapply) or of
    // qstream's lockstep round.
    const bool stream = mfma_bidir_streams_queries(d, m);
    const int64_t nwg = stream ? 256 : mfma_bidir_query_workgroups();
    const int64_t unit = stream ? mfma_bidir_stream_round() : 64;
    const int64_t want = (static_cast<int64_t>(L) * p->BH + nwg - 1) / nwg;
    int64_t qb = (want + unit - 1) / unit * unit;
    if (qb < 256) qb = stream ? unit : 256;
    p->qblk = static_cast<int32_t>(qb);
    p->off_T = off;    off = align256(off + BH * p->nseg * ncol * m * sizeof(float));
    p->off_cseg = off; off = align256(off + BH * p->nseg * m * sizeof(float));
    p->off_cP = off;   off = align256(off + static_cast<size_t>(m) * (d + 8) * 2);
    p->off_KV = off;   off = align256(off + BH * (d + 16) * (static_cast<size_t>(m) + 8) * 2);
    p->off_cfin = off; off = align256(off + BH * m * sizeof(float));
    p->bytes = off;
    return;
  }
  if (causal && mfma_causal_supported(d, m, dtype)) {
    p->path = kPathMfma;
    // Segments: about 512 scan work-groups in total, a multiple of the
    // 32-token chunk, at least 256 tokens each.
    int ns = (512 + p->BH - 1) / p->BH;
    const int maxs = (L + 255) / 256;
    ns = ns < 1 ? 1 : (ns > maxs ? maxs : ns);
    p->seg = ((L + ns - 1) / ns + 31) / 32 * 32;
    p->nseg = (L + p->seg - 1) / p->seg;
    p->off_T = off;    off = align256(off + BH * p->nseg * ncol * m * sizeof(float));
    p->off_cseg = off; off = align256(off + BH * p->nseg * m * sizeof(float));
    p->off_cP = off;   off = align256(off + BH * p->nseg * m * sizeof(float));
    p->off_KV = off;
    p->off_cfin = off;
    p->bytes = off;
    return;
  }
  make_generic_plan(p);
}

void make_generic_plan(Plan* p) {
  const size_t ncol = static_cast<size_t>(p->d) + 1;
  const size_t BH = static_cast<size_t>(p->BH);
  const size_t m = static_cast<size_t>(p->m);
  const int32_t causal = p->causal, L = p->L;
  size_t off = 0;
  p->path = kPathGeneric;
  // Sequence splits (bidirectional) and segments (causal); a multiple of the
  // 8-token tile of the generic kernels (a caller may preset a segment length).
  // Causal segments of 64 tokens (the masked in-segment term costs O(segment)
  // per token), doubled up to 256 while the segment states would pass 512 MB.
  if (p->seg <= 0) {
    if (causal) {
      p->seg = 64;
      while (p->seg < 256 && BH * ((static_cast<size_t>(L) + p->seg - 1) / p->seg) * m * ncol *
                                     sizeof(float) > (static_cast<size_t>(512) << 20))
        p->seg *= 2;
    } else {
      p->seg = 512;
    }
  }
  p->nseg = (L + p->seg - 1) / p->seg;
  p->off_T = off;    off = align256(off + BH * p->nseg * m * ncol * sizeof(float));
  p->off_cseg = off; off = align256(off + BH * p->nseg * m * sizeof(float));
  p->off_cP = off;   off = align256(off + (causal ? BH * p->nseg * m * sizeof(float) : 0));
  p->off_KV = off;   off = align256(off + (causal ? 0 : BH * m * ncol * sizeof(float)));
  p->off_cfin = off; off = align256(off + (causal ? 0 : BH * m * sizeof(float)));
  p->bytes = off;
}

void make_bwd_plan(int32_t B, int32_t H, int32_t L, int32_t d, int32_t m, int32_t dtype,
                   int32_t causal, Plan* p, BwdPlan* b) {
  std::memset(b, 0, sizeof(*b));
  if (mfma_bwd_supported(d, m, dtype, causal)) {
    make_plan(B, H, L, d, m, dtype, causal, p);   // the forward's key partials
    b->path = kPathMfma;
    const size_t BH = static_cast<size_t>(p->BH), mm = static_cast<size_t>(m);
    if (causal) {
      // The causal forward's segments; per query (L_i, p_i), and per
      // segment a query state of 66 rows.
      size_t off = p->bytes;
      b->off_ru = off; off = align256(off + BH * static_cast<size_t>(L) * 2 * 4);
      b->off_G = off;  off = align256(off + BH * p->nseg * 66 * mm * 4);
      b->bytes = off;
      return;
    }
    // Query blocks: about 512 work-groups in total, a multiple of 64 tokens.
    const int want = (512 + p->BH - 1) / p->BH;
    const int ntile = (L + 63) / 64;
    int nqb = want < ntile ? want : ntile;
    if (nqb < 1) nqb = 1;
    b->qblk = ((ntile + nqb - 1) / nqb) * 64;
    b->qblk = (b->qblk + 127) / 128 * 128;   // whole 128-query steps
    b->nqb = (L + b->qblk - 1) / b->qblk;
    // Key blocks: about 512 work-groups, a multiple of 128 keys.
    const int nstep = (L + 127) / 128;
    int nkb = want < nstep ? want : nstep;
    if (nkb < 1) nkb = 1;
    b->kblk = ((nstep + nkb - 1) / nkb) * 128;
    b->nkb = (L + b->kblk - 1) / b->kblk;
    size_t off = p->bytes;
    b->off_W16 = off; off = align256(off + mm * 64 * 2);
    b->off_WT = off;  off = align256(off + mm * 64 * 2);
    b->off_KzT = off; off = align256(off + BH * 2 * 80 * mm * 2);
    b->off_KzF = off; off = align256(off + BH * 2 * mm * 64 * 2);
    b->off_zf = off;  off = align256(off + BH * mm * 4);
    b->off_cf = off;  off = align256(off + BH * mm * 4);
    b->off_G = off;   off = align256(off + BH * b->nqb * mm * 65 * 4);
    b->off_GF = off;  off = align256(off + BH * 2 * mm * 64 * 2);
    b->off_GT = off;  off = align256(off + BH * mm * 64 * 2);
    b->off_Gz = off;  off = align256(off + BH * mm * 4);
    b->off_ru = off;  off = align256(off + BH * static_cast<size_t>(L) * 2 * 4);
    b->bytes = off;
    return;
  }
  b->path = kPathGeneric;
  // Causal: 64-token segments (the masked in-segment terms of the backward
  // cost O(segment) per token; the forward's 256 would quadruple them).
  make_generic_only_plan(B, H, L, d, m, dtype, causal, causal ? 64 : 0, p);
  const size_t ncol = static_cast<size_t>(d) + 1;
  const size_t BH = static_cast<size_t>(p->BH);
  size_t off = p->bytes;
  b->off_U = off;    off = align256(off + BH * L * ncol * sizeof(float));
  b->off_M = off;    off = align256(off + BH * L * sizeof(float));
  b->off_G = off;    off = align256(off + BH * p->nseg * m * ncol * sizeof(float));
  b->off_Gfin = off; off = align256(off + (causal ? 0 : BH * m * ncol * sizeof(float)));
  b->bytes = off;
}

}  // namespace favor

extern "C" {

int favor_workspace_bytes(int32_t B, int32_t H, int32_t L, int32_t d, int32_t m, int32_t dtype,
                          int32_t causal, size_t* bytes) {
  const int st = favor::check_shape(B, H, L, d, m, dtype);
  if (st != FAVOR_OK) return st;
  if (!bytes) return FAVOR_ERR_NULL;
  favor::Plan p;
  favor::make_plan(B, H, L, d, m, dtype, causal ? 1 : 0, &p, true);
  *bytes = p.bytes;
  if (p.path == favor::kPathFused) {
    // enough for the path the ReLU features take as well
    favor::make_plan(B, H, L, d, m, dtype, causal ? 1 : 0, &p, true, false);
    if (p.bytes > *bytes) *bytes = p.bytes;
  }
  return FAVOR_OK;
}

int favor_plan_describe(int32_t B, int32_t H, int32_t L, int32_t d, int32_t m, int32_t dtype,
                        int32_t causal, int32_t* path, int32_t* nseg, int32_t* seg) {
  const int st = favor::check_shape(B, H, L, d, m, dtype);
  if (st != FAVOR_OK) return st;
  if (!path || !nseg || !seg) return FAVOR_ERR_NULL;
  favor::Plan p;
  favor::make_plan(B, H, L, d, m, dtype, causal ? 1 : 0, &p, true);
  *path = p.path;
  *nseg = p.nseg;
  *seg = p.seg;
  return FAVOR_OK;
}

int favor_fwd_bidir(int32_t B, int32_t H, int32_t L, int32_t d, int32_t m, int32_t dtype,
                    const void* Q, const void* K, const void* V, const float* W, void* O,
                    void* workspace, size_t workspace_bytes, void* stream) {
  return favor::forward_call(B, H, L, d, m, dtype, 0, FAVOR_SOFTMAX, Q, K, V, W, O, workspace,
                        workspace_bytes, stream);
}

int favor_fwd_causal(int32_t B, int32_t H, int32_t L, int32_t d, int32_t m, int32_t dtype,
                     const void* Q, const void* K, const void* V, const float* W, void* O,
                     void* workspace, size_t workspace_bytes, void* stream) {
  return favor::forward_call(B, H, L, d, m, dtype, 1, FAVOR_SOFTMAX, Q, K, V, W, O, workspace,
                        workspace_bytes, stream);
}

int favor_fwd_attn(int32_t B, int32_t H, int32_t L, int32_t d, int32_t m, int32_t dtype,
                   int32_t causal, int32_t attn_kernel, const void* Q, const void* K,
                   const void* V, const float* W, void* O, void* workspace,
                   size_t workspace_bytes, void* stream) {
  return favor::forward_call(B, H, L, d, m, dtype, causal ? 1 : 0, attn_kernel, Q, K, V, W, O,
                        workspace, workspace_bytes, stream);
}

int favor_bwd_workspace_bytes(int32_t B, int32_t H, int32_t L, int32_t d, int32_t m,
                              int32_t dtype, int32_t causal, size_t* bytes) {
  const int st = favor::check_shape(B, H, L, d, m, dtype);
  if (st != FAVOR_OK) return st;
  if (!bytes) return FAVOR_ERR_NULL;
  favor::Plan p;
  favor::BwdPlan b;
  favor::make_bwd_plan(B, H, L, d, m, dtype, causal ? 1 : 0, &p, &b);
  *bytes = b.bytes;
  return FAVOR_OK;
}

int favor_bwd_attn(int32_t B, int32_t H, int32_t L, int32_t d, int32_t m, int32_t dtype,
                   int32_t causal, int32_t attn_kernel, const void* Q, const void* K,
                   const void* V, const float* W, const void* dO, void* dQ, void* dK, void* dV,
                   void* workspace, size_t workspace_bytes, void* stream) {
  return favor::backward(B, H, L, d, m, dtype, causal ? 1 : 0, attn_kernel, Q, K, V, W, dO, dQ,
                         dK, dV, workspace, workspace_bytes, stream);
}

int favor_state_bytes(int32_t B, int32_t H, int32_t d, int32_t m, size_t* bytes) {
  const int st = favor::check_state(B, H, d, m, FAVOR_SOFTMAX);
  if (st != FAVOR_OK) return st;
  if (!bytes) return FAVOR_ERR_NULL;
  *bytes = static_cast<size_t>(B) * H * m * (d + 4) * sizeof(float);
  return FAVOR_OK;
}

int favor_state_reset(int32_t B, int32_t H, int32_t d, int32_t m, float* state, void* stream) {
  const int st = favor::check_state(B, H, d, m, FAVOR_SOFTMAX);
  if (st != FAVOR_OK) return st;
  if (!state) return FAVOR_ERR_NULL;
  if (!favor::is_aligned(state, 16)) return FAVOR_ERR_ALIGN;
  const hipError_t e = favor::generic_state_reset(B * H, d, m, state,
                                                  static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return favor::fail_hip(e);
  return FAVOR_OK;
}

int favor_prefill_workspace_bytes(int32_t B, int32_t H, int32_t L, int32_t d, int32_t m,
                                  int32_t dtype, size_t* bytes) {
  const int st = favor::check_shape(B, H, L, d, m, dtype);
  if (st != FAVOR_OK) return st;
  if (!bytes) return FAVOR_ERR_NULL;
  favor::Plan p;
  favor::make_generic_only_plan(B, H, L, d, m, dtype, 1, favor::kPrefillSeg, &p);
  size_t need = p.bytes;
  favor::Plan pc, pb;
  size_t off_b = 0, mb = 0;
  if (favor::mfma_prefill_plans(B, H, L, d, m, dtype, &pc, &pb, &off_b, &mb) && mb > need)
    need = mb;
  *bytes = need;
  return FAVOR_OK;
}

int favor_prefill(int32_t B, int32_t H, int32_t L, int32_t d, int32_t m, int32_t dtype,
                  int32_t attn_kernel, const void* Q, const void* K, const void* V,
                  const float* W, void* O, const float* state_in, float* state_out,
                  void* workspace, size_t workspace_bytes, void* stream) {
  const int st = favor::check_shape(B, H, L, d, m, dtype);
  if (st != FAVOR_OK) return st;
  const float knorm = favor::norm_coefficient(attn_kernel);
  if (knorm < 0.f) return FAVOR_ERR_UNSUPPORTED;
  if (!Q || !K || !V || !W || !O || !workspace) return FAVOR_ERR_NULL;
  for (const void* x : {Q, K, V, static_cast<const void*>(W), static_cast<const void*>(O),
                        static_cast<const void*>(state_in), static_cast<const void*>(state_out)})
    if (x && !favor::is_aligned(x, 16)) return FAVOR_ERR_ALIGN;
  if (!favor::is_aligned(workspace, 256)) return FAVOR_ERR_ALIGN;
  if (state_in && state_out) {
    size_t sb = 0;
    favor_state_bytes(B, H, d, m, &sb);
    const auto* a = reinterpret_cast<const char*>(state_in);
    const auto* b = reinterpret_cast<const char*>(state_out);
    if (a < b + sb && b < a + sb) return FAVOR_ERR_ALIAS;
  }
  favor::Plan p;
  favor::make_generic_only_plan(B, H, L, d, m, dtype, 1, favor::kPrefillSeg, &p);
  size_t need = 0;
  if (favor_prefill_workspace_bytes(B, H, L, d, m, dtype, &need) != FAVOR_OK) return FAVOR_ERR_SHAPE;
  if (workspace_bytes < need) return FAVOR_ERR_WORKSPACE;
  p.knorm = knorm;
  p.relu = attn_kernel == FAVOR_RELU ? 1 : 0;
  favor::Plan pc, pb;
  size_t off_b = 0, mb = 0;
  if (favor::mfma_prefill_plans(B, H, L, d, m, dtype, &pc, &pb, &off_b, &mb)) {
    // On the matrix cores: the causal forward from the carried state, then
    // (if the state is wanted) the carried state plus the sum over every key.
    pc.knorm = pb.knorm = knorm;
    pc.relu = pb.relu = p.relu;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    bool exported = false;
    hipError_t e = favor::mfma_causal_forward(pc, Q, K, V, W, O, workspace, st, state_in,
                                              state_out, &exported);
    if (e == hipSuccess && state_out && !exported) {
      char* wb = static_cast<char*>(workspace) + off_b;
      e = favor::mfma_bidir_key_partials(pb, K, V, W, wb, st);
      if (e == hipSuccess) e = favor::mfma_state_export(pb, wb, state_in, state_out, st);
    }
    if (e != hipSuccess) return favor::fail_hip(e);
    return FAVOR_OK;
  }
  const hipError_t e = favor::generic_prefill(p, Q, K, V, W, O, state_in, state_out, workspace,
                                              static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return favor::fail_hip(e);
  return FAVOR_OK;
}

int favor_decode(int32_t B, int32_t H, int32_t d, int32_t m, int32_t dtype, int32_t attn_kernel,
                 const void* q, const void* k, const void* v, const float* W, void* o,
                 float* state, void* stream) {
  int st = favor::check_shape(B, H, 1, d, m, dtype);
  if (st != FAVOR_OK) return st;
  const float knorm = favor::norm_coefficient(attn_kernel);
  if (knorm < 0.f) return FAVOR_ERR_UNSUPPORTED;
  if (!q || !k || !v || !W || !o || !state) return FAVOR_ERR_NULL;
  for (const void* x : {q, k, v, static_cast<const void*>(W), static_cast<const void*>(o),
                        static_cast<const void*>(state)})
    if (!favor::is_aligned(x, 16)) return FAVOR_ERR_ALIGN;
  const hipError_t e = favor::generic_decode(B * H, d, m, dtype, knorm,
                                             attn_kernel == FAVOR_RELU ? 1 : 0, q, k, v, W, o,
                                             state, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return favor::fail_hip(e);
  return FAVOR_OK;
}

int favor_draw_projection_device(uint64_t seed, int32_t m, int32_t d, float* W, void* stream) {
  if (!W) return FAVOR_ERR_NULL;
  if (m < 1 || d < 1 || d > 128) return FAVOR_ERR_SHAPE;
  if (!favor::is_aligned(W, 16)) return FAVOR_ERR_ALIGN;
  const hipError_t e = favor::device_draw(seed, m, d, W, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return favor::fail_hip(e);
  return FAVOR_OK;
}

int favor_feature_map_attn(int32_t B, int32_t H, int32_t L, int32_t d, int32_t m, int32_t dtype,
                           int32_t attn_kernel, const void* X, const float* W, float* Xp,
                           void* stream) {
  const int st = favor::check_shape(B, H, L, d, m, dtype);
  if (st != FAVOR_OK) return st;
  const float knorm = favor::norm_coefficient(attn_kernel);
  if (knorm < 0.f) return FAVOR_ERR_UNSUPPORTED;
  if (!X || !W || !Xp) return FAVOR_ERR_NULL;
  if (!favor::is_aligned(X, 16) || !favor::is_aligned(W, 16) || !favor::is_aligned(Xp, 16))
    return FAVOR_ERR_ALIGN;
  const hipError_t e = favor::generic_feature_map(B * H, L, d, m, dtype, knorm,
                                                  attn_kernel == FAVOR_RELU ? 1 : 0, X, W, Xp,
                                                  static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return favor::fail_hip(e);
  return FAVOR_OK;
}

int favor_feature_map(int32_t B, int32_t H, int32_t L, int32_t d, int32_t m, int32_t dtype,
                      const void* X, const float* W, float* Xp, void* stream) {
  return favor_feature_map_attn(B, H, L, d, m, dtype, FAVOR_SOFTMAX, X, W, Xp, stream);
}

const char* favor_status_string(int status) {
  switch (status) {
    case FAVOR_OK: return "ok";
    case FAVOR_ERR_NULL: return "a required pointer is NULL";
    case FAVOR_ERR_SHAPE: return "invalid shape (B, H or L below 1, or tensor too large)";
    case FAVOR_ERR_UNSUPPORTED:
      return "unsupported configuration (d must be 16, 32, 64 or 128; m a multiple of 16 in "
             "[16, 1024]; dtype FAVOR_F32 or FAVOR_BF16; attention kernel FAVOR_SOFTMAX, "
             "FAVOR_GAUSSIAN or FAVOR_RELU)";
    case FAVOR_ERR_ALIGN:
      return "misaligned pointer (tensors need 16-byte, the workspace 256-byte alignment)";
    case FAVOR_ERR_WORKSPACE:
      return "workspace smaller than favor_workspace_bytes() (favor_bwd_workspace_bytes() for "
             "the backward pass)";
    case FAVOR_ERR_HIP: return "a HIP runtime call failed (see favor_last_hip_error)";
    case FAVOR_ERR_SCRATCH:
      return "favor_fwd_attn_noalloc: the shape needs more workspace than the static scratch "
             "(FAVOR_NOALLOC_SCRATCH_BYTES), or the stream is not on the current device";
    case FAVOR_ERR_ALIAS:
      return "two buffers that must be distinct overlap (favor_prefill: state_in and state_out)";
    default: return "unknown status";
  }
}

int favor_last_hip_error(void) { return favor::g_last_hip_error; }

}  // extern "C"
