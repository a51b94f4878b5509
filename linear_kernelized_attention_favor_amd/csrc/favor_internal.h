// Internal declarations shared by the C-ABI layer and the kernel files of
// libfavor.so.  Not installed; the public interface is include/favor.h.
#pragma once

#include <cstddef>
#include <cstdint>

#include <hip/hip_runtime.h>

namespace favor {

// ---------------------------------------------------------------------------
// Execution plan: which kernel path runs a shape, and the workspace layout.
// All offsets are in bytes from the workspace base and 256-byte aligned.
// ---------------------------------------------------------------------------
enum Path : int32_t {
  kPathGeneric = 0,  // fp32 FMA kernels, any supported shape and dtype
  kPathMfma = 1,     // bf16 MFMA kernels (see mfma_*_supported)
  kPathFused = 2,    // bf16 MFMA, bidirectional in one persistent kernel
};

struct Plan {
  int32_t B, H, L, d, m, dtype, causal;
  int32_t BH;
  int32_t path;
  int32_t seg;    // tokens per sequence split (bidirectional) or segment (causal)
  int32_t nseg;   // number of splits / segments per head
  int32_t qblk;   // tokens per query-side work-group (MFMA path)
  // Generic-path workspace (all fp32):
  //   T    [BH][nseg][m][d+1]  per-segment key state, then (causal) its
  //                            exclusive prefix over earlier segments
  //   cseg [BH][nseg][m]       per-feature key exponent reference of T
  //   cP   [BH][nseg][m]       reference of the exclusive prefix (causal)
  //   KV   [BH][m][d+1]        final key state (bidirectional)
  //   cfin [BH][m]             its per-feature reference
  // MFMA bidirectional path:
  //   T    [BH][nseg][d+1][m]  per-split partial state (row d = z), fp32
  //   cseg [BH][nseg][m]       per-feature references of the partials
  //   cP   [m][d+8]            W log2(e) in fp16 (query-side projection operand)
  //   KV   [BH][d+16][m+8]     combined state, bf16, query-side operand order
  //   cfin [BH][m]             combined per-feature references
  // MFMA causal path:
  //   T    [BH][nseg][d+1][m]  per-segment key state, then its exclusive
  //                            prefix over earlier segments (s >= 1), fp32
  //   cseg [BH][nseg][m]       per-feature references of the segment states
  //   cP   [BH][nseg][m]       references of the prefixes (s >= 1)
  size_t off_T, off_cseg, off_cP, off_KV, off_cfin;
  // Fused bidirectional path (path kPathFused: matrix cores, one persistent
  // kernel): cP (W' fp16 [m][d+8]), T and cseg (the splits' partial states
  // and references) as the MFMA bidirectional path, plus the work queues'
  // control block:
  //   ctrl [20 + BH] u32 words, 128 bytes apart
  size_t off_ctrl;
  size_t bytes;
  // Features (set per call): exp(w.k - knorm |k|^2) with knorm = 1/2 (softmax
  // kernel) or 1 (Gaussian kernel), or, with relu = 1, max(w.x, 0)
  // (generalized attention; knorm = 0).
  float knorm;
  int32_t relu;
};

// Fills *p for a validated shape (the C-ABI layer validates first).
// forward: the plan of a forward call (which may take the fused
// bidirectional path); other users (backward, prefill) get the
// three-kernel layout of the key partials.
void make_plan(int32_t B, int32_t H, int32_t L, int32_t d, int32_t m, int32_t dtype,
               int32_t causal, Plan* p, bool forward = false, bool allow_fused = true);
// Compute units the plans are laid out for (an MI355X has 256; the fused
// kernel's grid is the device's own count, its work queue adapts).
constexpr int kPlanCUs = 256;
// u32 words of the fused path's control block for BH heads.
inline size_t fused_ctrl_words(int32_t BH) { return 32 * (20 + static_cast<size_t>(BH)); }

// Backward pass: the generic path's key-state layout (Plan, path forced to
// kPathGeneric) followed by
//   U    [BH][L][d+1]         Ucat_i = [dO_i / den_i | -(dO_i . O_i) / den_i]
//   M    [BH][L]              the query rows' references
//   G    [BH][nseg][m][d+1]   per-segment query state sum_i Q~_ir Ucat_i, then
//                             (causal) its exclusive suffix over later segments
//   Gfin [BH][m][d+1]         bidirectional total of G
struct BwdPlan {
  int32_t path;   // kPathGeneric, or kPathMfma (bidirectional bf16, d = 64)
  size_t off_U, off_M, off_G, off_Gfin;
  // Matrix-core path (after the forward plan's key partials T, cseg):
  //   W16 [m][64] fp16 (W log2 e), WT [64][m] bf16 (W^T), KzT [BH][2][80][m]
  //   bf16 (state^T hi, lo; row 64 = z), KzF [BH][2][m][64] bf16 (state hi,
  //   lo), zf, cf [BH][m] fp32 (z and the references), G [BH][nqb][m][65]
  //   fp32 (per query block), GF [BH][2][m][64] (hi, lo), GT [BH][64][m] bf16
  //   and Gz [BH][m] fp32 (their sum).
  //   ru [BH][L][2] fp32 (1/den and u0 per query).
  size_t off_W16, off_WT, off_KzT, off_KzF, off_zf, off_cf, off_GF, off_GT, off_Gz, off_ru;
  int32_t nqb, qblk;   // query blocks per head and their length (multiple of 64)
  int32_t nkb, kblk;   // key blocks per head and their length (multiple of 128)
  size_t bytes;
};
// A generic-path plan whatever the shape (seg <= 0: the default segment length).
void make_generic_only_plan(int32_t B, int32_t H, int32_t L, int32_t d, int32_t m, int32_t dtype,
                            int32_t causal, int32_t seg, Plan* p);
void make_bwd_plan(int32_t B, int32_t H, int32_t L, int32_t d, int32_t m, int32_t dtype,
                   int32_t causal, Plan* p, BwdPlan* b);

// Generic path: enqueue the whole forward pass on `stream`.
hipError_t generic_forward(const Plan& p, const void* Q, const void* K, const void* V,
                           const float* W, void* O, void* ws, hipStream_t stream);
// Causal forward on the generic kernels carrying a state across calls:
// st_in (nullable) is the state before token 0, st_out (nullable) receives
// the state after token L-1; both fp32 [BH][m][d+4] rows [S~ | z~ | c | 0 | 0].
hipError_t generic_prefill(const Plan& p, const void* Q, const void* K, const void* V,
                           const float* W, void* O, const float* st_in, float* st_out, void* ws,
                           hipStream_t stream);
// Empty states (S~ = z~ = 0, c = -inf) for BH heads.
hipError_t generic_state_reset(int32_t BH, int32_t d, int32_t m, float* state,
                               hipStream_t stream);
// One decode step per head (q, k, v, o: [BH][d]); the state is updated in place.
hipError_t generic_decode(int32_t BH, int32_t d, int32_t m, int32_t dtype, float knorm,
                          int32_t relu, const void* q, const void* k, const void* v,
                          const float* W, void* o, float* state, hipStream_t stream);
// Its first two steps alone: the key state and references in the workspace.
hipError_t generic_key_state(const Plan& p, const void* K, const void* V, const float* W,
                             void* ws, hipStream_t stream);
// Matrix-core backward (bf16, d = 64, m in {64, 128, 192, 256}; both forms).
bool mfma_bwd_supported(int32_t d, int32_t m, int32_t dtype, int32_t causal);
hipError_t mfma_backward(const Plan& p, const BwdPlan& b, const void* Q, const void* K,
                         const void* V, const float* W, const void* dO, void* dQ, void* dK,
                         void* dV, void* ws, hipStream_t stream);
// Causal backward on the matrix cores (bf16, d = 64, m a multiple of 64 up
// to 256; the causal forward's plan p, workspace offsets off_ru (the
// per-query (L_i, p_i)) and off_G (the segments' query states) of b).
hipError_t mfma_causal_backward(const Plan& p, const BwdPlan& b, const void* Q, const void* K,
                                const void* V, const float* W, const void* dO, void* dQ, void* dK,
                                void* dV, void* ws, hipStream_t stream);
// Its first launches: every segment's key state and reference, the prefix
// states, and per query (L_i, p_i) as float pairs in lp (BH L pairs).
hipError_t mfma_causal_rowstats(const Plan& p, const void* Q, const void* K, const void* V,
                                const float* W, const void* dO, float* lp, void* ws,
                                hipStream_t stream);
// The exported causal state after every key (fp32 [BH][m][d+4], natural-log
// references) from the bidirectional key partials in `ws` (plan p), added to
// the imported state state_in (nullptr: empty; may not alias state).
hipError_t mfma_state_export(const Plan& p, const void* ws, const float* state_in, float* state,
                             hipStream_t stream);
// The bidirectional matrix-core path's key partials alone (kpart).
hipError_t mfma_bidir_key_partials(const Plan& p, const void* K, const void* V, const float* W,
                                   void* ws, hipStream_t stream);
// Generic backward: dQ, dK, dV of <dO, O> (same dtype as the inputs).
hipError_t generic_backward(const Plan& p, const BwdPlan& b, const void* Q, const void* K,
                            const void* V, const float* W, const void* dO, void* dQ, void* dK,
                            void* dV, void* ws, hipStream_t stream);

// MFMA path (bf16 inputs): shape support, and the bidirectional forward.
bool mfma_bidir_supported(int32_t d, int32_t m, int32_t dtype);
// Key-side token groups per work-group and feature blocks of the
// bidirectional MFMA path, and whether its query side streams the features
// through LDS (qstream) instead of holding them (qapply).
int mfma_bidir_token_groups(int32_t d, int32_t m);
int mfma_bidir_feature_blocks(int32_t d, int32_t m);
bool mfma_bidir_streams_queries(int32_t d, int32_t m);
int mfma_bidir_query_workgroups();   // query-side work-groups the plan aims for (qapply)
int mfma_bidir_stream_round();       // tokens per lockstep round of qstream
hipError_t mfma_bidir_forward(const Plan& p, const void* Q, const void* K, const void* V,
                              const float* W, void* O, void* ws, hipStream_t stream);

// Fused bidirectional path (bf16, d = 64, m = 256, at least 64 heads).
bool fused_bidir_supported(int32_t B, int32_t H, int32_t L, int32_t d, int32_t m, int32_t dtype);
// Splits (seg, nseg) and query blocks (qblk) for `cus` compute units.
void fused_bidir_layout(Plan* p, int cus);
// The causal form's segment key states (every segment but the last, or
// every segment when all_segments) in the layout of T and cseg, for d = 64,
// m = 256, bf16 inputs, softmax or Gaussian features.
bool fused_causal_keys_supported(int32_t d, int32_t m, int32_t dtype, int32_t relu);
hipError_t fused_causal_key_states(const Plan& p, const void* K, const void* V, const float* W,
                                   float* T, float* cs, hipStream_t st, bool all_segments = false);
hipError_t fused_bidir_forward(const Plan& p, const void* Q, const void* K, const void* V,
                               const float* W, void* O, void* ws, hipStream_t stream);

// MFMA path (bf16 inputs): shape support, and the causal forward.
bool mfma_causal_supported(int32_t d, int32_t m, int32_t dtype);
// state_in (exported layout, nullptr: none) is a carried state that every
// query also attends to.  state_out (nullptr: none): where the path can, the
// state after the last token (state_in plus every key) is written there in
// the exported layout and *exported set; otherwise *exported stays false
// and the caller forms it.
hipError_t mfma_causal_forward(const Plan& p, const void* Q, const void* K, const void* V,
                               const float* W, void* O, void* ws, hipStream_t stream,
                               const float* state_in = nullptr, float* state_out = nullptr,
                               bool* exported = nullptr);

// Measurement hooks behind favor_timing_*: each kernel launch is bracketed
// by timing_before / timing_after (no-ops unless this thread is recording).
// `kernel` must be a string literal.
void timing_before(hipStream_t st);
void timing_after(hipStream_t st, const char* kernel);

// The forward entry points' common body: validation, plan, workspace check
// and the launches on `stream` (a FAVOR_* status).
int forward_call(int32_t B, int32_t H, int32_t L, int32_t d, int32_t m, int32_t dtype,
                 int32_t causal, int32_t attn_kernel, const void* Q, const void* K, const void* V,
                 const float* W, void* O, void* ws, size_t ws_bytes, void* stream);

// Records a failed HIP call for favor_last_hip_error(); returns FAVOR_ERR_HIP.
int record_hip_error(hipError_t e);

// On-device draw of W [m, d] (fp32, device memory; 1 <= d <= 128), the host
// draw's distribution and random stream.
hipError_t device_draw(uint64_t seed, int32_t m, int32_t d, float* W, hipStream_t stream);

// Feature map test entry (generic fp32 arithmetic).
hipError_t generic_feature_map(int32_t BH, int32_t L, int32_t d, int32_t m, int32_t dtype,
                               float knorm, int32_t relu, const void* X, const float* W,
                               float* Xp, hipStream_t stream);

}  // namespace favor
