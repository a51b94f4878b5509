/*
 * favor.h -- C ABI of libfavor.so, the FAVOR+ attention forward pass for one
 * AMD Instinct MI355X (gfx950).
 *
 * What is computed (page: "FAVOR+", Code with Papers method page, section
 * "FAVOR+", the kernel definition and the FA-part equation; page: "Rethinking
 * Attention with Performers", abstract):
 *
 *   phi(x)_r = exp(w_r . x - |x|^2 / 2) / sqrt(m),   r = 0 .. m-1,
 *   rows of Q' and K' are phi(q_i) and phi(k_j),
 *   bidirectional:  O = D^-1 (Q' ((K')^T V)),  D = diag(Q' ((K')^T 1_L)),
 *   causal (masked self-attention; thesis record "Random Features for
 *   Efficient Attention Approximation", abstract): row i uses only keys and
 *   values j <= i (the diagonal included).
 *
 * The diagonal D is printed on the method page with (K')1_L; it is read as
 * (K')^T 1_L, the only product that type-checks.  The kernel is exp(x^T y)
 * with no internal 1/sqrt(d): callers who want softmax attention's usual
 * scale pre-multiply Q and K by d^-1/4.  The library applies no scaling.
 *
 * Exponent shifts ("stabilisers") are applied inside the kernels: a
 * per-feature reference on the key side, compensated on the query side, and a
 * per-query-row reference.  Such shifts cancel exactly in D^-1, so the result
 * is the formula above up to floating-point rounding.
 *
 * Conventions shared by every entry point below
 * ---------------------------------------------
 * Layout      Q, K, V and O are contiguous [B, H, L, d] (d at stride 1),
 *             16-byte aligned, in device memory.  O has the input dtype.
 *             W is fp32 [m, d] row-major, 16-byte aligned, in device memory.
 * dtype       FAVOR_F32 (fp32 inputs, fp32 arithmetic) or FAVOR_BF16 (bf16
 *             inputs and output, fp32 accumulation).
 * Shapes      B, H, L >= 1; d in {16, 32, 64, 128}; m a multiple of 16 with
 *             16 <= m <= 1024; B*H*L*d < 2^31.
 * Ownership   The caller owns every buffer, the workspace included.  The
 *             library allocates no device memory and keeps no pointer after
 *             a call returns.
 * Execution   Work is enqueued on the HIP stream `stream` (a hipStream_t;
 *             NULL is the default stream) and the call returns without
 *             waiting.  Inputs must stay valid until the stream reaches it.
 * Errors      Every argument is validated on the host before anything is
 *             enqueued; on error nothing is enqueued and a negative
 *             favor_status is returned.  A failed HIP launch returns
 *             FAVOR_ERR_HIP and records the HIP error code for
 *             favor_last_hip_error() (per thread).  NaN and Inf inputs are not
 *             checked; they propagate under IEEE rules.
 * Threads     Re-entrant; no global mutable state except the per-thread last
 *             HIP error and the per-thread timing record (favor_timing_*).  Calls that share a workspace must be ordered on one
 *             stream.
 */
#ifndef FAVOR_H
#define FAVOR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum favor_dtype {
  FAVOR_F32 = 0,
  FAVOR_BF16 = 1
};

/*
 * Attention kernel the features estimate (method page, section "FAVOR+": the
 * mechanism approximates softmax and Gaussian kernels; the paper's abstract
 * also names generalized kernelizable attention).  The features are
 * phi(x)_r = exp(w_r . x - c |x|^2) / sqrt(m) with c = 1/2 for the softmax
 * kernel exp(x . y) and c = 1 for the Gaussian kernel exp(-|x - y|^2 / 2)
 * (the softmax features times exp(-|x|^2 / 2)), and, for generalized
 * attention with f = ReLU (f is not named on the pages; this is the one
 * built), phi(x)_r = max(w_r . x, 0) / sqrt(m), whose expectation is the
 * first-order arc-cosine kernel.  The pages print none of the feature maps;
 * these are the readings taken.  With ReLU features a query whose features
 * are all zero (e.g. q = 0) has no defined output (0/0).
 */
enum favor_attn_kernel {
  FAVOR_SOFTMAX = 0,
  FAVOR_GAUSSIAN = 1,
  FAVOR_RELU = 2
};

enum favor_status {
  FAVOR_OK = 0,
  FAVOR_ERR_NULL = -1,        /* a required pointer is NULL                     */
  FAVOR_ERR_SHAPE = -2,       /* B, H or L < 1, or the tensor is too large      */
  FAVOR_ERR_UNSUPPORTED = -3, /* d, m, dtype or attention kernel outside the
                                 supported set                                  */
  FAVOR_ERR_ALIGN = -4,       /* a tensor base is not 16-byte aligned, or the
                                 workspace base is not 256-byte aligned         */
  FAVOR_ERR_WORKSPACE = -5,   /* workspace_bytes below favor_workspace_bytes()  */
  FAVOR_ERR_HIP = -6,         /* a HIP runtime call failed                      */
  FAVOR_ERR_ALIAS = -7,       /* two buffers that must be distinct overlap      */
  FAVOR_ERR_SCRATCH = -8      /* favor_fwd_attn_noalloc: the shape needs more
                                 than FAVOR_NOALLOC_SCRATCH_BYTES of workspace,
                                 or the stream is not on the current device    */
};

/*
 * Workspace size, in bytes, that favor_fwd_bidir (causal = 0) or
 * favor_fwd_causal (causal = 1) needs for this shape; written to *bytes.
 * The workspace holds the key-side state [(K')^T V | (K')^T 1_L] (m x (d+1)
 * fp32 per head, per sequence split or segment) and its per-feature exponent
 * references.  The size covers every attention kernel (favor_fwd_attn may
 * take another path for FAVOR_RELU than for the others).  Returns FAVOR_OK
 * or a validation error (bytes untouched).  Pure host function: no HIP call.
 */
int favor_workspace_bytes(int32_t B, int32_t H, int32_t L, int32_t d, int32_t m,
                          int32_t dtype, int32_t causal, size_t* bytes);

/*
 * The execution plan a forward call with these arguments would use:
 * *path = 0 (fp32 FMA kernels), 1 (bf16 matrix-core kernels) or 2 (bf16
 * matrix-core kernels, the bidirectional form in one persistent launch after
 * a small preparation launch: d = 64, m = 256, at least 64 heads, softmax and
 * Gaussian features; FAVOR_RELU features take path 1 there); *nseg and
 * *seg = the number of sequence splits (bidirectional) or segments (causal)
 * per head and their length in tokens.  Pure host function: no HIP call.
 * Returns FAVOR_OK, a validation error or FAVOR_ERR_NULL.
 */
int favor_plan_describe(int32_t B, int32_t H, int32_t L, int32_t d, int32_t m, int32_t dtype,
                        int32_t causal, int32_t* path, int32_t* nseg, int32_t* seg);

/*
 * Bidirectional FAVOR+ forward (FA-part equation of the method page):
 * O = D^-1 (Q' ((K')^T V)).  Q, K, V: [B,H,L,d] inputs; W: [m,d] fp32
 * projection; O: [B,H,L,d] output (may not alias Q, K, V); workspace of at
 * least favor_workspace_bytes(..., causal=0) bytes, 256-byte aligned.
 */
int favor_fwd_bidir(int32_t B, int32_t H, int32_t L, int32_t d, int32_t m, int32_t dtype,
                    const void* Q, const void* K, const void* V, const float* W,
                    void* O, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Causal (masked) FAVOR+ forward in prefix-sum form:
 * O_i = q'_i S_i / q'_i z_i with S_i = sum_{j<=i} k'_j v_j^T and
 * z_i = sum_{j<=i} k'_j.  Arguments as favor_fwd_bidir; workspace of at least
 * favor_workspace_bytes(..., causal=1) bytes.
 */
int favor_fwd_causal(int32_t B, int32_t H, int32_t L, int32_t d, int32_t m, int32_t dtype,
                     const void* Q, const void* K, const void* V, const float* W,
                     void* O, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Either form with any attention kernel: favor_fwd_bidir (causal = 0) or
 * favor_fwd_causal (causal != 0) with the features of `attn_kernel`
 * (FAVOR_SOFTMAX: exactly those entry points; FAVOR_GAUSSIAN: the key
 * features carry exp(-|k|^2), the query features' norm term cancels per
 * row; FAVOR_RELU: max(w . x, 0) features, no exponent references).
 * Arguments, workspace (favor_workspace_bytes does not depend on the kernel)
 * and errors as favor_fwd_bidir; an unknown attn_kernel gives
 * FAVOR_ERR_UNSUPPORTED before anything is enqueued.
 */
int favor_fwd_attn(int32_t B, int32_t H, int32_t L, int32_t d, int32_t m, int32_t dtype,
                   int32_t causal, int32_t attn_kernel, const void* Q, const void* K,
                   const void* V, const float* W, void* O, void* workspace,
                   size_t workspace_bytes, void* stream);

/*
 * favor_fwd_attn with no workspace argument, for callers that cannot
 * allocate device memory (code under stream capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The workspace is a static device array
 * of FAVOR_NOALLOC_SCRATCH_BYTES on each GPU the library runs on, held until
 * the process ends; this call allocates nothing.  It runs on the calling
 * thread's current device: `stream` (NULL: the null stream) must belong to
 * it.  Every call on one GPU shares that GPU's array, so calls that overlap
 * on one GPU (other streams, other threads) race and must be ordered by the
 * caller.  Errors as favor_fwd_attn, plus FAVOR_ERR_SCRATCH when
 * favor_workspace_bytes() for the shape exceeds the array (64 MiB: enough for
 * B*H = 64 heads of L = 4096 at d = 64, m = 256, in either form) or the
 * stream is on another device.
 */
#define FAVOR_NOALLOC_SCRATCH_BYTES (64 * 1024 * 1024)
int favor_fwd_attn_noalloc(int32_t B, int32_t H, int32_t L, int32_t d, int32_t m, int32_t dtype,
                           int32_t causal, int32_t attn_kernel, const void* Q, const void* K,
                           const void* V, const float* W, void* O, void* stream);

/*
 * Workspace size, in bytes, of favor_bwd_attn for this shape (written to
 * *bytes): the forward's key state and references plus, per query, the
 * scaled upstream gradient [dO/den | -(dO . O)/den] and its row reference,
 * and the per-segment query state.  Returns FAVOR_OK or a validation error
 * (bytes untouched).  Pure host function: no HIP call.
 */
int favor_bwd_workspace_bytes(int32_t B, int32_t H, int32_t L, int32_t d, int32_t m,
                              int32_t dtype, int32_t causal, size_t* bytes);

/*
 * Backward pass of favor_fwd_attn (the pages print none; it is the chain rule
 * through the same definitions, with W held fixed -- the pages redraw W, they
 * do not train it): for an upstream gradient dO [B,H,L,d] of the output,
 * writes dQ, dK, dV [B,H,L,d], the gradients of <dO, O> with respect to Q, K
 * and V, for either form (causal = 0 or 1) and any attn_kernel (the ReLU
 * derivative at exactly 0 is taken as 0).  Inputs and outputs share the
 * dtype; every buffer is in device memory, 16-byte aligned; the outputs may
 * not alias any input or each other.  The forward is recomputed inside the
 * call (no forward output is taken).  Workspace of at least
 * favor_bwd_workspace_bytes() bytes, 256-byte aligned.  Errors as
 * favor_fwd_attn.
 */
int favor_bwd_attn(int32_t B, int32_t H, int32_t L, int32_t d, int32_t m, int32_t dtype,
                   int32_t causal, int32_t attn_kernel, const void* Q, const void* K,
                   const void* V, const float* W, const void* dO, void* dQ, void* dK, void* dV,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * Incremental causal state (masked form in prefix-sum order; thesis record
 * "Random Features for Efficient Attention Approximation", abstract: masked
 * attention in linear time): the running sums S = sum_j phi(k_j) v_j^T and
 * z = sum_j phi(k_j) of the tokens seen so far, for streaming and
 * token-by-token decoding.
 *
 * Layout   fp32 [B*H][m][d+4] in device memory (16-byte aligned), one row
 *          per feature r: [S~_r (d values) | z~_r | c_r | 0 | 0], the true state
 *          [S | z]_r = exp(c_r) sqrt(m)^-1 [S~_r | z~_r] (c_r a per-feature
 *          exponent reference that keeps S~ in fp32 range; for FAVOR_RELU
 *          c_r = 0 once a token was added).  Empty state: S~ = z~ = 0,
 *          c = -inf.  The buffer is the export/import format: copy it to keep
 *          a stream's state, pass it back to continue it.  A state is tied to
 *          its (d, m, W, attn_kernel).
 */
/* Bytes of the states of B*H heads (B*H*m*(d+4)*4).  Pure host function. */
int favor_state_bytes(int32_t B, int32_t H, int32_t d, int32_t m, size_t* bytes);

/* Empty states for B*H heads (a fill kernel on `stream`, no memset node). */
int favor_state_reset(int32_t B, int32_t H, int32_t d, int32_t m, float* state, void* stream);

/* Workspace bytes of favor_prefill for this shape.  Pure host function. */
int favor_prefill_workspace_bytes(int32_t B, int32_t H, int32_t L, int32_t d, int32_t m,
                                  int32_t dtype, size_t* bytes);

/*
 * Causal forward over L new tokens that continues a state: O (as
 * favor_fwd_attn with causal = 1) where token i attends to the carried
 * tokens of state_in and to the new tokens j <= i.  state_in (NULL: empty)
 * and state_out (NULL: not written) are states as above and may not alias;
 * state_out receives the state after the last new token.  A prefill of
 * bf16 inputs with d = 64 and m a multiple of 64 up to 256 runs on the
 * matrix cores (the causal forward with state_in as the first segment's
 * carry, and the final state as state_in plus the sum over every key);
 * every other case on the fp32 FMA kernels.  Workspace of at least
 * favor_prefill_workspace_bytes() bytes, 256-byte aligned.  Errors as
 * favor_fwd_attn, and FAVOR_ERR_ALIAS when state_in and state_out
 * overlap (chunked prefill alternates two state buffers).
 */
int favor_prefill(int32_t B, int32_t H, int32_t L, int32_t d, int32_t m, int32_t dtype,
                  int32_t attn_kernel, const void* Q, const void* K, const void* V,
                  const float* W, void* O, const float* state_in, float* state_out,
                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * One decoding step for every head: the new token's k, v ([B,H,d] in
 * `dtype`) are added to `state` in place, then o = the causal output of the
 * new token's q over every token in the state (itself included).  One
 * work-group per head; no workspace.  Errors as favor_fwd_attn (L is 1).
 */
int favor_decode(int32_t B, int32_t H, int32_t d, int32_t m, int32_t dtype, int32_t attn_kernel,
                 const void* q, const void* k, const void* v, const float* W, void* o,
                 float* state, void* stream);

/*
 * The feature map alone, for testing the projection and exponent arithmetic:
 * Xp[b,h,l,r] = exp(w_r . x_{b,h,l} - |x_{b,h,l}|^2 / 2) / sqrt(m), fp32
 * [B,H,L,m] in device memory, with no exponent shift (the caller keeps the
 * exponents in fp32 range).  X: [B,H,L,d] in `dtype`.  Shapes and alignment
 * as above.
 */
int favor_feature_map(int32_t B, int32_t H, int32_t L, int32_t d, int32_t m, int32_t dtype,
                      const void* X, const float* W, float* Xp, void* stream);

/*
 * favor_feature_map with the features of `attn_kernel`:
 * Xp[b,h,l,r] = exp(w_r . x - c |x|^2) / sqrt(m), c = 1/2 (FAVOR_SOFTMAX, the
 * same as favor_feature_map) or 1 (FAVOR_GAUSSIAN), or max(w_r . x, 0) /
 * sqrt(m) (FAVOR_RELU).  Unknown attn_kernel: FAVOR_ERR_UNSUPPORTED.
 */
int favor_feature_map_attn(int32_t B, int32_t H, int32_t L, int32_t d, int32_t m, int32_t dtype,
                           int32_t attn_kernel, const void* X, const float* W, float* Xp,
                           void* stream);

/*
 * Draw the projection W [m, d] (fp32, row-major, host memory) from `seed`:
 * positive orthogonal random features (summary page "Key contributions";
 * limitation "m <= d" read as orthogonality within blocks of at most d
 * rows).  Block b (rows b*d ..) is the Gram-Schmidt orthonormalisation
 * (computed twice, fp64) of the columns of a d x d standard-normal matrix;
 * each row is then scaled by the norm of an independent d-dimensional
 * standard-normal vector (a chi(d) draw).  Normals come from a counter-based
 * SplitMix64 stream (Steele, Lea & Flood, OOPSLA 2014) through the Box-Muller
 * transform.  1 <= d <= 1024 and 1 <= m; W_host must hold m*d floats.
 * Pure host function: no HIP call.  Returns FAVOR_OK, FAVOR_ERR_NULL or
 * FAVOR_ERR_SHAPE.
 */
int favor_draw_projection(uint64_t seed, int32_t m, int32_t d, float* W_host);

/*
 * favor_draw_projection on the GPU: the same distribution, random stream and
 * stream order, written to W (fp32 [m, d], device memory, 16-byte aligned)
 * on `stream` (one work-group per block of d rows; no host work, no copy),
 * so that a redraw can be queued between forward calls.  The directions are
 * made orthonormal in fp64 by classical Gram-Schmidt applied twice, the host
 * by the one-at-a-time form: the two agree to fp64 rounding, and W to fp32
 * rounding.  1 <= d <= 128 and 1 <= m.  Returns FAVOR_OK, FAVOR_ERR_NULL,
 * FAVOR_ERR_SHAPE, FAVOR_ERR_ALIGN or FAVOR_ERR_HIP.
 */
int favor_draw_projection_device(uint64_t seed, int32_t m, int32_t d, float* W, void* stream);

/* Static English text for a favor_status value (never NULL). */
const char* favor_status_string(int status);

/* The hipError_t of this thread's last failed HIP call (0 if none). */
int favor_last_hip_error(void);

/*
 * Per-kernel GPU time, for measurement harnesses (not part of the method).
 * favor_timing_start() clears this host thread's record and turns recording
 * on: every favor_fwd_bidir / favor_fwd_causal call made afterwards by this
 * thread records a HIP event on its stream before and after each kernel it
 * launches.  favor_timing_stop() turns recording off, waits for the recorded
 * events, and reports up to max_kernels kernels in order of first launch:
 * names[k] (static strings owned by the library), ms[k] (summed
 * event-to-event milliseconds) and launches[k]; *n_kernels receives the
 * number of distinct kernels recorded.  Events are created on first use and
 * kept for reuse by this thread.  Returns FAVOR_OK, FAVOR_ERR_NULL (a NULL
 * output with max_kernels > 0, or n_kernels NULL) or FAVOR_ERR_HIP.
 */
int favor_timing_start(void);
int favor_timing_stop(int32_t max_kernels, const char** names, float* ms, int32_t* launches,
                      int32_t* n_kernels);

#ifdef __cplusplus
}
#endif

#endif /* FAVOR_H */
