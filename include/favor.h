/*
 * favor.h -- C ABI of the MI355X (gfx950) FAVOR attention library.
 *
 * FAVOR replaces softmax attention D^-1 A V, A = exp(Q K^T / sqrt(d)), by
 * the factorised kernel phi(q)^T phi(k) built from random features, and
 * re-associates the products so that no L x L matrix is formed: the keys
 * and values are first contracted into S = phi(K)^T V and z = phi(K)^T 1,
 * which are then left-multiplied by phi(Q) and normalised row by row.
 * The causal variant uses inclusive prefix sums of phi(k_j) v_j^T.
 * (FAVOR+ blog page "用随机特征“骗”过 softmax，Transformer 注意力也能跑成
 * 线性？", section 核心机制：FAVOR+; "Masked Language Modeling for Proteins
 * via Linearly Scalable Long-Context Transformers" summary pages, sections
 * Methodology / 方法论 and 核心创新.)
 *
 * Conventions shared by every entry point
 *  - All tensor pointers are device memory owned by the caller, except
 *    where an argument is documented as host memory.  The library never
 *    allocates or frees device memory.  Apart from favor_attention_noalloc
 *    (a fixed scratch array per device, shared by its calls) it keeps no
 *    mutable global state, and concurrent calls on different streams are
 *    safe.
 *  - Tensors are dense row-major.  Attention tensors are [B, H, L, d] with
 *    d fastest; Omega is [m, d] float32 and shared by every (b, h).
 *  - Device pointers (tensors and workspace) must be 16-byte aligned (the
 *    kernels move data in 16-byte vectors); a misaligned pointer returns
 *    FAVOR_ERR_INVALID_ARG.
 *  - `stream` is a hipStream_t (NULL = the legacy default stream).  Device
 *    work is enqueued on it asynchronously; no entry point synchronises.
 *  - Every argument check runs on the host before anything is enqueued and
 *    returns a negative favor_status; nothing is launched in that case.  A
 *    launch failure reported by the HIP runtime returns FAVOR_ERR_HIP.  No
 *    C++ exception crosses this interface.
 *  - Non-finite inputs propagate as IEEE values; a query whose estimated
 *    denominator phi(q)^T z is zero yields 0/0 = NaN (the method has no
 *    epsilon in the normaliser).
 */
#ifndef FAVOR_H_
#define FAVOR_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FAVOR_OK = 0,
  FAVOR_ERR_INVALID_ARG = -1,   /* null pointer, negative size, bad enum   */
  FAVOR_ERR_UNSUPPORTED = -2,   /* valid request this build cannot run     */
  FAVOR_ERR_WORKSPACE = -3,     /* workspace missing or smaller than asked */
  FAVOR_ERR_ALIAS = -4,         /* an output overlaps an input/workspace   */
  FAVOR_ERR_HIP = -5            /* the HIP runtime reported an error       */
} favor_status;

typedef enum { FAVOR_DTYPE_F32 = 0, FAVOR_DTYPE_BF16 = 1 } favor_dtype;

/* Feature maps.
 * TRIG: phi(x) = exp(|x~|^2/2) m^-1/2 [sin(Omega x~), cos(Omega x~)],
 *       F = 2m features, an unbiased estimate of exp(q.k/sqrt(d))
 *       (FAVOR+ blog page, section 核心机制：FAVOR+, trigonometric mode).
 * RELU: phi(x) = m^-1/2 max(Omega x~, 0), F = m features: generalized
 *       attention with ReLU as the kernel function (Chinese summary page,
 *       section 核心创新 item 2; English page, Technical Contribution).
 * POSITIVE: phi(x) = m^-1/2 exp(Omega x~ - |x~|^2/2), F = m non-negative
 *       features, also an unbiased estimate of exp(q.k/sqrt(d)) (the
 *       positive FAVOR+ variant named in the blog section; its form follows
 *       from the Gaussian moment-generating function).  The exponent is
 *       evaluated as one float32 value per feature: it never exceeds
 *       |omega|^2/2, and underflows only for |x~| far beyond the rows' norm.
 * In all, x~ = d^-1/4 x is applied by the library to the Q and K passed in. */
typedef enum {
  FAVOR_FEATURE_TRIG = 0,
  FAVOR_FEATURE_RELU = 1,
  FAVOR_FEATURE_POSITIVE = 2
} favor_feature_kind;

/* Kernel family selection for favor_attention_ex (AUTO = the fastest path
 * that supports the request).  MFMA requires bf16, d = 64 and m a multiple
 * of 32 with m <= 256, or m = 512 for the bidirectional forward; SMALL (the
 * forward of small bidirectional problems, float32 arithmetic) requires
 * d <= 32, m <= 128 and L <= 1024 -- with L <= 512, d a multiple of 8 and m
 * a multiple of 16 it is one launch whose matrix products take float32
 * operands as two bf16 parts each (relative error near 2^-17 per product,
 * float32 accumulation), otherwise two launches on the vector ALUs; the
 * choice depends on (L, d, m) only, never on B or H; GENERIC handles f32
 * and bf16 with d <= 64.  AUTO tries them in that order.  The backward pass
 * has MFMA and GENERIC families (SMALL returns FAVOR_ERR_UNSUPPORTED). */
typedef enum {
  FAVOR_PATH_AUTO = 0,
  FAVOR_PATH_GENERIC = 1,
  FAVOR_PATH_MFMA = 2,
  FAVOR_PATH_SMALL = 3
} favor_path;

/* Library version, (major << 16) | (minor << 8) | patch. */
int favor_version(void);

/* Static, human-readable text for a favor_status value. */
const char* favor_status_string(int status);

/*
 * favor_orf_omega -- orthogonal random features (HOST function).
 * Builds Omega [m, d] (float32, host memory, written by the call) from raw
 * Gaussian draws: for each d x d block of `gaussian` ([n_blocks, d, d]
 * float64, host, n_blocks = ceil(m / d)) the rows are orthonormalised in
 * order by modified Gram-Schmidt in float64; row r of the stacked result is
 * scaled to the chi(d) radius radii[r] ([m] float64, host) and rounded to
 * float32; the first m rows are kept.  Rows within a block are mutually
 * orthogonal and each row is marginally N(0, I_d) (FAVOR+ blog page,
 * section 核心机制：FAVOR+, orthogonal random directions; Chinese summary
 * page, section 方法详解).
 * Errors: FAVOR_ERR_INVALID_ARG for null pointers or m, d < 1, or a block
 * whose rows are linearly dependent.  Touches no device.
 */
int favor_orf_omega(const double* gaussian, const double* radii, int m, int d, float* omega);

/*
 * Workspace (device memory, bytes) that favor_attention needs for this
 * request; 0 is possible.  Returns 0 also for an invalid request (the call
 * itself then reports the error).  `path` as in favor_attention_ex.
 */
size_t favor_attention_workspace_bytes(int B, int H, int L, int d, int m, int dtype,
                                       int kind, int causal);
size_t favor_attention_workspace_bytes_ex(int B, int H, int L, int d, int m, int dtype,
                                          int kind, int causal, int path);

/*
 * favor_attention -- FAVOR attention, out = D^-1 (phi(Q) phi(K)^T) V
 * evaluated in linear order (FAVOR+ blog page, section 核心机制：FAVOR+).
 *   Q, K, V : [B, H, L, d] device, element type `dtype` (float32 or bf16)
 *   Omega   : [m, d] float32 device, shared by every (b, h)
 *   out     : [B, H, L, d] device, element type `dtype`; fully written.
 *             Must not overlap Q, K, V, Omega or the workspace.
 *   kind    : favor_feature_kind; causal: 0 = bidirectional,
 *             1 = causal (inclusive prefix over j <= i).
 *   workspace / workspace_bytes : device scratch of at least
 *             favor_attention_workspace_bytes(...) bytes (NULL if 0);
 *             contents on entry are ignored; clobbered.
 * B, H, L >= 0 (any zero makes the call a no-op returning FAVOR_OK);
 * d in [1, 64]; m >= 1 (m <= 1024).  Accumulation is float32 in every path.
 * Returns FAVOR_OK or a negative favor_status (see the conventions above).
 */
int favor_attention(const void* Q, const void* K, const void* V, const float* Omega, void* out,
                    int B, int H, int L, int d, int m, int dtype, int kind, int causal,
                    void* workspace, size_t workspace_bytes, void* stream);

/* As favor_attention, with an explicit kernel family (favor_path).  A path
 * that cannot run the request returns FAVOR_ERR_UNSUPPORTED. */
int favor_attention_ex(const void* Q, const void* K, const void* V, const float* Omega, void* out,
                       int B, int H, int L, int d, int m, int dtype, int kind, int causal,
                       void* workspace, size_t workspace_bytes, void* stream, int path);

/*
 * favor_attention_noalloc -- favor_attention_ex for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  It takes no workspace argument;
 * the kernels' scratch (the same buffers favor_attention_ex takes as its
 * workspace) is one fixed array of FAVOR_NOALLOC_SCRATCH_BYTES inside the
 * library, of which each device the library runs on holds its own copy
 * until the process ends.  The call allocates and frees nothing; the
 * first call on a device looks up that device's copy once.
 *   Arguments, layouts, results and errors as favor_attention_ex (the
 *   caller still owns Q, K, V, Omega and out).  The device is the one
 *   `stream` belongs to (the current device for a NULL stream).
 *   A request whose workspace (favor_attention_workspace_bytes_ex) exceeds
 *   FAVOR_NOALLOC_SCRATCH_BYTES returns FAVOR_ERR_WORKSPACE before
 *   anything is enqueued.
 *   Every call on one device shares that device's scratch, and its
 *   contents are whatever the last call left (the kernels never read
 *   scratch they have not written in the same call): calls that overlap
 *   in time on one device -- on different streams, or from different host
 *   threads -- race and must be ordered by the caller.
 */
#define FAVOR_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int favor_attention_noalloc(const void* Q, const void* K, const void* V, const float* Omega,
                            void* out, int B, int H, int L, int d, int m, int dtype, int kind,
                            int causal, void* stream, int path);

/*
 * favor_attention_train: favor_attention_ex that also writes the row
 * normaliser of the output, den[b, h, i] = D_ii = phi(q_i) . sum_j phi(k_j)
 * (j <= i when causal) with the full feature maps -- the diagonal of D in
 * D^-1 A V (FAVOR+ blog page, section 核心机制：FAVOR+).  Kept with `out`,
 * it lets favor_attention_backward_saved skip recomputing the forward.
 *   den: float32 [B, H, L] device memory, 4-byte aligned, written; it must
 *   not overlap any other argument (FAVOR_ERR_ALIAS).  Everything else as
 *   favor_attention_ex (same workspace size).  The trig map's causal MFMA
 *   path adds one small elementwise launch for den.
 */
int favor_attention_train(const void* Q, const void* K, const void* V, const float* Omega, void* out,
                          float* den, int B, int H, int L, int d, int m, int dtype, int kind,
                          int causal, void* workspace, size_t workspace_bytes, void* stream,
                          int path);

/* The favor_path that favor_attention_ex(..., path) would run (GENERIC,
 * MFMA or SMALL), or a negative favor_status if the request is
 * invalid/unsupported. */
int favor_attention_resolve_path(int B, int H, int L, int d, int m, int dtype, int kind,
                                 int causal, int path);

/*
 * favor_profile_attention -- per-kernel timing of favor_attention_ex.
 * Enqueues one call on `stream` in which every kernel (phase) whose result
 * depends only on the inputs and on earlier phases is launched `iters`
 * times back-to-back between a pair of HIP events (the generic causal
 * scan and readout, which update state in place, once), waits, and writes the mean duration of one launch
 * of each phase in milliseconds to phase_ms[0 .. *n_phases-1] and a short
 * name of each into names (max_phases entries of 48 bytes, NUL-terminated;
 * may be null).  `out` receives the call's result.  Creates and destroys
 * its own events; synchronises the stream.  Arguments as favor_attention_ex.
 */
int favor_profile_attention(const void* Q, const void* K, const void* V, const float* Omega,
                            void* out, int B, int H, int L, int d, int m, int dtype, int kind,
                            int causal, void* workspace, size_t workspace_bytes, void* stream,
                            int path, int iters, float* phase_ms, char* names, int max_phases,
                            int* n_phases);

/*
 * favor_attention_backward -- gradients of FAVOR attention.
 * The pages claim training-time speed-ups ("Masked Language Modeling for
 * Proteins ..." summary pages, Methodology) but print no backward pass;
 * this is the exact gradient of the computation favor_attention performs
 * (blog page "用随机特征“骗”过 softmax...", section 核心机制：FAVOR+),
 * the linear-order forms included.  For L = sum dOut . out it writes
 *   dQ = dL/dQ, dK = dL/dK, dV = dL/dV
 * with Omega fixed (no gradient).  With a_i = dOut_i / den_i and
 * b_i = -(dOut_i . out_i) / den_i: dphi(q_i) = S_i a_i + z_i b_i;
 * R_j = sum over queries i >= j (causal) or all i of phi(q_i) [a_i, b_i]^T;
 * dV_j = R_j[:, :d]^T phi(k_j) and dphi(k_j) = R_j [v_j, 1]; then the
 * chain rule through each feature map and x~ = d^-1/4 x.  The ReLU
 * derivative at 0 is 0; rows that are 0/0 in the forward give NaN.
 *   Q, K, V, dOut: [B, H, L, d] contiguous, dtype (read only).
 *   Omega: [m, d] float32 (read only).
 *   dQ, dK, dV: [B, H, L, d] contiguous, dtype (written; each element
 *   once, rounded to nearest even for bf16).  They must not overlap each
 *   other, any input or the workspace (FAVOR_ERR_ALIAS).
 *   workspace: device memory of at least
 *   favor_attention_backward_workspace_bytes(...) bytes, contents
 *   ignored and overwritten; float32 state, [a, b] and suffix buffers.
 * Every pointer is 16-byte aligned device memory owned by the caller.
 * Kernel families: MFMA (bf16, d = 64, m a multiple of 32 up to 256, both
 * directions; bidirectional: the forward's kernels plus a fused
 * feature-gradient kernel; causal: the forward's chunk kernel, which also
 * forms [a, b] and dV, and a chunked feature-gradient kernel that walks
 * prefix states for dQ and suffix states for dK) and generic (float32
 * arithmetic; d <= 64, m <= 1024, any L, both directions).  favor_attention_backward picks MFMA when it applies; the
 * _ex variants take a favor_path as for the forward (FAVOR_ERR_UNSUPPORTED
 * if the requested family cannot run the problem).  All checks run before
 * anything is enqueued; execution is asynchronous on `stream`.
 * B * H * L == 0 is a no-op.  The workspace size query returns 0 for an
 * invalid or unsupported request.
 */
size_t favor_attention_backward_workspace_bytes(int B, int H, int L, int d, int m, int dtype,
                                                int kind, int causal);
size_t favor_attention_backward_workspace_bytes_ex(int B, int H, int L, int d, int m, int dtype,
                                                   int kind, int causal, int path);
int favor_attention_backward(const void* Q, const void* K, const void* V, const float* Omega,
                             const void* dOut, void* dQ, void* dK, void* dV, int B, int H, int L,
                             int d, int m, int dtype, int kind, int causal, void* workspace,
                             size_t workspace_bytes, void* stream);
/*
 * favor_attention_backward_saved: favor_attention_backward_ex given the
 * forward's saved `out` and `den` (from favor_attention_train with the same
 * inputs).  The MFMA family then forms a_i = dOut_i / den_i and
 * b_i = -(dOut_i . out_i) / den_i in one elementwise pass instead of
 * recomputing the forward's readout; the generic family recomputes and
 * ignores them.  out: [B, H, L, d] dtype; den: float32 [B, H, L]; both
 * read only, must not overlap the gradients or the workspace.  Same
 * workspace size as favor_attention_backward_ex.
 */
int favor_attention_backward_saved(const void* Q, const void* K, const void* V,
                                   const float* Omega, const void* out, const float* den,
                                   const void* dOut, void* dQ, void* dK, void* dV, int B, int H,
                                   int L, int d, int m, int dtype, int kind, int causal,
                                   void* workspace, size_t workspace_bytes, void* stream, int path);
int favor_attention_backward_ex(const void* Q, const void* K, const void* V, const float* Omega,
                                const void* dOut, void* dQ, void* dK, void* dV, int B, int H,
                                int L, int d, int m, int dtype, int kind, int causal,
                                void* workspace, size_t workspace_bytes, void* stream, int path);

/*
 * Masked-LM attention block helpers (bf16), for the Performer block whose
 * attention is FAVOR ("Masked Language Modeling for Proteins ..." summary
 * pages, Methodology / 实验设计: protein sequences, multi-head attention).
 *
 * favor_embed_bf16: x[t, :] = table[ids[t], :] for t < n_tok.
 *   ids int32 [n_tok] device; table bf16 [vocab, E] device; x bf16
 *   [n_tok, E] device.  An id outside [0, vocab) writes a zero row.
 *   Requires E a multiple of 8 (FAVOR_ERR_UNSUPPORTED otherwise).
 */
int favor_embed_bf16(const int* ids, const void* table, void* x, int n_tok, int vocab, int E,
                     void* stream);

/*
 * favor_pack_weight_bf16: Wt[n, k] = W[k, n] for a bf16 weight W [K, N]
 * (row-major, the x W convention) -- the packed [out, in] layout the
 * projections below read (also PyTorch's Linear weight layout).  A layout
 * change, done once per weight; bit-exact.  Wt must not overlap W.
 */
int favor_pack_weight_bf16(const void* W, void* Wt, int K, int N, void* stream);

/*
 * favor_linear_bf16: Y = X Wt^T (bf16 operands, float32 accumulation on
 * MFMA, one round-to-nearest-even to bf16 at the end).  Wt is the packed
 * weight [N, K] row-major (favor_pack_weight_bf16 of a [K, N] W).
 *   X: logical [M, K].  in_heads == 0: X is [M, K] row-major.  in_heads > 0:
 *      X is head-split [M / seq_len, in_heads, seq_len, K / in_heads] and
 *      logical row r = b * seq_len + t gathers the heads' rows in order.
 *   Y: logical [M, N], stored row-major when out_heads == 0, or head-split
 *      [M / seq_len, out_heads, seq_len, N / out_heads] when out_heads > 0.
 * Requires M, N, K >= 1, N and K multiples of 8 (of 8 * heads when split)
 * and M a multiple of seq_len when a split is used; Y must not overlap X
 * or Wt.
 */
int favor_linear_bf16(const void* X, const void* Wt, void* Y, int M, int N, int K, int in_heads,
                      int out_heads, int seq_len, void* stream);

/*
 * favor_embed_linear_bf16: Y = X Wt^T with X[r, :] = table[ids[r], :] (a
 * zero row for ids outside [0, vocab)): the embedding gather fused into a
 * projection, so X is never stored.  Arithmetic as favor_linear_bf16.
 *   ids int32 [M]; table bf16 [vocab, K]; Wt bf16 [N, K] packed.
 *   Y: row-major [M, N] when out_heads == 0; else head-split in groups of
 *      G = out_heads * head_dim columns: column n of row r = b * seq_len + t
 *      goes to Y[n / G][b][h][t][n % head_dim], h = (n % G) / head_dim, a
 *      [N / G, M / seq_len, out_heads, seq_len, head_dim] tensor (Q, K and V
 *      of a block from one call with N = 3 * out_heads * head_dim).
 * Requires N and K multiples of 8; when split, head_dim a multiple of 8, N
 * a multiple of out_heads * head_dim and M of seq_len.  Y must not overlap
 * the other arguments.
 */
int favor_embed_linear_bf16(const int* ids, const void* table, int vocab, const void* Wt, void* Y,
                            int M, int N, int K, int out_heads, int head_dim, int seq_len,
                            void* stream);

#ifdef __cplusplus
}
#endif
#endif /* FAVOR_H_ */
