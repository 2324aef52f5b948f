/*
 * coda.h - C-ABI of the fused GEMM-Residual-RMSNorm-GEMM block and the fused
 * SwiGLU gate/up block, forward and backward, on one AMD Instinct MI355X
 * (gfx950).
 *
 * Sources (the pages are three news articles on the paper "CODA: Rewriting
 * Transformer Blocks as GEMM-Epilogue Programs"):
 *   [JA] toolin.ai blog "CODA：LLMと初心者が光速のGPUカーネルを書けるようにする"
 *   [RU] kucoin.com news flash (Russian) on the paper
 *   [FR] kucoin.com news flash (French) on the paper
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Tensors are row-major and contiguous, with shapes as written beside each
 * argument; a weight is stored [in, out].  Every pointer is a DEVICE pointer
 * (HIP device memory of the current device) unless it is marked host.  The
 * caller owns every buffer, including the workspace; the library allocates
 * no device memory and keeps no state between calls (apart from the optional
 * kernel tracing at the end of this header, and the built-in scratch of
 * coda_fwd_noalloc), so calls are reentrant.
 *
 * Element types: `dtype` is the type of every tensor argument except r,
 * dgamma and the workspace: CODA_BF16 (bfloat16, 2 bytes) or CODA_F32.
 * r and dgamma are always float32.  Arithmetic accumulates in float32; bf16
 * results are rounded to nearest even.
 *
 * Execution: work is enqueued on `stream` (a hipStream_t; NULL = the null
 * stream) and the call returns without waiting.  Results are ready when the
 * stream reaches that point.  Calls that share a workspace or outputs on
 * different streams race.
 *
 * Shapes: every size must be >= 1 and a multiple of 8 (bf16) or 4 (f32), so
 * that each row starts on a 16-byte boundary.  Sizes need not be multiples of
 * the kernels' tile sizes; edge tiles are masked.  The token count M may be up
 * to 2^23; every other size (K, d, N, F and 2F, V) up to 2^21; a tensor may be
 * larger than 2 GiB (e.g. LLaMA-3 logits, 16384 x 128256 bf16), up to 1 TiB.
 * Larger sizes return CODA_ERR_SHAPE.
 *
 * Errors: every argument is checked before anything is enqueued; a failing
 * check returns a non-zero coda_status and enqueues nothing.  A HIP launch
 * failure returns CODA_ERR_HIP.  No C++ exception crosses this interface.
 * coda_status_str() names each status.
 */
#ifndef CODA_H
#define CODA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CODA_OK = 0,
  CODA_ERR_NULL = 1,        /* a required pointer is NULL */
  CODA_ERR_SHAPE = 2,       /* a size is < 1, not a multiple of 8 (bf16) / 4 (f32), or too large */
  CODA_ERR_ALIGN = 3,       /* a tensor pointer is not 16-byte aligned */
  CODA_ERR_ALIAS = 4,       /* an output overlaps an input, another output or the workspace */
  CODA_ERR_DTYPE = 5,       /* dtype is not a coda_dtype value */
  CODA_ERR_EPS = 6,         /* eps is not finite or not > 0 */
  CODA_ERR_WORKSPACE = 7,   /* workspace is NULL or smaller than the matching *_workspace_bytes */
  CODA_ERR_UNSUPPORTED = 8, /* valid request this library does not implement (e.g. f32 backward) */
  CODA_ERR_HIP = 9          /* a HIP runtime call or kernel launch failed */
} coda_status;

typedef enum { CODA_F32 = 0, CODA_BF16 = 1 } coda_dtype;

/* Name of a status code (static string; never NULL). */
const char* coda_status_str(coda_status s);

/* Library version string, e.g. "coda-mi355x 0.1.0 gfx950" (static). */
const char* coda_version(void);

/* ------------------------------------------------------------------------
 * Forward of the GEMM-Residual-RMSNorm-GEMM block.
 *
 * Computes, per [RU] and [FR] insight sections ("CODA: В «Финале» спрятаны
 * сокровища" / "CODA : « La fin » cache un trésor") and [JA] 核心の洞察:
 *   y = X W1 + R                         (first GEMM, residual in its epilogue)
 *   r_i = (mean_j y_ij^2 + eps)^(-1/2)   (from per-tile partial sums of
 *                                         squares left by the first GEMM's
 *                                         epilogue, combined by a small kernel)
 *   z = diag(r) ((y diag(gamma)) W2)     (second GEMM; gamma is applied in
 *                                         the first GEMM's epilogue, which also
 *                                         writes y * gamma, and r in the second
 *                                         GEMM's epilogue)
 * which equals RMSNorm(y) * gamma @ W2 up to rounding.
 *
 *   X     [M,K]  in      W1 [K,d] in     R [M,d] in (residual)
 *   gamma [d]    in      W2 [d,N] in
 *   y     [M,d]  out     the residual stream X W1 + R, saved for the backward
 *                        (rounded to dtype; the partial sums use it unrounded)
 *   r     [M]    out     float32 row scales, saved for the backward
 *   z     [M,N]  out
 *   eps   > 0, finite
 *   workspace: >= coda_fwd_workspace_bytes(dtype, M, K, d, N) bytes, device,
 *              16-byte aligned, contents ignored; holds the partial sums
 *              [M, ceil(d/256)] (fp32) and y * gamma [M, d] during the call.
 * Outputs must not overlap inputs, each other or the workspace.
 * ---------------------------------------------------------------------- */
size_t coda_fwd_workspace_bytes(coda_dtype dtype, int64_t M, int64_t K, int64_t d, int64_t N);
coda_status coda_fwd(coda_dtype dtype, int64_t M, int64_t K, int64_t d, int64_t N, float eps,
                     const void* X, const void* W1, const void* R, const void* gamma,
                     const void* W2, void* y, float* r, void* z,
                     void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * coda_fwd for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same computation, arguments, checks and results as coda_fwd, without the
 * workspace: the partial sums and y * gamma go to a scratch array built into
 * the library (CODA_NOALLOC_SCRATCH_BYTES = 80 MiB, one copy per device,
 * held until the process ends).  The call allocates nothing; its first call
 * on a device looks up that device's copy (with the device current).
 *   Needs coda_fwd_workspace_bytes(dtype, M, K, d, N) <= 80 MiB, else returns
 *   CODA_ERR_WORKSPACE and enqueues nothing (the LLaMA-7B-shaped and
 *   70B-hidden-shaped forwards need about 64.5 MiB).
 * Every call on one device shares that device's scratch, and nothing in it
 * must start at zero: calls that overlap on one device (on different
 * streams, or from different threads without ordering) race and give wrong
 * results.  Calls ordered on one stream are safe.
 * ---------------------------------------------------------------------- */
#define CODA_NOALLOC_SCRATCH_BYTES ((size_t)80 << 20)
coda_status coda_fwd_noalloc(coda_dtype dtype, int64_t M, int64_t K, int64_t d, int64_t N,
                             float eps, const void* X, const void* W1, const void* R,
                             const void* gamma, const void* W2, void* y, float* r, void* z,
                             void* stream);

/* ------------------------------------------------------------------------
 * Backward of the same block: the exact gradient of L = <dz, z>, given the
 * tensors saved by coda_fwd (y, r).  The pages state that a block-local
 * forward gives a block-local backward ([RU]/[FR] insight sections) and quote
 * this kernel's speed-up ([JA] 実験結果, [RU] "Результаты эксперимента"); the
 * gradient itself is the calculus of the forward above:
 *   n = diag(r) y;  dW2 = diag(gamma) n^T dz;  dh = dz W2^T;
 *   dgamma_j = sum_i dh_ij n_ij;  dn = dh diag(gamma);  s_i = sum_j dn_ij y_ij;
 *   dy = diag(r) dn - diag(r^3 s / d) y;  dR = dy;
 *   dX = dy W1^T;  dW1 = X^T dy.
 *
 *   X [M,K], W1 [K,d], gamma [d], W2 [d,N], y [M,d], r [M] (float32),
 *   dz [M,N]: in.   dX [M,K], dW1 [K,d], dR [M,d], dW2 [d,N]: out (dtype).
 *   dgamma [d]: out, float32.
 *   workspace: >= coda_bwd_workspace_bytes(dtype, M, K, d, N) bytes.
 * CODA_F32 returns CODA_ERR_UNSUPPORTED in this library.
 * ---------------------------------------------------------------------- */
size_t coda_bwd_workspace_bytes(coda_dtype dtype, int64_t M, int64_t K, int64_t d, int64_t N);
coda_status coda_bwd(coda_dtype dtype, int64_t M, int64_t K, int64_t d, int64_t N,
                     const void* X, const void* W1, const void* gamma, const void* W2,
                     const void* y, const float* r, const void* dz,
                     void* dX, void* dW1, void* dR, void* dW2, float* dgamma,
                     void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * SwiGLU gate/up GEMM with the activation in its epilogue, then the
 * down-projection ([JA] 組み合わせ可能な5種類の「積み木」, [RU] "Пять
 * «кирпичиков»", [FR] "Cinq « blocs »": the elementwise-transform primitive
 * covers activations; the matrix-tile store primitive saves intermediates):
 *   gu = X W,  W = [W_gate | W_up]  (gate columns 0..F-1, up columns F..2F-1)
 *   a  = silu(g) * u,  silu(t) = t / (1 + exp(-t)),  g = gu[:, :F], u = gu[:, F:]
 *   z  = a Wd
 *
 *   X [M,d], W [d,2F], Wd [F,d]: in.   gu [M,2F], a [M,F]: out, saved for the
 *   backward.   z [M,d]: out.   No workspace is needed (pass NULL, 0).
 * CODA_F32 returns CODA_ERR_UNSUPPORTED in this library.
 * ---------------------------------------------------------------------- */
size_t coda_swiglu_fwd_workspace_bytes(coda_dtype dtype, int64_t M, int64_t d, int64_t F);
coda_status coda_swiglu_fwd(coda_dtype dtype, int64_t M, int64_t d, int64_t F,
                            const void* X, const void* W, const void* Wd,
                            void* gu, void* a, void* z,
                            void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * SwiGLU backward: exact gradient of L = <dz, z> given the saved gu and a
 * (the pages quote its speed-up: [JA] 実験結果, [RU] "Результаты
 * эксперимента"):
 *   da = dz Wd^T;  sg = sigmoid(g);
 *   dg = da u sg (1 + g (1 - sg));  du = da g sg;  dgu = [dg | du];
 *   dWd = a^T dz;  dW = X^T dgu;  dX = dgu W^T.
 *
 *   X [M,d], W [d,2F], Wd [F,d], gu [M,2F], a [M,F], dz [M,d]: in.
 *   dX [M,d], dW [d,2F], dWd [F,d]: out.
 *   workspace: >= coda_swiglu_bwd_workspace_bytes(...) bytes (holds dgu).
 * CODA_F32 returns CODA_ERR_UNSUPPORTED in this library.
 * ---------------------------------------------------------------------- */
size_t coda_swiglu_bwd_workspace_bytes(coda_dtype dtype, int64_t M, int64_t d, int64_t F);
coda_status coda_swiglu_bwd(coda_dtype dtype, int64_t M, int64_t d, int64_t F,
                            const void* X, const void* W, const void* Wd,
                            const void* gu, const void* a, const void* dz,
                            void* dX, void* dW, void* dWd,
                            void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * The two patterns chained as a LLaMA MLP sub-layer: projection + residual,
 * RMS normalisation, SwiGLU gate/up, down projection.  The pages name the
 * residual add and RMS normalisation around a matmul, and SwiGLU as the
 * activation epilogue, inside a transformer block ([RU]/[FR] insight
 * sections; [JA]/[RU]/[FR] primitives sections).  Here the normalised input
 * feeds the gate/up GEMM in place of the second GEMM of coda_fwd:
 *   y = X W1 + R;  r_i = (mean_j y_ij^2 + eps)^(-1/2);
 *   [g | u] = diag(r) (y diag(gamma)) W,  W = [W_gate | W_up];
 *   a = silu(g) * u;  z = a Wd.
 * The first GEMM's epilogue leaves the partial sums of squares and y*gamma;
 * the gate/up GEMM's epilogue forms r, scales both accumulators by it and
 * applies SwiGLU.
 *
 *   X [M,K], W1 [K,d], R [M,d], gamma [d], W [d,2F], Wd [F,d]: in.
 *   y [M,d], r [M] (float32), gu [M,2F] (the r-scaled [g | u]), a [M,F]:
 *   out, saved for the backward.   z [M,d]: out.
 *   workspace: >= coda_mlp_fwd_workspace_bytes(...) bytes, 16-byte aligned,
 *   contents ignored (partial sums and y*gamma).
 * Errors as coda_fwd; CODA_F32 returns CODA_ERR_UNSUPPORTED in this library.
 * ---------------------------------------------------------------------- */
size_t coda_mlp_fwd_workspace_bytes(coda_dtype dtype, int64_t M, int64_t K, int64_t d, int64_t F);
coda_status coda_mlp_fwd(coda_dtype dtype, int64_t M, int64_t K, int64_t d, int64_t F, float eps,
                         const void* X, const void* W1, const void* R, const void* gamma,
                         const void* W, const void* Wd, void* y, float* r, void* gu, void* a,
                         void* z, void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Backward of the MLP sub-layer: the exact gradient of
 * L = <dz, z> + <dy_in, y>, given the tensors saved by coda_mlp_fwd.  dy_in
 * is the gradient the residual stream y receives from later layers; it is
 * optional (NULL = zero) and is added to dy.
 *   da = dz Wd^T;  sg = sigmoid(g);  dgu = [da u sg (1 + g (1 - sg)) | da g sg];
 *   dWd = a^T dz;
 *   then the block backward of coda_bwd with dz := dgu and W2 := W:
 *   n = diag(r) y;  dW = diag(gamma) n^T dgu;  dh = dgu W^T;
 *   dgamma_j = sum_i dh_ij n_ij;  dn = dh diag(gamma);  s_i = sum_j dn_ij y_ij;
 *   dy = diag(r) dn - diag(r^3 s / d) y + dy_in;  dR = dy;
 *   dX = dy W1^T;  dW1 = X^T dy.
 *
 *   X [M,K], W1 [K,d], gamma [d], W [d,2F], Wd [F,d], y [M,d], r [M]
 *   (float32), gu [M,2F], a [M,F], dz [M,d], dy_in [M,d] or NULL: in.
 *   dX [M,K], dW1 [K,d], dR [M,d], dW [d,2F], dWd [F,d]: out (dtype).
 *   dgamma [d]: out, float32.
 *   workspace: >= coda_mlp_bwd_workspace_bytes(...) bytes (dgu, then the
 *   block backward's n, partial sums and c).
 * dy_in may not overlap an output (CODA_ERR_ALIAS).  Other errors as
 * coda_bwd; CODA_F32 returns CODA_ERR_UNSUPPORTED in this library.
 * ---------------------------------------------------------------------- */
size_t coda_mlp_bwd_workspace_bytes(coda_dtype dtype, int64_t M, int64_t K, int64_t d, int64_t F);
coda_status coda_mlp_bwd(coda_dtype dtype, int64_t M, int64_t K, int64_t d, int64_t F,
                         const void* X, const void* W1, const void* gamma, const void* W,
                         const void* Wd, const void* y, const float* r, const void* gu,
                         const void* a, const void* dz, const void* dy_in, void* dX, void* dW1,
                         void* dR, void* dW, void* dWd, float* dgamma, void* workspace,
                         size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * LM-head GEMM with cross-entropy.  The pages' stateful epilogue primitive
 * keeps a running max and sum of exponentials across the tiles of a row,
 * which cross-entropy uses ([JA]/[RU]/[FR] primitives sections):
 *   logits = h Wv;  lse_i = log sum_j exp(logits_ij);
 *   loss_i = lse_i - logits_i,labels_i     (one loss per row, no reduction).
 * The GEMM's epilogue stores the logits (bf16, saved for the backward) and
 * each 256-column tile's (max, sum-exp) pair per row from the fp32
 * accumulator, plus the label's fp32 logit; a small kernel combines the
 * pairs in tile order into lse and loss.
 *
 *   h [M,d], Wv [d,V]: in (dtype).  labels [M]: in, int32.  A label outside
 *   [0, V) (e.g. -100) marks an ignored row: its loss is 0 and coda_ce_bwd
 *   gives it a zero dlogits row; its lse is still the row's.  Labels are only
 *   compared, never used as an index.  A NaN logit makes its row's lse (and
 *   loss, unless ignored) NaN.
 *   logits [M,V]: out (dtype).   lse [M], loss [M]: out, float32.
 *   workspace: >= coda_ce_fwd_workspace_bytes(...) bytes (the tile pairs).
 * Errors as coda_fwd (no eps); CODA_F32 returns CODA_ERR_UNSUPPORTED.
 * ---------------------------------------------------------------------- */
size_t coda_ce_fwd_workspace_bytes(coda_dtype dtype, int64_t M, int64_t d, int64_t V);
coda_status coda_ce_fwd(coda_dtype dtype, int64_t M, int64_t d, int64_t V, const void* h,
                        const void* Wv, const int32_t* labels, void* logits, float* lse,
                        float* loss, void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Backward of the cross-entropy LM head: the exact gradient of
 * L = sum_i dloss_i loss_i given the saved logits and lse (for a mean over
 * rows, dloss_i = 1/M):
 *   dlogits = diag(dloss) (exp(logits - lse) - onehot(labels));
 *   dh = dlogits Wv^T;  dWv = h^T dlogits.
 * Rows whose label lies outside [0, V) are ignored (zero dlogits row).
 *
 *   h [M,d], Wv [d,V], labels [M] (int32), logits [M,V], lse [M] (float32),
 *   dloss [M] (float32): in.   dh [M,d], dWv [d,V]: out (dtype).
 *   workspace: >= coda_ce_bwd_workspace_bytes(...) bytes (holds dlogits).
 * CODA_F32 returns CODA_ERR_UNSUPPORTED in this library.
 * ---------------------------------------------------------------------- */
size_t coda_ce_bwd_workspace_bytes(coda_dtype dtype, int64_t M, int64_t d, int64_t V);
coda_status coda_ce_bwd(coda_dtype dtype, int64_t M, int64_t d, int64_t V, const void* h,
                        const void* Wv, const int32_t* labels, const void* logits,
                        const float* lse, const float* dloss, void* dh, void* dWv,
                        void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * QKV projection with rotary positions in its epilogue.  The pages list
 * position encodings among the elementwise transforms an epilogue carries
 * ([JA] 組み合わせ可能な5種類の「積み木」, [RU] "Пять «кирпичиков»", [FR]
 * "Cinq « blocs »"):
 *   P = X W;  for each D-wide head in the first N_rot columns (q and k) and
 *   i < D/2, with phi = (row mod S) * base^(-2i/D):
 *     Y[:, 2i] = P[:, 2i] cos phi - P[:, 2i+1] sin phi
 *     Y[:, 2i+1] = P[:, 2i] sin phi + P[:, 2i+1] cos phi
 *   the remaining columns (v) are copied.  Rows are S-token sequences one
 *   after another.
 *
 *   X [M,K], W [K,N]: in.  Y [M,N]: out.  D a multiple of 8 (<= 4096),
 *   N_rot a multiple of D and <= N, 1 <= S, base finite and > 0, else
 *   CODA_ERR_SHAPE.  workspace: >= coda_rope_fwd_workspace_bytes(...) bytes
 *   (the cos / sin table, S x D floats, built per call in double precision).
 * CODA_F32 returns CODA_ERR_UNSUPPORTED in this library.
 * ---------------------------------------------------------------------- */
size_t coda_rope_fwd_workspace_bytes(coda_dtype dtype, int64_t M, int64_t K, int64_t N,
                                     int64_t N_rot, int64_t D, int64_t S);
coda_status coda_rope_fwd(coda_dtype dtype, int64_t M, int64_t K, int64_t N, int64_t N_rot,
                          int64_t D, int64_t S, float base, const void* X, const void* W, void* Y,
                          void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Backward of the rotary QKV projection: the exact gradient of L = <dY, Y>.
 * The rotation is orthogonal, so dP is dY rotated back (by -phi) on the
 * first N_rot columns and dY elsewhere;  dX = dP W^T;  dW = X^T dP.
 *
 *   X [M,K], W [K,N], dY [M,N]: in.  dX [M,K], dW [K,N]: out.
 *   workspace: >= coda_rope_bwd_workspace_bytes(...) bytes (table and dP).
 * Arguments and errors as coda_rope_fwd.
 * ---------------------------------------------------------------------- */
size_t coda_rope_bwd_workspace_bytes(coda_dtype dtype, int64_t M, int64_t K, int64_t N,
                                     int64_t N_rot, int64_t D, int64_t S);
coda_status coda_rope_bwd(coda_dtype dtype, int64_t M, int64_t K, int64_t N, int64_t N_rot,
                          int64_t D, int64_t S, float base, const void* X, const void* W,
                          const void* dY, void* dX, void* dW, void* workspace,
                          size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * MXFP8 forward of the GEMM-Residual-RMSNorm-GEMM block, and the quantiser
 * that makes its operands.  The pages note that faster FP8 / FP4 matrix
 * units raise the relative cost of the memory-bound work around a GEMM ([JA]
 * 課題：大モデル訓練の「手抜き税」, [RU] "Налог на лень при обучении больших
 * моделей", [FR] "Le « impôt de la paresse » ...") but fix no format.  The
 * format here is OCP MXFP8: E4M3 elements (bias 7, largest finite 448, no
 * infinities) and one E8M0 scale byte s (value 2^(s-127)) per 32 consecutive
 * elements along the GEMM's contraction index.
 *
 * Quantisation of a 32-block (coda_mx8_quantize, and y * gamma inside
 * coda_fwd_mx8): shared exponent e = floor(log2(max |v|)) - 8, clamped to
 * [-127, 127] (-127 for an all-zero block); scale byte e + 127; each element
 * v / 2^e rounded to the nearest E4M3 value, ties to even, saturated to
 * +-448.
 *
 * Scale layout ("step-blocked", every scale tensor below): the scales of a
 * [rows, cols] MXFP8 tensor are [cols/128][rows][4] bytes; byte j of word
 * (t, r) is the scale of row r's 32-block 4t + j.  One K step (128) of the
 * GEMMs then reads each tile's scales as one contiguous run.  A row-major
 * [rows][cols/32] scale tensor s maps to it as s.reshape(rows, cols/128, 4)
 * with its first two axes swapped.
 *
 * coda_mx8_quantize: src [rows, cols] bf16 with row stride ld_src elements
 *   (ld_src >= cols, a multiple of 8, src 16-byte aligned) -> codes [rows,
 *   cols] E4M3 bytes (contiguous, 16-byte aligned) and scales (step-blocked,
 *   rows * cols/32 bytes).  cols a multiple of 128, rows >= 1.  Blocks run
 *   along each row, so a weight W [in, out] is quantised from its transpose
 *   [out, in].  Errors: CODA_ERR_NULL, CODA_ERR_SHAPE, CODA_ERR_ALIGN,
 *   CODA_ERR_ALIAS (codes or scales overlapping src or each other).
 *
 * coda_fwd_mx8 computes, with deq() the MXFP8 value of codes and scales:
 *   y = deq(X) deq(W1t)^T + R;   r_i = (mean_j y_ij^2 + eps)^(-1/2);
 *   (q, qs) = MXFP8(y diag(gamma))  (first GEMM's epilogue, blocks along d);
 *   z = diag(r) (deq(q, qs) deq(W2t)^T)   (r in the second GEMM's epilogue).
 * The rewrite of coda_fwd with both GEMMs on the MXFP8 matrix cores; what is
 * quantised for the second GEMM is y * gamma (the tensor the first GEMM's
 * epilogue holds), not the normalised RMSNorm(y) * gamma.
 *
 *   Xq   [M,K] E4M3 in    Xs   [K/128][M][4] E8M0 in (step-blocked)
 *   W1tq [d,K] E4M3 in    W1ts [K/128][d][4] in     (W1 stored [out, in])
 *   W2tq [N,d] E4M3 in    W2ts [d/128][N][4] in     (W2 stored [out, in])
 *   R [M,d] bf16 in, gamma [d] bf16 in
 *   y [M,d] bf16 out (saved for coda_bwd), r [M] float32 out, z [M,N] bf16 out
 *   M, N: >= 8 and multiples of 8; K, d: >= 128 and multiples of 128 (whole
 *   K steps of the MXFP8 main loop), else CODA_ERR_SHAPE.  Every pointer
 *   16-byte aligned.  eps > 0 and finite.
 *   workspace: >= coda_fwd_mx8_workspace_bytes(M, K, d, N) bytes: the partial
 *   sums [M, ceil(d/256)] fp32, then q [M, d] E4M3 at the next 256-byte
 *   boundary, then its scales qs (step-blocked, [d/128][M][4]) at the next
 *   256-byte boundary.
 * The backward is coda_bwd (bf16) or coda_bwd_mx8 (below) on the saved y and r.
 * ---------------------------------------------------------------------- */
coda_status coda_mx8_quantize(int64_t rows, int64_t cols, const void* src, int64_t ld_src,
                              void* codes, void* scales, void* stream);
size_t coda_fwd_mx8_workspace_bytes(int64_t M, int64_t K, int64_t d, int64_t N);
coda_status coda_fwd_mx8(int64_t M, int64_t K, int64_t d, int64_t N, float eps, const void* Xq,
                         const void* Xs, const void* W1tq, const void* W1ts, const void* R,
                         const void* gamma, const void* W2tq, const void* W2ts, void* y, float* r,
                         void* z, void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Backward of the block with every GEMM on the MXFP8 matrix units.  The pages
 * argue that faster FP8 matrix units make the memory-bound work around a
 * GEMM relatively costlier ([JA] 課題：大モデル訓練の「手抜き税」; [RU] "Налог
 * на лень при обучении больших моделей"), which is what the fused epilogues
 * remove.  Gradient: that of coda_bwd (the forward's quantisation passes it
 * straight through), with each of the four GEMMs on MXFP8 operands (the
 * format of coda_fwd_mx8) quantised along its own contraction index:
 *   dh  = dz W2^T          dz and W2 quantised along N;  epilogue as coda_bwd
 *                          (dn, n = r y, the partial sums of s and dgamma)
 *   dR  = dy = r dn - c y  (bf16, as coda_bwd)
 *   dW2 = diag(gamma) n^T dz   n and dz quantised along M
 *   dX  = dy W1^T          dy and W1 quantised along d
 *   dW1 = X^T dy           X and dy quantised along M
 * dn, n and dy are rounded to bf16 before they are quantised (dn and dy are
 * stored; n = r y is formed where it is quantised).  The weights and
 * activations come in bf16, as for coda_bwd (a training step keeps bf16
 * weights); the call quantises them itself.
 *
 *   Arguments as coda_bwd (bf16 tensors, r and dgamma float32).
 *   M, d, N: multiples of 128 (the contraction dimensions are whole 128-k
 *   steps); K: a multiple of 8.
 *   workspace: >= coda_bwd_mx8_workspace_bytes(M, K, d, N) bytes (every GEMM
 *   operand in MXFP8 and the partial sums), 16-byte aligned.
 * Errors as coda_bwd.
 * ---------------------------------------------------------------------- */
size_t coda_bwd_mx8_workspace_bytes(int64_t M, int64_t K, int64_t d, int64_t N);
coda_status coda_bwd_mx8(int64_t M, int64_t K, int64_t d, int64_t N, const void* X, const void* W1,
                         const void* gamma, const void* W2, const void* y, const float* r,
                         const void* dz, void* dX, void* dW1, void* dR, void* dW2, float* dgamma,
                         void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * The SwiGLU block (coda_swiglu_fwd / coda_swiglu_bwd) with every GEMM on the
 * MXFP8 matrix units, for the same reason as the block's MXFP8 entry points
 * ([JA] 課題：大モデル訓練の「手抜き税」; [RU] "Налог на лень при обучении
 * больших моделей").  Each GEMM's operands are quantised (the format of
 * coda_fwd_mx8) along its own contraction index:
 *   gu  = X W          X and W along d;   a = silu(g) u from the GEMM's fp32
 *                      result;  gu and a stored in bf16, a also quantised
 *                      along F in the epilogue
 *   z   = a Wd         a and Wd along F
 * and the backward is the gradient of the unquantised block (the forward's
 * quantisation passes it straight through), as coda_swiglu_bwd:
 *   da  = dz Wd^T      dz and Wd along d;  epilogue dgu from the saved gu
 *   dWd = a^T dz       a and dz along M
 *   dX  = dgu W^T      dgu and W along 2F
 *   dW  = X^T dgu      X and dgu along M
 * a and dgu are rounded to bf16 before they are quantised.  The tensors come
 * and go in bf16 (X [M,d], W [d,2F] gate columns first, Wd [F,d], gu [M,2F],
 * a [M,F], z and dz [M,d], dX [M,d], dW [d,2F], dWd [F,d]); the calls
 * quantise them.
 *   M, d, F: multiples of 128 (every contraction index is whole 128-k steps).
 *   workspace: >= the matching _workspace_bytes(M, d, F) bytes (every GEMM
 *   operand in MXFP8; dgu in the backward), 16-byte aligned; the query
 *   returns 0 for a shape the calls refuse.
 * Errors as coda_swiglu_fwd / coda_swiglu_bwd (CODA_ERR_SHAPE for a shape
 * that is not whole 128-blocks).
 * ---------------------------------------------------------------------- */
size_t coda_swiglu_fwd_mx8_workspace_bytes(int64_t M, int64_t d, int64_t F);
coda_status coda_swiglu_fwd_mx8(int64_t M, int64_t d, int64_t F, const void* X, const void* W,
                                const void* Wd, void* gu, void* a, void* z, void* workspace,
                                size_t workspace_bytes, void* stream);
size_t coda_swiglu_bwd_mx8_workspace_bytes(int64_t M, int64_t d, int64_t F);
coda_status coda_swiglu_bwd_mx8(int64_t M, int64_t d, int64_t F, const void* X, const void* W,
                                const void* Wd, const void* gu, const void* a, const void* dz, void* dX,
                                void* dW, void* dWd, void* workspace, size_t workspace_bytes,
                                void* stream);

/* ------------------------------------------------------------------------
 * The MLP sub-layer (coda_mlp_fwd / coda_mlp_bwd) with every GEMM on the
 * MXFP8 matrix units: the block's MXFP8 reading (coda_fwd_mx8,
 * coda_bwd_mx8) and the SwiGLU block's (coda_swiglu_fwd_mx8) composed.
 *   y  = X W1 + R          X and W1 along K; the epilogue stores y (bf16), the
 *                          partial sums of squares and y diag(gamma) quantised
 *                          along d (from the unrounded y)
 *   [g | u] = diag(r) (y diag(gamma)) W   along d; r from the partial sums in
 *                          the epilogue; gu, a = silu(g) u stored in bf16, a
 *                          also quantised along F
 *   z  = a Wd              along F
 * and the backward is the gradient of the unquantised sub-layer (with dy_in,
 * as coda_mlp_bwd): da = dz Wd^T (along d; dgu from the saved gu), dWd = a^T
 * dz (along M), then the block's MXFP8 backward with dz := dgu (rounded to
 * bf16) and W2 := W, dy_in added to dy.  Tensors bf16 as coda_mlp_fwd /
 * coda_mlp_bwd (r and dgamma float32); the calls quantise them.
 *   M, K, d, F: multiples of 128.  dy_in: [M,d] or NULL.
 *   workspace: >= the matching _workspace_bytes(M, K, d, F) bytes, 16-byte
 *   aligned; the query returns 0 for a shape the calls refuse.
 * Errors as coda_mlp_fwd / coda_mlp_bwd.
 * ---------------------------------------------------------------------- */
size_t coda_mlp_fwd_mx8_workspace_bytes(int64_t M, int64_t K, int64_t d, int64_t F);
coda_status coda_mlp_fwd_mx8(int64_t M, int64_t K, int64_t d, int64_t F, float eps, const void* X,
                             const void* W1, const void* R, const void* gamma, const void* W, const void* Wd,
                             void* y, float* r, void* gu, void* a, void* z, void* workspace,
                             size_t workspace_bytes, void* stream);
size_t coda_mlp_bwd_mx8_workspace_bytes(int64_t M, int64_t K, int64_t d, int64_t F);
coda_status coda_mlp_bwd_mx8(int64_t M, int64_t K, int64_t d, int64_t F, const void* X, const void* W1,
                             const void* gamma, const void* W, const void* Wd, const void* y, const float* r,
                             const void* gu, const void* a, const void* dz, const void* dy_in, void* dX,
                             void* dW1, void* dR, void* dW, void* dWd, float* dgamma, void* workspace,
                             size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Kernel tracing (measurement aid; off by default).
 *
 * coda_trace_start(capacity) creates 2*capacity timing events (host call,
 * allocates; do it before the region to be measured).  While tracing is on,
 * every kernel the entry points above enqueue is bracketed by two of those
 * events on the same stream, together with the kernel's name and its
 * algorithmic work: GEMM flops (2*M*N*K) and the minimum HBM bytes the
 * kernel must move.  Launches beyond `capacity` are not recorded.
 * coda_trace_count() = launches recorded; coda_trace_get(i, ...) waits for
 * launch i's events and returns its name (static string), elapsed
 * milliseconds, flops and bytes.  coda_trace_stop() destroys the events.
 * Tracing state is process-global and not thread-safe: while it is on, one
 * host thread at a time may call the library.  Returns CODA_ERR_HIP if an
 * event call fails, CODA_ERR_SHAPE for a bad capacity or index.
 * ---------------------------------------------------------------------- */
coda_status coda_trace_start(int capacity);
int coda_trace_count(void);
coda_status coda_trace_get(int index, const char** name, float* ms, double* flops, double* bytes);
coda_status coda_trace_stop(void);

#ifdef __cplusplus
}
#endif

#endif /* CODA_H */
