/*
 * muon_rocm.h -- C ABI of the MI355X (gfx950) Muon optimizer-step library.
 *
 * The library applies, to a set of 2-D fp32 weight matrices W of shape [A, B],
 *   - the Muon step of "Muon is Scalable for LLM Training" (Sec. 2.1 Eq. 1 momentum,
 *     Eq. 2 Newton-Schulz with X0 = M / ||M||_F and coefficients a, b, c, and
 *     Sec. 2.2 Eq. 4 update W <- W - lr * (0.2 * O * sqrt(max(A,B)) + wd * W)), and
 *   - the Periodic Row-wise variant of "Scaling Muon for Diffusion Transformers"
 *     (Periodic Row-wise paragraphs): NS5 once every K steps, and on the other steps
 *     Eq. 4 with O replaced by gamma * RowNorm(M), RowNorm scaling every row of M
 *     to unit l2 norm when A <= B and every column when A > B.
 * Tall matrices (A > B) run Newton-Schulz on M^T so the Gram matrix is min(A,B)^2.
 *
 * Conventions shared by every entry point:
 *   - All matrix buffers are DEVICE pointers owned by the caller, fp32, row-major,
 *     contiguous (leading dimension = cols), 16-byte aligned.
 *   - `workspace` is a caller-owned DEVICE buffer of at least the size that
 *     muon_workspace_bytes() reports for the same shapes, 256-byte aligned. Its
 *     contents need not be initialised and are garbage after the call.
 *   - `stream` is a hipStream_t (NULL = the legacy default stream). Calls only
 *     enqueue work on it and never synchronise; results are ready when the stream
 *     reaches that point. Concurrent calls must use distinct workspaces.
 *   - Every argument is validated on the host before anything is enqueued: on any
 *     error code no kernel runs and no buffer is touched.
 *   - Matrices with rows == 0 or cols == 0 are skipped (their pointers may be NULL);
 *     count == 0 is a no-op.
 *   - NaN / Inf in the inputs propagate to the outputs; they are not checked.
 *   - Results are deterministic: identical inputs give bitwise identical outputs.
 */
#ifndef MUON_ROCM_H
#define MUON_ROCM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MUON_ABI_VERSION 4

/* Status codes returned by every entry point. */
#define MUON_OK 0
#define MUON_ERR_INVALID_ARG (-1) /* NULL where a pointer is required, negative dims,
                                     count < 0, ns_steps < 1, period_k < 1, eps <= 0,
                                     unknown scale_mode, hidden < 1 under MUON_SCALE_HIDDEN */
#define MUON_ERR_WORKSPACE (-2)   /* workspace NULL or smaller than required */
#define MUON_ERR_ALIGN (-3)       /* matrix pointer not 16-byte aligned, workspace not 256,
                                     update_rms not 4 */
#define MUON_ERR_ALIAS (-4)       /* overlapping buffers that must be distinct */
#define MUON_ERR_HIP (-5)         /* a HIP runtime call or kernel launch failed */
#define MUON_ERR_TOO_LARGE (-6)   /* a dimension above 2^30 or a matrix above 2^40 elements */

/* Update-scale rules ("Muon is Scalable for LLM Training", Sec. 3.1). The update is
 * W <- W - lr (c U + wd W) with U = O on refresh steps and U = gamma R on RowNorm
 * steps, and the factor c is
 *   MUON_SCALE_MAX_DIM: rms_scale sqrt(max(A,B))     (Eq. 4, the same as Eq. 7)
 *   MUON_SCALE_HIDDEN:  rms_scale sqrt(hidden)        (Eq. 5, H = the model's hidden size)
 *   MUON_SCALE_RMS:     rms_scale / max(RMS(O), eps)  (Eq. 6) on refresh steps, where
 *                       RMS(O) = sqrt(mean(O^2)) is measured on the device; on RowNorm
 *                       steps rms_scale sqrt(max(A,B)), since RMS(R) = 1/sqrt(max(A,B))
 *                       exactly when every row (column) norm is >= eps. */
#define MUON_SCALE_MAX_DIM 0
#define MUON_SCALE_HIDDEN 1
#define MUON_SCALE_RMS 2

/* Hyperparameters. muon_default_hparams() fills the pages' defaults:
 * lr 1e-3, weight_decay 0.1, mu 0.95 (Muon notes Sec. 2.2), a, b, c =
 * 3.4445, -4.7750, 2.0315 (Sec. 2.1), rms_scale 0.2 (Eq. 4), gamma 0.15 and
 * period_k 3 (DiT paper, K/gamma sweep), eps 1e-7, ns_steps 5 (Sec. 2.2),
 * scale_mode MUON_SCALE_MAX_DIM, hidden 0. */
typedef struct muon_hparams {
    float lr;           /* eta */
    float weight_decay; /* lambda, decoupled (Eq. 3/4) */
    float mu;           /* momentum coefficient (Eq. 1) */
    float ns_a, ns_b, ns_c; /* Newton-Schulz polynomial coefficients (Eq. 2) */
    float rms_scale;    /* the 0.2 of Eq. 4 */
    float gamma;        /* RowNorm step relative to NS5 (Periodic variant) */
    float eps;          /* norms are divided as x / max(norm, eps) */
    int32_t ns_steps;   /* N, Newton-Schulz iterations (>= 1) */
    int32_t period_k;   /* K, refresh period (>= 1; 1 = vanilla Muon) */
    int32_t scale_mode; /* MUON_SCALE_* above */
    int32_t hidden;     /* H of MUON_SCALE_HIDDEN (>= 1 there, ignored otherwise) */
} muon_hparams;

/* One weight matrix with its optimizer state. All three are [rows, cols]. */
typedef struct muon_matrix {
    int64_t rows, cols;
    float* w;       /* weights, updated in place */
    float* m;       /* momentum (M_{t-1} in, M_t out), updated in place; zeros at t = 0 */
    const float* g; /* gradient, read only */
} muon_matrix;

/* Kernel classes reported by the optional timing facility. */
#define MUON_KCLASS_CAST 0          /* momentum + Frobenius partials + bf16 working copies */
#define MUON_KCLASS_FROB 1          /* per-matrix 1 / max(||M||_F, eps) */
#define MUON_KCLASS_GRAM 2          /* A = X X^T (symmetric tiles, bf16 MFMA; with its tail fixup) */
#define MUON_KCLASS_POLY 3          /* P = a I + b A + c A A (symmetric tiles, bf16 MFMA; with its tail fixup) */
#define MUON_KCLASS_APPLY 4         /* X' = P X = a X + (b A + c A A) X, iterations 1..N-1 (with its tail fixup) */
#define MUON_KCLASS_APPLY_FINAL 5   /* last iteration: O out, or the fused Eq. 4 update */
#define MUON_KCLASS_ROWNORM_ROWS 6  /* one-pass RowNorm step, flat / square matrices */
#define MUON_KCLASS_COLNORM_PARTIAL 7  /* tall: momentum + per-column partial sums */
#define MUON_KCLASS_COLNORM_FINALIZE 8 /* tall: per-column 1 / max(norm, eps) */
#define MUON_KCLASS_COLNORM_APPLY 9    /* tall: Eq. 4 update with the column-normalised M */
#define MUON_KCLASS_RMS_FINALIZE 10    /* per-matrix RMS(U): monitor value, Eq. 6 factor */
#define MUON_KCLASS_SCALED_UPDATE 11   /* Eq. 6 refresh: W <- decay W - coef O */
#define MUON_KCLASS_ADAMW 12           /* AdamW companion (non-matrix parameters) */
#define MUON_KCLASS_SPEC_GRAM 13       /* SVD entropy: fp64 Gram matrix (fp64 MFMA) */
#define MUON_KCLASS_SPEC_HOUSE 14      /* SVD entropy: Householder reflector per column */
#define MUON_KCLASS_SPEC_PASS 15       /* SVD entropy: trailing update + matrix-vector partials */
#define MUON_KCLASS_SPEC_REDUCE 16     /* SVD entropy: matrix-vector product from the partials */
#define MUON_KCLASS_SPEC_BISECT 17     /* SVD entropy: eigenvalues by Sturm bisection */
#define MUON_KCLASS_SPEC_ENTROPY 18    /* SVD entropy: normalisation and entropy */
#define MUON_KCLASS_COUNT 19

/* Returns MUON_ABI_VERSION. Host only. */
int muon_abi_version(void);

/* Static English text for a status code (never NULL). Host only. */
const char* muon_status_str(int status);

/* Detail of the last MUON_ERR_HIP (or other error) raised on this thread; "" if none. */
const char* muon_last_error(void);

/* Fills *hp with the defaults listed above. Host only; hp NULL is ignored. */
void muon_default_hparams(muon_hparams* hp);

/* Workspace size in bytes sufficient for muon_step, ns5_batched and rownorm_update
 * on `count` matrices of shapes rows[i] x cols[i]. Host only, touches no device.
 * Errors: INVALID_ARG (NULL bytes, count < 0, NULL rows/cols with count > 0, negative
 * dims), TOO_LARGE. */
int muon_workspace_bytes(const int64_t* rows, const int64_t* cols, int32_t count, size_t* bytes);

/* The GEMM plan of the Newton-Schulz stages (Eq. 2 of the Muon scaling paper: the Gram
 * X X^T, the polynomial P = a I + b A + c A A, the Apply P X = a X + (b A + c A A) X)
 * that ns5_batched and the refresh step of muon_step use for `count` matrices of
 * shapes rows[i] x cols[i].
 * Host only, touches no device; for tests and capacity planning. Nonempty matrices are
 * grouped as those calls group them: sorted by m = min(rows, cols), then by
 * n = max(rows, cols), both descending (stable), at most 16 per group. *groups receives
 * the number of groups. With capacity >= groups * MUON_PLAN_RECORD_INTS, `out` (host
 * array, caller-owned) receives one record of MUON_PLAN_RECORD_INTS values per group:
 *   [0]        matrices in the group;
 *   [1 .. 16]  their indices into rows / cols, -1 past that count;
 *   then 17 values for each of the Gram, the polynomial, the Apply of iterations
 *   1 .. N-1 and the last Apply, in that order: the tile width (128 or 256), then for
 *   XCD 0 .. 7 the number of its tiles that run as K chunks and the number of chunks
 *   (0 and 1 where the XCD does not split). A positive count h means the last h tiles
 *   of its sequence (tail split); a negative one, -h, its first h (head split, for a
 *   stage whose tiles fit one round and whose matrices differ in K).
 * capacity 0 only reports *groups (out may then be NULL).
 * Errors: INVALID_ARG (NULL groups, count < 0, NULL rows / cols with count > 0,
 * negative dims, capacity < 0, NULL out with capacity > 0, capacity below the
 * records), TOO_LARGE. */
#define MUON_PLAN_RECORD_INTS 85
int ns5_plan(const int64_t* rows, const int64_t* cols, int32_t count, int32_t* out, int32_t capacity,
             int32_t* groups);

/* One optimizer step at 0-based step index `step` for `count` matrices.
 * Periodic schedule (DiT paper, "NS5 once every K steps"; read here as a refresh
 * iff step % period_k == 0, so step 0 refreshes and period_k == 1 is vanilla Muon):
 *   refresh:  M <- mu M + G;  O = NS5(M);  W <- W - lr (c O + wd W), c per scale_mode
 *             (Eq. 4 and Eq. 5 fuse the update into the last Newton-Schulz GEMM;
 *             Eq. 6 writes O to the workspace, reduces RMS(O), then updates W)
 *   otherwise: exactly rownorm_update() below.
 * mats: host array of `count` descriptors.
 * update_rms: optional DEVICE array of `count` floats (NULL = not wanted). Entry i
 *   receives RMS(c U_i), the RMS of the update direction before the learning rate,
 *   weight decay excluded (about rms_scale under Eq. 4 by Lemma 1, exactly rms_scale
 *   under Eq. 6); entries of skipped empty matrices are left unchanged. It must not
 *   overlap any other buffer.
 * Errors: INVALID_ARG, ALIGN, ALIAS (any two of all w, m, g, update_rms ranges
 * overlap), WORKSPACE, TOO_LARGE, HIP. */
int muon_step(const muon_matrix* mats, int32_t count, const muon_hparams* hp, int64_t step,
              void* workspace, size_t workspace_bytes, float* update_rms, void* stream);

/* Newton-Schulz orthogonalisation alone ("Muon is Scalable", Sec. 2.1 Eq. 2):
 * o_out[i] = NS_N(m_in[i]) with X0 = M / max(||M||_F, eps), for [rows[i], cols[i]]
 * fp32 device matrices; the output has the input's shape and orientation. bf16 MFMA
 * products with fp32 accumulation; relative Frobenius error vs exact arithmetic is
 * about 1e-2. o_out[i] == m_in[i] (in place) is allowed; any other overlap is ALIAS.
 * m_in, o_out, rows, cols are host arrays of `count` entries. Only hp->ns_* and
 * hp->eps are used. Errors: INVALID_ARG, ALIGN, ALIAS, WORKSPACE, TOO_LARGE, HIP. */
int ns5_batched(const float* const* m_in, float* const* o_out, const int64_t* rows,
                const int64_t* cols, int32_t count, const muon_hparams* hp,
                void* workspace, size_t workspace_bytes, void* stream);

/* The Periodic variant's non-refresh step (DiT paper, Periodic Row-wise and
 * distributed-implementation paragraphs), fp32 throughout, in one pass for flat and
 * square matrices and three short kernels for tall ones:
 *   M <- mu M + G
 *   R = M / max(row l2 norms, eps)     if rows <= cols
 *   R = M / max(column l2 norms, eps)  if rows >  cols
 *   W <- W - lr (c gamma R + wd W), c = rms_scale sqrt(max(A,B)) or rms_scale sqrt(hidden)
 * update_rms as for muon_step (here RMS(c gamma R), one more small kernel when given).
 * hp->period_k is not used. Errors as muon_step. */
int rownorm_update(const muon_matrix* mats, int32_t count, const muon_hparams* hp,
                   void* workspace, size_t workspace_bytes, float* update_rms, void* stream);

/* ---- Allocation-free RowNorm step ---------------------------------------------------
 * For callers that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc. The same step as rownorm_update() (the
 * same kernels in the same order: bitwise identical results), with its workspace taken
 * from a fixed array of MUON_NOALLOC_SCRATCH_BYTES in device memory that the library
 * holds: one copy on each GPU it runs on, kept until the process ends. The call
 * allocates nothing (no hipMalloc, hipFree or allocating library routine) and creates
 * no timing events.
 * Limit: the RowNorm workspace of the matrices must fit the array. Per group of up to
 * 16 matrices (the same grouping as muon_step) it is the sum over the group of
 *   tall [A, B] (A > B):  4 B (ceil(A / 64) + 2) bytes,
 *   flat [A, B]:          4 A bytes,
 * each part rounded up to 256 bytes; sixteen [30720, 5120] matrices take 158 MB. Beyond
 * it the call returns MUON_ERR_WORKSPACE and nothing runs.
 * Every call on one GPU uses that GPU's single array: calls that overlap in time on one
 * GPU (other streams, other threads) race and corrupt each other's results; serialise
 * them. The array keeps the last call's contents; no part of it needs to start at zero.
 * Errors: as rownorm_update (WORKSPACE for the limit), HIP when the current device or the
 * array's address cannot be looked up. */
#define MUON_NOALLOC_SCRATCH_BYTES ((size_t)160 << 20)
int rownorm_update_noalloc(const muon_matrix* mats, int32_t count, const muon_hparams* hp,
                           float* update_rms, void* stream);

/* ---- One GPU's share of a row-sharded RowNorm step --------------------------------
 * "Scaling Muon for Diffusion Transformers", distributed-implementation paragraph: with
 * the weights sharded by rows (dim 0) across GPUs, the rows of a flat matrix (A <= B)
 * are whole on every GPU, so rownorm_update() on a GPU's block of rows is already its
 * share of the step (the block's sqrt(max(rows, B)) = sqrt(B) is the whole matrix's
 * scale). A tall matrix (A > B) normalises columns, which span the GPUs. Its step is
 * split in two calls around the caller's reduction:
 *   1. rownorm_shard_colsq: M <- mu M + G on the block, and colsq[c] = sum over the
 *      block's rows of M[r][c]^2;
 *   2. the caller sums colsq over the GPUs holding the matrix (an all-reduce; with
 *      one block per matrix, nothing);
 *   3. rownorm_shard_apply: W <- W - lr (c gamma M / max(sqrt(total[c]), eps) + wd W)
 *      with c = rms_scale sqrt(full_rows), or rms_scale sqrt(hidden) under
 *      MUON_SCALE_HIDDEN (MUON_SCALE_RMS takes the max-dimension form, as rownorm_update).
 * Concatenating the blocks reproduces rownorm_update() on the whole matrix up to the
 * summation order of the column sums. */
typedef struct muon_shard {
    int64_t rows, cols;  /* this GPU's block: `rows` rows of the matrix, all `cols` columns */
    int64_t full_rows;   /* A of the whole matrix: must exceed cols (tall) and be >= rows */
    float* w;            /* [rows, cols] block of W, updated by rownorm_shard_apply */
    float* m;            /* [rows, cols] block of M, updated by rownorm_shard_colsq */
    const float* g;      /* [rows, cols] block of G, read by rownorm_shard_colsq (apply: unused, may be NULL) */
} muon_shard;

/* Workspace in bytes for either shard call on these blocks (about 4 cols ceil(rows / 256)
 * bytes per block for up to 16 blocks at a time). Host only.
 * Errors: INVALID_ARG (NULL bytes or shards, count < 0, negative dims, full_rows <= cols,
 * rows > full_rows), TOO_LARGE. Blocks with cols == 0 are skipped. */
int rownorm_shard_workspace_bytes(const muon_shard* shards, int32_t count, size_t* bytes);

/* Step 1 for `count` blocks (host array). colsq: host array of `count` DEVICE pointers,
 * each to cols floats (4-byte aligned), written; a block with rows == 0 writes zeros.
 * Errors: as rownorm_update, plus INVALID_ARG for NULL colsq entries. */
int rownorm_shard_colsq(const muon_shard* shards, int32_t count, const muon_hparams* hp,
                        float* const* colsq, void* workspace, size_t workspace_bytes, void* stream);

/* Step 3. colsq_total: host array of `count` DEVICE pointers to the reduced column sums
 * (cols floats each), read only. M must hold step 1's output. Blocks with rows == 0 are
 * left alone. Errors: as rownorm_shard_colsq. */
int rownorm_shard_apply(const muon_shard* shards, int32_t count, const muon_hparams* hp,
                        const float* const* colsq_total, void* workspace, size_t workspace_bytes,
                        void* stream);

/* ---- AdamW companion for the parameters Muon does not take -------------------------
 * "Scaling Muon for Diffusion Transformers" (setup paragraph) keeps biases,
 * normalisation parameters and everything outside the transformer blocks on AdamW,
 * an auxiliary group at lr 1e-4; "Muon is Scalable for LLM Training" (Sec. 2.2,
 * matching-update-RMS paragraph) pairs Muon with AdamW for non-matrix parameters.
 * The pages do not restate AdamW; this is Adam with bias-corrected moments and
 * decoupled weight decay in Eq. 3's form, at 0-based step s (t = s + 1):
 *   m <- b1 m + (1 - b1) g;  v <- b2 v + (1 - b2) g^2
 *   W <- W - lr (m / (1 - b1^t) / (sqrt(v / (1 - b2^t)) + eps) + wd W)
 * adamw_default_hparams(): lr 1e-4 (the DiT paper's auxiliary group), beta1 0.9,
 * beta2 0.999, eps 1e-8 (PyTorch's AdamW defaults), weight_decay 0.1 (shared with Muon). */
typedef struct adamw_hparams {
    float lr;
    float beta1, beta2; /* in [0, 1) */
    float eps;          /* > 0 */
    float weight_decay;
} adamw_hparams;

/* One parameter tensor of any shape, as `numel` contiguous fp32 elements. w, m
 * (first moment), v (second moment) are DEVICE pointers updated in place (zeros at
 * s = 0); g is read only. All four 16-byte aligned; numel == 0 entries are skipped. */
typedef struct adamw_param {
    int64_t numel;
    float* w;
    float* m;
    float* v;
    const float* g;
} adamw_param;

/* Fills *hp with the defaults above. Host only; hp NULL is ignored. */
void adamw_default_hparams(adamw_hparams* hp);

/* One AdamW step at 0-based step `step` for `count` tensors (host array of
 * descriptors), enqueued on `stream`: one launch per 48 tensors, 28 bytes of HBM
 * traffic per element. fp32 throughout; no workspace.
 * Errors: INVALID_ARG (NULL hp / params / pointers, count < 0, numel < 0, step < 0,
 * beta outside [0, 1), eps <= 0, non-finite lr or wd), ALIGN, ALIAS (any two of all
 * w, m, v, g ranges overlap), TOO_LARGE (numel above 2^40), HIP. */
int adamw_step(const adamw_param* params, int32_t count, const adamw_hparams* hp, int64_t step,
               void* stream);

/* ---- Singular-spectrum diagnostic ----------------------------------------------------
 * SVD entropy of "Muon is Scalable for LLM Training", Sec. 3.4 (Dynamics of Singular
 * Spectrum): for W [A, B] with singular values sigma_1..sigma_n, n = min(A, B),
 *   q_i = sigma_i^2 / sum_j sigma_j^2,   H = -(1 / log n) sum_i q_i log q_i,
 * 1 for a flat spectrum and 0 for rank one. Zero singular values contribute 0; n = 1
 * gives 0; an all-zero matrix gives NaN (nothing to normalise).
 * Computed in fp64 on the device: sigma_i^2 are the eigenvalues of the Gram matrix
 * X X^T (X = W, or W^T when A > B), reduced to tridiagonal form by Householder
 * reflections and solved by Sturm-count bisection. The cost is about
 * min(A,B)^2 max(A,B) fp64 MFMA flops plus 8 min(A,B)^3 / 3 bytes of memory traffic
 * (the upper triangle of the shrinking trailing block, read and written once per
 * column), so this is an occasional diagnostic, not a per-step call. */

/* Workspace in bytes for svd_entropy on `count` matrices of shapes rows[i] x cols[i]
 * (about 8.25 min(A,B)^2 bytes per matrix for up to 16 matrices at a time). Host only.
 * Errors: INVALID_ARG (NULL bytes, count < 0, NULL rows/cols with count > 0, negative
 * dims), TOO_LARGE (as muon_workspace_bytes, or min(A, B) above 65536). */
int svd_entropy_workspace_bytes(const int64_t* rows, const int64_t* cols, int32_t count, size_t* bytes);

/* entropy[i] = H(w[i]) for the fp32 DEVICE matrices w[i] of shape rows[i] x cols[i]
 * (host arrays of `count` entries; row-major, 16-byte aligned, read only).
 * entropy: DEVICE array of `count` doubles, 8-byte aligned.
 * sigma_sq: optional DEVICE array (NULL = not wanted) of sum_i min(rows[i], cols[i])
 *   doubles, 8-byte aligned; matrix i's sigma^2 in descending order start at
 *   sum_{k<i} min(rows[k], cols[k]). Eigenvalues below 0 by rounding are reported as 0.
 * Empty matrices are skipped (their entropy entry is left unchanged). Outputs must not
 * overlap each other, the inputs or the workspace.
 * Errors: INVALID_ARG, ALIGN, ALIAS, WORKSPACE, TOO_LARGE, HIP. */
int svd_entropy(const float* const* w, const int64_t* rows, const int64_t* cols, int32_t count,
                void* workspace, size_t workspace_bytes, double* entropy, double* sigma_sq,
                void* stream);

/* ---- Attainable ceilings ------------------------------------------------------------
 * Yardsticks for the two rooflines the step is measured against, timed by the caller
 * (HIP events on `stream`) on the same GPU; neither is part of the optimizer step.
 * muon_ceiling_copy: dst[i] = src[i] for n fp32 elements (DEVICE pointers, 16-byte
 *   aligned, not overlapping), streamed as the step's HBM-bound passes stream: 256
 *   threads, 32 KiB contiguous per block, all loads of a thread before its stores,
 *   non-temporal hints. 8 n bytes of HBM traffic. Errors: INVALID_ARG, ALIGN, ALIAS,
 *   TOO_LARGE, HIP.
 * muon_ceiling_mfma: `blocks` blocks of four waves; every wave issues `iters` rounds of
 *   16 independent v_mfma_f32_32x32x16_bf16 on register operands into 16 fp32 32 x 32
 *   accumulators (the register budget of a Newton-Schulz GEMM wave), then writes one
 *   checksum to out[4 block + wave] (DEVICE, 4 blocks floats, 4-byte aligned). *flops
 *   (host, may be NULL) receives the dense flop count, blocks * 4 * iters * 16 * 32768.
 *   One block per compute unit (256 blocks) keeps one wave on every SIMD, as the GEMMs
 *   do. Errors: INVALID_ARG, ALIGN, HIP. */
int muon_ceiling_copy(const float* src, float* dst, int64_t n, void* stream);
int muon_ceiling_mfma(float* out, int32_t blocks, int32_t iters, double* flops, void* stream);

/* Optional per-kernel-class timing. While enabled (enable != 0), every kernel the
 * library enqueues is bracketed by HIP events recorded on the caller's stream (a GEMM
 * stage that splits its last tiles over K is bracketed together with its fixup
 * launch, and counts as one launch).
 * muon_timing_read() waits for the recorded events, adds their durations into
 * ms[MUON_KCLASS_COUNT] and launch counts into launches[MUON_KCLASS_COUNT] (either
 * may be NULL), and clears the record. muon_timing_enable(0) discards the record.
 * Process-global; not meant for concurrent callers. Errors: HIP. */
int muon_timing_enable(int enable);
int muon_timing_read(double* ms, int64_t* launches);

#ifdef __cplusplus
}
#endif

#endif /* MUON_ROCM_H */
