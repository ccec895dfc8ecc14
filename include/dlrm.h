/*
 * dlrm.h -- C ABI of libdlrm.so, the DLRM hot path on one AMD Instinct
 * MI355X (gfx950).
 *
 * The model (cited by web page and section):
 *   [EXPL] "Deep Learning Recommendation Model (DLRM)" explainer
 *          (nadeemcite.github.io): Core Idea; Key Method Details
 *          (Embedding tables, Bottom MLP, Interaction layer, Top MLP, Loss).
 *   [SU]   "DLRM - Deep Learning Recommendation Model" (briansu.co/recsys/dlrm):
 *          How it works; Key equations (Interaction, Output);
 *          Limitations & trade-offs (memory-bound, one shared d).
 *
 * Conventions shared by every entry point
 *   - Pointers are DEVICE pointers unless the comment says "host".
 *   - The caller owns all memory.  The library never allocates, frees or
 *     synchronises; scratch space is passed in as a workspace whose size a
 *     *_workspace_size query returns.
 *   - Every call enqueues work on `stream` and returns an int status:
 *       DLRM_OK (0), DLRM_E_INVALID (null pointer, size or alignment out of
 *       range), DLRM_E_WORKSPACE (workspace too small), DLRM_E_HIP (a launch
 *       failed; dlrm_last_hip_error() returns the hipError_t),
 *       DLRM_E_UNSUPPORTED (valid but not implemented, e.g. key width).
 *     Arguments are checked on the host before anything is enqueued; on an
 *     error nothing is enqueued.
 *   - Index values are a precondition (0 <= idx < rows of its table,
 *     offsets non-decreasing); they are not checked on the hot path.
 *     dlrm_check_indices() validates them on the device.
 *   - Results are bitwise deterministic run to run.  Calls on different
 *     streams are safe when their outputs do not overlap.
 *   - Row-major everywhere.  "ld" arguments are leading dimensions in
 *     elements of the array's own type.
 */
#ifndef DLRM_H_
#define DLRM_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DLRM_ABI_VERSION 5

enum {
  DLRM_OK = 0,
  DLRM_E_INVALID = -1,
  DLRM_E_WORKSPACE = -2,
  DLRM_E_HIP = -3,
  DLRM_E_UNSUPPORTED = -4
};

/* element types (DLRM_I8: table rows only, with a per-row fp32 scale and bias) */
enum { DLRM_F32 = 0, DLRM_BF16 = 1, DLRM_I8 = 2 };

/* activation after a layer */
enum { DLRM_ACT_NONE = 0, DLRM_ACT_RELU = 1 };

int dlrm_abi_version(void);
const char* dlrm_strerror(int status);
/* hipError_t of the last failed launch on this thread (0 if none). */
int dlrm_last_hip_error(void);

/*
 * Embedding lookup with sum pooling (forward).
 * [EXPL] Key Method Details, "Embedding tables"; [SU] How it works: each
 * categorical feature k has its own table T_k of m_k rows of width d and
 * looks up rows by integer id.  Several ids in one bag are summed; a bag of
 * one id is exactly the row lookup.
 *
 *   tables   device array of K device pointers; T_k is fp32 [m_k][d],
 *            16-byte aligned.
 *   indices  int64 [nnz], table-major.
 *   offsets  int64 [K*B + 1], non-decreasing, offsets[0] = 0: bag (k, b)
 *            owns indices[offsets[k*B+b] .. offsets[k*B+b+1]).
 *   nnz      offsets[K*B] if the caller knows it on the host, else -1: it
 *            only sizes the work split (bags per lane group) and never
 *            bounds a read.
 *   out      fp32; bag (k, b) is written to
 *            out[b*out_ld + out_col0 + k*d + c], c < d (out_ld >= out_col0
 *            + K*d; out and out_ld*4, out_col0*4 must keep 16-byte alignment).
 *   Result:  out = sum over the bag's ids in ascending position of the rows,
 *            accumulated in fp32 from +0.0 (empty bag: +0.0).  Bit-exact.
 *   Limits:  d % 4 == 0, 4 <= d <= 1024, K >= 1, B >= 1.
 */
int dlrm_embbag_fwd(const float* const* tables, int32_t K, int32_t d, const int64_t* indices,
                    const int64_t* offsets, int64_t B, int64_t nnz, float* out, int64_t out_ld, int64_t out_col0,
                    hipStream_t stream);

/*
 * Embedding lookup with sum pooling from low-precision table rows.
 * Quantised tables are what a bandwidth-bound recommendation model gains
 * from ([ML1] "Deep Learning Recommendation Model for Personalization and
 * Recommendation Systems", mlsanity summary, Citations in the corpus: a
 * survey of quantisation methods cites the model as a bandwidth-bound
 * problem where quantisation pays).  Each value read is first turned into fp32, then
 * pooled exactly as dlrm_embbag_fwd (fp32, bag order, from +0.0):
 *   DLRM_BF16  T_k is bf16 [m_k][d] (2 bytes per value): widened exactly.
 *   DLRM_I8    T_k is int8 [m_k][d] (1 byte per value) and scale_bias[k] is
 *              fp32 [m_k][2] = (s, z) per row: value = (s * q) + z, rounded
 *              to fp32 after the product and again after the sum (no fused
 *              multiply-add).
 * Bit-exact.  Arguments as dlrm_embbag_fwd; tables hold K device pointers to
 * 16-byte aligned tables of table_dtype; scale_bias (DLRM_I8 only, else
 * ignored) K device pointers to 8-byte aligned fp32 [m_k][2].  Other
 * table_dtype values: DLRM_E_INVALID.
 */
int dlrm_embbag_fwd_lp(const void* const* tables, int32_t table_dtype, const float* const* scale_bias, int32_t K,
                       int32_t d, const int64_t* indices, const int64_t* offsets, int64_t B, int64_t nnz, float* out,
                       int64_t out_ld, int64_t out_col0, hipStream_t stream);

/*
 * Pairwise dot-product interaction, packed strict lower triangle, concat.
 * [SU] Key equations, Interaction: Z = tril(X X^T), X = [x_dense; e_1..e_K]
 * of shape n x d, n = K + 1.  [EXPL] Key Method Details, "Interaction
 * layer": only pairs of distinct vectors, n(n-1)/2 values.  [SU] Key
 * equations, Output: the top MLP input is [x_dense, vec(Z)].
 *
 *   X        fp32, sample b's matrix at X + b*x_ld, rows of d floats
 *            (x_ld >= n*d, x_ld % 4 == 0, 16-byte aligned).
 *   out      DLRM_F32 or DLRM_BF16 (out_dtype), sample b's row at
 *            out + b*out_ld: out[c] = X_b[0][c] for c < d, then
 *            out[d + i(i-1)/2 + j] = sum_c X_b[i][c] X_b[j][c] for j < i < n.
 *            out_ld >= d + n(n-1)/2.  Columns beyond that (up to out_ld) are
 *            written with zeros up to the next multiple of 8.
 *   Accuracy: every fp32 value is split exactly into three bf16 parts
 *            (x = h + m + l) and the six products hh, hm, mh, hl, mm, lh are
 *            summed in fp32 by bf16 MFMAs; the dropped terms (ml, lm, ll)
 *            are below 2^-20 |x_ic x_jc| each, so
 *            |err| <= (2^-20 d + 2^-24 (d + 24)) sum_c |x_ic x_jc|, below
 *            1e-5 sum_c |x_ic x_jc| for d <= 256.  Small integers (and other
 *            values with at most 8 significant bits) give exact results.
 *   Limits:  2 <= n <= 128, d % 4 == 0, 4 <= d <= 256.
 */
int dlrm_interact_fwd(const float* X, int64_t B, int32_t n, int32_t d, int64_t x_ld, void* out,
                      int32_t out_dtype, int64_t out_ld, hipStream_t stream);

/*
 * Pairwise dot-product interaction, backward.
 * The training pass through the interaction above: [SU] Key equations,
 * Interaction and Output give the forward map X -> [X_0, Z]; the model is
 * trained on binary cross-entropy ([EXPL] Key Method Details, Loss), so the
 * top MLP returns g, the gradient of its input row, and by the chain rule
 *   dX[i][c] = [i == 0] g[c] + sum over j != i of g_pair(i, j) * X[j][c],
 *   g_pair(i, j) = g[d + a(a-1)/2 + b], a = max(i, j), b = min(i, j).
 * dX rows 1..n-1 are the gradients of the pooled embeddings (the input of
 * dlrm_embbag_bwd_sgd), row 0 the gradient of the bottom MLP's output.
 *
 *   X        fp32, sample b's forward input at X + b*x_ld, rows of d floats
 *            (x_ld >= n*d, x_ld % 4 == 0, 16-byte aligned).
 *   g        fp32, sample b's gradient row at g + b*g_ld, g_ld >= d + n(n-1)/2.
 *   dX       fp32 out, sample b's rows at dX + b*dx_ld (dx_ld >= n*d).
 *   Accuracy: fp32 products and accumulation
 *            (|err| <= n u (sum over j of |g_pair(i, j) X[j][c]| + |g[c]|)).
 *   Limits:  2 <= n <= 128, d % 4 == 0, 4 <= d <= 256, and one sample's
 *            n (d + 16) + n(n-1)/2 floats within the 160 KB of LDS
 *            (DLRM_E_UNSUPPORTED otherwise, e.g. n = 128 with d = 256).
 */
int dlrm_interact_bwd(const float* X, int64_t B, int32_t n, int32_t d, int64_t x_ld, const float* g, int64_t g_ld,
                      float* dX, int64_t dx_ld, hipStream_t stream);

/*
 * Fused pooled lookup and interaction (forward).
 * The same result as dlrm_embbag_fwd into X rows 1..K followed by
 * dlrm_interact_fwd, with X row 0 = x_dense, but X never goes to memory:
 * each sample's K pooled rows are summed straight into the registers that
 * feed the Gram MFMAs.  Pooled values are bit-identical to dlrm_embbag_fwd
 * (fp32, bag order, from +0) and the output bit-identical to the two-call
 * path.  ([SU] Limitations & trade-offs: the model is memory-bound, so the
 * round trip of X through HBM is the cost this call removes.)
 *
 *   x_dense  fp32 [B][xd_ld], d floats per sample (the bottom MLP output).
 *   tables, K, d, indices, offsets, B: as dlrm_embbag_fwd.
 *   out, out_dtype, out_ld: as dlrm_interact_fwd with n = K + 1.
 *   Limits:  K + 1 <= 128, d % 4 == 0, 4 <= d <= 256, and
 *            ceil((K+1)/16) * ceil(d/16) <= 32 (register-resident layout);
 *            DLRM_E_UNSUPPORTED otherwise.
 */
int dlrm_embbag_interact_fwd(const float* x_dense, int64_t xd_ld, const float* const* tables, int32_t K, int32_t d,
                             const int64_t* indices, const int64_t* offsets, int64_t B, void* out, int32_t out_dtype,
                             int64_t out_ld, hipStream_t stream);

/*
 * Fused pooled lookup and interaction from low-precision table rows: the
 * rows of dlrm_embbag_fwd_lp (bf16 widened exactly, or int8 with per-row
 * scale and bias, two fp32 roundings) pooled as dlrm_embbag_fwd_lp (bit for
 * bit, in registers) and interacted as dlrm_embbag_interact_fwd, with one
 * difference: each lane feeds the Gram MFMAs eight consecutive columns of a
 * row (one load of a low-precision row), so the pairs are summed in another
 * order than by dlrm_interact_fwd and agree with it within the same
 * dot-product bound, not bit for bit.  table_dtype and scale_bias as
 * dlrm_embbag_fwd_lp; other arguments as dlrm_embbag_interact_fwd.  The
 * output must be bf16 (the top MLP's input) and d a multiple of 32 (each
 * lane loads eight consecutive columns of a row), DLRM_E_UNSUPPORTED
 * otherwise.
 */
int dlrm_embbag_interact_fwd_lp(const float* x_dense, int64_t xd_ld, const void* const* tables, int32_t table_dtype,
                                const float* const* scale_bias, int32_t K, int32_t d, const int64_t* indices,
                                const int64_t* offsets, int64_t B, void* out, int32_t out_dtype, int64_t out_ld,
                                hipStream_t stream);

/*
 * Multilayer perceptron, forward.
 * [EXPL] Key Method Details, "Bottom MLP" (FC layers with ReLU, output
 * width d) and "Top MLP" (FC layers with ReLU ending in a sigmoid); [SU] Key
 * equations, Output: y = sigma(MLP_top(...)).
 *
 * Layer l (0 <= l < L) maps width dims[l] to dims[l+1]:
 *     y = act(x W_l^T + b_l),  act = ReLU for l < L-1, last_act for l = L-1.
 *   in       [B][in_ld] of in_dtype (DLRM_F32 or DLRM_BF16), 16-byte aligned
 *            when bf16 with in_ld % 8 == 0 (other layouts take a slower path).
 *   dims     host [L+1].
 *   W        host array of L device pointers, W_l is w_dtype [dims[l+1]][w_ld[l]].
 *   w_ld     host [L] or NULL (then w_ld[l] = dims[l]).
 *   bias     host array of L device pointers, fp32 [dims[l+1]].
 *   w_dtype  DLRM_BF16: inputs of every layer are rounded to bf16 (nearest
 *            even), products are exact, sums fp32 (MFMA); hidden activations
 *            are stored as bf16.  DLRM_F32: everything fp32.
 *   out      fp32 [B][out_ld], the last layer's output (the logit when
 *            dims[L] == 1 and last_act == DLRM_ACT_NONE).
 *   prob     nullable fp32 [B]; when dims[L] == 1 receives 1/(1+exp(-out)).
 *   ws       workspace of dlrm_mlp_workspace_size() bytes (256-byte aligned).
 *   save_acts != 0 keeps every layer's input in ws for dlrm_mlp_bwd.
 *   bf16 networks ending in a hidden layer of at most 256 outputs and a
 *   single-output layer run those two layers as one launch: the hidden
 *   values are rounded to bf16 exactly as when stored, and the logit is
 *   their fp32 sum of products with the last weight row (a fixed order:
 *   per lane over its columns, then lane pairs, then four column groups)
 *   plus the bias; its last bits can differ from dlrm_linear_fwd's
 *   single-output kernel.  The hidden rows are written to ws only with
 *   save_acts.
 */
size_t dlrm_mlp_workspace_size(int64_t B, int32_t L, const int32_t* dims, int32_t w_dtype, int32_t save_acts);
int dlrm_mlp_fwd(const void* in, int32_t in_dtype, int64_t in_ld, int64_t B, int32_t L, const int32_t* dims,
                 const void* const* W, const int32_t* w_ld, const float* const* bias, int32_t w_dtype,
                 int32_t last_act, float* out, int64_t out_ld, float* prob, void* ws, size_t ws_bytes,
                 int32_t save_acts, hipStream_t stream);

/*
 * One fully connected bf16 layer, the building block of the bf16 MLPs above
 * (dlrm_mlp_fwd runs each of its bf16 layers with the same kernels, except
 * a last hidden layer of at most 256 outputs and the single-output layer
 * after it, which share one launch):
 *     C = act(A W^T + b)
 * ([EXPL] Key Method Details, "Bottom MLP" / "Top MLP": FC layers with ReLU.)
 *   A        bf16 [M][lda] (lda >= K), the layer input.
 *   W        bf16 [N][ldw] (ldw >= K), one K-contiguous row per output.
 *   bias     nullable fp32 [N] (NULL: zero).
 *   C        out_dtype DLRM_F32 or DLRM_BF16 (bf16: rounded to nearest
 *            even after bias and activation), [M][ldc], ldc >= N.
 *   act      DLRM_ACT_NONE or DLRM_ACT_RELU.
 *   Products of bf16 values are exact; they are summed in fp32 (MFMA),
 *   starting from the bias.  N == 1 takes a dot-product kernel (fp32 output
 *   only; DLRM_E_INVALID for bf16) that adds the bias last.  16-byte aligned A and W with lda, ldw
 *   multiples of 8 take the fast MFMA kernel, anything else a generic one.
 *   Limits: M >= 1, N >= 1, K >= 1, M, N, K < 2^31.
 */
int dlrm_linear_fwd(const void* A, int64_t lda, const void* W, int64_t ldw, const float* bias, void* C,
                    int32_t out_dtype, int64_t ldc, int64_t M, int32_t N, int32_t K, int32_t act,
                    hipStream_t stream);

/*
 * Multilayer perceptron, backward (bf16 networks).
 * Training minimises binary cross-entropy ([EXPL] Key Method Details,
 * "Loss"); the caller passes dY = dLoss/d(out) (for BCE on the logit,
 * (sigma(logit) - y) / B).
 *
 *   fwd_ws   the workspace of a dlrm_mlp_fwd call with save_acts != 0 and the
 *            same B, L, dims; out/out_ld that call's output (used for the
 *            last layer's ReLU mask when last_act == DLRM_ACT_RELU).
 *   dY       fp32 [B][dy_ld].
 *   dW       host array of L device pointers, fp32 [dims[l+1]][dims[l]]:
 *            dW_l = delta_l^T x_l (overwritten).
 *   db       host array of L device pointers, fp32 [dims[l+1]] (overwritten).
 *   dX       nullable fp32 [B][dx_ld], gradient w.r.t. the MLP input.
 *   delta_l = g_l * 1[y_l > 0] on ReLU layers; g_{l-1} = delta_l W_l.  The
 *   GEMMs take bf16 operands (delta rounded to bf16) with fp32 sums.
 *   db_l sums delta_l over the batch in fp32: the fp32 delta of the last
 *   layer, the bf16-rounded delta (the GEMM operand) of the others.
 *   ws       dlrm_mlp_bwd_workspace_size() bytes: the two delta buffers
 *            and, per layer, its weight-gradient partials (one slice of the
 *            batch each) and bias-gradient partials, which one launch after
 *            the last layer adds up in a fixed order (dW and db are written
 *            only then).
 */
size_t dlrm_mlp_bwd_workspace_size(int64_t B, int32_t L, const int32_t* dims);
int dlrm_mlp_bwd(int64_t B, int32_t L, const int32_t* dims, const void* const* W, const int32_t* w_ld,
                 int32_t last_act, const void* fwd_ws, const float* out, int64_t out_ld, const float* dY,
                 int64_t dy_ld, float* const* dW, float* const* db, float* dX, int64_t dx_ld, void* ws,
                 size_t ws_bytes, hipStream_t stream);

/*
 * Gradient of the mean binary cross-entropy w.r.t. the logit.
 * [EXPL] Key Method Details, "Loss": binary cross-entropy on the click
 * probability sigma(logit) ([SU] Key equations, Output).  For
 *   loss = -(1/B) sum_b [y_b log s_b + (1 - y_b) log(1 - s_b)],  s_b = sigma(logit_b)
 * the derivative is dY[b] = (s_b - y_b) / B.
 *   logit    fp32 [B] with stride logit_ld; y fp32 [B] (0 or 1); dY fp32 [B].
 */
int dlrm_bce_grad(const float* logit, int64_t logit_ld, const float* y, int64_t B, float* dY, hipStream_t stream);

/*
 * Sparse embedding backward with row-wise SGD, in place.
 * Sum pooling passes each bag's gradient unchanged to every row it looked
 * up, once per occurrence ([EXPL] Key Method Details, Embedding tables;
 * Loss).  For every row r of table k that the batch touches, with x_i =
 * G[b(p_i)*g_ld + g_col0 + k*d + c] for r's occurrences p_0 < p_1 < ... in
 * table k's bags:
 *     S_j = x_{128j} + ... + x_{128j+127} (to the last occurrence), in
 *           order, fp32 from +0.0
 *     g   = S_0 + S_1 + ..., in order, fp32 from +0.0
 *     T_k[r][c] <- T_k[r][c] - (lr * g[c])         (two fp32 roundings)
 * (the pages fix no order for the sum; up to 129 occurrences this is the
 * plain left-to-right sum).  Computed by a stable radix sort of (table,
 * row) keys and a run-length segmentation; the blocks of long rows are
 * summed in parallel.  Untouched rows are not written.  Bit-exact and
 * deterministic.
 *
 *   tables   device array of K device pointers, fp32 [m_k][d], updated.
 *   rows     host [K], m_k (bounds the key width: K * max m_k < 2^32).
 *   indices, offsets, B as for dlrm_embbag_fwd; nnz = offsets[K*B] (host).
 *   G        fp32 [B][g_ld]; bag (k, b)'s gradient at G[b*g_ld + g_col0 + k*d].
 *            B * g_ld * 4 < 2^31.
 *   ws       dlrm_embbag_bwd_sgd_workspace_size() bytes for this d (256-byte
 *            aligned).
 *   Limits:  d % 4 == 0, 4 <= d <= 1024, nnz < 2^31.
 */
size_t dlrm_embbag_bwd_sgd_workspace_size(int32_t K, int64_t B, int64_t nnz, int32_t d);
int dlrm_embbag_bwd_sgd(float* const* tables, int32_t K, int32_t d, const int64_t* rows, const int64_t* indices,
                        const int64_t* offsets, int64_t B, int64_t nnz, const float* G, int64_t g_ld,
                        int64_t g_col0, float lr, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * dlrm_embbag_bwd_sgd in two calls, for callers that overlap the index work
 * with the forward and dense backward: the sort, segmentation and hot-row
 * list depend on the indices only, not on the gradient.
 *
 * dlrm_embbag_bwd_sgd_prepare: the (table, row) keys, their stable radix
 *   sort, the segments and the list of long segments, into ws.  Reads
 *   indices and offsets only (K, rows, indices, offsets, B, nnz as for
 *   dlrm_embbag_bwd_sgd).
 * dlrm_embbag_bwd_sgd_apply: the per-row gradient sums and the update, from
 *   a workspace that a prepare call with the same K, rows, B and nnz filled
 *   and that nothing changed since (the caller orders the two calls, e.g.
 *   by an event when they run on different streams).  The result is bit for
 *   bit that of dlrm_embbag_bwd_sgd; the workspace stays prepared, so
 *   applying it again updates the same rows again (a second SGD step with
 *   the same indices).
 *   side (nullable): a second stream of the caller.  NULL: everything runs
 *   on `stream`.  Otherwise the long segments (Zipf heads) run on `stream`
 *   and the short ones on `side` at the same time; the two touch disjoint
 *   rows.  The caller orders `side` after everything the call depends on
 *   (e.g. hipStreamWaitEvent(side, e) on an event e recorded on `stream`
 *   just before the call) and its later work after both streams (the same
 *   in reverse).  The library creates no stream and no event.
 * Same arguments, limits and error codes as dlrm_embbag_bwd_sgd.
 */
int dlrm_embbag_bwd_sgd_prepare(int32_t K, const int64_t* rows, const int64_t* indices, const int64_t* offsets,
                                int64_t B, int64_t nnz, void* ws, size_t ws_bytes, hipStream_t stream);
int dlrm_embbag_bwd_sgd_apply(float* const* tables, int32_t K, int32_t d, const int64_t* rows, int64_t B, int64_t nnz,
                              const float* G, int64_t g_ld, int64_t g_col0, float lr, void* ws, size_t ws_bytes,
                              hipStream_t stream, hipStream_t side);

/*
 * dlrm_embbag_bwd_sgd without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving or
 * training loops, harnesses that forbid allocation).  The workspace lives
 * in a static device array of DLRM_NOALLOC_SCRATCH_MB MiB inside the
 * library: each GPU the library runs on holds one until the process ends.
 * The call allocates nothing (no hipMalloc, no hipFree).  Arguments, limits
 * and results as dlrm_embbag_bwd_sgd (bit for bit the same table rows);
 * nnz needing more scratch than the array holds (about 8.0 million lookups
 * at d = 128, 10.2 million at d = 16, 3.0 million at d = 1024) returns
 * DLRM_E_WORKSPACE before anything is enqueued.  Every call on one
 * GPU shares that GPU's array and leaves its contents behind: calls that
 * overlap on one GPU (on different streams, or from different threads
 * without ordering) race and are not allowed.
 */
#define DLRM_NOALLOC_SCRATCH_MB 256
int dlrm_embbag_bwd_sgd_noalloc(float* const* tables, int32_t K, int32_t d, const int64_t* rows,
                                const int64_t* indices, const int64_t* offsets, int64_t B, int64_t nnz,
                                const float* G, int64_t g_ld, int64_t g_col0, float lr, hipStream_t stream);

/*
 * Validate indices and offsets on the device.  rows_dev: device int64 [K].
 * Adds to *bad_count (device int64, caller zeroes it) the number of indices
 * outside [0, rows[k]) plus the number of decreasing offset steps, plus one
 * if offsets[0] != 0.
 */
int dlrm_check_indices(const int64_t* indices, const int64_t* offsets, int32_t K, int64_t B,
                       const int64_t* rows_dev, int64_t* bad_count, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* DLRM_H_ */
