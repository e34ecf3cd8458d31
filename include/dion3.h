/*
 * dion3.h -- C ABI of the MI355X (gfx950) Dion3 optimizer-step hot path.
 *
 * The method is the one described in "Dion3: Full-Stack Orthogonal Updates"
 * (paper text; section numbers inferred from its cross-references):
 *   momentum   M <- M + G                                  (Section 6)
 *   selection  the k = ceil(f n) rows of largest l1 norm   (Section 6)
 *   Gram Newton-Schulz of M[S,:], restart after iter 2     (Section 4)
 *   update     W[S,:] <- W[S,:] - eta O, one rounding;     (Section 6)
 *              M[S,:] <- mu M[S,:]  (error feedback)
 *
 * Conventions shared by every entry point:
 *   - Matrices are row-major; a "group" is `batch` matrices of one shape laid
 *     out `batch_stride` elements apart.
 *   - Canonical orientation: the selection axis has length n and the other
 *     axis length m.  sel_axis 0 selects rows (n = rows, m = cols), 1 selects
 *     columns (n = cols, m = rows); -1 picks the smaller dimension, rows on a
 *     tie (Section 6: select along the smaller dimension when not sharded).
 *   - All tensor pointers are device pointers owned by the caller; the
 *     library never allocates, frees or retains them.  Scalars and parameter
 *     structs are host values read during the call.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call is
 *     asynchronous and stream-ordered, does no host synchronisation and no
 *     allocation, and is deterministic run to run.  The exceptions are
 *     stated at their declarations: the whole-step calls create the
 *     library's own streams and events when a step on a device first needs
 *     them, dion3_step_graph_create creates graphs, dion3_timing_enable
 *     creates events, dion3_timing_report waits for the recorded events, and
 *     dion3_release waits for and destroys what the library created.
 *   - Return value: DION3_OK (0) or a negative status.  Arguments are
 *     validated before anything is launched; on an error nothing is written.
 *     DION3_ERR_HIP means a launch failed (hipGetLastError was not success).
 *   - A workspace must not be used by two calls that may run concurrently.
 */
#ifndef DION3_H
#define DION3_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { DION3_F32 = 0, DION3_F16 = 1, DION3_BF16 = 2 } dion3_dtype;

enum {
  DION3_OK = 0,
  DION3_ERR_INVALID_ARG = -1,   /* null pointer, size <= 0, k outside [1, n], bad dtype */
  DION3_ERR_UNSUPPORTED = -2,   /* valid but not implemented (e.g. n > 32768 in top-k) */
  DION3_ERR_WORKSPACE = -3,     /* workspace missing or smaller than required */
  DION3_ERR_HIP = -4,           /* a HIP launch or runtime call failed */
  DION3_ERR_TOO_LARGE = -5      /* needs more than the fixed scratch of a no-allocation entry point */
};

/* A batch of same-shape matrices (W, G and M share this description). */
typedef struct {
  int rows, cols;              /* stored shape of each matrix, leading dimension = cols */
  int batch;                   /* number of matrices */
  long long batch_stride;      /* elements between consecutive matrices, >= rows*cols */
  int dtype;                   /* dion3_dtype of W, G and M: DION3_F32 or DION3_BF16 */
  int sel_axis;                /* -1 auto, 0 rows, 1 columns */
} dion3_group;

/* Newton-Schulz parameters (Section 2 polynomial p_t(x) = a_t x + b_t x^3 + c_t x^5;
 * Section 4 restart).  coeffs is a host array [T][3] of (a_t, b_t, c_t).
 * Bit t of restart_mask (1 <= t < T) restarts after iteration t; the pages'
 * setting is T = 5, restart_mask = 1u << 2.  eps guards X / (||X||_F + eps).
 * ns_dtype is the storage type of every Newton-Schulz intermediate:
 * DION3_F16 (the pages' half-precision choice) or DION3_F32. */
typedef struct {
  int T;
  const double* coeffs;
  unsigned restart_mask;
  float eps;
  int ns_dtype;
} dion3_ns_params;

/* Optional finite check (Appendix B, Figure 11: the half-precision Gram
 * iteration without restarts ends with non-finite outputs).  Adds the number
 * of NaN and +-Inf entries of x (n elements of dtype DION3_F32, DION3_F16 or
 * DION3_BF16, device memory, any alignment) to *count, a device uint64 the
 * caller zeroes beforehand; asynchronous on `stream`, allocates nothing.
 * DION3_ERR_INVALID_ARG for a null pointer, n == 0 or another dtype. */
int dion3_count_nonfinite(const void* x, int dtype, size_t n, unsigned long long* count, void* stream);

/* ---------------------------------------------------------------- helpers */

/* k = ceil(f * n) for the exact product of the given double f and n, clamped
 * to [1, n] (Section 6).  Returns k, or DION3_ERR_INVALID_ARG unless n >= 1
 * and 0 < f <= 1. */
int dion3_k_from_fraction(int n, double f);

/* Canonical sizes of a group: *n = length of the selection axis, *m = the
 * other axis, *axis = 0 (rows) or 1 (columns).  Any output pointer may be NULL. */
int dion3_canonical(const dion3_group* g, int* n, int* m, int* axis);

/* Human-readable name of a status code (static storage). */
const char* dion3_status_string(int status);

/* ------------------------------------------------ momentum and selection */

/* Workspace bytes dion3_momentum_rowsel needs for this group (>= 256). */
size_t dion3_rowsel_workspace_bytes(const dion3_group* g);

/* Momentum accumulation fused with the selection keys, then top-k (Section 6).
 *   M      [batch][rows][cols], updated in place: M <- round(M + G), where the
 *          sum is formed in fp32 and rounded once to the storage type.
 *   G      [batch][rows][cols], read only.
 *   idx    out [batch][k] int32: per matrix the k canonical lines with the
 *          largest l1 norm (ties to the lower index, a NaN norm counts as
 *          +infinity), listed in ascending order.
 *   keys   out [batch][n] fp64 l1 norms of the canonical lines (may be NULL).
 *   sel_sqnorm out [batch] fp64: sum of squares of the selected lines of M,
 *          i.e. ||M[S,:]||_F^2 (may be NULL).
 * Norms are accumulated in fp64 in a fixed order.  Requires n <= 32768. */
int dion3_momentum_rowsel(const dion3_group* g, void* M, const void* G, int k,
                          int32_t* idx, double* keys, double* sel_sqnorm,
                          void* ws, size_t ws_bytes, void* stream);

/* Deferred error feedback (Section 6 decays the selected lines of M by mu after
 * the update; this entry point applies that decay at the start of the next
 * step instead, inside the same pass over M).  As dion3_momentum_rowsel, and in
 * addition, when prev_idx is not NULL, every canonical line listed in prev_idx
 * ([batch][prev_k] ascending, the previous step's selection) is first decayed:
 *   M <- round(round(mu * M) + G)        on those lines,
 *   M <- round(M + G)                    on the others,
 * which is bit-identical to decaying after the previous step and accumulating
 * now.  prev_idx may alias idx (it is read before idx is written).  mu is fp32;
 * the product is rounded once. */
int dion3_momentum_rowsel_ef(const dion3_group* g, void* M, const void* G, int k,
                             int32_t* idx, double* keys, double* sel_sqnorm,
                             const int32_t* prev_idx, int prev_k, float mu,
                             void* ws, size_t ws_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): exactly
 * dion3_momentum_rowsel_ef, with its scratch (the per-line partial sums of
 * the selection) in a fixed per-GPU array of DION3_NOALLOC_SCRATCH_BYTES
 * (64 MiB) inside the library instead of a caller's workspace.  Nothing is
 * allocated, freed or cleared by the call; the array is set up on the first
 * call on each device (its address looked up while that device is current)
 * and held until the process ends.  A group whose
 * dion3_rowsel_workspace_bytes exceeds the array returns DION3_ERR_TOO_LARGE
 * before anything is launched (split the batch).  Every call on one GPU uses
 * the same array: calls that may overlap on one GPU (on different streams,
 * or from different threads) race and must be ordered by the caller. */
#define DION3_NOALLOC_SCRATCH_BYTES (64ull << 20)
int dion3_momentum_rowsel_noalloc(const dion3_group* g, void* M, const void* G, int k,
                                  int32_t* idx, double* keys, double* sel_sqnorm,
                                  const int32_t* prev_idx, int prev_k, float mu, void* stream);

/* ------------------------------------------------------- gather + scale */

/* X[b] = M[b][S_b, :] / (sqrt(sel_sqnorm[b]) + eps) in canonical orientation
 * (Section 2: Frobenius normalisation of the Newton-Schulz input).
 *   X      out [batch][k][m] in x_dtype (DION3_F16 or DION3_F32), packed.
 *   sel_sqnorm  [batch] fp64 as produced by dion3_momentum_rowsel. */
int dion3_gather_rows(const dion3_group* g, const void* M, const int32_t* idx, int k,
                      const double* sel_sqnorm, float eps, int x_dtype, void* X,
                      void* stream);

/* -------------------------------------------------- Gram Newton-Schulz */

/* Workspace bytes dion3_gram_ns needs for k selected lines of this group
 * (0 if the arguments are invalid, e.g. k > m). */
size_t dion3_gram_ns_workspace_bytes(const dion3_group* g, int k, const dion3_ns_params* p);

/* One workspace size that serves both dion3_momentum_rowsel and dion3_gram_ns
 * for this group and k (the larger of the two). */
size_t dion3_workspace_bytes(const dion3_group* g, int k, const dion3_ns_params* p);

/* Gram Newton-Schulz of every matrix's selected submatrix (Section 2: the
 * input is normalised by its Frobenius norm; Section 4: Gram iteration with
 * restarts).  Per matrix b, with S = idx[b] ([batch][k] ascending canonical
 * lines, as produced by dion3_momentum_rowsel):
 *   X0 = M[S,:] / (||M[S,:]||_F + p->eps)   (norm accumulated in fp64, fixed
 *        order; X0 rounded once to p->ns_dtype), then dion3_gram_ns_gathered.
 *   M   [batch][rows][cols] in g->dtype (DION3_F32 or DION3_BF16), read only.
 *   O   out [batch][k][m] in p->ns_dtype, canonical orientation, packed.
 * Requires k <= m.  ws holds the sums of squares, X0 and the iteration's
 * buffers (dion3_gram_ns_workspace_bytes).  An index outside [0, n) is
 * treated as an all-zero line. */
int dion3_gram_ns(const dion3_group* g, const void* M, const int32_t* idx, int k,
                  const dion3_ns_params* p, void* O, void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes dion3_gram_ns_gathered needs. */
size_t dion3_gram_ns_gathered_workspace_bytes(int batch, int k, int m, int ns_dtype);

/* Gram Newton-Schulz with restarts (Section 4) on already gathered and
 * normalised inputs (dion3_gather_rows); the whole-step driver uses this form.
 *   X0  [batch][k][m] in p->ns_dtype, k <= m, read only.
 *   O   out [batch][k][m] in p->ns_dtype: the Newton-Schulz output.
 * Per pass on R = X X^T:  Z = a I + b R + c R^2;  Q = Z (first iteration) or
 * Q Z;  R = Z R Z (except on the last iteration); the pass ends X <- Q X.
 * Symmetric products compute the lower triangle and mirror it. */
int dion3_gram_ns_gathered(int batch, int k, int m, const dion3_ns_params* p, const void* X0,
                           void* O, void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes dion3_standard_ns needs. */
size_t dion3_standard_ns_workspace_bytes(int batch, int k, int m, int ns_dtype);

/* Standard Newton-Schulz on the symmetric kernels (Section 2 for the
 * iteration; Section 4 and Appendix C.3: the fall-back used when the aspect
 * ratio m / k is 1).  Arguments as dion3_gram_ns_gathered; p->restart_mask is
 * ignored.
 * Per iteration t: A = X X^T, Z = a_t I + b_t A + c_t A^2, X <- Z X, i.e.
 * X <- a_t X + (b_t A + c_t A^2) X with the a_t X term carried by Z. */
int dion3_standard_ns(int batch, int k, int m, const dion3_ns_params* p, const void* X0,
                      void* O, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------- symmetric building blocks
 * (Section 5: triangular tile schedule, mirrored write-back, diagonal tiles
 * written once.)  dtype: DION3_F16, DION3_BF16 or DION3_F32 for operands and
 * result; accumulation is fp32.  Matrices are packed (leading dim = cols). */

/* C = alpha A A^T + beta C, A [batch][n][kdim], C [batch][n][n] symmetric.
 * With beta == 0, C is not read. */
int dion3_syrk(int batch, int n, int kdim, int dtype, const void* A, long long strideA,
               void* C, long long strideC, float alpha, float beta, void* stream);

/* C = alpha A A + beta B + gamma I for symmetric A, B [batch][n][n]. */
int dion3_sym_sq_add(int batch, int n, int dtype, const void* A, long long strideA,
                     const void* B, long long strideB, void* C, long long strideC,
                     float alpha, float beta, float gamma, void* stream);

/* C = alpha A B for symmetric A, B whose product is symmetric (commuting
 * polynomials of one Gram matrix); the lower triangle is computed and mirrored. */
int dion3_sym_mul(int batch, int n, int dtype, const void* A, long long strideA,
                  const void* B, long long strideB, void* C, long long strideC,
                  float alpha, void* stream);

/* Y = alpha Q X for symmetric Q [batch][k][k] and X [batch][k][m] (the
 * rectangular multiply closing a Gram Newton-Schulz pass).  in_dtype is the
 * dtype of Q and X, out_dtype that of Y (DION3_F16 or DION3_F32 with f16 in,
 * same as input otherwise). */
int dion3_gemm(int batch, int k, int m, int in_dtype, const void* Q, long long strideQ,
               const void* X, long long strideX, int out_dtype, void* Y, long long strideY,
               float alpha, void* stream);

/* ------------------------------------------------------------ the update */

/* Fused-rounding update and error feedback (Section 6).  With
 * u = fp32(1 - eta*wd):
 *   every line of W (only if wd != 0):  a = fp32(u * w)
 *   selected lines:   W <- round(fp32(a - eta * O))   (one fp32 rounding, one cast)
 *                     M <- round(mu * M)              (exact product, one rounding)
 *   other lines:      W <- round(a) if wd != 0, M untouched.
 *   O   [batch] slices of [k][m] (o_stride elements apart), canonical
 *       orientation, o_dtype DION3_F16 or DION3_F32.  eta, wd, mu are fp32.
 *   M may be NULL: W is updated and the decay of M[S,:] is left to the caller
 *   (deferred error feedback, see dion3_momentum_rowsel_ef / dion3_decay_rows). */
int dion3_apply_rows(const dion3_group* g, void* W, void* M, const int32_t* idx, int k,
                     const void* O, int o_dtype, long long o_stride,
                     float eta, float wd, float mu, void* stream);

/* dion3_apply_rows with a factor per row of O (the NorMuon flavour): every
 * selected line uses fp32(row_scale[b][i] * O[b][i][j]) in place of O[b][i][j]
 * (one fp32 product, then the same fused update).  row_scale [batch][k] fp32,
 * may be NULL (then exactly dion3_apply_rows). */
int dion3_apply_rows_scaled(const dion3_group* g, void* W, void* M, const int32_t* idx, int k,
                            const void* O, int o_dtype, long long o_stride, const float* row_scale,
                            float eta, float wd, float mu, void* stream);

/* NorMuon flavour (Section 2: each row of the orthogonalised update is divided
 * by the root of its second moment, an exponential moving average, and the
 * update is rescaled to Muon's Frobenius norm; Section 6: only the selected
 * lines' moments are updated, in fp32).  Per matrix b, selected row i:
 *   q = sum_j O_ij^2 / m;  V[b][idx_i] <- fma(beta2, V[b][idx_i], fp32(1-beta2) * q)
 *   d_i = 1 / (sqrt(V[b][idx_i]) + eps);  r = ||O||_F / ||diag(d) O||_F (1 if 0)
 *   row_scale[b][i] = d_i r
 *   O    [batch] slices of [k][m] (o_stride elements apart), canonical, F16 or F32.
 *   V    in/out [batch][n] fp32: second moment of every line of the selection axis.
 *   row_scale out [batch][k] fp32, for dion3_apply_rows_scaled.
 * 0 <= beta2 <= 1, eps >= 0.  Deterministic (fixed-order reductions). */
int dion3_normuon_scale(const dion3_group* g, const int32_t* idx, int k, const void* O, int o_dtype,
                        long long o_stride, float* V, float beta2, float eps, float* row_scale,
                        void* stream);

/* The error-feedback decay alone, M[S,:] <- round(mu * M[S,:]) for the lines
 * in idx ([batch][k] ascending), one rounding (Section 6).  Completes a
 * deferred decay, e.g. before M is read or saved. */
int dion3_decay_rows(const dion3_group* g, void* M, const int32_t* idx, int k, float mu,
                     void* stream);

/* ------------------------------------------------------------ whole step */

/* Workspace bytes dion3_step needs for these groups (k[i] per group). */
size_t dion3_step_workspace_bytes(int n_groups, const dion3_group* groups, const int* k,
                                  const dion3_ns_params* p);

/* One optimizer step over several groups (Muon flavour of the update rule,
 * Section 6, with Gram Newton-Schulz, Section 4).  For every group i:
 * dion3_momentum_rowsel, dion3_gather_rows; groups whose canonical (k, m)
 * agree are then orthogonalised in one batched dion3_gram_ns call (the pages'
 * megabatching of same-shape matrices, on one GPU; dion3_standard_ns when
 * k = m, the aspect-ratio-1 fall-back of Section 4); finally
 * dion3_apply_rows.  W[i], M[i], G[i] are the group tensors, idx[i] receives
 * the [batch][k[i]] selected indices.  eta, wd, mu as in dion3_apply_rows
 * (one value for all groups).
 * The (k, m) classes are processed in order of increasing momentum traffic
 * (bytes of M of their groups), whatever the order of the groups.
 * Streams: the first class's momentum pass and gather and the last class's
 * update are enqueued on `stream`; the Newton-Schulz products run on a side
 * stream, and the other momentum passes, gathers and updates on a third
 * stream, so that they overlap another class's products; that stream is
 * limited to half of the compute units when those momentum passes move at
 * least 8 GB, and uses every unit otherwise.
 * The library streams belong to the current device; the library creates each
 * (with an event pool) when a step on the device first needs it and keeps
 * them until dion3_release or the end of the process.
 * Graph capture is not supported: a call on a capturing stream
 * returns DION3_ERR_UNSUPPORTED and enqueues nothing (a query of the capture
 * state that fails, e.g. on the legacy null stream while another stream
 * captures, returns DION3_ERR_HIP).  Events order all three against `stream`: when the call
 * returns, everything it enqueued is ordered before later work on `stream`,
 * as if all of it had been enqueued there; `stream` must belong to the
 * current device.  Concurrent calls on one device are serialised while they
 * enqueue.  The workspace (dion3_step_workspace_bytes) holds the selected
 * sums of squares and the NorMuon row factors of every group and, with two or
 * more (k, m) classes, two gathered inputs and two Newton-Schulz outputs, so
 * that the next class's gather and this class's update overlap this class's
 * products. */
int dion3_step(int n_groups, const dion3_group* groups, void* const* W, void* const* M,
               const void* const* G, const int* k, int32_t* const* idx,
               const dion3_ns_params* p, float eta, float wd, float mu,
               void* ws, size_t ws_bytes, void* stream);

/* dion3_step with deferred error feedback: the decay of each step's selected
 * lines is applied by the next step's momentum pass, so the update never
 * touches M.  On entry idx[i] holds the previous step's selection when
 * has_prev != 0 (it is decayed, then overwritten by this step's selection);
 * pass has_prev = 0 on the first step.  After a call, M[i] still owes the
 * decay of the lines in idx[i]: dion3_decay_rows completes it.  The sequence
 * of W, M (once completed) and idx is bit-identical to dion3_step's.  Since
 * the update then leaves M alone, the last Newton-Schulz product of a
 * row-selected bf16 group (whole 256 x 256 tiles) updates W itself instead
 * of writing O, with the same arithmetic as dion3_apply_rows. */
int dion3_step_deferred(int n_groups, const dion3_group* groups, void* const* W, void* const* M,
                        const void* const* G, const int* k, int32_t* const* idx, int has_prev,
                        const dion3_ns_params* p, float eta, float wd, float mu,
                        void* ws, size_t ws_bytes, void* stream);

/* The deferred step as HIP graphs (Section 6: the step's launches have the
 * same dependencies every step, so recorded graphs replace them; the pages
 * replay the step to cut the host time per step).  Nothing is recorded by
 * stream capture: dion3_step_deferred runs once with these arguments while
 * its launches are collected; the kernels one stream receives between two
 * event operations on that stream become one graph (kernel nodes in a
 * chain), instantiated once.  dion3_graph_launch replays the step in the
 * driver's order: each such graph launched on its stream (`stream` for the
 * caller's part, the library's streams, with their compute-unit masks, for
 * the rest) and the driver's event records and waits between them, about a
 * tenth of the eager call's host calls.  It performs exactly that step (same
 * pointers, scalars and has_prev; the buffers' current contents), ordered
 * after earlier work on `stream`; the returned work is complete once
 * `stream` reaches it.  Creation allocates the graphs; launching allocates
 * nothing.  Results are bit-identical to the eager call.  Launch on the
 * device the graph was created on (else DION3_ERR_INVALID_ARG); after
 * dion3_release the graph cannot be launched (DION3_ERR_INVALID_ARG) and
 * should be destroyed.  A graph must not be launched while another launch of
 * it, or an eager step on the same tensors or workspace, may run
 * concurrently.  Steady state: run the first step eagerly (has_prev = 0),
 * then launch a graph created with has_prev = 1 every step.
 * flags: 0, or DION3_GRAPH_ONE for a single graph of the whole step whose
 * stream branches HIP schedules itself (one host call per step; the
 * library's streams and compute-unit masks are not used; faster for small
 * steps, slower for large ones).  Other bits: DION3_ERR_INVALID_ARG. */
#define DION3_GRAPH_ONE 1u
typedef struct dion3_graph_s* dion3_graph;
int dion3_step_graph_create(int n_groups, const dion3_group* groups, void* const* W, void* const* M,
                            const void* const* G, const int* k, int32_t* const* idx, int has_prev,
                            const dion3_ns_params* p, float eta, float wd, float mu,
                            void* ws, size_t ws_bytes, unsigned flags, dion3_graph* out);
int dion3_graph_launch(dion3_graph g, void* stream);
int dion3_graph_destroy(dion3_graph g);

/* The whole step in the NorMuon flavour: dion3_step (deferred = 0) or
 * dion3_step_deferred (deferred = 1, has_prev as there) with
 * dion3_normuon_scale before each group's update.  V[i] is group i's
 * [batch][n] fp32 second-moment state (zero before the first step); beta2 and
 * nm_eps as in dion3_normuon_scale.  Same streams, workspace query and
 * capture restriction as dion3_step. */
int dion3_step_normuon(int n_groups, const dion3_group* groups, void* const* W, void* const* M,
                       const void* const* G, const int* k, int32_t* const* idx, float* const* V,
                       int deferred, int has_prev, const dion3_ns_params* p, float eta, float wd,
                       float mu, float beta2, float nm_eps, void* ws, size_t ws_bytes, void* stream);

/* The deferred NorMuon step (dion3_step_normuon with deferred = 1) as HIP
 * graphs: built, launched (dion3_graph_launch) and destroyed
 * (dion3_graph_destroy) exactly as dion3_step_graph_create's, with V, beta2
 * and nm_eps as in dion3_step_normuon; a launch performs that step on the
 * buffers' current contents, bit-identical to the eager call. */
int dion3_step_normuon_graph_create(int n_groups, const dion3_group* groups, void* const* W, void* const* M,
                                    const void* const* G, const int* k, int32_t* const* idx, float* const* V,
                                    int has_prev, const dion3_ns_params* p, float eta, float wd, float mu,
                                    float beta2, float nm_eps, void* ws, size_t ws_bytes, unsigned flags,
                                    dion3_graph* out);

/* ------------------------------------------------------------- teardown */

/* Destroys what the library created by itself: the whole-step streams and
 * event pool of every device that ran a step, and the timing events.  Call it
 * before the process's HIP runtime shuts down (the Python binding does, at
 * interpreter exit); work already enqueued on the library streams completes
 * first.  A later call of a whole-step entry point creates them again.  Not
 * to be called while another thread runs a library call.  Returns DION3_OK or
 * DION3_ERR_HIP. */
int dion3_release(void);

/* ------------------------------------------------------------ measurement */

/* Per-kernel timing with hipEvents, for benchmarks.  dion3_timing_enable(n)
 * creates a pool of n event pairs (n = 0 disables and frees it); while enabled
 * every launch of the library records an event pair on its stream (none
 * while a step graph is being built).  dion3_timing_report writes one line
 * per kernel name, "name count total_ms\n", into buf (synchronising on the
 * recorded events) and clears the pool.  Returns the bytes written or a
 * negative status.  The pool is process-wide and unsynchronised: enable
 * timing only while one thread issues library calls. */
int dion3_timing_enable(int max_launches);
int dion3_timing_report(char* buf, size_t buf_bytes);

#ifdef __cplusplus
}
#endif

#endif /* DION3_H */
