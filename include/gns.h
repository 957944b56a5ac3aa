/*
 * gns.h -- C ABI of the MI355X (gfx950) Gram Newton-Schulz library.
 *
 * The library orthogonalises batches of n x m matrices the way the
 * Muon family of optimisers does: it approximates polar(X) = U V^T
 * ("Dion3: Full-Stack Orthogonal Updates", §2.1 Definition 1) with a fixed
 * number T of odd quintic steps p_t(x) = a_t x + b_t x^3 + c_t x^5
 * (same paper, §2.2).  Two algorithms are exported:
 *
 *   gns_gram_batched      Gram Newton-Schulz (Dion3 §4, Algorithms 2 and 3):
 *                         iterate on the n x n Gram matrix R = X X^T and the
 *                         accumulated polynomial Q, restart at the given
 *                         iterations (§4.2, Appendix B.2), return Q_T X.
 *   gns_standard_batched  standard Newton-Schulz (Dion3 §2.2, Algorithm 1),
 *                         the comparison path.
 *
 * Both optionally work on a row subset of every matrix (Dion3 §6,
 * Algorithm 4: orthogonalise M[S,:] only).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers marked (device) are HIP device pointers; (host) are host
 *   pointers read before the call returns.
 * - X and out are contiguous row-major [batch][n][m] in the I/O dtype.
 * - The caller owns every buffer, including the workspace; the library never
 *   allocates or frees device memory and never synchronises the stream
 *   (GNS_OPT_DEBUG_CHECKS and a first GNS_OPT_TILE_AUTOTUNE call aside).
 *   The call returns once its work is enqueued; results are ready when
 *   `stream` is.  With batch >= 2 (and without GNS_OPT_ONE_STREAM) the two
 *   halves of the batch run on two streams that the library creates once per
 *   device: they start after everything already enqueued on `stream`, and
 *   `stream` waits for both before anything enqueued on it later, so the
 *   caller sees the same ordering as if all work ran on `stream`.  The
 *   halves then fill each other's idle CUs in the last, partial wave of
 *   tiles of every launch.  Every host thread has its own two streams per
 *   device (created on its first such call, kept until the process ends),
 *   so calls from different threads neither serialise on shared streams nor
 *   enter another thread's graph capture.
 * - Argument errors are detected on the host before anything is enqueued
 *   (no partial work) and reported as a status code; nothing throws across
 *   the ABI.  A failed kernel launch returns GNS_E_HIP.  Faults inside
 *   kernels surface at the caller's next synchronisation.
 * - out may be the same buffer as X (in place): no product reads X after
 *   the final product starts writing out.  Where the final product would
 *   otherwise read X itself (16-bit X in the compute type, whole 256-edge
 *   tiles, no restart), the input pass first copies X into the workspace;
 *   results are bit-identical to the out-of-place call.  A partial overlap
 *   of X and out returns GNS_E_ALIAS, as does any overlap of the workspace
 *   with X or out.
 * - Results are deterministic for a fixed shape, dtype and option set (no
 *   atomics, fixed reduction order).
 * - batch == 0 is a no-op that returns GNS_OK (pointers may then be NULL).
 * - Calls that share one workspace must be ordered on one stream; calls with
 *   separate workspaces are independent and thread-safe.
 */
#ifndef GNS_H_
#define GNS_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GNS_ABI_VERSION 2   /* 2: gns_plan_info gained gram_tile */

typedef enum {
  GNS_F32 = 0,   /* IEEE binary32                          */
  GNS_BF16 = 1,  /* bfloat16 (8-bit exponent, 7-bit mantissa) */
  GNS_F16 = 2,   /* IEEE binary16                          */
  GNS_BF16X3 = 3 /* compute type only: every matrix the method forms is kept
                    as a pair of bf16 planes hi + lo (hi = bf16(v), lo =
                    bf16(v - hi)), and every product sums the three bf16
                    MFMA terms hi*hi + hi*lo + lo*hi in fp32.  About 16
                    significant bits at three times the bf16 MFMA work: the
                    accurate mode for ill-conditioned inputs, where forming
                    X X^T squares the condition number ("Dion3", Appendix
                    B.2.2).  Uses 128-edge tiles. */
} gns_dtype;

typedef enum {
  GNS_OK = 0,
  GNS_E_NULL = 1,      /* a required pointer is NULL                          */
  GNS_E_SHAPE = 2,     /* n < 1, m < 1, k not in [1, n], or too large        */
  GNS_E_DTYPE = 3,     /* unknown dtype                                       */
  GNS_E_COEFF = 4,     /* T < 1, T > GNS_MAX_ITERS, or a non-finite coeff.    */
  GNS_E_RESTART = 5,   /* restart list not strictly increasing in [1, T-1]    */
  GNS_E_ROWIDX = 6,    /* row index out of range or repeated (check call)     */
  GNS_E_ALIAS = 7,     /* workspace overlaps X or out, or out overlaps X
                          without being the same buffer                      */
  GNS_E_WORKSPACE = 8, /* workspace NULL or smaller than gns_*_workspace_bytes */
  GNS_E_HIP = 9,       /* a HIP launch or runtime call failed                 */
  GNS_E_FLAGS = 10,    /* unknown option bit, or GNS_OPT_DEBUG_CHECKS on a
                          stream that is being captured into a graph         */
  GNS_E_PARAM = 11,    /* non-finite update hyperparameter, or eps <= 0 with
                          NorMuon (gns_dion3_step); bad safety factor        */
  GNS_E_NONFINITE = 12 /* GNS_OPT_DEBUG_CHECKS only: the result holds Inf or
                          NaN.  Half-precision Gram Newton-Schulz without
                          restarts can blow up this way ("Dion3", Appendix
                          B.1, Figs. 11-12); a restart, or a second one,
                          usually cures it (Appendix B.2).                   */
} gns_status;

#define GNS_MAX_ITERS 64

/* Option bits for gns_gram_batched. */
#define GNS_OPT_NAIVE_ALGEBRA 0x1u /* Algorithm 2 algebra: Z = aI + bR + cR^2,
                                      Q <- QZ, R <- ZRZ (default: Algorithm 3's
                                      reformulation with explicit a-terms,
                                      Dion3 Appendix B.2.3); gns_gram_batched only */
#define GNS_OPT_NO_SQUARE_FALLBACK 0x2u /* run Gram NS even when the orthogonalised
                                      matrix is square (by default a square
                                      problem runs standard NS, which costs the
                                      same there, Dion3 §4.1); gns_gram_batched only */
#define GNS_OPT_ONE_STREAM 0x4u    /* enqueue everything on `stream` itself
                                      instead of splitting the batch over the
                                      library's two streams (see below)      */
#define GNS_OPT_TILE_128 0x10u     /* force 128 x 128 output tiles            */
#define GNS_OPT_TILE_256 0x20u     /* force 256 x 256 output tiles            */
#define GNS_OPT_TILE_AUTOTUNE 0x40u /* pick the tiles by timing (see
                                      gns_tuned_tile); gns_gram_batched and
                                      gns_standard_batched only, not with
                                      another TILE bit                        */
#define GNS_OPT_TILE_MIXED 0x80u   /* 256 x 256 tiles for the products Q X
                                      (restart and final), 128 x 128 tiles for
                                      the symmetric ones (Gram matrix, n x n
                                      iteration)                              */
#define GNS_OPT_DEBUG_CHECKS 0x100u /* synchronous checks (gns_gram_batched,
                                      gns_standard_batched, gns_dion3_step):
                                      before enqueueing, a row subset is
                                      checked (GNS_E_ROWIDX on a repeated or
                                      out-of-range index; rows <= 65536 only);
                                      after the call, the output (the selected
                                      rows of out; for gns_dion3_step the update
                                      O, before it reaches W) is checked for Inf
                                      and NaN (GNS_E_NONFINITE).  Both
                                      synchronise `stream`, so the bit is
                                      refused while `stream` is being captured
                                      (GNS_E_FLAGS).  A debugging aid: the
                                      default mode never synchronises. */
/* At most one TILE bit.  Without one the library picks from the problem
   size: 256-edge tiles once the symmetric products have 64 upper 256-edge
   tiles over the batch; of those, the symmetric products run 128-edge tiles
   while they have fewer 256-edge tiles than the GPU has compute units (256)
   and the orthogonalised side is at most 2048, so that they fill it.  The
   tile edges do not change the arithmetic.  fp32 and split-bf16 compute
   always run 128-edge tiles (GNS_OPT_TILE_256 and GNS_OPT_TILE_MIXED are
   ignored there). */

/* Version of this ABI (GNS_ABI_VERSION). */
int gns_abi_version(void);

/* Static string naming a status code. */
const char *gns_status_str(gns_status s);

/*
 * Workspace bytes that gns_gram_batched needs for this problem.
 *   rows = k when a row subset is used, else n.  Returns 0 for invalid
 *   arguments (rows < 1, m < 1, unknown dtype) and for batch == 0.
 */
size_t gns_gram_workspace_bytes(gns_dtype compute_dtype, int64_t batch, int64_t rows, int64_t m);

/* Same for gns_standard_batched. */
size_t gns_standard_workspace_bytes(gns_dtype compute_dtype, int64_t batch, int64_t rows, int64_t m);

/*
 * Gram Newton-Schulz on a batch (Dion3 §4.2, Algorithm 3; §4 Algorithm 2
 * with GNS_OPT_NAIVE_ALGEBRA).
 *
 *   X          (device) [batch][n][m], io_dtype, read only.
 *   out        (device) [batch][n][m], io_dtype.  Without a row subset every
 *              element is written.  With a row subset only the selected rows
 *              are written; the others keep what the caller put there.
 *   batch      number of matrices (>= 0).
 *   n, m       matrix shape (n, m >= 1).  Dion3 (§2) takes rows <= m without
 *              loss of generality; a tall problem (rows > m, rows = n or k)
 *              is orthogonalised through its transpose, polar(X) =
 *              polar(X^T)^T: the iteration runs on m x m Gram matrices of
 *              X_hat^T (the transposed copy the normalisation writes anyway)
 *              and the last product X_hat Q writes the caller's layout.
 *   io_dtype   dtype of X and out.
 *   compute_dtype  dtype of the matrix products' operands (GNS_BF16 or
 *              GNS_F16: MFMA with fp32 accumulation; GNS_F32: fp32 MFMA;
 *              GNS_BF16X3: hi/lo bf16 pairs, three bf16 MFMAs per product).
 *              Every product accumulates in fp32, applies its a/b/c terms
 *              in fp32 and rounds its result once to compute_dtype (for
 *              GNS_BF16X3: splits it once into hi and lo).
 *   coeffs     (host) T x 3 doubles, row t = (a_t, b_t, c_t) of
 *              p_t(x) = a_t x + b_t x^3 + c_t x^5 (used as given: a safety
 *              factor s is applied by the caller as (a/s, b/s^3, c/s^5),
 *              Dion3 Appendix B.2.2).
 *   T          number of iterations, 1..GNS_MAX_ITERS.
 *   restart_after (host) n_restart iterations s, strictly increasing, each in
 *              [1, T-1]: before iteration s+1 the input is replaced by
 *              Q_s X, R is re-formed from it and Q is reset to I (Dion3
 *              §4.2; its default is {2} for T = 5).  May be NULL when
 *              n_restart == 0.
 *   row_idx    (device) [batch][k] int64 or NULL.  When given, rows
 *              row_idx[b][0..k) of X_b form one k x m matrix, normalised by
 *              its own Frobenius norm (Dion3 §6, Algorithm 4), and its
 *              orthogonalised rows are written to the same rows of out_b.
 *              Indices must be distinct and in [0, n): this is a
 *              precondition (checkable with gns_check_row_idx); kernels
 *              never access memory outside X or out for a bad index (an
 *              out-of-range row reads as zeros and is not written).
 *   k          rows per matrix when row_idx != NULL (1 <= k <= n); ignored
 *              otherwise.
 *   opts       GNS_OPT_* bits.
 *   workspace  (device) >= gns_gram_workspace_bytes(compute_dtype, batch,
 *              rows, m) bytes, 256-byte aligned; contents on entry do not
 *              matter and are clobbered.
 *   stream     HIP stream (hipStream_t) or NULL for the default stream.
 */
gns_status gns_gram_batched(const void *X, void *out, int64_t batch, int64_t n, int64_t m,
                            gns_dtype io_dtype, gns_dtype compute_dtype,
                            const double *coeffs, int T,
                            const int *restart_after, int n_restart,
                            const int64_t *row_idx, int64_t k, unsigned opts,
                            void *workspace, size_t workspace_bytes, void *stream);

/*
 * Standard Newton-Schulz on a batch (Dion3 §2.2, Algorithm 1) with the
 * symmetric products computed once per pair of mirrored tiles (Dion3 §5,
 * Appendix C.3): per iteration A = X X^T, B = b A + c A^2, X <- a X + B X.
 * Arguments as for gns_gram_batched (no restarts; opts takes the TILE bits
 * and GNS_OPT_ONE_STREAM).
 */
gns_status gns_standard_batched(const void *X, void *out, int64_t batch, int64_t n, int64_t m,
                                gns_dtype io_dtype, gns_dtype compute_dtype,
                                const double *coeffs, int T,
                                const int64_t *row_idx, int64_t k, unsigned opts,
                                void *workspace, size_t workspace_bytes, void *stream);

/*
 * The host-side plan of a gns_gram_batched (standard = 0) or
 * gns_standard_batched (standard = 1) call with these arguments, without
 * enqueueing anything and without a workspace or stream: argument errors are
 * returned exactly as the call would return them (workspace checks aside).
 * X and out are compared and their alignment examined, never dereferenced.
 * With GNS_OPT_TILE_AUTOTUNE the plan of the kept choice is reported, or of
 * the size rule while the shape is untuned.  batch == 0 reports zeros.
 */
typedef struct {
  int standard;         /* 1: runs standard Newton-Schulz (that entry point,
                           or the square fallback of gns_gram_batched)        */
  int tile;             /* edge of the rectangular products (128 or 256)      */
  int sym_tile;         /* edge of the symmetric products                     */
  int gram_parts;       /* parts of a Gram matrix split along its contraction
                           (1: not split)                                     */
  int direct_input;     /* 1: the products read X itself, scaled in their
                           epilogues, instead of a normalised copy            */
  int kmajor_products;  /* 1: Q X reads X row-major (no transposed copy)      */
  int input_copy;       /* 1: on the direct path, the input pass copies X
                           (a row subset: its selected rows) into the
                           workspace and the products read the copy: for a
                           row subset, and in place when the final product
                           would read X                                       */
  int split_streams;    /* 1: the batch is split over the library's streams   */
  int autotune_timed;   /* 1: the call would time the tile choices            */
  size_t workspace_bytes; /* workspace this plan uses                         */
  int gram_tile;        /* edge of the Gram matrix's tiles (the size rule
                           keeps 256 where a 128-edge grid would overflow one
                           round of the GPU; else sym_tile)                   */
} gns_plan_info;

gns_status gns_call_plan(int standard, const void *X, const void *out, int64_t batch, int64_t n,
                         int64_t m, gns_dtype io_dtype, gns_dtype compute_dtype,
                         const double *coeffs, int T, const int *restart_after, int n_restart,
                         const int64_t *row_idx, int64_t k, unsigned opts, gns_plan_info *info);

/*
 * gns_gram_batched for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  The workspace is a device array inside the library of
 * GNS_NOALLOC_SCRATCH_BYTES (128 MiB), one per GPU, held from the library's
 * first use of it on that GPU until the process ends; its device address is
 * looked up once per device.  Arguments as for gns_gram_batched, without
 * the workspace.  The call allocates nothing and creates no streams or
 * events: it always runs on `stream` (GNS_OPT_ONE_STREAM is implied) with
 * the size rule's tiles.
 *   - A problem whose gns_gram_workspace_bytes exceeds the array returns
 *     GNS_E_WORKSPACE before anything is enqueued (for example 4 x 1024x4096
 *     bf16 needs 156 MiB; 2 x 1024x4096, 78 MiB, fits).
 *   - GNS_OPT_TILE_AUTOTUNE and GNS_OPT_DEBUG_CHECKS return GNS_E_FLAGS.
 *   - Every call on one GPU shares that GPU's array and leaves its contents
 *     behind; nothing in it needs to start at zero.  Calls that overlap in
 *     time on one GPU (two streams, or two host threads) race on the array
 *     and give wrong results: order them on one stream.
 */
#define GNS_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
gns_status gns_gram_batched_noalloc(const void *X, void *out, int64_t batch, int64_t n, int64_t m,
                                    gns_dtype io_dtype, gns_dtype compute_dtype,
                                    const double *coeffs, int T, const int *restart_after,
                                    int n_restart, const int64_t *row_idx, int64_t k, unsigned opts,
                                    void *stream);

/*
 * Row selection of the Dion3 update ("Dion3: Full-Stack Orthogonal Updates",
 * §6, Algorithm 4, selection step): for every matrix M_b, the indices of the
 * k rows with the largest l1 norm sum_j |M_b[i][j]|, written to
 * row_idx[b][0..k) in ascending order, ready for gns_gram_batched's row
 * subset.  Dion3 (§6, Algorithm 4) takes k = ceil(f n) for a fraction f in (0, 1].
 *   M          (device) [batch][n][m] in dtype (GNS_F32, GNS_BF16, GNS_F16).
 *   row_idx    (device) [batch][k] int64, written.
 *   workspace  (device) >= gns_select_workspace_bytes(batch, n) bytes,
 *              256-byte aligned (the fp64 row norms); clobbered.
 * The row norms are fp64 sums in a fixed order; for 16-bit inputs whose
 * values in a row span less than 2^31 in magnitude they are exact.  Rows
 * with equal norms are taken in index order (the smaller index first), so
 * the selection is deterministic.  Needs 1 <= k <= n, batch <= 65535.
 */
size_t gns_select_workspace_bytes(int64_t batch, int64_t n);
gns_status gns_select_rows_l1(const void *M, int64_t batch, int64_t n, int64_t m, gns_dtype dtype,
                              int64_t k, int64_t *row_idx, void *workspace, size_t workspace_bytes,
                              void *stream);

/*
 * One Dion3 update of a batch of weight matrices ("Dion3: Full-Stack
 * Orthogonal Updates", §6, Algorithm 4), with Gram Newton-Schulz as its
 * orthogonalisation and, when `normuon` is set, the NorMuon steps of §2.1,
 * eq. (2).  For every matrix b, in this order:
 *   1. M <- M + G                              (fp32 additions, stored)
 *   2. S = the k rows of M with the largest l1 norm, ascending (as
 *      gns_select_rows_l1; written to row_idx[b][0..k))
 *   3. O = Gram Newton-Schulz of the k x m matrix M[S,:], normalised by its
 *      own Frobenius norm (as gns_gram_batched with that row subset; square
 *      k = m falls back to standard NS unless GNS_OPT_NO_SQUARE_FALLBACK)
 *   4. NorMuon (optional): v[S_i] <- beta2 v[S_i] + (1 - beta2) mean_j O_ij^2,
 *      O_i <- O_i / (sqrt(v[S_i]) + eps), then O is rescaled to the Frobenius
 *      norm it had before the division (left zero when that is zero)
 *   5. W <- (1 - lr * weight_decay) W          (every row)
 *   6. W[S_i] <- W[S_i] - lr O_i               (selected rows)
 *   7. M[S_i] <- mu M[S_i]                     (error feedback, selected rows)
 *
 *   W          (device) [batch][n][m] fp32, updated in place.
 *   G          (device) [batch][n][m] in grad_dtype (GNS_F32, GNS_BF16 or
 *              GNS_F16), read only.
 *   M          (device) [batch][n][m] fp32 momentum, updated in place.
 *   v          (device) [batch][n] fp32 row second moments, updated at the
 *              selected rows; may be NULL without NorMuon.
 *   n, m, k    matrix shape and rows selected per matrix (1 <= k <= n; the
 *              pages take k = ceil(f n) for a fraction f in (0, 1]).
 *   compute_dtype, coeffs, T, restart_after, n_restart, opts
 *              as for gns_gram_batched (opts: GNS_OPT_NAIVE_ALGEBRA,
 *              GNS_OPT_NO_SQUARE_FALLBACK, GNS_OPT_ONE_STREAM, TILE bits).
 *   lr, weight_decay, mu, beta2, eps
 *              eta, wd, the error-feedback factor mu, and the NorMuon decay
 *              and epsilon; all finite, eps > 0 with NorMuon.
 *   row_idx    (device) [batch][k] int64, written (the selection S).
 *   workspace  (device) >= gns_dion3_workspace_bytes(compute_dtype, batch, n,
 *              m, k) bytes, 256-byte aligned, clobbered.
 * W, G, M, v, row_idx and the workspace must not overlap (GNS_E_ALIAS).
 * Needs batch <= 65535.  Row l1 norms are fp64 sums in a fixed order, so
 * near-equal norms may order differently from an exactly rounded sum; equal
 * norms take the smaller index first.  Everything is enqueued on `stream`
 * (the orthogonalisation may fan out over the library's two streams, as in
 * gns_gram_batched); nothing allocates and nothing synchronises, so the whole
 * step can be captured in a HIP graph.
 */
size_t gns_dion3_workspace_bytes(gns_dtype compute_dtype, int64_t batch, int64_t n, int64_t m,
                                 int64_t k);
gns_status gns_dion3_step(float *W, const void *G, float *M, float *v, int64_t batch, int64_t n,
                          int64_t m, gns_dtype grad_dtype, gns_dtype compute_dtype, int64_t k,
                          const double *coeffs, int T, const int *restart_after, int n_restart,
                          double lr, double weight_decay, double mu, double beta2, double eps,
                          int normuon, int64_t *row_idx, unsigned opts, void *workspace,
                          size_t workspace_bytes, void *stream);

/*
 * Enqueue a check of a row subset: writes to *result (device int32) 0 when
 * every row_idx[b][i] is in [0, n) and the k indices of each matrix are
 * distinct, 1 when an index is out of range, 2 when an index repeats.
 * The caller reads *result after synchronising the stream.  Needs k <= n
 * and n <= 65536.
 */
gns_status gns_check_row_idx(const int64_t *row_idx, int64_t batch, int64_t k, int64_t n,
                             int32_t *result, void *stream);

/*
 * Enqueue a finite check of a [batch][rows][cols] row-major array A in
 * dtype (GNS_F32, GNS_BF16 or GNS_F16): writes to *result (device int32) 1
 * when an element is Inf or NaN, else 0.  With row_idx ([batch][k] int64,
 * device) only those rows are checked (indices outside [0, rows) are
 * skipped).  The caller reads *result after synchronising the stream.  Half
 * precision Gram Newton-Schulz can return Infs ("Dion3", Appendix B.1); this
 * is the enqueue-only form of the check that GNS_OPT_DEBUG_CHECKS runs
 * synchronously.  Needs batch <= 65535.
 */
gns_status gns_check_finite(const void *A, gns_dtype dtype, int64_t batch, int64_t rows, int64_t cols,
                            const int64_t *row_idx, int64_t k, int32_t *result, void *stream);

/*
 * Rows a Dion3 update orthogonalises ("Dion3", §6, Algorithm 4): k = ceil(f
 * n) for a fraction f in (0, 1], clamped to [1, n]; 0 for n < 1 or f outside
 * (0, 1].
 */
int64_t gns_select_count(int64_t n, double fraction);

/*
 * Safety factor ("Dion3", Appendix B.2.2): the coefficients of p_t(x / s),
 * (a_t / s, b_t / s^3, c_t / s^5), so that singular values up to s still
 * converge (the pages use s = 1.02, or 1.05 to be conservative).
 *   coeffs, out  (host) T x 3 doubles (may be the same array).
 * GNS_E_NULL, GNS_E_COEFF (T outside 1..GNS_MAX_ITERS) or GNS_E_PARAM (s not
 * finite and positive).
 */
gns_status gns_safety_scale(const double *coeffs, int T, double s, double *out);

/*
 * Shape-keyed tile autotuning ("DMuon: Efficient Distributed Muon Training
 * with Near-Adam Overhead", §3.3: the best tile shape of the batched Gram NS
 * kernels varies by shape, so it is chosen per shape by measurement).  With
 * GNS_OPT_TILE_AUTOTUNE, the first call of a shape -- entry point, compute
 * and I/O dtypes, batch, rows (k with a row subset, else n) and m -- runs
 * the whole call with each tile choice (128-edge, 256-edge and mixed tiles,
 * see GNS_OPT_TILE_MIXED, and the size rule's own plan, which alone may also
 * cut a small Gram matrix into parts along its contraction), twice each, on
 * `stream` and blocks the host until they end; the choice with the smallest time is kept in a process-wide
 * table, and the caller's `out` holds the result of a run with that choice.
 * Later calls of the shape run the kept choice with no timing.  fp32 and
 * split-bf16 compute have one choice (128) and are never timed.  While
 * `stream` is being captured into a graph, an untuned shape runs the
 * size-based choice and stays untuned.  A failing run returns its status
 * and keeps nothing.  An in-place call (out == X) is never timed (each
 * timed run would orthogonalise the previous run's output again): it runs
 * the kept choice, or the size rule while the shape is untuned, and keeps
 * nothing.
 *
 * gns_tuned_tile returns the kept tile edge of the rectangular products for
 * a shape (standard = 0 for gns_gram_batched, 1 for gns_standard_batched),
 * or 0 if the shape has not been tuned; when sym_edge is not NULL it
 * receives the edge of the symmetric products (0 if untuned).
 * gns_autotune_clear forgets every shape.  Both are thread-safe.
 */
int gns_tuned_tile(int standard, gns_dtype compute_dtype, gns_dtype io_dtype, int64_t batch,
                   int64_t rows, int64_t m, int *sym_edge);
void gns_autotune_clear(void);

/*
 * Optional per-launch timing for measurement tools.  While enabled, every
 * kernel that a gns_*_batched call enqueues is bracketed by HIP events on the
 * call's stream.  gns_timing_read synchronises those events and returns,
 * for each kernel launched since the last reset, its name (static string),
 * its algorithmic FLOP count (2 per multiply-add, symmetric products
 * counted once per output pair), its algorithmic HBM bytes and its duration
 * in milliseconds.  Returns the number of records available (it may exceed
 * cap; only cap are copied).  Not thread-safe; for benchmarking only.
 */
typedef struct {
  const char *name;   /* step of the method, e.g. "syrk", "q_update"       */
  const char *kernel; /* kernel that ran it, e.g. "gemm_nt<bf16,256,sym>" */
  double flops;
  double bytes;
  float ms;
} gns_launch_record;

void gns_timing_enable(int on);
int gns_timing_read(gns_launch_record *records, int cap);
void gns_timing_reset(void);

#ifdef __cplusplus
}
#endif
#endif /* GNS_H_ */
