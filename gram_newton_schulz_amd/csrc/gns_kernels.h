// Internal interface between the host orchestration (gns_host.cpp) and the
// device kernels (gns_kernels.hip).  Not part of the public ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gns {

// DT_BF16X3 is a compute type only: every matrix is stored as two bf16
// planes hi + lo, and every product sums hi*hi + hi*lo + lo*hi.
enum DType : int { DT_F32 = 0, DT_BF16 = 1, DT_F16 = 2, DT_BF16X3 = 3 };

inline int dtype_size(int dt) { return dt == DT_F32 ? 4 : 2; }
inline int dtype_planes(int dt) { return dt == DT_BF16X3 ? 2 : 1; }

// Epilogue of the NT product kernel.
enum GemmMode : int {
  MODE_SYM = 0,   // symmetric result: upper tiles computed, mirrored, diagonal
                  // tiles symmetrised so that the stored matrix is exactly
                  // symmetric; optional second output C2 = C + diag2 * I
  MODE_GEN = 1,   // general result in row layout, optional transposed copy
  MODE_FINAL = 2  // general result converted into the caller's output
};

// C = alpha * (A . B^T) + beta * D over a batch (computed as
// alpha * (A . B^T + (beta/alpha) D), or with K = 0 when alpha = 0), A and B row-major with the
// contraction index contiguous.  All internal buffers are padded to whole
// tiles and zero-filled there, so the kernel needs no bounds checks except
// for the caller's output in MODE_FINAL.
struct GemmParams {
  const void *A; int64_t lda, sA;   // leading dim and batch stride (elements)
  const void *B; int64_t ldb, sB;
  // split storage (DT_BF16X3): element offset from each hi plane to its lo
  // plane; unused otherwise
  int64_t pA, pB, pDT, pC, pC2, pCT;
  int K;                            // contraction length, multiple of 128 bytes
  int tiles_m, tiles_n;             // output tiles per matrix along rows / cols
  int tiles_per_mat;                // sym: tiles_m*(tiles_m+1)/2
  int sym_block, sym_half;          // sym: tile order (0 = column-major triangle;
                                    // else blocks of sym_block, bands of sym_half rows)
  // K split of a symmetric result (256-edge 16-bit tiles): the first pass runs
  // k_parts slices of K (grid = tiles x batch x k_parts; whole 32-element
  // stages, the last part taking the remainder)
  // and writes raw fp32 accumulators to part_out [k_parts][batch][tiles][256*256];
  // the second pass (K = 0) starts from the sum of parts_in such parts in
  // part_in and runs the normal epilogue.
  int k_parts;
  float *part_out;
  const float *part_in;
  int parts_in;
  int batch;
  int xcd_chunk;                    // tiles per run dealt to one XCD (see gemm_nt);
                                    // must divide (grid & ~7) / 8
  float alpha;                      // C = alpha * (acc)
  const float *alpha_vec;           // optional per-matrix factor on alpha (device, [batch])
  float init_scale;                 // acc starts at init_scale * D
  const void *DT; int64_t lddt, sDT;  // D read transposed: D(i,j) = DT[j*lddt + i];
                                      // may be null (D = 0)
  int d_rows;                       // D read in row layout instead: D(i,j) = DT[i*lddt + j]
                                    // (16-bit unsplit types)
  int b_kmajor;                     // B stored K-major (B[k][n], n contiguous): C = A B
                                    // (MODE_GEN / MODE_FINAL, 256-edge 16-bit tiles)
  const void *DT2;                  // optional second term init_scale2 * D2, same
  float init_scale2;                //   layout as DT (needs DT)
  int64_t pDT2;
  void *C; int64_t ldc, sC;
  void *C2; int64_t sC2;            // MODE_SYM second output (ld = ldc); may be null
  float diag1, diag2;               // MODE_SYM: added to C / C2 on the diagonal
  int n_real;                       // diagonal entries i < n_real get diag1/diag2
  void *CT; int64_t ldct, sCT;      // MODE_GEN transposed copy; may be null
  // MODE_FINAL
  void *out; int out_dtype;
  int64_t out_rows;                 // rows of each caller matrix (n)
  int64_t out_cols;                 // m
  int64_t rows_eff;                 // rows actually computed (n or k)
  const int64_t *row_idx;           // [batch][rows_eff] or null
};

// Launchers (return hipGetLastError() after the launch).
hipError_t launch_gemm(int compute_dtype, int tile, int mode, const GemmParams &p,
                       hipStream_t s);
const char *gemm_kernel_name(int compute_dtype, int tile, int mode, bool b_kmajor = false);

hipError_t launch_norm_partial(int io_dtype, const void *X, int64_t batch, int64_t n,
                               int64_t m, int64_t rows_eff, const int64_t *row_idx,
                               int parts, double *partials, hipStream_t s);

// X_hat = X / (||X||_F + eps) in the compute type, row-major into Xh and
// transposed into XT (skipped when XT is null); for DT_BF16X3 the lo planes
// sit plane_h / plane_t elements after Xh / XT.
hipError_t launch_scale_transpose(int io_dtype, int compute_dtype, const void *X,
                                  int64_t batch, int64_t n, int64_t m, int64_t rows_eff,
                                  const int64_t *row_idx, const double *partials,
                                  int parts, double eps, void *Xh, void *XT, int64_t Np,
                                  int64_t Mp, int64_t plane_h, int64_t plane_t, hipStream_t s);

// Dion3 selection: keys[b][i] = sum_j |M_b[i][j]| (fp64), then out[b][0..k) =
// indices of the k largest keys in ascending order (ties: smaller index).
hipError_t launch_select_rows_l1(int io_dtype, const void *M, int64_t batch, int64_t n, int64_t m,
                                 int64_t k, double *keys, int64_t *out, hipStream_t s);

// Unscaled transpose of 16-bit X (n, m multiples of 128, 16-byte aligned) into
// XT [m][n] per matrix (skipped when XT is null), and the sum of squares of
// every 128x128 tile into partials[b][tile] (fp64).
// With Xcopy set, X is also copied row-major into Xcopy ([b][n][m]).
// With row_idx ([batch][n]), the n x m matrix of batch entry b is rows
// row_idx[b][0..n) of the n_src x m matrix X_b (an index outside [0, n_src)
// reads as a zero row).
hipError_t launch_transpose_sumsq(int dtype, const void *X, int64_t batch, int64_t n, int64_t m,
                                  void *XT, void *Xcopy, double *partials, const int64_t *row_idx,
                                  int64_t n_src, hipStream_t s);
// inv[b] = 1 / (sqrt(sum_i partials[b][i]) + eps) and inv2[b] = inv[b]^2 (fixed-order sums).
hipError_t launch_norm_finish(const double *partials, int64_t batch, int64_t parts, double eps,
                              float *inv, float *inv2, hipStream_t s);

// *result = 1 if any element of the [batch][rows][cols] array A (dtype DT_F32,
// DT_BF16 or DT_F16) is Inf or NaN, else 0; with row_idx ([batch][k]) only
// those rows are checked.
hipError_t launch_check_finite(int dtype, const void *A, int64_t batch, int64_t rows, int64_t cols,
                               const int64_t *row_idx, int64_t k, int32_t *result, hipStream_t s);

hipError_t launch_check_rows(const int64_t *row_idx, int64_t batch, int64_t k, int64_t n,
                             int32_t *result, hipStream_t s);

// Dion3 update (Algorithm 4 around the orthogonalisation).
// M <- M + G (fp32) and keys[b][i] = sum_j |M_b[i][j]| (fp64); with sumsq
// also sumsq[b][i] = sum_j M_b[i][j]^2 (fp64).
hipError_t launch_momentum_l1(int grad_dtype, float *M, const void *G, int64_t batch, int64_t n,
                              int64_t m, double *keys, double *sumsq, hipStream_t s);
// partials[b][p] (p < parts) = sum over the rows r of part p (ceil(k / parts)
// consecutive entries of row_idx[b], in order) of rowsq[b][row_idx[b][r]]:
// the norm partials of a row subset whose per-row sums of squares are known.
hipError_t launch_row_partials(const double *rowsq, const int64_t *row_idx, int64_t batch, int64_t n,
                               int64_t k, int parts, double *partials, hipStream_t s);
// out[b][0..k) = indices of the k largest keys, ascending (ties: smaller index).
hipError_t launch_select_topk(const double *keys, int64_t batch, int64_t n, int64_t k, int64_t *out,
                              hipStream_t s);
// Row factors of the k x m update O: NorMuon (v updated in place at rows S)
// with the Frobenius rescale, or all ones without NorMuon.
hipError_t launch_normuon(const float *O, int64_t batch, int64_t k, int64_t m, float *v,
                          const int64_t *S, int64_t n, double beta2, double eps, int normuon,
                          double *rowsq, double *factor, hipStream_t s);
// W <- decay W everywhere, W[S_i] -= lr factor_i O_i, M[S_i] *= mu (S ascending).
hipError_t launch_dion3_update(float *W, float *M, const float *O, const int64_t *S,
                               const double *factor, int64_t batch, int64_t n, int64_t m, int64_t k,
                               float decay, double lr, float mu, hipStream_t s);

}  // namespace gns
