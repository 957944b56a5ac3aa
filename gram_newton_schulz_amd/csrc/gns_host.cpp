// Host side of the C ABI declared in include/gns.h: argument validation,
// workspace carving and the launch sequence of Gram Newton-Schulz
// ("Dion3: Full-Stack Orthogonal Updates", §4.2 Algorithm 3, with the
// Algorithm 2 algebra as an option) and of standard Newton-Schulz (§2.2,
// Algorithm 1).  Everything is enqueued on the caller's stream; nothing
// allocates, nothing synchronises.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <map>
#include <mutex>
#include <tuple>
#include <vector>

#include "../../include/gns.h"
#include "gns_kernels.h"

namespace {

using gns::GemmParams;

constexpr double kEps = 1e-7;  // added to the Frobenius norm (Algorithms 1-3)
constexpr size_t kAlign = 256;

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
int64_t round_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

bool valid_dtype(int dt) { return dt == GNS_F32 || dt == GNS_BF16 || dt == GNS_F16; }
bool valid_compute(int dt) { return valid_dtype(dt) || dt == GNS_BF16X3; }

// --------------------------------------------------------------------------
// problem plan: tile edge, padded sizes, workspace layout
// --------------------------------------------------------------------------
// The method works on Y with r <= c: Y = X_hat (r = rows, c = m) for a wide
// or square problem, Y = X_hat^T (r = m, c = rows) for a tall one
// (polar(X) = polar(X^T)^T; "Dion3" §2 assumes n <= m without loss of
// generality).  Buffers: xh = Y row-major [Np][Mp], xt = Y^T row-major [Mp][Np].
struct Plan {
  int tile = 128;                      // tile edge of the rectangular products
  int sym_tile = 128;                  // and of the symmetric ones
  int gram_tile = 128;                 // and of the Gram matrix (gram_tile_edge)
  int syrk_parts = 1;                  // K parts of the Gram matrix (256-edge tiles)
  int syrk_parts_room = 1;             // parts the workspace has room for
  int64_t batch = 0, rows = 0, m = 0;  // the caller's (selected) rows and columns
  int64_t r = 0, c = 0;                // short and long side of Y
  bool tall = false;                   // rows > m
  int64_t Np = 0, Mp = 0;              // r and c padded to whole tiles
  int parts = 1;
  int esz = 2;
  int planes = 1;                      // 2: split hi/lo storage (GNS_BF16X3)
  size_t off_partials = 0, off_inv = 0, off_xh = 0, off_xt0 = 0, off_xt1 = 0;
  int64_t tile_parts = 0;              // 128x128 tiles per matrix (direct input path)
  size_t off_sq[5] = {0, 0, 0, 0, 0};  // R, Z, RZ, Q0, Q1 (standard NS: A, B)
  size_t off_part = 0;                 // fp32 partial Gram tiles of a K split
  size_t off_flag = 0;                 // int32 result of the debug checks
  size_t bytes = 0;
};

int choose_tile(int cdt, int64_t batch, int64_t rows) {
  if (cdt == GNS_F32 || cdt == GNS_BF16X3) return 128;
  // 256-edge tiles halve operand traffic per FLOP and win as soon as the
  // symmetric products have some 64 upper tiles over the batch: measured
  // 2-31% faster on 16x1024x4096, 8x1024x16384, 4x2048x8192, 32x1024x4096,
  // 8x2048x4096 and 2x4096x16384 (80 to 320 tiles), slower on 16x512x8192
  // (48 tiles), where the n x n products would leave most CUs idle.
  const int64_t t256 = (rows + 255) / 256;
  const int64_t work = t256 * (t256 + 1) / 2 * batch;
  return work >= 64 ? 256 : 128;
}

int choose_parts(int64_t batch, int64_t rows) {
  int64_t p = (2048 + batch - 1) / std::max<int64_t>(batch, 1);
  p = std::min<int64_t>(p, 1024);
  p = std::min<int64_t>(p, rows);
  return static_cast<int>(std::max<int64_t>(p, 1));
}

// Tile request: 0 = choose from the size, 128 or 256 = that edge for every
// product, kTileMixed = 256 for the rectangular and 128 for the symmetric
// products.
constexpr int kTileMixed = 384;

// The symmetric products switch to 128-edge tiles when their 256-edge grid
// has fewer upper tiles over the batch than the GPU has compute units and
// the n x n contractions are short (n <= 2048): the fuller grid then wins
// (8 x 1024x16384: 2.02 -> 1.61 ms per call, the 1024 selected rows of
// 8 x 4096x16384: 2.38 -> 2.03, 4 x 2048x8192: 1.99 -> 1.82, 16 x 1024x4096:
// 1.40 -> 1.31).  With n = 4096 the 256 edge stays faster even on 136 tiles
// (1 x 4096x16384: 3.25 against 3.61 ms), as on every larger grid measured.
int choose_sym_tile(int64_t batch, int64_t rows) {
  const int64_t t256 = (rows + 255) / 256;
  return (t256 * (t256 + 1) / 2 * batch < 256 && rows <= 2048) ? 128 : 256;
}

// The Gram matrix contracts over the long side.  When its 256-edge upper
// tiles over the batch fill at most half of the GPU's 256 compute units, its
// contraction is cut into parts so that tiles x parts come close to one full
// round (each part at least 2048 long); a second short pass adds the parts.
// The 1024 selected rows of 8 x 4096x16384: 80 tiles, 3 parts.
int choose_syrk_parts(int cdt, int64_t batch, int64_t Np256, int64_t Mp256) {
  if (cdt != GNS_BF16 && cdt != GNS_F16) return 1;
  const int64_t t = Np256 / 256;
  const int64_t tiles = t * (t + 1) / 2 * batch;
  if (tiles < 1 || tiles > 128) return 1;
  int64_t parts = std::min<int64_t>(256 / tiles, 4);
  parts = std::min<int64_t>(parts, Mp256 / 2048);
  return parts >= 2 ? static_cast<int>(parts) : 1;
}

// Under the size rule the Gram matrix keeps 256-edge tiles where the n x n
// products take 128 but its own 128-edge grid would not fit one round of two
// workgroups per compute unit: 16 x 1024x4096 has 576 upper 128-edge tiles
// for 512 slots, and its 160 256-edge tiles run in one round instead (1.14 ->
// 1.10-1.11 ms per call, 1.26 -> 1.20 on one stream; outputs identical, as
// the tile edge changes no sum).  Forced tile requests keep their edges.
int gram_tile_edge(int tile_request, int tile, int sym_tile, int64_t batch, int64_t r) {
  if (tile_request != 0 || tile != 256 || sym_tile != 128) return sym_tile;
  const int64_t t128 = round_up(r, 256) / 128;
  return t128 * (t128 + 1) / 2 * batch > 2 * 256 ? 256 : 128;
}

// tile_request: see kTileMixed.  Workspace sizes are quoted
// for 256-padded buffers so that any tile choice fits.
bool make_plan(int cdt, int64_t batch, int64_t rows, int64_t m, int n_square, int tile_request,
               Plan *pl) {
  if (!valid_compute(cdt) || batch < 0 || rows < 1 || m < 1) return false;
  pl->tall = rows > m;
  pl->r = std::min(rows, m);
  pl->c = std::max(rows, m);
  if (tile_request == 0) {
    pl->tile = choose_tile(cdt, batch, pl->r);
    pl->sym_tile = pl->tile == 256 ? choose_sym_tile(batch, pl->r) : 128;
  } else if (tile_request == kTileMixed) {
    pl->tile = 256;
    pl->sym_tile = 128;
  } else {
    pl->tile = pl->sym_tile = tile_request;
  }
  // the fp32 and split-plane kernels exist for 128-edge tiles only
  if (cdt == GNS_F32 || cdt == GNS_BF16X3) pl->tile = pl->sym_tile = 128;
  pl->gram_tile = gram_tile_edge(tile_request, pl->tile, pl->sym_tile, batch, pl->r);
  pl->batch = batch;
  pl->rows = rows;
  pl->m = m;
  pl->Np = round_up(pl->r, pl->tile);
  pl->Mp = round_up(pl->c, pl->tile);
  // per-matrix element offsets stay within int range of the kernels' math
  if (pl->Np * pl->Mp > (int64_t(1) << 31)) return false;
  // operand panels (256 rows of a padded buffer) are addressed with 32-bit
  // buffer offsets
  if (int64_t(256) * std::max(pl->Np, pl->Mp) * gns::dtype_size(cdt) >= (int64_t(1) << 31)) return false;
  pl->parts = choose_parts(batch, rows);
  pl->esz = gns::dtype_size(cdt);
  pl->planes = gns::dtype_planes(cdt);
  size_t off = 0;
  pl->off_partials = off;
  // norm partials: per row block (normalised-copy path) or per 128x128 tile
  // (direct path), whichever needs more
  pl->tile_parts = (pl->Np / 128) * (pl->Mp / 128);
  off = align_up(off + sizeof(double) * batch * std::max<int64_t>(pl->parts, pl->tile_parts), kAlign);
  pl->off_inv = off;                   // 1/(||X||+eps) and its square, per matrix
  off = align_up(off + 2 * sizeof(float) * batch, kAlign);
  // every region holds `planes` planes of `batch` matrices, lo after hi
  const size_t rect = static_cast<size_t>(pl->planes) * batch * pl->Np * pl->Mp * pl->esz;
  const size_t sq = static_cast<size_t>(pl->planes) * batch * pl->Np * pl->Np * pl->esz;
  pl->off_xh = off;
  off = align_up(off + rect, kAlign);
  pl->off_xt0 = off;
  off = align_up(off + rect, kAlign);
  pl->off_xt1 = off;
  off = align_up(off + rect, kAlign);
  for (int i = 0; i < n_square; ++i) {
    pl->off_sq[i] = off;
    off = align_up(off + sq, kAlign);
  }
  // room for a K split of the Gram matrix, from the 256-edge geometry (the
  // same for every tile request, so that quoted sizes fit the size rule)
  {
    const int64_t Np256 = round_up(pl->r, 256), Mp256 = round_up(pl->c, 256);
    pl->syrk_parts_room = pl->tall ? 1 : choose_syrk_parts(cdt, batch, Np256, Mp256);
    pl->syrk_parts = (tile_request == 0 && pl->tile == 256) ? pl->syrk_parts_room : 1;
    if (pl->syrk_parts > 1) pl->gram_tile = 256;   // the K split runs 256-edge tiles
    pl->off_part = off;
    if (pl->syrk_parts_room > 1) {
      const int64_t t = Np256 / 256;
      off = align_up(off + sizeof(float) * static_cast<size_t>(pl->syrk_parts_room) * batch * (t * (t + 1) / 2) *
                               256 * 256,
                     kAlign);
    }
  }
  pl->off_flag = off;
  off = align_up(off + sizeof(int32_t), kAlign);
  pl->bytes = off;
  return true;
}

// --------------------------------------------------------------------------
// optional per-launch timing (benchmarking aid)
// --------------------------------------------------------------------------
struct TimedLaunch {
  const char *name;
  const char *kernel;
  double flops, bytes;
  hipEvent_t start, stop;
};
std::mutex g_tmu;
bool g_timing = false;
std::vector<TimedLaunch> g_launches;
std::vector<hipEvent_t> g_event_pool;

hipEvent_t pooled_event() {
  if (!g_event_pool.empty()) {
    hipEvent_t e = g_event_pool.back();
    g_event_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

struct LaunchScope {
  hipStream_t s;
  TimedLaunch rec{};
  bool on = false;
  LaunchScope(hipStream_t st, const char *name, const char *kernel, double flops, double bytes)
      : s(st) {
    if (!g_timing) return;
    rec = TimedLaunch{name, kernel, flops, bytes, pooled_event(), pooled_event()};
    if (rec.start && rec.stop && hipEventRecord(rec.start, s) == hipSuccess) on = true;
  }
  void done() {
    if (!on) return;
    if (hipEventRecord(rec.stop, s) == hipSuccess) {
      std::lock_guard<std::mutex> lk(g_tmu);
      g_launches.push_back(rec);
    }
  }
};

// --------------------------------------------------------------------------
// launch helpers
// --------------------------------------------------------------------------
// One sub-batch: matrices [b0, b0 + batch) of a call, enqueued on stream s.
// Every workspace region is strided per matrix, so a sub-batch addresses its
// share with a plain offset.
struct Ctx {
  const Plan *pl;
  int cdt;
  int64_t batch;
  int64_t b0;
  unsigned char *ws;
  hipStream_t s;
  // Direct input path: X (already in the compute type, whole tiles) is read
  // as it is instead of through a normalised copy; products that read it
  // apply 1/(||X||_F + eps) per matrix in their epilogues.
  bool direct = false;
  const void *xin = nullptr;           // this sub-batch's X
  // The input pass also copies X row-major into the workspace (xcopy), and
  // every later product reads that copy, for a row subset (the copy holds the
  // selected rows, unscaled) and for in-place calls whose final product would
  // read X (so that no product reads X while the final one writes it).  Null
  // otherwise.
  void *xcopy = nullptr;
  const void *xsrc() const { return xcopy ? xcopy : xin; }
  // The rectangular products of Gram NS read X row-major (K-major B operand,
  // LDS transpose reads), so no transposed copy of X is written.
  bool nn = false;
  // Per-row sums of squares of this sub-batch's X ([batch][n], fp64), known
  // before the call (the Dion3 update's momentum pass forms them): a row
  // subset's norm then adds those of its rows instead of reading the rows.
  const double *row_sumsq = nullptr;
  // Fan-out stagger: recorded on `s` once the input is normalised; the next
  // part's stream waits for it (see run_batches).  Null when unused.
  hipEvent_t stagger = nullptr;
  gns_status mark_stagger() const {
    if (stagger && hipEventRecord(stagger, s) != hipSuccess) return GNS_E_HIP;
    return GNS_OK;
  }
  int64_t sq_stride() const { return pl->Np * pl->Np; }
  int64_t rect_stride() const { return pl->Np * pl->Mp; }
  void *sq(int i) const { return ws + pl->off_sq[i] + b0 * sq_stride() * pl->esz; }
  void *xh() const { return ws + pl->off_xh + b0 * rect_stride() * pl->esz; }
  void *xt(int i) const { return ws + (i ? pl->off_xt1 : pl->off_xt0) + b0 * rect_stride() * pl->esz; }
  double *partials() const {
    return reinterpret_cast<double *>(ws + pl->off_partials) + b0 * pl->parts;
  }
  double *tile_partials() const {
    return reinterpret_cast<double *>(ws + pl->off_partials) + b0 * pl->tile_parts;
  }
  float *inv() const { return reinterpret_cast<float *>(ws + pl->off_inv) + b0; }
  // this sub-batch's partial Gram tiles: [parts][batch][tiles][256 * 256]
  float *part() const {
    const int64_t t = pl->Np / 256;
    return reinterpret_cast<float *>(ws + pl->off_part) +
           b0 * static_cast<int64_t>(pl->syrk_parts_room) * (t * (t + 1) / 2) * 256 * 256;
  }
  float *inv2() const { return reinterpret_cast<float *>(ws + pl->off_inv) + pl->batch + b0; }
  // element offset from a hi plane to its lo plane (split storage only)
  int64_t plane_sq() const { return pl->planes == 2 ? pl->batch * sq_stride() : 0; }
  int64_t plane_rect() const { return pl->planes == 2 ? pl->batch * rect_stride() : 0; }
};

// alpha * (A B^T) + beta * D is evaluated as alpha * (A B^T + (beta/alpha) D);
// with alpha = 0 the product is skipped (K = 0) and the result is beta * D.
void set_scale(GemmParams *p, float alpha, float beta) {
  if (alpha != 0.0f) {
    p->alpha = alpha;
    p->init_scale = beta / alpha;
  } else {
    p->alpha = 1.0f;
    p->init_scale = beta;
    p->K = 0;
  }
}

// Runs of tiles dealt to one XCD (the kernel's xcd_chunk): 1/xpm of a matrix
// per run so that xpm XCDs share each matrix, or with xpm = 1 (and whenever
// the sizes do not divide) one contiguous run per XCD, which holds whole
// matrices when the batch is a multiple of 8.  Products use xpm = 4 (a
// quarter matrix per run): measured on 8 x 4096x16384 bf16 against 1, 2 and 8
// per product kind, it keeps the matrices in flight within the shared
// last-level cache while each XCD's L2 still sees a compact block of tiles.
// The n x n products of matrices of at
// most 2 MiB (half an XCD's L2) use xpm = 1 instead, so that one XCD's L2
// holds every operand of its matrix (16 x 1024x4096 bf16: 1.08 -> 1.06 ms
// a call; 64 x 2048x7168 unchanged).
int xcd_chunk(int64_t tiles_per_mat, int64_t batch, int xpm) {
  const int64_t S = ((tiles_per_mat * batch) & ~int64_t(7)) / 8;
  if (S == 0) return 1;
  if (xpm > 1 && tiles_per_mat % xpm == 0) {
    const int64_t c = tiles_per_mat / xpm;
    if (S % c == 0) return static_cast<int>(c);
  }
  return static_cast<int>(S);
}

// Tile order of the symmetric products (the kernel's sym_tile): the Gram
// matrix runs in blocks of 4 x 4 tiles taken in bands of 2 rows, so that each
// XCD's run of tiles streams few operand panels through its L2 (8 x 4096x16384
// bf16: 4.44 -> 4.06 ms for the two Gram matrices of a call; blocks of 8 with
// bands of 4 or 8, and of 4 with bands of 4, measured 4.11-4.15); the n x n
// products keep the column-major triangle, which measured 1% faster for them
// than blocks of 4.  The band height must divide the block edge.
constexpr int kSyrkBlock = 4, kSyrkBand = 2;
constexpr int kSymmBlock = 0, kSymmBand = 1;

// Launch layout of a symmetric product over nt x nt tiles.  (With 256-edge
// 16-bit tiles a diagonal tile costs three quarters of a tile; running the
// diagonal tiles last on every XCD, to fill the partial last round, measured
// slower: 4.04 -> 4.79 ms for the two Gram matrices of an 8 x 4096x16384
// call, as a diagonal tile shares no operand panel with the tiles around it.)
void sym_layout(GemmParams *p, const Ctx &c, int nt, int xpm, int block, int band) {
  p->tiles_m = p->tiles_n = nt;
  p->tiles_per_mat = nt * (nt + 1) / 2;
  p->sym_block = block;
  p->sym_half = band;
  p->xcd_chunk = xcd_chunk(p->tiles_per_mat, c.batch, xpm);
}

GemmParams base_params(const Ctx &c) {
  GemmParams p;
  std::memset(&p, 0, sizeof(p));
  p.batch = static_cast<int>(c.batch);
  p.alpha = 1.0f;
  p.n_real = static_cast<int>(c.pl->r);
  return p;
}

// C = alpha * A B + beta * D (+ beta2 * D2) for n x n iterates (B
// symmetric), mirrored.
gns_status symm(const Ctx &c, const void *A, const void *B, float alpha, float beta, const void *D,
                void *C, void *C2, float diag1, float diag2, const char *what, double flops,
                const void *D2 = nullptr, float beta2 = 0.0f) {
  GemmParams p = base_params(c);
  const int64_t N = c.pl->Np;
  const int nt = static_cast<int>(N / c.pl->sym_tile);
  // The 256-edge kernels add beta D from the operand stream when D is the B
  // operand (D = B, a symmetric iterate: each wave takes its D entries from
  // the B panel's stages as they pass through LDS).  A product whose D is its
  // A operand (R Z with D = R, Q Z with D = Q) therefore runs as B A^T: A and
  // B are polynomials in the same R, so both orders give the same product up
  // to rounding, and the stored result (upper tiles, mirrored) is exactly
  // symmetric either way.
  if (D && D == A && D != B) std::swap(A, B);
  p.A = A; p.lda = N; p.sA = c.sq_stride();
  p.B = B; p.ldb = N; p.sB = c.sq_stride();
  p.K = static_cast<int>(N);
  const int xpm = N * N * c.pl->esz * c.pl->planes <= (int64_t(2) << 20) ? 1 : 4;
  sym_layout(&p, c, nt, xpm, kSymmBlock, kSymmBand);
  set_scale(&p, alpha, beta);
  if (D) { p.DT = D; p.lddt = N; p.sDT = c.sq_stride(); }   // D is symmetric
  if (D && D2) {
    p.DT2 = D2;
    p.init_scale2 = alpha != 0.0f ? beta2 / alpha : beta2;
    p.pDT2 = c.plane_sq();
  }
  p.C = C; p.ldc = N; p.sC = c.sq_stride();
  p.C2 = C2; p.sC2 = c.sq_stride();
  p.pA = p.pB = p.pDT = p.pC = p.pC2 = c.plane_sq();
  p.diag1 = diag1; p.diag2 = diag2;
  const double n = static_cast<double>(c.pl->r);
  const double bytes = c.batch * n * n * c.pl->esz * (3.0 + (D ? 1.0 : 0.0) + (D2 ? 1.0 : 0.0) + (C2 ? 1.0 : 0.0));
  LaunchScope ls(c.s, what, gns::gemm_kernel_name(c.cdt, c.pl->sym_tile, gns::MODE_SYM), flops * c.batch,
                 bytes);
  hipError_t e = gns::launch_gemm(c.cdt, c.pl->sym_tile, gns::MODE_SYM, p, c.s);
  ls.done();
  return e == hipSuccess ? GNS_OK : GNS_E_HIP;
}

// R = X X^T from the row-layout buffer, or (from_input on the direct path)
// from the caller's X with 1/(||X||+eps)^2 applied in the epilogue.
// xrow: the row-layout X to use instead of the normalised copy (the restarted
// X of a K-major-B call lives in one of two row buffers).
// The Gram matrix in two passes (see choose_syrk_parts): 256-edge tiles
// over `parts` slices of the contraction write raw fp32 partial tiles, then a
// pass with no contraction sums them in part order and runs the usual
// epilogue (normalisation factor, rounding, mirror).
gns_status syrk_split(const Ctx &c, void *R, bool from_input, const void *xrow) {
  const int parts = c.pl->syrk_parts;
  const int64_t N = c.pl->Np, M = c.pl->Mp;
  const int nt = static_cast<int>(N / 256);
  const bool direct = from_input && c.direct;
  const void *Xh = direct ? c.xsrc() : (xrow ? xrow : c.xh());
  GemmParams p = base_params(c);
  p.A = Xh; p.lda = M; p.sA = c.rect_stride();
  p.B = Xh; p.ldb = M; p.sB = c.rect_stride();
  p.K = static_cast<int>(M);
  p.tiles_m = p.tiles_n = nt;
  p.tiles_per_mat = nt * (nt + 1) / 2;
  p.sym_block = kSyrkBlock;
  p.sym_half = kSyrkBand;
  p.xcd_chunk = xcd_chunk(p.tiles_per_mat, c.batch * parts, 4);
  p.k_parts = parts;
  p.part_out = c.part();
  const double n = static_cast<double>(c.pl->r), m = static_cast<double>(c.pl->c);
  const double part_bytes = 4.0 * parts * c.batch * p.tiles_per_mat * 256.0 * 256.0;
  {
    LaunchScope ls(c.s, "syrk", gns::gemm_kernel_name(c.cdt, 256, gns::MODE_SYM), n * n * m * c.batch,
                   c.batch * n * m * c.pl->esz + part_bytes);
    const hipError_t e = gns::launch_gemm(c.cdt, 256, gns::MODE_SYM, p, c.s);
    ls.done();
    if (e != hipSuccess) return GNS_E_HIP;
  }
  GemmParams q = base_params(c);
  if (direct) q.alpha_vec = c.inv2();
  q.K = 0;
  q.tiles_m = q.tiles_n = nt;
  q.tiles_per_mat = p.tiles_per_mat;
  q.sym_block = kSyrkBlock;
  q.sym_half = kSyrkBand;
  q.xcd_chunk = xcd_chunk(q.tiles_per_mat, c.batch, 4);
  q.part_in = c.part();
  q.parts_in = parts;
  q.C = R; q.ldc = N; q.sC = c.sq_stride();
  q.pC = c.plane_sq();
  LaunchScope ls(c.s, "syrk", gns::gemm_kernel_name(c.cdt, 256, gns::MODE_SYM), 0.0,
                 part_bytes + c.batch * n * n * c.pl->esz);
  const hipError_t e = gns::launch_gemm(c.cdt, 256, gns::MODE_SYM, q, c.s);
  ls.done();
  return e == hipSuccess ? GNS_OK : GNS_E_HIP;
}

gns_status syrk(const Ctx &c, void *R, bool from_input = false, const void *xrow = nullptr) {
  if (c.pl->syrk_parts > 1) return syrk_split(c, R, from_input, xrow);
  GemmParams p = base_params(c);
  const int64_t N = c.pl->Np, M = c.pl->Mp;
  const int nt = static_cast<int>(N / c.pl->gram_tile);
  const bool direct = from_input && c.direct;
  const void *Xh = direct ? c.xsrc() : (xrow ? xrow : c.xh());
  if (direct) p.alpha_vec = c.inv2();
  p.A = Xh; p.lda = M; p.sA = c.rect_stride();
  p.B = Xh; p.ldb = M; p.sB = c.rect_stride();
  p.K = static_cast<int>(M);
  sym_layout(&p, c, nt, 4, kSyrkBlock, kSyrkBand);
  p.C = R; p.ldc = N; p.sC = c.sq_stride();
  p.pA = p.pB = c.plane_rect();
  p.pC = c.plane_sq();
  const double n = static_cast<double>(c.pl->r), m = static_cast<double>(c.pl->c);
  LaunchScope ls(c.s, "syrk", gns::gemm_kernel_name(c.cdt, c.pl->gram_tile, gns::MODE_SYM), n * n * m * c.batch,
                 c.batch * (n * m + n * n) * c.pl->esz);
  hipError_t e = gns::launch_gemm(c.cdt, c.pl->gram_tile, gns::MODE_SYM, p, c.s);
  ls.done();
  return e == hipSuccess ? GNS_OK : GNS_E_HIP;
}

// Y = S X (+ beta * X) with S an n x n iterate and X read through its
// transposed copy XT_in.  Either writes the row layout in place plus the
// transposed copy XT_out, or (final) the caller's output.
gns_status apply(const Ctx &c, const void *S, const void *XT_in, void *XT_out, float beta,
                 bool final, void *out, int io_dtype, int64_t n_total, const int64_t *row_idx,
                 const char *what, const float *alpha_vec = nullptr) {
  GemmParams p = base_params(c);
  p.alpha_vec = alpha_vec;           // 1/(||X||+eps) when X^T is the unscaled input
  const int64_t N = c.pl->Np, M = c.pl->Mp;
  const int tm = static_cast<int>(N / c.pl->tile), tn = static_cast<int>(M / c.pl->tile);
  void *Xh = c.xh();
  p.A = S; p.lda = N; p.sA = c.sq_stride();
  p.B = XT_in; p.ldb = N; p.sB = c.rect_stride();
  p.K = static_cast<int>(N);
  p.tiles_m = tm; p.tiles_n = tn;
  p.tiles_per_mat = tm * tn;
  p.xcd_chunk = xcd_chunk(p.tiles_per_mat, c.batch, 4);
  set_scale(&p, 1.0f, beta);
  // the beta term reads X through its transposed copy, the B operand
  if (beta != 0.0f) { p.DT = XT_in; p.lddt = N; p.sDT = c.rect_stride(); }
  p.pA = c.plane_sq();
  p.pB = p.pDT = p.pC = p.pCT = c.plane_rect();
  const double n = static_cast<double>(c.pl->r), m = static_cast<double>(c.pl->c);
  double bytes = c.batch * (n * n + n * m) * c.pl->esz;
  if (final) {
    if (c.pl->tall) {
      // out = (S Y + beta Y)^T = Y^T S + beta Y^T, written in the caller's
      // layout: A = Y^T rows, B = S (symmetric), the beta term read through
      // Y itself
      p.A = XT_in; p.lda = N; p.sA = c.rect_stride();
      p.B = S; p.ldb = N; p.sB = c.sq_stride();
      p.tiles_m = tn; p.tiles_n = tm;
      if (beta != 0.0f) { p.DT = Xh; p.lddt = M; p.sDT = c.rect_stride(); }
      p.pA = p.pDT = c.plane_rect();
      p.pB = c.plane_sq();
    }
    p.out = out; p.out_dtype = io_dtype; p.out_rows = n_total; p.out_cols = c.pl->m;
    p.rows_eff = c.pl->rows; p.row_idx = row_idx;
    bytes += c.batch * n * m * gns::dtype_size(io_dtype);
  } else {
    p.C = Xh; p.ldc = M; p.sC = c.rect_stride();
    p.CT = XT_out; p.ldct = N; p.sCT = c.rect_stride();
    bytes += 2.0 * c.batch * n * m * c.pl->esz;
  }
  if (beta != 0.0f) bytes += c.batch * n * m * c.pl->esz;
  LaunchScope ls(c.s, what,
                 gns::gemm_kernel_name(c.cdt, c.pl->tile, final ? gns::MODE_FINAL : gns::MODE_GEN),
                 2.0 * n * n * m * c.batch, bytes);
  hipError_t e = gns::launch_gemm(c.cdt, c.pl->tile, final ? gns::MODE_FINAL : gns::MODE_GEN, p, c.s);
  ls.done();
  return e == hipSuccess ? GNS_OK : GNS_E_HIP;
}

// Y = S X (+ beta * X) with S an n x n iterate and X row-major [rows][m]
// (pitch ld_in): the K-major-B form of the product, whose kernel reads X
// through LDS transpose loads.  Writes the row layout Y into Xrow_out, or
// (final) the caller's output.
gns_status apply_nn(const Ctx &c, const void *S, const void *Xrow_in, int64_t ld_in, void *Xrow_out,
                    float beta, bool final, void *out, int io_dtype, int64_t n_total,
                    const int64_t *row_idx, const char *what, const float *alpha_vec = nullptr) {
  GemmParams p = base_params(c);
  p.alpha_vec = alpha_vec;           // 1/(||X||+eps) when X is the unscaled input
  const int64_t N = c.pl->Np, M = c.pl->Mp;
  const int tm = static_cast<int>(N / c.pl->tile), tn = static_cast<int>(M / c.pl->tile);
  p.A = S; p.lda = N; p.sA = c.sq_stride();
  p.B = Xrow_in; p.ldb = ld_in; p.sB = c.rect_stride();
  p.b_kmajor = 1;
  p.K = static_cast<int>(N);
  p.tiles_m = tm; p.tiles_n = tn;
  p.tiles_per_mat = tm * tn;
  p.xcd_chunk = xcd_chunk(p.tiles_per_mat, c.batch, 4);
  set_scale(&p, 1.0f, beta);
  if (beta != 0.0f) { p.DT = Xrow_in; p.lddt = ld_in; p.sDT = c.rect_stride(); p.d_rows = 1; }
  const double n = static_cast<double>(c.pl->r), m = static_cast<double>(c.pl->c);
  double bytes = c.batch * (n * n + n * m) * c.pl->esz;
  if (final) {
    p.out = out; p.out_dtype = io_dtype; p.out_rows = n_total; p.out_cols = c.pl->m;
    p.rows_eff = c.pl->rows; p.row_idx = row_idx;
    bytes += c.batch * n * m * gns::dtype_size(io_dtype);
  } else {
    p.C = Xrow_out; p.ldc = M; p.sC = c.rect_stride();
    bytes += c.batch * n * m * c.pl->esz;
  }
  if (beta != 0.0f) bytes += c.batch * n * m * c.pl->esz;
  const int mode = final ? gns::MODE_FINAL : gns::MODE_GEN;
  LaunchScope ls(c.s, what, gns::gemm_kernel_name(c.cdt, c.pl->tile, mode, true), 2.0 * n * n * m * c.batch,
                 bytes);
  hipError_t e = gns::launch_gemm(c.cdt, c.pl->tile, mode, p, c.s);
  ls.done();
  return e == hipSuccess ? GNS_OK : GNS_E_HIP;
}

// Norm + scale + cast (+ transpose, where a path reads X^T) of the
// (row-selected) input.  On the direct path: the per-matrix scale factors and,
// unless the products read X row-major, the unscaled transpose X^T.
gns_status normalize(const Ctx &c, const void *X, int io, int64_t n_total, const int64_t *row_idx) {
  double *partials = c.partials();
  const double rows = static_cast<double>(c.pl->rows), m = static_cast<double>(c.pl->m);
  if (c.direct) {
    {
      LaunchScope ls(c.s, "transpose_sumsq", "transpose_sumsq", 2.0 * rows * m * c.batch,
                     c.batch * rows * m * (c.nn ? 1.0 : 2.0) * gns::dtype_size(io) +
                         (c.xcopy ? c.batch * rows * m * gns::dtype_size(io) : 0.0));
      hipError_t e = gns::launch_transpose_sumsq(io, X, c.batch, c.pl->rows, c.pl->m,
                                                 c.nn ? nullptr : c.xt(0), c.xcopy, c.tile_partials(), row_idx,
                                                 n_total, c.s);
      ls.done();
      if (e != hipSuccess) return GNS_E_HIP;
    }
    LaunchScope ls(c.s, "norm_finish", "norm_finish", 1.0 * c.batch * c.pl->tile_parts,
                   8.0 * c.batch * c.pl->tile_parts);
    hipError_t e = gns::launch_norm_finish(c.tile_partials(), c.batch, c.pl->tile_parts, kEps, c.inv(),
                                           c.inv2(), c.s);
    ls.done();
    return e == hipSuccess ? GNS_OK : GNS_E_HIP;
  }
  if (c.row_sumsq && row_idx) {
    LaunchScope ls(c.s, "row_partials", "row_partials", rows * c.batch, 16.0 * rows * c.batch);
    hipError_t e = gns::launch_row_partials(c.row_sumsq, row_idx, c.batch, n_total, c.pl->rows, c.pl->parts,
                                            partials, c.s);
    ls.done();
    if (e != hipSuccess) return GNS_E_HIP;
  } else {
    LaunchScope ls(c.s, "norm_partial", "norm_partial", 2.0 * rows * m * c.batch,
                   c.batch * rows * m * gns::dtype_size(io));
    hipError_t e = gns::launch_norm_partial(io, X, c.batch, n_total, c.pl->m, c.pl->rows, row_idx,
                                            c.pl->parts, partials, c.s);
    ls.done();
    if (e != hipSuccess) return GNS_E_HIP;
  }
  {
    // reads X once, writes X_hat (all planes) and, unless the products read X
    // row-major, its transpose
    LaunchScope ls(c.s, "scale_transpose", "scale_transpose", rows * m * c.batch,
                   c.batch * rows * m *
                       (gns::dtype_size(io) + (c.nn ? 1.0 : 2.0) * c.pl->planes * c.pl->esz));
    // X_hat row-major [rows][m] and its transpose; for a tall problem X_hat is
    // Y^T (the xt buffer) and its transpose is Y (the xh buffer)
    void *dst_rows = c.pl->tall ? c.xt(0) : c.xh();
    void *dst_cols = c.nn ? nullptr : (c.pl->tall ? c.xh() : c.xt(0));
    const int64_t rows_pad = c.pl->tall ? c.pl->Mp : c.pl->Np;
    const int64_t cols_pad = c.pl->tall ? c.pl->Np : c.pl->Mp;
    hipError_t e = gns::launch_scale_transpose(io, c.cdt, X, c.batch, n_total, c.pl->m, c.pl->rows,
                                               row_idx, partials, c.pl->parts, kEps,
                                               dst_rows, dst_cols, rows_pad, cols_pad,
                                               c.plane_rect(), c.plane_rect(), c.s);
    ls.done();
    if (e != hipSuccess) return GNS_E_HIP;
  }
  return GNS_OK;
}

gns_status parse_opts(unsigned opts, unsigned allowed, int *tile) {
  allowed |= GNS_OPT_TILE_128 | GNS_OPT_TILE_256 | GNS_OPT_TILE_MIXED | GNS_OPT_ONE_STREAM;
  if (opts & ~allowed) return GNS_E_FLAGS;
  const unsigned tile_bits =
      opts & (GNS_OPT_TILE_128 | GNS_OPT_TILE_256 | GNS_OPT_TILE_MIXED | GNS_OPT_TILE_AUTOTUNE);
  if (tile_bits & (tile_bits - 1)) return GNS_E_FLAGS;   // at most one
  *tile = (opts & GNS_OPT_TILE_128) ? 128
          : (opts & GNS_OPT_TILE_256) ? 256
          : (opts & GNS_OPT_TILE_MIXED) ? kTileMixed
                                        : 0;
  return GNS_OK;
}

bool ranges_overlap(const void *a, size_t na, const void *b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

gns_status check_coeffs(const double *coeffs, int T) {
  if (!coeffs) return GNS_E_NULL;
  if (T < 1 || T > GNS_MAX_ITERS) return GNS_E_COEFF;
  for (int i = 0; i < 3 * T; ++i)
    if (!std::isfinite(coeffs[i])) return GNS_E_COEFF;
  return GNS_OK;
}

gns_status parse_restarts(const int *restart_after, int n_restart, int T, std::vector<char> *at) {
  if (n_restart < 0 || (n_restart > 0 && !restart_after)) return GNS_E_RESTART;
  at->assign(T + 2, 0);
  for (int i = 0; i < n_restart; ++i) {
    const int r = restart_after[i];
    if (r < 1 || r > T - 1 || (i > 0 && r <= restart_after[i - 1])) return GNS_E_RESTART;
    (*at)[r] = 1;
  }
  return GNS_OK;
}

gns_status common_checks(const void *X, const void *out, int64_t batch, int64_t n, int64_t m,
                         gns_dtype io, gns_dtype cdt, const double *coeffs, int T,
                         const int64_t *row_idx, int64_t k, int64_t *rows) {
  if (!valid_dtype(io) || !valid_compute(cdt)) return GNS_E_DTYPE;
  if (batch < 0 || n < 1 || m < 1) return GNS_E_SHAPE;
  if (row_idx) {
    if (k < 1 || k > n) return GNS_E_SHAPE;
    *rows = k;
  } else {
    *rows = n;
  }
  const gns_status cs = check_coeffs(coeffs, T);
  if (cs != GNS_OK) return cs;
  if (batch > 0 && (!X || !out)) return GNS_E_NULL;
  if (batch > (int64_t(1) << 24)) return GNS_E_SHAPE;
  return GNS_OK;
}

gns_status workspace_checks(const void *X, const void *out, int64_t batch, int64_t n, int64_t m,
                            gns_dtype io, const Plan &pl, void *ws, size_t ws_bytes) {
  if (!ws || ws_bytes < pl.bytes || (reinterpret_cast<uintptr_t>(ws) & (kAlign - 1))) return GNS_E_WORKSPACE;
  const size_t io_bytes = static_cast<size_t>(batch) * n * m * gns::dtype_size(io);
  if (ranges_overlap(ws, pl.bytes, X, io_bytes) || ranges_overlap(ws, pl.bytes, out, io_bytes))
    return GNS_E_ALIAS;
  return GNS_OK;
}

// Standard Newton-Schulz (Dion3 §2.2, Algorithm 1) on a validated problem;
// the symmetric products go through the mirrored kernel (Appendix C.3).
// Rows row_idx of X (all rows when null) are orthogonalised; row i of the
// result goes to row out_idx[i] of out (row i when null), out having
// out_rows rows per matrix.
gns_status enqueue_standard(const Ctx &c, const void *X, void *out, int io, int64_t n,
                            const double *coeffs, int T, const int64_t *row_idx,
                            const int64_t *out_idx, int64_t out_rows) {
  const Plan &pl = *c.pl;
  void *A = c.sq(0), *B = c.sq(1);
  void *XT[2] = {c.xt(0), c.xt(1)};
  int xcur = 0;
  const double nn = static_cast<double>(pl.r);
  gns_status st;
  if ((st = normalize(c, X, io, n, row_idx)) != GNS_OK) return st;
  // on the direct path the first iteration reads X itself (syrk) and its
  // unscaled transpose (apply), both with the normalisation as a factor
  const float *x_scale = c.direct ? c.inv() : nullptr;
  if ((st = c.mark_stagger()) != GNS_OK) return st;
  for (int t = 1; t <= T; ++t) {
    const float a = static_cast<float>(coeffs[3 * (t - 1) + 0]);
    const float b = static_cast<float>(coeffs[3 * (t - 1) + 1]);
    const float cc = static_cast<float>(coeffs[3 * (t - 1) + 2]);
    if ((st = syrk(c, A, t == 1)) != GNS_OK) return st;                           // A = X X^T
    st = symm(c, A, A, cc, b, A, B, nullptr, 0.0f, 0.0f, "std_poly", nn * nn * nn);  // B = bA + cA^2
    if (st != GNS_OK) return st;
    if (t < T) {
      st = apply(c, B, XT[xcur], XT[xcur ^ 1], a, false, nullptr, io, n, nullptr, "std_apply", x_scale);
      xcur ^= 1;
    } else {
      st = apply(c, B, XT[xcur], nullptr, a, true, out, io, out_rows, out_idx, "std_final_apply", x_scale);
    }
    x_scale = nullptr;
    if (st != GNS_OK) return st;
  }
  return GNS_OK;
}

// Gram Newton-Schulz (Dion3 §4.2, Algorithm 3; Algorithm 2 algebra when
// `naive`) on one sub-batch of a validated problem; rows, out_idx and
// out_rows as for enqueue_standard.
gns_status enqueue_gram(const Ctx &c, const void *X, void *out, int io, int64_t n,
                        const double *coeffs, int T, const std::vector<char> &restart_at,
                        const int64_t *row_idx, const int64_t *out_idx, int64_t out_rows, bool naive) {
  gns_status st;
  void *R = c.sq(0), *Z = c.sq(1), *RZ = c.sq(2);
  void *Qb[2] = {c.sq(3), c.sq(4)};
  void *XT[2] = {c.xt(0), c.xt(1)};
  int qcur = 0, xcur = 0;
  bool q_is_identity = true;
  float q_shift = 0.0f;   // Q is Qb[qcur] + q_shift I (nonzero right after an identity Q)
  const double nn = static_cast<double>(c.pl->r);
  const double n3 = nn * nn * nn;

  if ((st = normalize(c, X, io, n, row_idx)) != GNS_OK) return st;
  if ((st = c.mark_stagger()) != GNS_OK) return st;
  if ((st = syrk(c, R, true)) != GNS_OK) return st;                  // R_0 = X X^T
  // K-major form: X in row layout, the caller's X on the direct path, else
  // the normalised copy; restarts alternate between two row buffers (the
  // transposed-copy buffers, unused in this form, hold the second one)
  void *rows[2] = {c.xh(), c.xt(0)};
  const void *xrow = c.direct ? c.xsrc() : c.xh();
  int64_t xrow_ld = c.direct ? c.pl->m : c.pl->Mp;
  int rcur = c.direct ? 0 : 1;
  // the unscaled input (row-major, or its transpose) carries the normalisation as a factor
  const float *x_scale = c.direct ? c.inv() : nullptr;
  for (int t = 1; t <= T; ++t) {
    const float a = static_cast<float>(coeffs[3 * (t - 1) + 0]);
    const float b = static_cast<float>(coeffs[3 * (t - 1) + 1]);
    const float cc = static_cast<float>(coeffs[3 * (t - 1) + 2]);
    if (t > 1 && restart_at[t - 1]) {
      // restart: X <- Q X, R <- X X^T, Q <- I.  Transposed form: the row
      // layout is written in place and the transposed copy swapped; K-major
      // form: the row layout goes to the other row buffer.
      if (c.nn) {
        st = apply_nn(c, Qb[qcur], xrow, xrow_ld, rows[rcur], q_shift, false, nullptr, io, n, nullptr,
                      "restart_apply", x_scale);
        xrow = rows[rcur];
        xrow_ld = c.pl->Mp;
        rcur ^= 1;
      } else {
        st = apply(c, Qb[qcur], XT[xcur], XT[xcur ^ 1], q_shift, false, nullptr, io, n, nullptr, "restart_apply",
                   x_scale);
        xcur ^= 1;
      }
      x_scale = nullptr;
      q_shift = 0.0f;
      if (st != GNS_OK) return st;
      if ((st = syrk(c, R, false, c.nn ? xrow : nullptr)) != GNS_OK) return st;
      q_is_identity = true;
    }
    const bool need_r = (t < T) && !restart_at[t];
    if (!naive) {
      // Z = b R + c R^2.  With Q = I the Q update is Z + a I (Dion3 §4.1:
      // the first product is free); it stays implicit: Z goes into the Q
      // buffer and the next product that uses Q adds the a I term itself.
      const void *Zt = Z;
      if (q_is_identity) {
        st = symm(c, R, R, cc, b, R, Qb[qcur], nullptr, 0.0f, 0.0f, "poly_q", n3);
        Zt = Qb[qcur];
        q_shift = a;                   // Q = Qb[qcur] + q_shift I
        q_is_identity = false;
      } else {
        st = symm(c, R, R, cc, b, R, Z, nullptr, 0.0f, 0.0f, "poly", n3);
        if (st == GNS_OK) {
          if (q_shift != 0.0f) {
            // (Zq + s I) Z + a (Zq + s I) = Zq Z + a Zq + s Z + a s I
            st = symm(c, Qb[qcur], Z, 1.0f, a, Qb[qcur], Qb[qcur ^ 1], nullptr, a * q_shift, 0.0f,
                      "q_update", n3, Z, q_shift);
            q_shift = 0.0f;
          } else {
            st = symm(c, Qb[qcur], Z, 1.0f, a, Qb[qcur], Qb[qcur ^ 1], nullptr, 0.0f, 0.0f, "q_update", n3);
          }
          qcur ^= 1;
        }
      }
      if (st != GNS_OK) return st;
      if (need_r) {
        if ((st = symm(c, R, Zt, 1.0f, a, R, RZ, nullptr, 0.0f, 0.0f, "rz", n3)) != GNS_OK) return st;
        if ((st = symm(c, Zt, RZ, 1.0f, a, RZ, R, nullptr, 0.0f, 0.0f, "r_update", n3)) != GNS_OK) return st;
      }
    } else {
      // Algorithm 2 algebra: Z = a I + b R + c R^2, Q <- Q Z, R <- Z R Z
      if (q_is_identity) {
        st = symm(c, R, R, cc, b, R, Z, Qb[qcur], a, a, "poly_q", n3);
        q_is_identity = false;
      } else {
        st = symm(c, R, R, cc, b, R, Z, nullptr, a, 0.0f, "poly", n3);
        if (st == GNS_OK) {
          st = symm(c, Qb[qcur], Z, 1.0f, 0.0f, nullptr, Qb[qcur ^ 1], nullptr, 0.0f, 0.0f, "q_update", n3);
          qcur ^= 1;
        }
      }
      if (st != GNS_OK) return st;
      if (need_r) {
        if ((st = symm(c, R, Z, 1.0f, 0.0f, nullptr, RZ, nullptr, 0.0f, 0.0f, "rz", n3)) != GNS_OK) return st;
        if ((st = symm(c, Z, RZ, 1.0f, 0.0f, nullptr, R, nullptr, 0.0f, 0.0f, "r_update", n3)) != GNS_OK) return st;
      }
    }
  }
  // out = Q_T X
  if (c.nn)
    return apply_nn(c, Qb[qcur], xrow, xrow_ld, nullptr, q_shift, true, out, io, out_rows, out_idx, "final_apply",
                    x_scale);
  return apply(c, Qb[qcur], XT[xcur], nullptr, q_shift, true, out, io, out_rows, out_idx, "final_apply",
               x_scale);
}

// Gram NS runs its rectangular products with X row-major (K-major B) for
// unsplit 16-bit compute types on 256-edge tiles when the problem is wide and
// a whole X fits the 32-bit range of a buffer descriptor.  Against the
// transposed copies this drops two HBM writes of X per call (the input
// transpose and the restart's second layout).
bool kmajor_products(const Plan &pl, int cdt) {
  return (cdt == GNS_BF16 || cdt == GNS_F16) && pl.planes == 1 && pl.tile == 256 && !pl.tall &&
         pl.Np * pl.Mp * pl.esz < (int64_t(1) << 31);
}

// The direct input path applies when X can stand in for its normalised copy:
// X is already in the (16-bit, unsplit) compute type, the matrices (or their
// row subsets) fill whole tiles, and X is 16-byte aligned.
bool direct_input(const Plan &pl, const void *X, int io, int cdt) {
  return io == cdt && (cdt == GNS_BF16 || cdt == GNS_F16) && pl.planes == 1 &&
         !pl.tall && pl.rows % pl.tile == 0 && pl.m % pl.tile == 0 &&
         (reinterpret_cast<uintptr_t>(X) & 15) == 0;
}

// --------------------------------------------------------------------------
// sub-batch fan-out
// --------------------------------------------------------------------------
// A call's matrices are independent, so a batch is split into two halves that
// run the whole sequence on two library-owned streams.  The kernels of one
// half then fill the CUs that the other half's launch leaves idle in its last,
// partial wave of tiles.  The caller's stream forks to both streams and waits
// for both before anything it enqueues later, so ordering is as if every
// kernel ran on the caller's stream.
// The second half starts once the first has normalised its input.  Two
// halves in step would run every product side by side and end their partial
// last waves together; shifted by about half a product, one half's last wave
// overlaps the other's full ones (8 x 4096x16384 bf16: 21.39 -> 21.11 ms with
// the blocked Gram-matrix order; no change without it).
constexpr int kSplit = 2;   // 3 and 4 parts measured slower (22.9 and 24.0 vs 22.0 ms per call)
constexpr int kMaxDevices = 64;

// The streams and events belong to one host thread and one device.  Calls
// from different threads therefore never share them: they do not serialise
// on each other, and a call on one thread never enqueues into streams that
// another thread's open graph capture has joined.
struct Fanout {
  bool tried = false, ok = false;
  hipStream_t s[kSplit] = {};
  hipEvent_t fork = nullptr;
  hipEvent_t join[kSplit] = {};
  hipEvent_t stagger[kSplit] = {};
};
thread_local Fanout t_fanout[kMaxDevices];

// This thread's streams and events for the current device, created on first
// use (default priority, non-blocking; kept until the process ends); nullptr
// when the device cannot provide them.
Fanout *fanout_for_current_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  Fanout *f = &t_fanout[dev];
  if (!f->tried) {
    f->tried = true;
    bool ok = hipEventCreateWithFlags(&f->fork, hipEventDisableTiming) == hipSuccess;
    for (int i = 0; i < kSplit && ok; ++i) {
      ok = hipStreamCreateWithFlags(&f->s[i], hipStreamNonBlocking) == hipSuccess &&
           hipEventCreateWithFlags(&f->join[i], hipEventDisableTiming) == hipSuccess &&
           hipEventCreateWithFlags(&f->stagger[i], hipEventDisableTiming) == hipSuccess;
    }
    f->ok = ok;
  }
  return f->ok ? f : nullptr;
}

// Enqueues body(ctx) for the whole batch on `caller`, or for two halves on the
// fan-out streams.  body enqueues the matrices [ctx.b0, ctx.b0 + ctx.batch).
template <class Body>
gns_status run_batches(const Plan &pl, int cdt, int64_t batch, void *workspace,
                       hipStream_t caller, bool split, Body &&body) {
  unsigned char *ws = static_cast<unsigned char *>(workspace);
  Fanout *f = (split && batch >= 2) ? fanout_for_current_device() : nullptr;
  if (!f) return body(Ctx{&pl, cdt, batch, 0, ws, caller});
  if (hipEventRecord(f->fork, caller) != hipSuccess) return GNS_E_HIP;
  gns_status st = GNS_OK;
  const int parts = static_cast<int>(std::min<int64_t>(kSplit, batch));
  for (int i = 0; i < parts; ++i) {
    const int64_t b0 = batch * i / parts;
    const int64_t nb = batch * (i + 1) / parts - b0;
    if (hipStreamWaitEvent(f->s[i], f->fork, 0) != hipSuccess) { st = GNS_E_HIP; continue; }
    // part i starts after part i-1 has normalised (recorded while its body
    // was enqueued, so the event is always recorded before this wait)
    if (i > 0 && st == GNS_OK && hipStreamWaitEvent(f->s[i], f->stagger[i - 1], 0) != hipSuccess) {
      st = GNS_E_HIP;
      continue;
    }
    Ctx c{&pl, cdt, nb, b0, ws, f->s[i]};
    if (i + 1 < parts) c.stagger = f->stagger[i];
    if (st == GNS_OK) st = body(c);
  }
  // always join, so that the caller's stream orders after whatever was enqueued
  for (int i = 0; i < parts; ++i) {
    if (hipEventRecord(f->join[i], f->s[i]) != hipSuccess ||
        hipStreamWaitEvent(caller, f->join[i], 0) != hipSuccess)
      st = GNS_E_HIP;
  }
  return st;
}

// --------------------------------------------------------------------------
// Dion3 update: workspace layout after the orthogonalisation's own workspace
// --------------------------------------------------------------------------
struct Dion3Layout {
  size_t off_keys = 0, off_msq = 0, off_o = 0, off_rowsq = 0, off_factor = 0, bytes = 0;
};

// The orthogonalisation's region is sized for 256-padded buffers (any tile
// choice fits), so the regions after it do not depend on the tile.
bool dion3_layout(int cdt, int64_t batch, int64_t n, int64_t m, int64_t k, Dion3Layout *d) {
  Plan pl;
  if (batch <= 0 || n < 1 || k < 1 || k > n || !make_plan(cdt, batch, k, m, 5, 256, &pl)) return false;
  size_t off = align_up(pl.bytes, kAlign);
  d->off_keys = off;                                  // fp64 row keys [batch][n]
  off = align_up(off + sizeof(double) * batch * n, kAlign);
  d->off_msq = off;                                   // fp64 row sums of M^2 [batch][n]
  off = align_up(off + sizeof(double) * batch * n, kAlign);
  d->off_o = off;                                     // fp32 update O [batch][k][m]
  off = align_up(off + sizeof(float) * batch * k * m, kAlign);
  d->off_rowsq = off;                                 // fp64 row sums of O^2 [batch][k]
  off = align_up(off + sizeof(double) * batch * k, kAlign);
  d->off_factor = off;                                // fp64 row factors [batch][k]
  off = align_up(off + sizeof(double) * batch * k, kAlign);
  d->bytes = off;
  return true;
}

// ---------------------------------------------------------------- autotune
// Shape-keyed table of measured tile choices (GNS_OPT_TILE_AUTOTUNE); the
// value is the TILE option bit that won, or kRuleChoice for the size rule's
// own plan (which alone may also split the Gram matrix along K).
constexpr unsigned kRuleChoice = 0x80000000u;
struct TuneKey {
  int standard, cdt, io;
  int64_t batch, rows, m;
  bool operator<(const TuneKey &o) const {
    return std::tie(standard, cdt, io, batch, rows, m) <
           std::tie(o.standard, o.cdt, o.io, o.batch, o.rows, o.m);
  }
};
std::mutex g_tune_mu;
std::map<TuneKey, unsigned> g_tune;

unsigned tuned_choice(const TuneKey &key) {
  std::lock_guard<std::mutex> lk(g_tune_mu);
  const auto it = g_tune.find(key);
  return it == g_tune.end() ? 0u : it->second;
}

void keep_choice(const TuneKey &key, unsigned bit) {
  std::lock_guard<std::mutex> lk(g_tune_mu);
  g_tune[key] = bit;
}

// run(bits) enqueues the whole call with the tile bits `bits` (0: size-based
// choice).  An untuned shape is timed with every choice, twice each (the
// first runs also pay one-time costs such as stream creation), and the
// winner's result is left in the output.
template <class Run>
gns_status autotune(const TuneKey &key, hipStream_t s, Run run) {
  const unsigned kept = tuned_choice(key);
  if (kept) return run(kept == kRuleChoice ? 0u : kept);
  if (key.cdt == GNS_F32 || key.cdt == GNS_BF16X3) {   // one tile edge only
    const gns_status st = run(GNS_OPT_TILE_128);
    if (st == GNS_OK) keep_choice(key, GNS_OPT_TILE_128);
    return st;
  }
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &cs) != hipSuccess) return GNS_E_HIP;
  if (cs != hipStreamCaptureStatusNone) return run(0);   // no timing inside a capture
  hipEvent_t ev[2] = {nullptr, nullptr};
  if (hipEventCreate(&ev[0]) != hipSuccess || hipEventCreate(&ev[1]) != hipSuccess) {
    if (ev[0]) (void)hipEventDestroy(ev[0]);
    return GNS_E_HIP;
  }
  constexpr int kChoices = 4;
  const unsigned bits[kChoices] = {GNS_OPT_TILE_128, GNS_OPT_TILE_256, GNS_OPT_TILE_MIXED, kRuleChoice};
  float best[kChoices] = {INFINITY, INFINITY, INFINITY, INFINITY};
  gns_status st = GNS_OK;
  for (int rep = 0; rep < 2 && st == GNS_OK; ++rep)
    for (int i = 0; i < kChoices && st == GNS_OK; ++i) {
      float ms = 0.0f;
      if (hipEventRecord(ev[0], s) != hipSuccess) { st = GNS_E_HIP; break; }
      if ((st = run(bits[i] == kRuleChoice ? 0u : bits[i])) != GNS_OK) break;
      if (hipEventRecord(ev[1], s) != hipSuccess || hipEventSynchronize(ev[1]) != hipSuccess ||
          hipEventElapsedTime(&ms, ev[0], ev[1]) != hipSuccess) {
        st = GNS_E_HIP;
        break;
      }
      best[i] = std::min(best[i], ms);
    }
  (void)hipEventDestroy(ev[0]);
  (void)hipEventDestroy(ev[1]);
  if (st != GNS_OK) return st;
  int win = 0;
  for (int i = 1; i < kChoices; ++i)
    if (best[i] < best[win]) win = i;
  // the last run used the last choice: leave the winner's result in the output
  if (win != kChoices - 1 && (st = run(bits[win] == kRuleChoice ? 0u : bits[win])) != GNS_OK) return st;
  keep_choice(key, bits[win]);
  return GNS_OK;
}

// --------------------------------------------------------------- call plan
// Everything a gns_gram_batched / gns_standard_batched call decides on the
// host before it enqueues anything (also reported by gns_call_plan).
struct CallPlan {
  Plan pl;
  int64_t rows = 0;
  bool standard = false;     // runs standard NS (that entry point, or the square fallback)
  bool naive = false;        // Algorithm 2 algebra
  bool direct = false;       // the products read X itself (no normalised copy)
  bool nn = false;           // Q X reads X row-major (K-major B operand)
  bool inplace = false;      // out is X
  bool copy_input = false;   // the input pass copies X into the workspace (Ctx::xcopy)
  bool split = false;        // the batch may be split over the library's streams
  bool autotune = false;     // GNS_OPT_TILE_AUTOTUNE
  bool timed = false;        // this call would time an untuned shape
  bool debug = false;        // GNS_OPT_DEBUG_CHECKS
  std::vector<char> restart_at;
};

gns_status plan_call(bool standard_entry, const void *X, const void *out, int64_t batch, int64_t n, int64_t m,
                     gns_dtype io, gns_dtype cdt, const double *coeffs, int T, const int *restart_after,
                     int n_restart, const int64_t *row_idx, int64_t k, unsigned opts, CallPlan *cp) {
  int64_t rows = 0;
  gns_status st = common_checks(X, out, batch, n, m, io, cdt, coeffs, T, row_idx, k, &rows);
  if (st != GNS_OK) return st;
  int tile_req = 0;
  const unsigned allowed = GNS_OPT_TILE_AUTOTUNE | GNS_OPT_DEBUG_CHECKS |
                           (standard_entry ? 0u : GNS_OPT_NAIVE_ALGEBRA | GNS_OPT_NO_SQUARE_FALLBACK);
  if ((st = parse_opts(opts, allowed, &tile_req)) != GNS_OK) return st;
  if (standard_entry) {
    cp->restart_at.assign(T + 2, 0);
  } else if ((st = parse_restarts(restart_after, n_restart, T, &cp->restart_at)) != GNS_OK) {
    return st;
  }
  cp->rows = rows;
  if (batch == 0) return GNS_OK;
  // out is either X itself or a separate buffer: a partial overlap would let
  // the output of one matrix overwrite input another still reads
  const size_t io_bytes = static_cast<size_t>(batch) * n * m * gns::dtype_size(io);
  cp->inplace = X == out;
  if (!cp->inplace && ranges_overlap(X, io_bytes, out, io_bytes)) return GNS_E_ALIAS;
  cp->autotune = (opts & GNS_OPT_TILE_AUTOTUNE) != 0;
  cp->debug = (opts & GNS_OPT_DEBUG_CHECKS) != 0;
  cp->split = !(opts & GNS_OPT_ONE_STREAM);
  cp->naive = (opts & GNS_OPT_NAIVE_ALGEBRA) != 0;
  if (cp->autotune) {
    // the plan of the kept choice, or of the size rule until the shape is
    // tuned; an in-place call is never timed (every timed run would
    // orthogonalise the previous run's output again)
    const unsigned kept = tuned_choice(TuneKey{standard_entry ? 1 : 0, cdt, io, batch, rows, m});
    const bool one_edge = cdt == GNS_F32 || cdt == GNS_BF16X3;
    cp->timed = !kept && !cp->inplace && !one_edge;
    unsigned bits = kept == kRuleChoice ? 0u : kept;
    if (one_edge) bits = GNS_OPT_TILE_128;
    parse_opts(bits, 0, &tile_req);
  }
  if (!make_plan(cdt, batch, rows, m, standard_entry ? 2 : 5, tile_req, &cp->pl)) return GNS_E_SHAPE;
  // Square matrices: both algorithms cost the same and standard NS needs
  // fewer launches and never forms X X^T of an ill-conditioned square
  // matrix, so Dion3 falls back to it (§4.1, last paragraph).
  cp->standard = standard_entry || (rows == m && !(opts & GNS_OPT_NO_SQUARE_FALLBACK));
  cp->nn = !cp->standard && kmajor_products(cp->pl, cdt);
  // A row subset takes the direct path in the K-major form only: its input
  // pass gathers the rows, unscaled, into a workspace region that form never
  // uses (elsewhere that region holds the second transposed copy).
  cp->direct = direct_input(cp->pl, X, io, cdt) && (!row_idx || cp->nn);
  // In place on the direct path, the final Q X reads X (K-major form) when
  // no restart has replaced it by a workspace buffer: the input pass then
  // copies X, and the products read the copy.  (The transposed form and
  // standard NS read X only in their first product, before any output is
  // written; a normalised copy is never X.)  A row subset always reads its
  // gathered copy.
  const bool restarted = std::find(cp->restart_at.begin(), cp->restart_at.end(), 1) != cp->restart_at.end();
  cp->copy_input = cp->direct && cp->nn && ((cp->inplace && !restarted) || row_idx != nullptr);
  return GNS_OK;
}

// Enqueues a planned, validated call (no autotune, no debug checks).
gns_status enqueue_call(const CallPlan &cp, int cdt, const void *X, void *out, int64_t batch, int64_t n,
                        int64_t m, int io, const double *coeffs, int T, const int64_t *row_idx, int64_t k,
                        void *workspace, hipStream_t caller) {
  const size_t io_mat = static_cast<size_t>(n) * m * gns::dtype_size(io);
  return run_batches(cp.pl, cdt, batch, workspace, caller, cp.split, [&](const Ctx &c0) {
    const unsigned char *Xs = static_cast<const unsigned char *>(X) + c0.b0 * io_mat;
    Ctx c = c0;
    c.direct = cp.direct;
    c.nn = cp.nn;
    c.xin = Xs;
    if (cp.copy_input) c.xcopy = c.xt(1);   // a region the K-major form never uses
    const int64_t *ri = row_idx ? row_idx + c.b0 * k : nullptr;
    unsigned char *os = static_cast<unsigned char *>(out) + c.b0 * io_mat;
    if (cp.standard) return enqueue_standard(c, Xs, os, io, n, coeffs, T, ri, ri, n);
    return enqueue_gram(c, Xs, os, io, n, coeffs, T, cp.restart_at, ri, ri, n, cp.naive);
  });
}

// Synchronous read of the debug-check flag in the workspace (4 bytes).
gns_status read_flag(const int32_t *flag, hipStream_t s, int32_t *value) {
  if (hipMemcpyAsync(value, flag, sizeof(int32_t), hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return GNS_E_HIP;
  return GNS_OK;
}

gns_status orthogonalise(bool standard_entry, const void *X, void *out, int64_t batch, int64_t n, int64_t m,
                         gns_dtype io, gns_dtype cdt, const double *coeffs, int T, const int *restart_after,
                         int n_restart, const int64_t *row_idx, int64_t k, unsigned opts, void *workspace,
                         size_t workspace_bytes, void *stream) {
  CallPlan cp;
  gns_status st = plan_call(standard_entry, X, out, batch, n, m, io, cdt, coeffs, T, restart_after, n_restart,
                            row_idx, k, opts, &cp);
  if (st != GNS_OK || batch == 0) return st;
  if ((st = workspace_checks(X, out, batch, n, m, io, cp.pl, workspace, workspace_bytes)) != GNS_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t *flag = reinterpret_cast<int32_t *>(static_cast<unsigned char *>(workspace) + cp.pl.off_flag);
  if (cp.debug) {
    // the checks synchronise the stream, which a graph capture cannot do
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &cs) != hipSuccess) return GNS_E_HIP;
    if (cs != hipStreamCaptureStatusNone) return GNS_E_FLAGS;
    if (row_idx && n <= 65536) {
      int32_t bad = 0;
      if (gns::launch_check_rows(row_idx, batch, k, n, flag, s) != hipSuccess) return GNS_E_HIP;
      if ((st = read_flag(flag, s, &bad)) != GNS_OK) return st;
      if (bad) return GNS_E_ROWIDX;
    }
  }
  if (cp.autotune) {
    const unsigned inner = opts & ~(GNS_OPT_TILE_AUTOTUNE | GNS_OPT_DEBUG_CHECKS);
    auto run = [&](unsigned bits) {
      return orthogonalise(standard_entry, X, out, batch, n, m, io, cdt, coeffs, T, restart_after, n_restart,
                           row_idx, k, inner | bits, workspace, workspace_bytes, stream);
    };
    const TuneKey key{standard_entry ? 1 : 0, cdt, io, batch, cp.rows, m};
    st = cp.inplace ? run(tuned_choice(key) == kRuleChoice ? 0u : tuned_choice(key)) : autotune(key, s, run);
  } else {
    st = enqueue_call(cp, cdt, X, out, batch, n, m, io, coeffs, T, row_idx, k, workspace, s);
  }
  if (st != GNS_OK || !cp.debug) return st;
  int32_t bad = 0;
  if (gns::launch_check_finite(io, out, batch, n, m, row_idx, k, flag, s) != hipSuccess) return GNS_E_HIP;
  if ((st = read_flag(flag, s, &bad)) != GNS_OK) return st;
  return bad ? GNS_E_NONFINITE : GNS_OK;
}

}  // namespace

// ==========================================================================
// exported ABI
// ==========================================================================
extern "C" {

int gns_abi_version(void) { return GNS_ABI_VERSION; }

const char *gns_status_str(gns_status s) {
  switch (s) {
    case GNS_OK: return "ok";
    case GNS_E_NULL: return "required pointer is NULL";
    case GNS_E_SHAPE: return "invalid shape";
    case GNS_E_DTYPE: return "unsupported dtype";
    case GNS_E_COEFF: return "invalid iteration count or coefficient";
    case GNS_E_RESTART: return "restart iterations must be strictly increasing in [1, T-1]";
    case GNS_E_ROWIDX: return "row index out of range or repeated";
    case GNS_E_ALIAS: return "buffers overlap (workspace with X or out, or out partly with X)";
    case GNS_E_WORKSPACE: return "workspace missing, misaligned or too small";
    case GNS_E_HIP: return "HIP launch failed";
    case GNS_E_FLAGS: return "unknown option bits";
    case GNS_E_PARAM: return "invalid update hyperparameter";
    case GNS_E_NONFINITE: return "result holds Inf or NaN (debug checks)";
  }
  return "unknown status";
}

size_t gns_gram_workspace_bytes(gns_dtype cdt, int64_t batch, int64_t rows, int64_t m) {
  Plan pl;
  if (batch <= 0 || !make_plan(cdt, batch, rows, m, 5, 256, &pl)) return 0;
  return pl.bytes;
}

size_t gns_standard_workspace_bytes(gns_dtype cdt, int64_t batch, int64_t rows, int64_t m) {
  Plan pl;
  if (batch <= 0 || !make_plan(cdt, batch, rows, m, 2, 256, &pl)) return 0;
  return pl.bytes;
}

gns_status gns_gram_batched(const void *X, void *out, int64_t batch, int64_t n, int64_t m,
                            gns_dtype io, gns_dtype cdt, const double *coeffs, int T,
                            const int *restart_after, int n_restart, const int64_t *row_idx,
                            int64_t k, unsigned opts, void *workspace, size_t workspace_bytes,
                            void *stream) {
  return orthogonalise(false, X, out, batch, n, m, io, cdt, coeffs, T, restart_after, n_restart, row_idx, k,
                       opts, workspace, workspace_bytes, stream);
}

gns_status gns_standard_batched(const void *X, void *out, int64_t batch, int64_t n, int64_t m,
                                gns_dtype io, gns_dtype cdt, const double *coeffs, int T,
                                const int64_t *row_idx, int64_t k, unsigned opts, void *workspace,
                                size_t workspace_bytes, void *stream) {
  return orthogonalise(true, X, out, batch, n, m, io, cdt, coeffs, T, nullptr, 0, row_idx, k, opts, workspace,
                       workspace_bytes, stream);
}

gns_status gns_call_plan(int standard, const void *X, const void *out, int64_t batch, int64_t n, int64_t m,
                         gns_dtype io, gns_dtype cdt, const double *coeffs, int T, const int *restart_after,
                         int n_restart, const int64_t *row_idx, int64_t k, unsigned opts, gns_plan_info *info) {
  if (!info) return GNS_E_NULL;
  CallPlan cp;
  const gns_status st = plan_call(standard != 0, X, out, batch, n, m, io, cdt, coeffs, T, restart_after,
                                  n_restart, row_idx, k, opts, &cp);
  if (st != GNS_OK) return st;
  std::memset(info, 0, sizeof(*info));
  if (batch == 0) return GNS_OK;
  info->standard = cp.standard ? 1 : 0;
  info->tile = cp.pl.tile;
  info->sym_tile = cp.pl.sym_tile;
  info->gram_tile = cp.pl.gram_tile;
  info->gram_parts = cp.pl.syrk_parts;
  info->direct_input = cp.direct ? 1 : 0;
  info->kmajor_products = cp.nn ? 1 : 0;
  info->input_copy = cp.copy_input ? 1 : 0;
  info->split_streams = (cp.split && batch >= 2) ? 1 : 0;
  info->autotune_timed = cp.timed ? 1 : 0;
  info->workspace_bytes = cp.pl.bytes;
  return GNS_OK;
}

int gns_tuned_tile(int standard, gns_dtype cdt, gns_dtype io, int64_t batch, int64_t rows, int64_t m,
                   int *sym_edge) {
  const unsigned bit = tuned_choice(TuneKey{standard ? 1 : 0, cdt, io, batch, rows, m});
  int rect = bit == GNS_OPT_TILE_128 ? 128 : bit ? 256 : 0;
  int sym = bit == GNS_OPT_TILE_256 ? 256 : bit ? 128 : 0;
  Plan pl;
  if (bit == kRuleChoice && make_plan(cdt, batch, rows, m, standard ? 2 : 5, 0, &pl)) {
    rect = pl.tile;
    sym = pl.sym_tile;
  }
  if (sym_edge) *sym_edge = sym;
  return rect;
}

void gns_autotune_clear(void) {
  std::lock_guard<std::mutex> lk(g_tune_mu);
  g_tune.clear();
}

size_t gns_select_workspace_bytes(int64_t batch, int64_t n) {
  if (batch <= 0 || n < 1) return 0;
  return align_up(sizeof(double) * static_cast<size_t>(batch) * static_cast<size_t>(n), kAlign);
}

gns_status gns_select_rows_l1(const void *M, int64_t batch, int64_t n, int64_t m, gns_dtype dtype,
                              int64_t k, int64_t *row_idx, void *workspace, size_t workspace_bytes,
                              void *stream) {
  if (!valid_dtype(dtype)) return GNS_E_DTYPE;
  if (batch < 0 || n < 1 || m < 1 || k < 1 || k > n || batch > 65535 ||
      n > (int64_t(1) << 31) - 1024)
    return GNS_E_SHAPE;
  if (batch == 0) return GNS_OK;
  if (!M || !row_idx) return GNS_E_NULL;
  if (!workspace || workspace_bytes < gns_select_workspace_bytes(batch, n) ||
      (reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)))
    return GNS_E_WORKSPACE;
  const size_t in_bytes = static_cast<size_t>(batch) * n * m * gns::dtype_size(dtype);
  const size_t ws_used = gns_select_workspace_bytes(batch, n);
  if (ranges_overlap(workspace, ws_used, M, in_bytes) ||
      ranges_overlap(workspace, ws_used, row_idx, sizeof(int64_t) * batch * k))
    return GNS_E_ALIAS;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const double bytes = static_cast<double>(in_bytes);
  LaunchScope ls(s, "select_rows_l1", "row_l1+select_topk", 2.0 * batch * n * m, bytes);
  hipError_t e = gns::launch_select_rows_l1(dtype, M, batch, n, m, k, static_cast<double *>(workspace),
                                            row_idx, s);
  ls.done();
  return e == hipSuccess ? GNS_OK : GNS_E_HIP;
}

size_t gns_dion3_workspace_bytes(gns_dtype cdt, int64_t batch, int64_t n, int64_t m, int64_t k) {
  Dion3Layout d;
  if (!dion3_layout(cdt, batch, n, m, k, &d)) return 0;
  return d.bytes;
}

gns_status gns_dion3_step(float *W, const void *G, float *M, float *v, int64_t batch, int64_t n,
                          int64_t m, gns_dtype grad_dtype, gns_dtype cdt, int64_t k,
                          const double *coeffs, int T, const int *restart_after, int n_restart,
                          double lr, double weight_decay, double mu, double beta2, double eps,
                          int normuon, int64_t *row_idx, unsigned opts, void *workspace,
                          size_t workspace_bytes, void *stream) {
  if (!valid_dtype(grad_dtype) || !valid_compute(cdt)) return GNS_E_DTYPE;
  if (batch < 0 || n < 1 || m < 1 || k < 1 || k > n || batch > 65535 || n > (int64_t(1) << 30))
    return GNS_E_SHAPE;
  gns_status st = check_coeffs(coeffs, T);
  if (st != GNS_OK) return st;
  if (!std::isfinite(lr) || !std::isfinite(weight_decay) || !std::isfinite(mu) || !std::isfinite(beta2) ||
      !std::isfinite(eps) || (normuon && !(eps > 0.0)))
    return GNS_E_PARAM;
  int tile_req = 0;
  if ((st = parse_opts(opts, GNS_OPT_NAIVE_ALGEBRA | GNS_OPT_NO_SQUARE_FALLBACK | GNS_OPT_DEBUG_CHECKS,
                       &tile_req)) != GNS_OK)
    return st;
  std::vector<char> restart_at;
  if ((st = parse_restarts(restart_after, n_restart, T, &restart_at)) != GNS_OK) return st;
  if (batch == 0) return GNS_OK;
  if (!W || !G || !M || !row_idx || (normuon && !v)) return GNS_E_NULL;
  const bool debug = (opts & GNS_OPT_DEBUG_CHECKS) != 0;
  Plan pl;
  Dion3Layout d;
  if (!make_plan(cdt, batch, k, m, 5, tile_req, &pl) || !dion3_layout(cdt, batch, n, m, k, &d))
    return GNS_E_SHAPE;
  if (!workspace || workspace_bytes < d.bytes || (reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)))
    return GNS_E_WORKSPACE;
  const size_t elems = static_cast<size_t>(batch) * n * m;
  struct Range { const void *p; size_t bytes; };
  const Range user[] = {{W, elems * 4}, {M, elems * 4}, {G, elems * gns::dtype_size(grad_dtype)},
                        {row_idx, sizeof(int64_t) * batch * k},
                        {normuon ? v : nullptr, sizeof(float) * batch * n}};
  for (const Range &r : user)
    if (r.p && ranges_overlap(workspace, d.bytes, r.p, r.bytes)) return GNS_E_ALIAS;
  for (int i = 0; i < 5; ++i)
    for (int j = i + 1; j < 5; ++j)
      if (user[i].p && user[j].p && ranges_overlap(user[i].p, user[i].bytes, user[j].p, user[j].bytes))
        return GNS_E_ALIAS;

  hipStream_t s = static_cast<hipStream_t>(stream);
  if (debug) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &cs) != hipSuccess) return GNS_E_HIP;
    if (cs != hipStreamCaptureStatusNone) return GNS_E_FLAGS;
  }
  unsigned char *ws = static_cast<unsigned char *>(workspace);
  double *keys = reinterpret_cast<double *>(ws + d.off_keys);
  double *msq = reinterpret_cast<double *>(ws + d.off_msq);
  float *O = reinterpret_cast<float *>(ws + d.off_o);
  double *rowsq = reinterpret_cast<double *>(ws + d.off_rowsq);
  double *factor = reinterpret_cast<double *>(ws + d.off_factor);
  const double bn = static_cast<double>(batch) * n, bk = static_cast<double>(batch) * k;
  const double gsz = gns::dtype_size(grad_dtype);
  // Algorithm 4, first two steps: M <- M + G, then the k rows of largest l1
  // norm (the same pass keeps every row's sum of squares for the norm of the
  // selected rows)
  {
    LaunchScope ls(s, "momentum_l1", "momentum_l1", 4.0 * bn * m, bn * m * (8.0 + gsz));
    hipError_t e = gns::launch_momentum_l1(grad_dtype, M, G, batch, n, m, keys, msq, s);
    ls.done();
    if (e != hipSuccess) return GNS_E_HIP;
  }
  {
    LaunchScope ls(s, "select_topk", "select_topk", bn, 8.0 * bn * 8.0 + 8.0 * bk);
    hipError_t e = gns::launch_select_topk(keys, batch, n, k, row_idx, s);
    ls.done();
    if (e != hipSuccess) return GNS_E_HIP;
  }
  // orthogonalise M[S,:] into the k x m update O (fp32, not scattered)
  const size_t in_mat = static_cast<size_t>(n) * m;
  const size_t o_mat = static_cast<size_t>(k) * m;
  const bool naive = (opts & GNS_OPT_NAIVE_ALGEBRA) != 0;
  const bool square = (k == m) && !(opts & GNS_OPT_NO_SQUARE_FALLBACK);
  st = run_batches(pl, cdt, batch, workspace, s, !(opts & GNS_OPT_ONE_STREAM), [&](const Ctx &c) {
    const float *Xs = M + c.b0 * in_mat;
    float *Os = O + c.b0 * o_mat;
    const int64_t *ri = row_idx + c.b0 * k;
    Ctx cg = c;
    cg.row_sumsq = msq + c.b0 * n;
    if (square) return enqueue_standard(cg, Xs, Os, GNS_F32, n, coeffs, T, ri, nullptr, k);
    cg.nn = kmajor_products(pl, cdt);
    return enqueue_gram(cg, Xs, Os, GNS_F32, n, coeffs, T, restart_at, ri, nullptr, k, naive);
  });
  if (st != GNS_OK) return st;
  if (debug) {
    // a non-finite update is reported before it reaches W, v or the error
    // feedback (M then holds M + G, row_idx the selection)
    int32_t *flag = reinterpret_cast<int32_t *>(ws + pl.off_flag);
    int32_t bad = 0;
    if (gns::launch_check_finite(GNS_F32, O, batch, k, m, nullptr, 0, flag, s) != hipSuccess) return GNS_E_HIP;
    if ((st = read_flag(flag, s, &bad)) != GNS_OK) return st;
    if (bad) return GNS_E_NONFINITE;
  }
  // NorMuon row factors (second moment v at the selected rows), then the
  // decay, the update of the selected rows and the error feedback
  {
    LaunchScope ls(s, "normuon", "row_sumsq+normuon_factors", normuon ? 2.0 * bk * m : 0.0,
                   normuon ? bk * m * 4.0 + bk * 16.0 : bk * 8.0);
    hipError_t e = gns::launch_normuon(O, batch, k, m, v, row_idx, n, beta2, eps, normuon, rowsq, factor, s);
    ls.done();
    if (e != hipSuccess) return GNS_E_HIP;
  }
  {
    const float decay = static_cast<float>(1.0 - lr * weight_decay);
    const double rows_w = decay != 1.0f ? bn : bk;
    LaunchScope ls(s, "dion3_update", "dion3_update", 3.0 * bk * m, rows_w * m * 8.0 + bk * m * 12.0);
    hipError_t e = gns::launch_dion3_update(W, M, O, row_idx, factor, batch, n, m, k, decay, lr,
                                            static_cast<float>(mu), s);
    ls.done();
    if (e != hipSuccess) return GNS_E_HIP;
  }
  return GNS_OK;
}

gns_status gns_check_row_idx(const int64_t *row_idx, int64_t batch, int64_t k, int64_t n,
                             int32_t *result, void *stream) {
  if (!row_idx || !result) return GNS_E_NULL;
  if (batch < 0 || k < 1 || n < 1 || k > n || n > 65536) return GNS_E_SHAPE;
  if (batch == 0) return GNS_OK;
  hipError_t e = gns::launch_check_rows(row_idx, batch, k, n, result, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? GNS_OK : GNS_E_HIP;
}

gns_status gns_check_finite(const void *A, gns_dtype dtype, int64_t batch, int64_t rows, int64_t cols,
                            const int64_t *row_idx, int64_t k, int32_t *result, void *stream) {
  if (!valid_dtype(dtype)) return GNS_E_DTYPE;
  if (batch < 0 || rows < 1 || cols < 1 || batch > 65535 || (row_idx && (k < 1 || k > rows))) return GNS_E_SHAPE;
  if (!result || (batch > 0 && !A)) return GNS_E_NULL;
  const hipError_t e = gns::launch_check_finite(dtype, A, batch, rows, cols, row_idx, k, result,
                                                static_cast<hipStream_t>(stream));
  return e == hipSuccess ? GNS_OK : GNS_E_HIP;
}

int64_t gns_select_count(int64_t n, double fraction) {
  if (n < 1 || !(fraction > 0.0) || !(fraction <= 1.0)) return 0;
  const double k = std::ceil(fraction * static_cast<double>(n));
  return std::max<int64_t>(1, std::min<int64_t>(n, static_cast<int64_t>(k)));
}

gns_status gns_safety_scale(const double *coeffs, int T, double s, double *out) {
  if (!coeffs || !out) return GNS_E_NULL;
  if (T < 1 || T > GNS_MAX_ITERS) return GNS_E_COEFF;
  if (!std::isfinite(s) || !(s > 0.0)) return GNS_E_PARAM;
  const double s3 = s * s * s, s5 = s3 * s * s;
  for (int t = 0; t < T; ++t) {
    const double a = coeffs[3 * t], b = coeffs[3 * t + 1], c = coeffs[3 * t + 2];
    out[3 * t] = a / s;
    out[3 * t + 1] = b / s3;
    out[3 * t + 2] = c / s5;
  }
  return GNS_OK;
}

void gns_timing_enable(int on) {
  std::lock_guard<std::mutex> lk(g_tmu);
  g_timing = on != 0;
}

void gns_timing_reset(void) {
  std::lock_guard<std::mutex> lk(g_tmu);
  for (auto &l : g_launches) {
    g_event_pool.push_back(l.start);
    g_event_pool.push_back(l.stop);
  }
  g_launches.clear();
}

int gns_timing_read(gns_launch_record *records, int cap) {
  std::lock_guard<std::mutex> lk(g_tmu);
  const int n = static_cast<int>(g_launches.size());
  for (int i = 0; i < n && i < cap && records; ++i) {
    const TimedLaunch &l = g_launches[i];
    float ms = -1.0f;
    if (hipEventSynchronize(l.stop) == hipSuccess && hipEventElapsedTime(&ms, l.start, l.stop) != hipSuccess)
      ms = -1.0f;
    records[i] = gns_launch_record{l.name, l.kernel, l.flops, l.bytes, ms};
  }
  return n;
}

}  // extern "C"
