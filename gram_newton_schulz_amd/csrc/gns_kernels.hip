// Device kernels of the Gram Newton-Schulz library, written for CDNA4 (gfx950).
//
// * norm_partial     -- Frobenius norm, first stage: per-workgroup sums of
//                       squares in fixed order (HBM-bound, vector loads).
// * scale_transpose  -- X_hat = X / (||X||_F + eps) rounded once to the
//                       compute dtype, written row-major [n][m] and, where a
//                       path reads it, transposed [m][n] (zero padded to whole
//                       tiles); the second stage of the norm reduction runs in
//                       its prologue.
// * transpose_sumsq  -- input already in the compute type: per-tile sums of
//                       squares (and the transposed copy, where one is read).
// * gemm_nt          -- C = alpha * A B^T + beta * D on bf16/fp16 (32x32x16)
//                       or fp32 (32x32x2) MFMA with fp32 accumulation, or on
//                       split hi/lo bf16 pairs (three bf16 MFMAs per product).
//                       256x256 workgroup tiles with 8 waves in ping-pong, or
//                       128x128 tiles with 4 waves; operands reach LDS by
//                       LDS-DMA buffer loads into a 5-stage ring of 32-element
//                       K stages, XOR-swizzled.  Symmetric results compute only
//                       the upper tiles and mirror them ("Dion3: Full-Stack
//                       Orthogonal Updates", §5 and App. C.1-C.2).  With a
//                       K-major B (BK = 1) the same kernel computes C = A B.
// * row_l1, select_topk, momentum_l1, row_sumsq, normuon_factors,
//   dion3_update     -- the HBM-bound steps of the Dion3 update around the
//                       orthogonalisation (Dion3 §6, Algorithm 4).
//
// Every product of the method reads its operands row-major: X X^T directly;
// products of two n x n iterates as A B^T, because every stored iterate is
// exactly symmetric (so its rows are its columns); Q X either with X as a
// K-major B (16-bit 256-edge tiles, LDS transpose reads) or, on the other
// paths, as A B^T through the transposed copy of X kept beside it.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <type_traits>

#include "gns_kernels.h"

namespace gns {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// ---------------------------------------------------------------------------
// element types
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}
// Round to nearest even; NaN stays NaN.  gfx950 converts in hardware
// (v_cvt_pk_bf16_f32, two values per instruction): checked against the
// integer rounding (u + 0x7fff + lsb) >> 16 on every fp32 bit pattern, in
// both halves, on the GPU.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{lo, hi}), bf16x2_t));
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return static_cast<uint16_t>(f32x2_to_bf16x2(f, 0.0f));
}
__device__ __forceinline__ float f16_to_f32(uint16_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, h));
}
__device__ __forceinline__ uint16_t f32_to_f16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
}
__device__ __forceinline__ uint32_t f32x2_to_f16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{lo, hi}), f16x2_t));
}

struct EBF16 {
  using S = uint16_t;
  static constexpr int code = DT_BF16;
  __device__ static float ld(S v) { return bf16_to_f32(v); }
  __device__ static S st(float f) { return f32_to_bf16(f); }
  // two values rounded into one packed pair (lo in bits 0-15)
  __device__ static uint32_t st2(float lo, float hi) { return f32x2_to_bf16x2(lo, hi); }
};
struct EF16 {
  using S = uint16_t;
  static constexpr int code = DT_F16;
  __device__ static float ld(S v) { return f16_to_f32(v); }
  __device__ static S st(float f) { return f32_to_f16(f); }
  __device__ static uint32_t st2(float lo, float hi) { return f32x2_to_f16x2(lo, hi); }
};
struct EF32 {
  using S = float;
  static constexpr int code = DT_F32;
  __device__ static float ld(S v) { return v; }
  __device__ static S st(float f) { return f; }
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// Type tag (selects the 16-bit type an epilogue rounds to).
template <class T> struct Tag { using type = T; };

// Streaming passes that read and write every element once give their loads
// and stores the non-temporal hint, which moves these mixed read/write
// streams faster (Dion3 momentum pass 4.7 -> 5.1 TB/s, update 4.7 -> 5.2,
// row sums 4.3 -> 5.4).
__device__ __forceinline__ void st_once(float4 *p, float4 x) {
  typedef float v4f __attribute__((ext_vector_type(4)));
  __builtin_nontemporal_store(v4f{x.x, x.y, x.z, x.w}, reinterpret_cast<v4f *>(p));
}
__device__ __forceinline__ float4 ld_once(const float4 *p) {
  typedef float v4f __attribute__((ext_vector_type(4)));
  const v4f v = __builtin_nontemporal_load(reinterpret_cast<const v4f *>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 ld_once(const uint2 *p) {
  typedef unsigned v2u __attribute__((ext_vector_type(2)));
  const v2u v = __builtin_nontemporal_load(reinterpret_cast<const v2u *>(p));
  return make_uint2(v.x, v.y);
}


// Streaming passes keep kUnroll 16-byte pieces per lane in flight: all their
// loads are issued before the first use, which one piece at a time (a single
// load round trip per wave) left at about two thirds of HBM bandwidth.
constexpr int kUnroll = 4;

// One lane's share of a 16-deep slice of the contraction: 8 consecutive
// elements (one 16-byte chunk for 16-bit types, two for fp32).  A and B
// fragments use the same element -> k mapping, so the products pair up
// correctly whatever k numbering the instruction uses internally.
// `load` reads slice s of a 128-byte LDS row whose chunks are XOR-swizzled
// by `sw`; lanes 32..63 (h = 1) take the second half of the slice.
template <class E>
struct Mma;

template <>
struct Mma<EBF16> {
  static constexpr int kInstr = 1;
  typedef u32x4 Frag;
  __device__ static __forceinline__ Frag load(const unsigned char *row, int s, int h, int sw) {
    return *reinterpret_cast<const u32x4 *>(row + (((2 * s + h) ^ sw) << 4));
  }
  __device__ static __forceinline__ f32x16_t run(Frag a, Frag b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
};
template <>
struct Mma<EF16> {
  static constexpr int kInstr = 1;
  typedef u32x4 Frag;
  __device__ static __forceinline__ Frag load(const unsigned char *row, int s, int h, int sw) {
    return *reinterpret_cast<const u32x4 *>(row + (((2 * s + h) ^ sw) << 4));
  }
  __device__ static __forceinline__ f32x16_t run(Frag a, Frag b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  }
};
template <>
struct Mma<EF32> {
  static constexpr int kInstr = 8;
  struct Frag {
    u32x4 lo, hi;
  };
  __device__ static __forceinline__ Frag load(const unsigned char *row, int s, int h, int sw) {
    Frag f;
    f.lo = *reinterpret_cast<const u32x4 *>(row + (((4 * s + 2 * h) ^ sw) << 4));
    f.hi = *reinterpret_cast<const u32x4 *>(row + (((4 * s + 2 * h + 1) ^ sw) << 4));
    return f;
  }
  __device__ static __forceinline__ f32x16_t run(Frag a, Frag b, f32x16_t c) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.lo[e]), __uint_as_float(b.lo[e]), c, 0, 0, 0);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.hi[e]), __uint_as_float(b.hi[e]), c, 0, 0, 0);
    return c;
  }
};

__device__ __forceinline__ void store_out(void *base, int64_t idx, int dt, float v) {
  if (dt == DT_F32) {
    static_cast<float *>(base)[idx] = v;
  } else if (dt == DT_BF16) {
    static_cast<uint16_t *>(base)[idx] = f32_to_bf16(v);
  } else {
    static_cast<uint16_t *>(base)[idx] = f32_to_f16(v);
  }
}

template <int I, int N, class F>
__device__ __forceinline__ void static_for(F &&f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// XOR swizzle of the four 16-byte chunks of a 64-byte LDS row.  Fragment
// reads take one chunk from each of 32 consecutive rows; with this swizzle
// the rows that share a bank window (r, r+2, r+4, r+6 for 32 banks; r, r+4,
// r+8, r+12 for 64 banks) always use four different chunks.
__device__ __forceinline__ int swz(int row) { return ((row >> 1) ^ (row >> 2)) & 3; }

// ---------------------------------------------------------------------------
// NT product with fused epilogues
// ---------------------------------------------------------------------------
// Wave layout per tile edge: 256 -> 8 waves (two per SIMD) in a 4 x 2 grid of
// 64 x 128 wave tiles; 128 -> 4 waves in a 2 x 2 grid of 64 x 64.  Two waves
// per SIMD let one wave's MFMAs run while the other waits on LDS or memory.
// With a K-major B (BK = 1) the 256-edge grid is 2 x 4 (128 x 64 wave tiles):
// each wave then reads two column blocks of B through the 8-byte transpose
// reads instead of four, and four row blocks of A through 16-byte reads
// instead of two, 16 LDS reads per stage instead of 20 for the same bytes.
// That shortens the load phase, which was the longer half of the ping-pong
// for these products (8 x 4096x16384 bf16: the two Q X products 6.92 -> 6.67
// ms per call).
template <int TILE, int BK = 0>
struct WaveLayout {
  static constexpr int WGM = TILE == 256 ? (BK ? 2 : 4) : 2;   // wave rows
  static constexpr int WGN = TILE == 256 ? (BK ? 4 : 2) : 2;   // wave columns
  static constexpr int THREADS = 64 * WGM * WGN;
};

// Split storage (PL = 2): a value v is kept as two bf16 planes, hi = bf16(v)
// and lo = bf16(v - hi), the lo plane `plane` elements after the hi plane.
// Products take the three significant terms hi*hi + hi*lo + lo*hi.
template <class E, int PL>
struct Store {
  using S = typename E::S;
  __device__ static __forceinline__ void put(S *base, int64_t idx, int64_t plane, float v) {
    const S h = E::st(v);
    base[idx] = h;
    if constexpr (PL == 2) base[idx + plane] = E::st(v - E::ld(h));
  }
  // four consecutive entries of a row
  __device__ static __forceinline__ void put4(S *base, int64_t idx, int64_t plane, const float *v) {
    static_assert(sizeof(S) == 2, "16-bit storage only");
    S h[4], l[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      h[q] = E::st(v[q]);
      l[q] = E::st(v[q] - E::ld(h[q]));
    }
    uint2 pk;
    pk.x = static_cast<uint32_t>(h[0]) | (static_cast<uint32_t>(h[1]) << 16);
    pk.y = static_cast<uint32_t>(h[2]) | (static_cast<uint32_t>(h[3]) << 16);
    *reinterpret_cast<uint2 *>(base + idx) = pk;
    if constexpr (PL == 2) {
      pk.x = static_cast<uint32_t>(l[0]) | (static_cast<uint32_t>(l[1]) << 16);
      pk.y = static_cast<uint32_t>(l[2]) | (static_cast<uint32_t>(l[3]) << 16);
      *reinterpret_cast<uint2 *>(base + idx + plane) = pk;
    }
  }
  __device__ static __forceinline__ float get(const S *base, int64_t idx, int64_t plane) {
    float v = E::ld(base[idx]);
    if constexpr (PL == 2) v += E::ld(base[idx + plane]);
    return v;
  }
};

// Upper-triangle tile t (0 <= t < nt (nt + 1) / 2) of an nt x nt tile grid.
// With bb = 0 the order is the column-major triangle: column j holds tiles
// (0..j, j).  With bb > 0 the grid is cut into bb x bb blocks taken
// column-major over the block triangle; a diagonal block is a column-major
// triangle, an off-diagonal block is taken in bands of hh rows, each band
// column by column.  Consecutive tiles then share few row and column panels
// (for nt = 16, bb = 8, hh = 4: at most 14 panels per run of 34 tiles, 10.5 on
// average, against 12.25 for the plain triangle), which is what the XCD runs
// below keep together in one L2.
__device__ __forceinline__ void sym_tile(int t, int nt, int bb, int hh, int *ti, int *tj) {
  int base = 0, J = 0, w = nt;
  if (bb > 0) {
    const int nb = (nt + bb - 1) / bb;
    for (; J < nb - 1; ++J) {
      const int wj = min(bb, nt - J * bb);
      const int cnt = J * bb * wj + wj * (wj + 1) / 2;
      if (t < base + cnt) break;
      base += cnt;
    }
    w = min(bb, nt - J * bb);
    int r = t - base;
    const int off = J * bb * w;            // tiles of the off-diagonal blocks of block column J
    if (r < off) {
      const int I = r / (bb * w);
      r -= I * bb * w;
      const int h = r / (hh * w);
      r -= h * hh * w;
      *ti = I * bb + h * hh + r % hh;
      *tj = J * bb + r / hh;
      return;
    }
    base += off;
  }
  const int r = t - base;                  // column-major triangle of edge w at (J bb, J bb)
  int bj = static_cast<int>((sqrtf(8.0f * static_cast<float>(r) + 1.0f) - 1.0f) * 0.5f);
  while ((bj + 1) * (bj + 2) / 2 <= r) ++bj;
  while (bj * (bj + 1) / 2 > r) --bj;
  *tj = J * bb + bj;
  *ti = J * bb + r - bj * (bj + 1) / 2;
}

// Timeline build (compiled with GNS_TIMELINE; the build script's --timeline
// option makes libgns_timeline.so): every GEMM workgroup records the
// constant 100 MHz clock (s_memrealtime) at entry, when its prologue is done,
// when its main loop is done and when its last store has completed, the
// shader-clock cycles in between (s_memtime), its tile, and the CU and queue
// it ran on.  The work itself is unchanged; in the library build the marks
// compile to nothing.
#ifdef GNS_TIMELINE
constexpr unsigned kTimelineMax = 1u << 18;   // records (64 bytes each)
__device__ unsigned long long g_timeline[kTimelineMax][8];
__device__ unsigned int g_timeline_n;
struct Timeline {
  unsigned long long t0, t1, t2, c0, tile;
  int mode, K;
  __device__ __forceinline__ Timeline(int mode_, int K_) : tile(0), mode(mode_), K(K_) {
    t0 = t1 = t2 = __builtin_amdgcn_s_memrealtime();
    c0 = __builtin_amdgcn_s_memtime();
  }
  __device__ __forceinline__ void prologue_done() { t1 = __builtin_amdgcn_s_memrealtime(); }
  __device__ __forceinline__ void loop_done() { t2 = __builtin_amdgcn_s_memrealtime(); }
  __device__ __forceinline__ void set_tile(int ti, int tj, int mat) {
    tile = static_cast<unsigned long long>(ti) | (static_cast<unsigned long long>(tj) << 16) |
           (static_cast<unsigned long long>(mat) << 32);
  }
  // at every exit of the kernel: every wave's stores have completed
  __device__ __forceinline__ ~Timeline() {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    const unsigned long long t3 = __builtin_amdgcn_s_memrealtime();
    const unsigned long long c3 = __builtin_amdgcn_s_memtime();
    unsigned hw = 0, xcc = 0;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_HW_ID)" : "=s"(hw));
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
    if (threadIdx.x == 0) {
      const unsigned slot = atomicAdd(&g_timeline_n, 1u);
      if (slot < kTimelineMax) {
        unsigned long long *r = g_timeline[slot];
        r[0] = t0; r[1] = t1; r[2] = t2; r[3] = t3;
        r[4] = c3 - c0;
        r[5] = tile;
        r[6] = static_cast<unsigned long long>(static_cast<unsigned>(K)) |
               (static_cast<unsigned long long>(gridDim.x & 0xffffffu) << 32) |
               (static_cast<unsigned long long>(mode) << 56);
        r[7] = static_cast<unsigned long long>(hw) | (static_cast<unsigned long long>(xcc) << 32);
      }
    }
  }
};
#else
struct Timeline {
  __device__ __forceinline__ Timeline(int, int) {}
  __device__ __forceinline__ void prologue_done() {}
  __device__ __forceinline__ void loop_done() {}
  __device__ __forceinline__ void set_tile(int, int, int) {}
};
#endif

// BK = 0: both operands row-major along K (C = A B^T).  BK = 1: B is stored
// K-major, B[k][n] row-major with n contiguous (C = A B), read with the LDS
// transpose load; 256-edge 16-bit tiles, general results only.
// KS: 0 = one pass; K split of a symmetric result: 1 = a part's raw
// accumulators out, 2 = sum of the parts in, then the usual epilogue.
template <class E, int TILE, int MODE, int PL, int BK = 0, int KS = 0>
__global__ void __launch_bounds__((WaveLayout<TILE, BK>::THREADS))
gemm_nt(GemmParams p) {
  Timeline tl(MODE | (BK << 2) | (KS << 3) | ((TILE == 256) << 5), p.K);
  using S = typename E::S;
  using St = Store<E, PL>;
  constexpr int ESZ = sizeof(S);
  constexpr int SB = 64;                  // bytes of one row of one K stage
  constexpr int BKE = SB / ESZ;           // contraction elements per stage
  constexpr int SUB = BKE / 16;           // 16-deep slices per stage (2, or 1 for fp32)
  constexpr int WGM = WaveLayout<TILE, BK>::WGM;
  constexpr int WGN = WaveLayout<TILE, BK>::WGN;
  constexpr int NT = WaveLayout<TILE, BK>::THREADS;
  constexpr int WTM = TILE / WGM;         // wave tile rows
  constexpr int WTN = TILE / WGN;         // wave tile columns
  constexpr int NBI = WTM / 32;           // 32x32 blocks per wave, rows
  constexpr int NBJ = WTN / 32;           // 32x32 blocks per wave, columns
  constexpr int OPB = TILE * SB;          // bytes of one operand plane in one stage
  constexpr int STB = 2 * PL * OPB;       // bytes of one stage: A planes, then B planes
  constexpr int NST = 5;                  // LDS ring depth (stages)
  constexpr int NW = NT / 64;             // waves
  constexpr int BPW = (TILE / 16) / NW;   // 1 KiB LDS blocks per wave per plane per stage
  constexpr int LPS = 2 * PL * BPW;       // DMA instructions per wave per stage
  static_assert(BPW * NW * 16 == TILE, "blocks must cover the tile");
  static_assert(PL == 1 || (ESZ == 2 && NW == 4), "split planes: 16-bit types, 128-edge tiles");
  static_assert(BK == 0 || (TILE == 256 && ESZ == 2 && PL == 1 && NW == 8 && MODE != MODE_SYM),
                "K-major B: 256-edge 16-bit tiles, general results");
  static_assert(NST * STB <= 160 * 1024, "LDS budget");
  static_assert(KS == 0 || (MODE == MODE_SYM && TILE == 256 && ESZ == 2 && PL == 1 && NW == 8),
                "K split: symmetric 256-edge 16-bit tiles");

  __shared__ __attribute__((aligned(16))) unsigned char lds[NST * STB];

  // Workgroup -> tile.  Consecutive tiles share operand panels; the hardware
  // deals workgroups round-robin over the 8 XCDs (one L2 each), so ids are
  // regrouped: the logical tile order is cut into runs of xcd_chunk tiles,
  // run r goes to XCD r % 8, and each XCD works through its runs in order.
  // Long runs keep one matrix per XCD (most L2 reuse); runs of a fraction of
  // a matrix let several XCDs work on the same matrix at once, which keeps
  // the set of matrices in flight small enough for the shared last-level
  // cache (the host uses a quarter matrix per run).
  const int G = gridDim.x;
  const int w = blockIdx.x;
  const int G8 = G & ~7;
  int mat, ti, tj, t;
  // K split (symmetric results): the grid holds k_parts copies of the tile
  // set, part kp contracting over its own slice of K
  const int kparts = KS == 1 ? p.k_parts : 1;
  int kp = 0;
  {
    int lw = w;
    if (w < G8 && p.xcd_chunk > 0) {
      const int c = p.xcd_chunk, slot = w >> 3;
      lw = ((slot / c) * 8 + (w & 7)) * c + slot % c;
      if (lw >= G8) lw = w;   // only when xcd_chunk does not divide G8 / 8 (a host error)
    }
    if (kparts > 1) {
      const int tb = p.tiles_per_mat * p.batch;
      kp = lw / tb;
      lw -= kp * tb;
    }
    mat = lw / p.tiles_per_mat;
    t = lw - mat * p.tiles_per_mat;
    if (MODE == MODE_SYM) {
      sym_tile(t, p.tiles_m, p.sym_block, p.sym_half, &ti, &tj);
    } else {
      // grouped raster: runs of 32 consecutive tiles form 4 x 8 blocks, so
      // the tiles that one XCD runs together touch 4 A panels and 8 B panels
      constexpr int GM = 4;
      const int group = t / (GM * p.tiles_n);
      const int first = group * GM;
      const int gm = (p.tiles_m - first) < GM ? (p.tiles_m - first) : GM;
      const int r = t - group * GM * p.tiles_n;
      ti = first + r % gm;
      tj = r / gm;
    }
  }

  tl.set_tile(ti, tj, mat);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  // A diagonal tile of a symmetric result needs only its upper triangle.
  // With 256-edge tiles and 8 waves, waves 0-3 keep their 64 x 128 tiles
  // (rows 0-127, every column) and waves 4-7 take 64 x 64 tiles of the
  // lower-right quadrant (rows 128-255, columns 128-255); the lower-left
  // quadrant is never computed.  Wave w runs on SIMD w % 4, so every SIMD
  // does 12 of its usual 16 blocks: the tile costs three quarters of a tile.
  constexpr bool kHalfDiag = (MODE == MODE_SYM && TILE == 256 && NW == 8 && PL == 1);
  const bool half = kHalfDiag && ti == tj && wave >= 4;
  const int wr = (wave / WGN) * WTM;
  const int wc = half ? 128 + (wave % 2) * 64 : (wave % WGN) * WTN;

  const int64_t ldaB = p.lda * ESZ;
  const int64_t ldbB = p.ldb * ESZ;

  // Operands move from HBM/L2 straight into LDS with the LDS-DMA form of the
  // buffer load: one instruction fills 1 KiB (16 rows x 64 bytes) of a stage,
  // lane l writing bytes 16 l .. 16 l + 15.  Lane l therefore fetches row
  // l / 4 of its block and the logical chunk that the swizzle places at
  // physical chunk l % 4.  Wave w fills blocks w, w + NW, ... of each plane.
  const int dma_row = lane >> 2;
  const int dma_chunk = (lane & 3) ^ swz(dma_row);
  const int vA = dma_row * static_cast<int>(ldaB) + dma_chunk * 16;
  // K-major B: a stage is 32 K rows of TILE elements (512 bytes each), and
  // one DMA instruction fills two of them (block blk = rows 2 blk, 2 blk + 1).
  // The 16-byte chunks of row r are XOR-swizzled by (r & 3) << 2, so that
  // the transpose reads of four consecutive rows hit four different bank
  // quarters.  A wave's blocks all have the parity of the wave index.
  int vB;
  if constexpr (BK) {
    const int r = 2 * (wave & 1) + (lane >> 5);          // (2 blk + lane / 32) & 3
    vB = (lane >> 5) * static_cast<int>(ldbB) + (((lane & 31) ^ (r << 2)) * 16);
  } else {
    vB = dma_row * static_cast<int>(ldbB) + dma_chunk * 16;
  }
  // buffer descriptors over this tile's A and B panels, one per plane
  // (hardware range check: loads past the panel return zeros; the values are
  // wave-uniform, readfirstlane puts them in SGPRs for the asm)
  auto descriptor = [&](const void *base, int64_t panel_off, int64_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(static_cast<const unsigned char *>(base) + panel_off * ESZ);
    const i32x4 r = {__builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(a))),
                     __builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(a >> 32) & 0xffff)),
                     __builtin_amdgcn_readfirstlane(static_cast<int>(bytes)), 0x00020000};
    return r;
  };
  // K part kp: stages kp * base .. (the last part also takes the remainder)
  const int kbase = (p.K / BKE) / kparts;
  const int64_t kofs = static_cast<int64_t>(kp) * kbase * BKE;
  const int64_t offA = static_cast<int64_t>(mat) * p.sA + static_cast<int64_t>(ti) * TILE * p.lda + kofs;
  // K-major B: the panel is columns tj*TILE .. of all K rows
  const int64_t offB = static_cast<int64_t>(mat) * p.sB +
                       (BK ? static_cast<int64_t>(tj) * TILE : static_cast<int64_t>(tj) * TILE * p.ldb + kofs);
  i32x4 rA[PL], rB[PL];
#pragma unroll
  for (int pl = 0; pl < PL; ++pl) {
    rA[pl] = descriptor(p.A, offA + pl * p.pA, TILE * ldaB);
    rB[pl] = descriptor(p.B, offB + pl * p.pB, BK ? static_cast<int64_t>(p.K) * ldbB : TILE * ldbB);
  }
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int ldaB32 = __builtin_amdgcn_readfirstlane(static_cast<int>(ldaB));
  const int ldbB32 = __builtin_amdgcn_readfirstlane(static_cast<int>(ldbB));
  const uint32_t lds_base =
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) unsigned char *)(lds)));

  // fragment read coordinates: block b of a wave covers rows wr/wc + b*32 + lane%32
  const int lr = lane & 31;
  const int lh = lane >> 5;
  const int fsw = swz(lr);
  // K-major B transpose reads: lane j (of its group of 16) reads K row
  // j / 4 (+ the slice's base) and the 8 bytes of columns n0 + 4 (j % 4) ..
  // + 3, with n0 = 16 (group % 2); chunk index tr_c and byte tr_half within
  // the 16-byte chunk.
  const int tr_rsub = (lane & 15) >> 2;
  const int tr_c = 2 * ((lane >> 4) & 1) + ((lane >> 1) & 1);
  const int tr_half = 8 * (lane & 1);

  // Accumulators start at (beta/alpha) * D so that the epilogue is a plain
  // scale-and-store (except where D comes from the operand stream, see
  // op_d below).  D is read through its transposed copy DT (D itself
  // for symmetric D), where the four rows held by a lane are contiguous.
  // The D loads are issued right after the main loop's first DMA stages, so
  // that those stages do not queue behind the D requests and the two
  // latencies overlap (8 x 4096x16384 bf16, one stream: 20.42 -> 20.27 ms
  // per call; with the 16-byte D loads below 20.09 ms).
  f32x16_t acc[NBI][NBJ];
#pragma unroll
  for (int i = 0; i < NBI; ++i)
#pragma unroll
    for (int j = 0; j < NBJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  // Second pass of a K split: the accumulators start as the sum of the
  // parts' raw accumulators, added in part order (lane-major layout: element
  // ((wave * NBI + ib) * NBJ + jb) * 16 + r of a tile at lane offset).
  if constexpr (KS == 2) {
    const int64_t tile_off = (static_cast<int64_t>(mat) * p.tiles_per_mat + t) * (TILE * TILE);
    const int64_t part_stride = static_cast<int64_t>(p.tiles_per_mat) * p.batch * (TILE * TILE);
#pragma unroll 1
    for (int q = 0; q < p.parts_in; ++q) {
      const float *src = p.part_in + q * part_stride + tile_off + (threadIdx.x >> 6) * (NBI * NBJ * 16 * 64) +
                         (threadIdx.x & 63);
#pragma unroll
      for (int i = 0; i < NBI; ++i)
#pragma unroll
        for (int j = 0; j < NBJ; ++j) {
          // one block at a time (keeps the loads from piling up in registers)
          float v[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) v[r] = __builtin_nontemporal_load(src + ((i * NBJ + j) * 16 + r) * 64);
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[i][j][r] += v[r];
          __builtin_amdgcn_sched_barrier(0);
        }
    }
  }
  using RawD = typename std::conditional<ESZ == 2, uint2, float4>::type;
  RawD draw[PL][NBI][NBJ][4];
  const bool has_d = p.DT != nullptr;
  auto load_d = [&]() {
    const S *DTm = static_cast<const S *>(p.DT) + static_cast<int64_t>(mat) * p.sDT;
    const int64_t i_base = static_cast<int64_t>(ti) * TILE + wr + 4 * lh;
    const int64_t j_base = static_cast<int64_t>(tj) * TILE + wc + lr;
    if constexpr (ESZ == 2 && PL == 1) {
      if (p.d_rows) {
        // D in row layout, D(i,j) = DT[i * lddt + j]: the four rows of a lane
        // are four 2-byte loads (consecutive lanes on consecutive columns)
#pragma unroll
        for (int i = 0; i < NBI; ++i)
#pragma unroll
          for (int j = 0; j < NBJ; ++j) {
            if (half && j >= 2) continue;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const S *src = DTm + (i_base + i * 32 + 8 * g) * p.lddt + j_base + j * 32;
              uint32_t e[4];
#pragma unroll
              for (int q = 0; q < 4; ++q) e[q] = src[q * p.lddt];
              draw[0][i][j][g] = RawD{e[0] | (e[1] << 16), e[2] | (e[3] << 16)};
            }
          }
        return;
      }
    }
    if constexpr (ESZ == 2 && PL == 1) {
      // 16-byte loads: lane (lr, lh) reads the 8 rows of block rows 16u + 8lh
      // .. + 7 of its column (g = 2u + lh, both row halves), then the lane
      // halves swap 8 bytes so that each lane holds its own four rows of
      // g = 2u and g = 2u + 1.  permlane32_swap(x, y) returns x with lanes
      // 32-63 replaced by y's lanes 0-31, and y with lanes 0-31 replaced by
      // x's lanes 32-63 (checked with an in-bounds probe on the GPU).  Half
      // the load instructions of 8-byte gathers, each row's 16 bytes in one
      // request (one stream: 20.42 -> 20.04 ms per call).
      const int64_t i0 = static_cast<int64_t>(ti) * TILE + wr + 8 * lh;
#pragma unroll
      for (int i = 0; i < NBI; ++i)
#pragma unroll
        for (int j = 0; j < NBJ; ++j) {
          if (half && j >= 2) continue;
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const S *src = DTm + (j_base + j * 32) * p.lddt + i0 + i * 32 + 16 * u;
            const u32x4 v = *reinterpret_cast<const u32x4 *>(src);
            const auto s0 = __builtin_amdgcn_permlane32_swap(v[0], v[2], false, false);
            const auto s1 = __builtin_amdgcn_permlane32_swap(v[1], v[3], false, false);
            draw[0][i][j][2 * u] = RawD{s0[0], s1[0]};
            draw[0][i][j][2 * u + 1] = RawD{s0[1], s1[1]};
          }
        }
      return;
    }
#pragma unroll
    for (int i = 0; i < NBI; ++i)
#pragma unroll
      for (int j = 0; j < NBJ; ++j) {
        if (half && j >= 2) continue;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const S *src = DTm + (j_base + j * 32) * p.lddt + i_base + i * 32 + 8 * g;
#pragma unroll
          for (int pl = 0; pl < PL; ++pl) draw[pl][i][j][g] = *reinterpret_cast<const RawD *>(src + pl * p.pDT);
        }
      }
  };
  // d1 = false: the D term itself comes from the operand stream (below) and
  // only a second term is loaded here
  auto init_from_d = [&](bool d1) {
#pragma unroll
    for (int i = 0; i < NBI; ++i)
#pragma unroll
      for (int j = 0; j < NBJ; ++j) {
        if (!d1 || (half && j >= 2)) continue;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          float v[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int pl = 0; pl < PL; ++pl) {
            const RawD u = draw[pl][i][j][g];
            if constexpr (ESZ == 2) {
              v[0] += E::ld(static_cast<S>(u.x & 0xffffu));
              v[1] += E::ld(static_cast<S>(u.x >> 16));
              v[2] += E::ld(static_cast<S>(u.y & 0xffffu));
              v[3] += E::ld(static_cast<S>(u.y >> 16));
            } else {
              v[0] = u.x; v[1] = u.y; v[2] = u.z; v[3] = u.w;
            }
          }
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[i][j][4 * g + q] = p.init_scale * v[q];
        }
      }
    if (p.DT2) {
      // second term (only the Q update that follows an identity Q has one):
      // loaded and added here
      const S *D2m = static_cast<const S *>(p.DT2) + static_cast<int64_t>(mat) * p.sDT;
      const int64_t i_base = static_cast<int64_t>(ti) * TILE + wr + 4 * lh;
      const int64_t j_base = static_cast<int64_t>(tj) * TILE + wc + lr;
#pragma unroll
      for (int i = 0; i < NBI; ++i)
#pragma unroll
        for (int j = 0; j < NBJ; ++j) {
          if (half && j >= 2) continue;
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const S *src = D2m + (j_base + j * 32) * p.lddt + i_base + i * 32 + 8 * g;
#pragma unroll
            for (int pl = 0; pl < PL; ++pl) {
              const RawD u = *reinterpret_cast<const RawD *>(src + pl * p.pDT2);
              float v[4];
              if constexpr (ESZ == 2) {
                v[0] = E::ld(static_cast<S>(u.x & 0xffffu));
                v[1] = E::ld(static_cast<S>(u.x >> 16));
                v[2] = E::ld(static_cast<S>(u.y & 0xffffu));
                v[3] = E::ld(static_cast<S>(u.y >> 16));
              } else {
                v[0] = u.x; v[1] = u.y; v[2] = u.z; v[3] = u.w;
              }
#pragma unroll
              for (int q = 0; q < 4; ++q) acc[i][j][4 * g + q] += p.init_scale2 * v[q];
            }
          }
        }
    }
  };

  // Main loop over K stages of 64 bytes per row in an NST-deep LDS ring.
  // The loads bypass the compiler's wait bookkeeping (inline assembly), so
  // the waits are explicit counts of this wave's outstanding loads.
  // (wave-uniform: the loop index feeds the scalar operands of the DMA)
  // (the summing pass has no contraction: no main loop is compiled for it)
  const int nk = KS == 2   ? 0
                 : KS == 0 ? p.K / BKE
                           : __builtin_amdgcn_readfirstlane(kp < kparts - 1 ? kbase : p.K / BKE - kbase * (kparts - 1));
  // beta * D from the operand stream.  When D is the B operand of a
  // symmetric product (D = B: the same exactly symmetric iterate), the lane's
  // D entries D(e + q, j), e = wr + 32 ib + 8 g + 4 lh, j = wc + 32 jb + lr,
  // equal B(tj TILE + j, ti TILE + e + q): 8 contiguous bytes of row j of the
  // B panel in the stage holding K = ti TILE + wr + 32 ib.  That stage passes
  // through LDS anyway, so the wave adds them to its accumulators there (two
  // stages per wave, one per row block ib): D costs no memory traffic and no
  // wait before the first stage.  The D loads of the prologue took 12.8 of a
  // tile's 118 us on 8 x 4096x16384 bf16; n x n products with short K gain
  // most (64 x 2048x7168: 20.10 -> 19.80 ms per call).  The stage index is
  // made wave-uniform (readfirstlane): taken as divergent, the tests on it
  // turned the K loop into an exec-masked loop with its indices on the VALU.
  // (both the 8-wave 256-edge and the 4-wave 128-edge symmetric kernels)
  constexpr bool kOpD = (ESZ == 2 && PL == 1 && BK == 0 && KS == 0 && MODE == MODE_SYM &&
                         ((TILE == 256 && NW == 8) || (TILE == 128 && NW == 4)));
  const bool op_d = kOpD && has_d && p.DT == p.B && p.lddt == p.ldb && p.sDT == p.sB && !p.d_rows &&
                    nk >= (ti + 1) * (TILE / BKE);
  const int ds0 = __builtin_amdgcn_readfirstlane((ti * TILE + wr) / BKE);   // this wave's first D stage
  if (nk > 0) {
    using Frag = typename Mma<E>::Frag;
    // The loop issues NST - 1 stages past the last one, so that every stage
    // waits on the same count of loads.  Those go through descriptors with an
    // empty range: out-of-range loads complete without fetching anything, and
    // the ring slots they fill are never read.
    i32x4 rAz[PL], rBz[PL];
#pragma unroll
    for (int pl = 0; pl < PL; ++pl) {
      rAz[pl] = rA[pl];
      rAz[pl][2] = 0;
      rBz[pl] = rB[pl];
      rBz[pl][2] = 0;
    }
    auto dma_stage = [&](int stage) {
      const uint32_t buf_lds = lds_base + static_cast<uint32_t>((stage % NST) * STB);
      const bool live = stage < nk;
      const int st = live ? stage : nk - 1;
#pragma unroll
      for (int q = 0; q < BPW; ++q) {
        const int blk = wave_u + q * NW;
        const int soA = blk * 16 * ldaB32 + st * SB;
        const int soB = BK ? (32 * st + 2 * blk) * ldbB32 : blk * 16 * ldbB32 + st * SB;
#pragma unroll
        for (int pl = 0; pl < PL; ++pl) {
          asm volatile(
              "s_mov_b32 m0, %0\n\t"
              "buffer_load_dwordx4 %1, %2, %3 offen lds"
              :: "s"(buf_lds + pl * OPB + blk * 1024), "v"(vA), "s"(live ? rA[pl] : rAz[pl]), "s"(soA)
              : "memory", "m0");
          asm volatile(
              "s_mov_b32 m0, %0\n\t"
              "buffer_load_dwordx4 %1, %2, %3 offen lds"
              :: "s"(buf_lds + (PL + pl) * OPB + blk * 1024), "v"(vB), "s"(live ? rB[pl] : rBz[pl]), "s"(soB)
              : "memory", "m0");
        }
      }
    };
    Frag fa[2][PL][NBI], fb[2][PL][NBJ];
    // NJ: column blocks this wave computes (NBJ, or 2 for a half wave of a
    // diagonal tile)
    auto fload = [&](int slot, int buf, int sub, auto nj) {
      constexpr int NJ = decltype(nj)::value;
      const unsigned char *la = lds + buf * STB;
#pragma unroll
      for (int pl = 0; pl < PL; ++pl) {
#pragma unroll
        for (int b = 0; b < NBI; ++b)
          fa[slot][pl][b] = Mma<E>::load(la + pl * OPB + (wr + b * 32 + lr) * SB, sub, lh, fsw);
        if constexpr (BK) {
          // Transpose reads: in every group of 16 lanes, lane 4a + b receives
          // element b of the 8-byte pieces addressed by lanes a, 4 + a, 8 + a
          // and 12 + a.  Lane j of a group addresses K row kb + j / 4 and
          // columns n0 + 4 (j % 4) .. + 3, so lane i ends with column n0 + i
          // at rows kb .. kb + 3; two reads give the 8 K values of the
          // fragment in the same order as the A fragment.
          const unsigned char *lb = la + (PL + pl) * OPB;
#pragma unroll
          for (int b = 0; b < NJ; ++b) {
            typedef short v4s __attribute__((ext_vector_type(4)));
            typedef __attribute__((address_space(3))) v4s lv4s;
            uint2 h2[2];
#pragma unroll
            for (int q = 0; q < 2; ++q) {
              const int row = 16 * sub + 8 * lh + 4 * q + tr_rsub;
              const int chunk = ((wc >> 3) + 4 * b + tr_c) ^ (tr_rsub << 2);
              const unsigned char *addr = lb + row * 512 + chunk * 16 + tr_half;
              const v4s t = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                  (lv4s *)((__attribute__((address_space(3))) unsigned char *)(addr)));
              h2[q] = __builtin_bit_cast(uint2, t);
            }
            fb[slot][pl][b] = u32x4{h2[0].x, h2[0].y, h2[1].x, h2[1].y};
          }
        } else {
#pragma unroll
          for (int b = 0; b < NJ; ++b)
            fb[slot][pl][b] = Mma<E>::load(la + (PL + pl) * OPB + (wc + b * 32 + lr) * SB, sub, lh, fsw);
        }
      }
    };
    auto mma = [&](int slot, auto nj) {
      constexpr int NJ = decltype(nj)::value;
#pragma unroll
      for (int ii = 0; ii < NBI; ++ii)
#pragma unroll
        for (int jj = 0; jj < NJ; ++jj) {
          if constexpr (PL == 2) {
            // small terms first
            acc[ii][jj] = Mma<E>::run(fa[slot][1][ii], fb[slot][0][jj], acc[ii][jj]);
            acc[ii][jj] = Mma<E>::run(fa[slot][0][ii], fb[slot][1][jj], acc[ii][jj]);
          }
          acc[ii][jj] = Mma<E>::run(fa[slot][0][ii], fb[slot][0][jj], acc[ii][jj]);
        }
    };

    // D entries of row block IB from the B plane of the stage in buffer buf
    // (chunk g of a row holds K elements 8 g .. 8 g + 7, swizzled like the
    // fragments)
    auto add_d = [&](int buf, auto ibc, auto nj) {
      constexpr int IB = decltype(ibc)::value;
      constexpr int NJ = decltype(nj)::value;
      const unsigned char *lb = lds + buf * STB + OPB;
#pragma unroll
      for (int jb = 0; jb < NJ; ++jb) {
        const unsigned char *rowp = lb + (wc + jb * 32 + lr) * SB + 8 * lh;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const uint2 v = *reinterpret_cast<const uint2 *>(rowp + ((g ^ fsw) << 4));
          acc[IB][jb][4 * g + 0] += p.init_scale * E::ld(static_cast<S>(v.x & 0xffffu));
          acc[IB][jb][4 * g + 1] += p.init_scale * E::ld(static_cast<S>(v.x >> 16));
          acc[IB][jb][4 * g + 2] += p.init_scale * E::ld(static_cast<S>(v.y & 0xffffu));
          acc[IB][jb][4 * g + 3] += p.init_scale * E::ld(static_cast<S>(v.y >> 16));
        }
      }
    };
    if constexpr (NW == 8) {
      // Ping-pong over the two waves of every SIMD.  Every wave runs the same
      // stream per stage i -- L(i): read its fragments of stage i, then issue
      // its DMA share of stage i+NST-1 (reads first, so that a DMA issue
      // stalled by a busy memory path does not delay them); barrier; C(i):
      // the MFMAs of stage i; barrier -- but waves 4-7 start one barrier
      // later than waves 0-3.
      // At every barrier the two waves of a SIMD are therefore in opposite
      // phases: one multiplies while the other reads, and the matrix core
      // never drains at a barrier.  Stage i+NST-1 goes into the buffer of
      // stage i-1, which both groups finished reading one barrier earlier;
      // at the end of L(i) each wave waits for its share of stage i+1, which
      // the other group reads one barrier later at the earliest.
      const bool g1 = wave_u >= 4;
      constexpr int kWait = LPS * (NST - 2);   // this wave's loads of stages i+2 .. i+NST-1
      static_assert(kWait < 64, "wait count out of range");
#pragma unroll
      for (int j = 0; j < NST - 1; ++j) dma_stage(j);
      if (has_d && !op_d) { load_d(); init_from_d(true); }
      else if (op_d && p.DT2) init_from_d(false);
      asm volatile("s_waitcnt vmcnt(%0)" :: "n"(kWait) : "memory");
      __syncthreads();
      if (g1) __syncthreads();
      tl.prologue_done();
      // the same barrier sequence in both versions of the loop: the half
      // waves of a diagonal tile run the one that skips column blocks 2, 3
      auto loop = [&](auto nj) {
        int buf = 0;                        // buffer of stage i
        auto stage_body = [&](int i, auto dk) {
          static_for<0, SUB>([&](auto sc) { fload(decltype(sc)::value, buf, decltype(sc)::value, nj); });
          dma_stage(i + NST - 1);           // into the buffer of stage i-1
          if constexpr (decltype(dk)::value >= 0) add_d(buf, dk, nj);
          asm volatile("s_waitcnt vmcnt(%0)" :: "n"(kWait) : "memory");
          __syncthreads();
          __builtin_amdgcn_s_setprio(1);
          static_for<0, SUB>([&](auto sc) { mma(decltype(sc)::value, nj); });
          __builtin_amdgcn_s_setprio(0);
          __syncthreads();
          buf = buf == NST - 1 ? 0 : buf + 1;
        };
        // the two stages that carry this wave's D rows run outside the main
        // loop, so that the loop itself keeps the code of a product without D
        const int lo = op_d ? ds0 : nk;
        int i = 0;
        for (; i < lo; ++i) stage_body(i, std::integral_constant<int, -1>{});
        if (op_d) {
          stage_body(i++, std::integral_constant<int, 0>{});
          stage_body(i++, std::integral_constant<int, 1>{});
        }
        for (; i < nk; ++i) stage_body(i, std::integral_constant<int, -1>{});
      };
      if constexpr (kHalfDiag) {
        if (half) loop(std::integral_constant<int, 2>{});
        else loop(std::integral_constant<int, NBJ>{});
      } else {
        loop(std::integral_constant<int, NBJ>{});
      }
      if (!g1) __syncthreads();
    } else {
      // Iteration i multiplies stage i; its last slice already reads the
      // first fragments of stage i+1, so at the start of every iteration
      // stages i and i+1 are complete and NST-3 later stages are in flight.
      // After the barrier that closes iteration i, the buffer of stage i is
      // refilled with stage i+NST, which gives each load NST-2 iterations to
      // arrive.  Before that barrier every wave waits until its share of
      // stage i+2 has landed.
      // prologue: all NST stages in flight; wait for stages 0 and 1
#pragma unroll
      for (int j = 0; j < NST; ++j) dma_stage(j);
      if (has_d && !op_d) { load_d(); init_from_d(true); }
      else if (op_d && p.DT2) init_from_d(false);
      static_assert(LPS * (NST - 2) < 64, "wait count out of range");
      asm volatile("s_waitcnt vmcnt(%0)" :: "n"(LPS * (NST - 2)) : "memory");
      __syncthreads();
      tl.prologue_done();
      fload(0, 0, 0, std::integral_constant<int, NBJ>{});

      int buf = 0;                            // buffer of stage i
      auto stage_body = [&](int i, auto dk) {
        const int bnext = buf == NST - 1 ? 0 : buf + 1;
        static_for<0, SUB>([&](auto sc) {
          constexpr int s = decltype(sc)::value;
          constexpr int cur = s & 1;
          if constexpr (s + 1 < SUB) {
            fload(cur ^ 1, buf, s + 1, std::integral_constant<int, NBJ>{});
          } else {
            fload(cur ^ 1, bnext, 0, std::integral_constant<int, NBJ>{});
          }
          __builtin_amdgcn_sched_barrier(0);
          mma(cur, std::integral_constant<int, NBJ>{});
          __builtin_amdgcn_sched_barrier(0);
        });
        if constexpr ((SUB & 1) == 1) {
#pragma unroll
          for (int pl = 0; pl < PL; ++pl) {
#pragma unroll
            for (int b = 0; b < NBI; ++b) fa[0][pl][b] = fa[1][pl][b];
#pragma unroll
            for (int b = 0; b < NBJ; ++b) fb[0][pl][b] = fb[1][pl][b];
          }
        }
        // this wave's D rows of row block dk from stage i (still in its buffer)
        if constexpr (decltype(dk)::value >= 0) add_d(buf, dk, std::integral_constant<int, NBJ>{});
        // stage i+2 must be complete before the barrier; stages i+3 .. i+NST-1
        // may still be in flight
        asm volatile("s_waitcnt vmcnt(%0)" :: "n"(LPS * (NST - 3)) : "memory");
        __syncthreads();
        dma_stage(i + NST);
        buf = bnext;
      };
      // as in the 8-wave loop, the two stages that carry this wave's D rows
      // run outside the main loop
      const int lo = op_d ? ds0 : nk;
      int i = 0;
      for (; i < lo; ++i) stage_body(i, std::integral_constant<int, -1>{});
      if constexpr (kOpD) {
        if (op_d) {
          stage_body(i++, std::integral_constant<int, 0>{});
          stage_body(i++, std::integral_constant<int, 1>{});
        }
      }
      for (; i < nk; ++i) stage_body(i, std::integral_constant<int, -1>{});
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    tl.loop_done();
  } else if (has_d) {
    load_d();
    init_from_d(true);
  }
  // First pass of a K split: this part's raw accumulators go to part_out
  // (the second pass sums the parts and runs the epilogue).
  if constexpr (KS == 1) {
    const int64_t tb = static_cast<int64_t>(p.tiles_per_mat) * p.batch;
    float *dst = p.part_out + ((kp * tb + static_cast<int64_t>(mat) * p.tiles_per_mat + t) * (TILE * TILE)) +
                 (threadIdx.x >> 6) * (NBI * NBJ * 16 * 64) + (threadIdx.x & 63);
#pragma unroll
    for (int i = 0; i < NBI; ++i)
#pragma unroll
      for (int j = 0; j < NBJ; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) __builtin_nontemporal_store(acc[i][j][r], dst + ((i * NBJ + j) * 16 + r) * 64);
    return;
  }

  // ---------------------------------------------------------------- epilogue
  // 32x32 accumulator layout: lane l, register r holds row
  // 8*(r/4) + 4*(l/32) + r%4 and column l%32 of its block.
  const int64_t row_base = static_cast<int64_t>(ti) * TILE + wr;
  const int64_t col_base = static_cast<int64_t>(tj) * TILE + wc;
  const float alpha = p.alpha_vec ? p.alpha * p.alpha_vec[mat] : p.alpha;

  // Outputs of unsplit 16-bit tiles go through LDS: the accumulator layout
  // gives each lane scattered 2-byte elements (direct layout) or 8-byte
  // pieces of 32 different rows (transposed layout), so the tile is first
  // written into LDS (rows of TILE + 8 elements, either layout) and the whole
  // workgroup then stores it as full rows, 16 bytes per lane.  Both layouts
  // of every output are stored this way.
  constexpr bool kStage = ((TILE == 256 || TILE == 128) && PL == 1 && ESZ == 2);
  constexpr int TP = TILE + 8;                         // staged row pitch (elements)
  static_assert(!kStage || TILE * TP * 2 <= NST * STB, "staging tile fits the ring");
  S *const Ts = reinterpret_cast<S *>(lds);
  // The staged paths round every accumulator once into packed pairs:
  // pk[ib][jb][2 g + h] holds rows 8 g + 4 lh + 2 h and + 1 (low half first)
  // of column lr in block (ib, jb).  The fp32 accumulators then die, which
  // keeps the epilogue within the register budget of two waves per SIMD.
  // A diagonal symmetric tile also keeps, per row block ib, the unrounded
  // diagonal entry this lane holds (dv[ib]; see fix_diag).
  uint32_t pk[NBI][NBJ][8];
  float dv[NBI];
  // tag: the 16-bit type to round to (the compute type, or the caller's
  // output type for the final product)
  auto pack = [&](bool keep_diag, auto tag) {
    using T = typename decltype(tag)::type;
    const int dreg = 4 * (lr >> 3) + (lr & 3);
#pragma unroll
    for (int ib = 0; ib < NBI; ++ib) {
      dv[ib] = 0.0f;
#pragma unroll
      for (int jb = 0; jb < NBJ; ++jb) {
        if (half && jb >= 2) continue;
        if (keep_diag && wr + 32 * ib == wc + 32 * jb) {
          float v = acc[ib][jb][0];
#pragma unroll
          for (int r = 1; r < 16; ++r) v = r == dreg ? acc[ib][jb][r] : v;
          dv[ib] = alpha * v;
        }
#pragma unroll
        for (int h = 0; h < 8; ++h) pk[ib][jb][h] = T::st2(alpha * acc[ib][jb][2 * h], alpha * acc[ib][jb][2 * h + 1]);
      }
    }
  };
  // Ts[c][r] = tile(r, c)
  auto stage_transposed = [&]() {
    __syncthreads();   // the ring (or the previous staged tile) is no longer read
#pragma unroll
    for (int ib = 0; ib < NBI; ++ib)
#pragma unroll
      for (int jb = 0; jb < NBJ; ++jb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int c = wc + jb * 32 + lr;
          const int r0 = wr + ib * 32 + 8 * g + 4 * lh;
          uint2 v;
          v.x = pk[ib][jb][2 * g];
          v.y = pk[ib][jb][2 * g + 1];
          *reinterpret_cast<uint2 *>(Ts + c * TP + r0) = v;
        }
    __syncthreads();
  };
  // Ts[r][c] = tile(r, c)
  auto stage_direct = [&]() {
    __syncthreads();
    S *const base = Ts + (wr + 4 * lh) * TP + wc + lr;
#pragma unroll
    for (int ib = 0; ib < NBI; ++ib)
#pragma unroll
      for (int jb = 0; jb < NBJ; ++jb) {
        if (half && jb >= 2) continue;
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            base[(ib * 32 + 8 * g + q) * TP + jb * 32] =
                static_cast<S>(pk[ib][jb][2 * g + q / 2] >> (16 * (q & 1)));
      }
    __syncthreads();
  };
  // Diagonal tile: entry (r, r) of the staged direct tile becomes
  // alpha * acc + diag, rounded once (rows r < n_real only).  In a 32 x 32
  // block that lies on the diagonal, lane (lr, lh) holds entry (lr, lr) when
  // bit 2 of lr equals lh (in register 4 (lr / 8) + lr % 4, kept as dv).
  auto fix_diag = [&](float diag) {
    __syncthreads();
    if (((lr >> 2) & 1) == lh) {
#pragma unroll
      for (int ib = 0; ib < NBI; ++ib) {
        const int rc = wr + 32 * ib + lr;
        if (rc >= wc && rc < wc + (half ? 64 : WTN) && static_cast<int64_t>(ti) * TILE + rc < p.n_real)
          Ts[rc * TP + rc] = E::st(dv[ib] + diag);
      }
    }
    __syncthreads();
  };
  // staged row k -> row (row0 + k) of dst, columns col0 .. col0 + TILE - 1;
  // with `upper`, element (k, c) with k > c is taken from (c, k) instead
  // (the stored form of a diagonal symmetric tile)
  auto store_staged = [&](S *dst, int64_t ld, int64_t row0, int64_t col0, bool upper) {
    constexpr int CPR = TILE / 8;                      // 16-byte pieces per row
#pragma unroll 4
    for (int k = tid; k < TILE * CPR; k += NT) {
      const int rr = k / CPR;
      const int cc = (k % CPR) * 8;
      u32x4 v;
      if (!upper || cc >= rr) {
        v = *reinterpret_cast<const u32x4 *>(Ts + rr * TP + cc);
      } else {
        S e[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int c = cc + q;
          e[q] = c >= rr ? Ts[rr * TP + c] : Ts[c * TP + rr];
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = static_cast<uint32_t>(e[2 * q]) | (static_cast<uint32_t>(e[2 * q + 1]) << 16);
      }
      // streaming (non-temporal) store: the output is not read again by this
      // launch, so it should not displace operand panels from the L2
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(dst + (row0 + rr) * ld + col0 + cc));
    }
  };
  const int64_t tr0 = static_cast<int64_t>(ti) * TILE, tc0 = static_cast<int64_t>(tj) * TILE;

  if (MODE == MODE_SYM) {
    S *Cm = static_cast<S *>(p.C) + static_cast<int64_t>(mat) * p.sC;
    S *C2m = p.C2 ? static_cast<S *>(p.C2) + static_cast<int64_t>(mat) * p.sC2 : nullptr;
    const bool diag_tile = (ti == tj);
    if constexpr (kStage) {
      pack(diag_tile, Tag<E>{});
      if (!diag_tile) {
        // C and its mirror; C2 equals C off the diagonal
        stage_direct();
        store_staged(Cm, p.ldc, tr0, tc0, false);
        if (C2m) store_staged(C2m, p.ldc, tr0, tc0, false);
        stage_transposed();
        store_staged(Cm, p.ldc, tc0, tr0, false);
        if (C2m) store_staged(C2m, p.ldc, tc0, tr0, false);
      } else {
        // diagonal tile: the upper-triangle value of every pair, written to
        // both places, each entry exactly once
        stage_direct();
        if (p.diag1 != 0.0f) fix_diag(p.diag1);
        store_staged(Cm, p.ldc, tr0, tc0, true);
        if (C2m) {
          if (p.diag2 != p.diag1) fix_diag(p.diag2);
          store_staged(C2m, p.ldc, tr0, tc0, true);
        }
      }
      return;
    }
#pragma unroll
    for (int ib = 0; ib < NBI; ++ib)
#pragma unroll
      for (int jb = 0; jb < NBJ; ++jb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int64_t i0 = row_base + ib * 32 + 8 * g + 4 * lh;
          const int64_t j = col_base + jb * 32 + lr;
          float v[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) v[q] = alpha * acc[ib][jb][4 * g + q];
          if (!diag_tile) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              St::put(Cm, (i0 + q) * p.ldc + j, p.pC, v[q]);
              if (C2m) St::put(C2m, (i0 + q) * p.ldc + j, p.pC2, v[q]);
            }
            // mirrored copy: four consecutive entries of row j
            if constexpr (ESZ == 2) {
              St::put4(Cm, j * p.ldc + i0, p.pC, v);
              if (C2m) St::put4(C2m, j * p.ldc + i0, p.pC2, v);
            } else {
              float4 pk = make_float4(v[0], v[1], v[2], v[3]);
              *reinterpret_cast<float4 *>(Cm + j * p.ldc + i0) = pk;
              if (C2m) *reinterpret_cast<float4 *>(C2m + j * p.ldc + i0) = pk;
            }
          } else {
            // Diagonal tile: keep the upper-triangle value of each pair and
            // write it to both places, each entry exactly once.
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int64_t i = i0 + q;
              if (i > j) continue;
              const float dg = (i == j && i < p.n_real) ? 1.0f : 0.0f;
              const float v1 = v[q] + dg * p.diag1;
              St::put(Cm, i * p.ldc + j, p.pC, v1);
              if (i != j) St::put(Cm, j * p.ldc + i, p.pC, v1);
              if (C2m) {
                const float v2 = v[q] + dg * p.diag2;
                St::put(C2m, i * p.ldc + j, p.pC2, v2);
                if (i != j) St::put(C2m, j * p.ldc + i, p.pC2, v2);
              }
            }
          }
        }
  } else if (MODE == MODE_GEN) {
    S *Cm = static_cast<S *>(p.C) + static_cast<int64_t>(mat) * p.sC;
    S *CTm = p.CT ? static_cast<S *>(p.CT) + static_cast<int64_t>(mat) * p.sCT : nullptr;
    if constexpr (kStage) {
      pack(false, Tag<E>{});
      stage_direct();
      store_staged(Cm, p.ldc, tr0, tc0, false);
      if (CTm) {
        stage_transposed();
        store_staged(CTm, p.ldct, tc0, tr0, false);
      }
      return;
    }
#pragma unroll
    for (int ib = 0; ib < NBI; ++ib)
#pragma unroll
      for (int jb = 0; jb < NBJ; ++jb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int64_t i0 = row_base + ib * 32 + 8 * g + 4 * lh;
          const int64_t j = col_base + jb * 32 + lr;
          float v[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            v[q] = alpha * acc[ib][jb][4 * g + q];
            St::put(Cm, (i0 + q) * p.ldc + j, p.pC, v[q]);
          }
          if (CTm) {
            if constexpr (ESZ == 2) {
              St::put4(CTm, j * p.ldct + i0, p.pCT, v);
            } else {
              *reinterpret_cast<float4 *>(CTm + j * p.ldct + i0) = make_float4(v[0], v[1], v[2], v[3]);
            }
          }
        }
  } else {  // MODE_FINAL
    const int64_t *ridx = p.row_idx ? p.row_idx + static_cast<int64_t>(mat) * p.rows_eff : nullptr;
    const int64_t obase = static_cast<int64_t>(mat) * p.out_rows * p.out_cols;
    const bool plain = !ridx && p.out_dtype == E::code;
    if constexpr (kStage) {
      // 16-bit output with 16-byte aligned rows: rounded once to the output
      // type, staged, and written as row pieces, each row to its destination
      // row (through row_idx if given); rows past rows_eff and pieces past
      // out_cols (a multiple of 8) are padding and skipped
      // (fp16 products also round to a bf16 output here; bf16 products with
      // an fp16 output take the element path below, as a second rounding
      // there would make the bf16 kernels spill)
      constexpr bool kToBf16 = std::is_same<E, EF16>::value;
      if ((p.out_dtype == E::code || (kToBf16 && p.out_dtype == DT_BF16)) && (p.out_cols & 7) == 0 &&
          (reinterpret_cast<uintptr_t>(p.out) & 15) == 0) {
        constexpr int CPR = TILE / 8;                      // 16-byte pieces per row
        constexpr int NPC = TILE * CPR / NT;               // pieces per thread
        static_assert(TILE * CPR % NT == 0, "whole pieces per thread");
        // the destination rows of this thread's pieces, loaded before the
        // tile is rounded and staged so that their latency overlaps that work
        // (-1: not a row of the output)
        int64_t dest[NPC];
#pragma unroll
        for (int j = 0; j < NPC; ++j) {
          const int64_t i = tr0 + (tid + j * NT) / CPR;
          dest[j] = i < p.rows_eff ? (ridx ? ridx[i] : i) : -1;
        }
        if constexpr (kToBf16) {
          if (p.out_dtype == DT_BF16) pack(false, Tag<EBF16>{});
          else pack(false, Tag<E>{});
        } else {
          pack(false, Tag<E>{});
        }
        stage_direct();
        S *O = static_cast<S *>(p.out) + obase;
#pragma unroll
        for (int j = 0; j < NPC; ++j) {
          const int k = tid + j * NT;
          const int rr = k / CPR;
          const int cc = (k % CPR) * 8;
          const int64_t row = dest[j];
          if (row < 0 || row >= p.out_rows || tc0 + cc >= p.out_cols) continue;
          const u32x4 v = *reinterpret_cast<const u32x4 *>(Ts + rr * TP + cc);
          __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(O + row * p.out_cols + tc0 + cc));
        }
        return;
      }
      // fp32 output (not rounded to the compute type): the same, in two
      // halves of 128 rows (waves 0-3 hold rows 0-127, waves 4-7 rows
      // 128-255), each staged as fp32 with a 260-float row pitch.  bf16
      // products only: with fp16 the path makes the kernel spill.
      if (std::is_same<E, EBF16>::value && p.out_dtype == DT_F32 && (p.out_cols & 3) == 0 &&
          (reinterpret_cast<uintptr_t>(p.out) & 15) == 0) {
        constexpr int HR = TILE / 2;                       // rows per half
        constexpr int TPF = TILE + 4;                      // fp32 row pitch
        static_assert(HR * TPF * 4 <= NST * STB, "fp32 half tile fits the ring");
        float *const Tf = reinterpret_cast<float *>(lds);
        float *O = static_cast<float *>(p.out) + obase;
        constexpr int CPR = TILE / 4;                      // 16-byte pieces per row
        for (int h = 0; h < 2; ++h) {
          __syncthreads();                                 // ring / previous half no longer read
          if ((wr >= HR) == (h == 1)) {
            float *const tw = Tf + (wr - HR * h + 4 * lh) * TPF + wc + lr;
#pragma unroll
            for (int ib = 0; ib < NBI; ++ib)
#pragma unroll
              for (int jb = 0; jb < NBJ; ++jb)
#pragma unroll
                for (int g = 0; g < 4; ++g)
#pragma unroll
                  for (int q = 0; q < 4; ++q)
                    tw[(ib * 32 + 8 * g + q) * TPF + jb * 32] = alpha * acc[ib][jb][4 * g + q];
          }
          __syncthreads();
#pragma unroll 4
          for (int k = tid; k < HR * CPR; k += NT) {
            const int rr = k / CPR;
            const int cc = (k % CPR) * 4;
            const int64_t i = tr0 + HR * h + rr;
            if (i >= p.rows_eff || tc0 + cc >= p.out_cols) continue;
            const int64_t row = ridx ? ridx[i] : i;
            if (row < 0 || row >= p.out_rows) continue;
            const float4 v = *reinterpret_cast<const float4 *>(Tf + rr * TPF + cc);
            st_once(reinterpret_cast<float4 *>(O + row * p.out_cols + tc0 + cc), v);
          }
        }
        return;
      }
    }
    if (plain && row_base + WTM <= p.rows_eff && col_base + WTN <= p.out_cols) {
      // the whole wave tile lies inside the caller's matrix and needs no
      // conversion: plain stores, consecutive lanes on consecutive columns
      S *O = static_cast<S *>(p.out) + obase;
#pragma unroll
      for (int ib = 0; ib < NBI; ++ib)
#pragma unroll
        for (int jb = 0; jb < NBJ; ++jb)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int64_t i0 = row_base + ib * 32 + 8 * g + 4 * lh;
            const int64_t j = col_base + jb * 32 + lr;
#pragma unroll
            for (int q = 0; q < 4; ++q) O[(i0 + q) * p.out_cols + j] = E::st(alpha * acc[ib][jb][4 * g + q]);
          }
      return;
    }
#pragma unroll
    for (int ib = 0; ib < NBI; ++ib)
#pragma unroll
      for (int jb = 0; jb < NBJ; ++jb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int64_t i0 = row_base + ib * 32 + 8 * g + 4 * lh;
          const int64_t j = col_base + jb * 32 + lr;
          if (j >= p.out_cols) continue;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int64_t i = i0 + q;
            if (i >= p.rows_eff) continue;
            const float v = alpha * acc[ib][jb][4 * g + q];
            const int64_t row = ridx ? ridx[i] : i;
            if (row < 0 || row >= p.out_rows) continue;
            store_out(p.out, obase + row * p.out_cols + j, p.out_dtype, v);
          }
        }
  }
}

// ---------------------------------------------------------------------------
// Frobenius norm, stage 1: per-workgroup partial sums of squares
// ---------------------------------------------------------------------------
template <class TIn>
__global__ void __launch_bounds__(256)
norm_partial(const void *X, int64_t n, int64_t m, int64_t rows_eff, const int64_t *row_idx,
             int parts, double *partials) {
  using S = typename TIn::S;
  const int b = blockIdx.y;
  const int part = blockIdx.x;
  const int64_t rpp = (rows_eff + parts - 1) / parts;
  const int64_t r0 = part * rpp;
  const int64_t r1 = (r0 + rpp < rows_eff) ? r0 + rpp : rows_eff;
  const S *Xb = static_cast<const S *>(X) + static_cast<int64_t>(b) * n * m;
  constexpr int VE = 16 / sizeof(S);  // elements per 16-byte vector
  const bool vec = ((m * static_cast<int64_t>(sizeof(S))) % 16 == 0) &&
                   ((reinterpret_cast<uintptr_t>(X) & 15) == 0);
  double dacc = 0.0;
  for (int64_t r = r0; r < r1; ++r) {
    const int64_t row = row_idx ? row_idx[static_cast<int64_t>(b) * rows_eff + r] : r;
    if (row < 0 || row >= n) continue;
    const S *xr = Xb + row * m;
    float s = 0.0f;
    if (vec) {
      const uint4 *xv = reinterpret_cast<const uint4 *>(xr);
      const int64_t nv = m / VE;
      for (int64_t v = threadIdx.x; v < nv; v += blockDim.x) {
        const uint4 u = xv[v];
        const S *e = reinterpret_cast<const S *>(&u);
#pragma unroll
        for (int q = 0; q < VE; ++q) {
          const float f = TIn::ld(e[q]);
          s += f * f;
        }
      }
    } else {
      for (int64_t c = threadIdx.x; c < m; c += blockDim.x) {
        const float f = TIn::ld(xr[c]);
        s += f * f;
      }
    }
    dacc += static_cast<double>(s);
  }
  // fixed-order reduction: wave tree, then the four waves in order
  for (int off = 32; off > 0; off >>= 1) dacc += __shfl_down(dacc, off, 64);
  __shared__ double wsum[4];
  if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = dacc;
  __syncthreads();
  if (threadIdx.x == 0)
    partials[static_cast<int64_t>(b) * parts + part] = ((wsum[0] + wsum[1]) + wsum[2]) + wsum[3];
}

// ---------------------------------------------------------------------------
// X_hat = X / (||X||_F + eps), rounded to the compute dtype, in both layouts
// ---------------------------------------------------------------------------
// PL = 2 (split storage) also writes the lo planes X - hi, plane_h and
// plane_t elements after the hi planes.
template <class TIn, class TCmp, int PL>
__global__ void __launch_bounds__(256)
scale_transpose(const void *X, int64_t n, int64_t m, int64_t rows_eff, const int64_t *row_idx,
                const double *partials, int parts, double eps, void *Xh, void *XT, int64_t Np,
                int64_t Mp, int64_t plane_h, int64_t plane_t) {
  using SI = typename TIn::S;
  using SC = typename TCmp::S;
  const int b = blockIdx.z;
  const int64_t c0 = static_cast<int64_t>(blockIdx.x) * 64;
  const int64_t r0 = static_cast<int64_t>(blockIdx.y) * 64;
  __shared__ float inv_s;
  __shared__ SC tileT[PL][64][65];

  if (threadIdx.x < 64) {  // norm stage 2, same fixed order in every workgroup
    double s = 0.0;
    for (int i = threadIdx.x; i < parts; i += 64) s += partials[static_cast<int64_t>(b) * parts + i];
    for (int off = 32; off > 0; off >>= 1) s += __shfl_down(s, off, 64);
    if (threadIdx.x == 0) inv_s = static_cast<float>(1.0 / (sqrt(s) + eps));
  }
  __syncthreads();
  const float inv = inv_s;

  const SI *Xb = static_cast<const SI *>(X) + static_cast<int64_t>(b) * n * m;
  SC *Xhb = static_cast<SC *>(Xh) + static_cast<int64_t>(b) * Np * Mp;
  SC *XTb = static_cast<SC *>(XT) + static_cast<int64_t>(b) * Mp * Np;
  const int col = threadIdx.x & 63;
  const int rg = threadIdx.x >> 6;
#pragma unroll 4
  for (int rr = 0; rr < 16; ++rr) {
    const int r = rg + 4 * rr;
    const int64_t gr = r0 + r;
    const int64_t gc = c0 + col;
    float v = 0.0f;
    if (gr < rows_eff && gc < m) {
      const int64_t row = row_idx ? row_idx[static_cast<int64_t>(b) * rows_eff + gr] : gr;
      if (row >= 0 && row < n) v = TIn::ld(Xb[row * m + gc]) * inv;
    }
    const SC sv = TCmp::st(v);
    Xhb[gr * Mp + gc] = sv;
    if (XT) tileT[0][col][r] = sv;
    if constexpr (PL == 2) {
      const SC sl = TCmp::st(v - TCmp::ld(sv));
      Xhb[plane_h + gr * Mp + gc] = sl;
      if (XT) tileT[PL - 1][col][r] = sl;
    }
  }
  if (!XT) return;   // row layout only
  __syncthreads();
#pragma unroll 4
  for (int rr = 0; rr < 16; ++rr) {
    const int c = rg + 4 * rr;
#pragma unroll
    for (int pl = 0; pl < PL; ++pl) XTb[pl * plane_t + (c0 + c) * Np + r0 + col] = tileT[pl][c][col];
  }
}

// Same operation for fp32 input, a 16-bit compute type and the row layout
// only (no transposed copy), with m a multiple of 4 and X 16-byte aligned:
// one wave per row of X_hat (gathered through row_idx), 16-byte loads and
// 8-byte stores, zeros in the padding up to Np x Mp.  The same norm and the
// same rounding as above.
template <class TCmp>
__global__ void __launch_bounds__(256)
scale_rows_f32(const float *X, int64_t n, int64_t m, int64_t rows_eff, const int64_t *row_idx,
               const double *partials, int parts, double eps, void *Xh, int64_t Np, int64_t Mp) {
  using SC = typename TCmp::S;
  const int b = blockIdx.y;
  __shared__ float inv_s;
  if (threadIdx.x < 64) {  // norm stage 2, same fixed order in every workgroup
    double s = 0.0;
    for (int i = threadIdx.x; i < parts; i += 64) s += partials[static_cast<int64_t>(b) * parts + i];
    for (int off = 32; off > 0; off >>= 1) s += __shfl_down(s, off, 64);
    if (threadIdx.x == 0) inv_s = static_cast<float>(1.0 / (sqrt(s) + eps));
  }
  __syncthreads();
  const float inv = inv_s;
  const int lane = threadIdx.x & 63;
  const int64_t r = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (r >= Np) return;
  SC *dst = static_cast<SC *>(Xh) + (static_cast<int64_t>(b) * Np + r) * Mp;
  const float *src = nullptr;
  if (r < rows_eff) {
    const int64_t row = row_idx ? row_idx[static_cast<int64_t>(b) * rows_eff + r] : r;
    if (row >= 0 && row < n) src = X + (static_cast<int64_t>(b) * n + row) * m;
  }
  const int64_t m4 = src ? m / 4 : 0;
  for (int64_t v = lane; v < Mp / 4; v += 64) {
    float4 x = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    if (v < m4) x = ld_once(reinterpret_cast<const float4 *>(src) + v);
    const uint32_t lo = static_cast<uint32_t>(TCmp::st(x.x * inv)) | (static_cast<uint32_t>(TCmp::st(x.y * inv)) << 16);
    const uint32_t hi = static_cast<uint32_t>(TCmp::st(x.z * inv)) | (static_cast<uint32_t>(TCmp::st(x.w * inv)) << 16);
    reinterpret_cast<uint2 *>(dst)[v] = make_uint2(lo, hi);
  }
}

// Same operation for 16-bit input and compute types with m a multiple of 8:
// 16-byte loads and stores on every global access (rows of X and X_hat, and
// 8-row runs of each X^T row), transposed through a padded LDS tile.
template <class TIn, class TCmp, int PL>
__global__ void __launch_bounds__(256)
scale_transpose16(const void *X, int64_t n, int64_t m, int64_t rows_eff, const int64_t *row_idx,
                  const double *partials, int parts, double eps, void *Xh, void *XT, int64_t Np,
                  int64_t Mp, int64_t plane_h, int64_t plane_t) {
  static_assert(sizeof(typename TIn::S) == 2 && sizeof(typename TCmp::S) == 2, "16-bit types only");
  const int b = blockIdx.z;
  const int64_t c0 = static_cast<int64_t>(blockIdx.x) * 64;
  const int64_t r0 = static_cast<int64_t>(blockIdx.y) * 64;
  __shared__ float inv_s;
  __shared__ __attribute__((aligned(16))) uint16_t tile[PL][64][72];   // 144-byte rows

  if (threadIdx.x < 64) {  // norm stage 2, same fixed order in every workgroup
    double sum = 0.0;
    for (int i = threadIdx.x; i < parts; i += 64) sum += partials[static_cast<int64_t>(b) * parts + i];
    for (int off = 32; off > 0; off >>= 1) sum += __shfl_down(sum, off, 64);
    if (threadIdx.x == 0) inv_s = static_cast<float>(1.0 / (sqrt(sum) + eps));
  }
  __syncthreads();
  const float inv = inv_s;

  const uint16_t *Xb = static_cast<const uint16_t *>(X) + static_cast<int64_t>(b) * n * m;
  uint16_t *Xhb = static_cast<uint16_t *>(Xh) + static_cast<int64_t>(b) * Np * Mp;
  uint16_t *XTb = static_cast<uint16_t *>(XT) + static_cast<int64_t>(b) * Mp * Np;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int v = threadIdx.x + 256 * h;
    const int row = v >> 3;
    const int cv = (v & 7) * 8;
    const int64_t gr = r0 + row;
    const int64_t gc = c0 + cv;
    u32x4 in = {0u, 0u, 0u, 0u};
    if (gr < rows_eff && gc < m) {
      const int64_t src = row_idx ? row_idx[static_cast<int64_t>(b) * rows_eff + gr] : gr;
      if (src >= 0 && src < n) in = *reinterpret_cast<const u32x4 *>(Xb + src * m + gc);
    }
    // each 32-bit word holds two consecutive elements (even one in the low half)
    u32x4 o[PL];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float f0 = TIn::ld(static_cast<uint16_t>(in[q] & 0xffffu)) * inv;
      const float f1 = TIn::ld(static_cast<uint16_t>(in[q] >> 16)) * inv;
      const uint16_t h0 = TCmp::st(f0), h1 = TCmp::st(f1);
      o[0][q] = static_cast<uint32_t>(h0) | (static_cast<uint32_t>(h1) << 16);
      if constexpr (PL == 2)
        o[PL - 1][q] = static_cast<uint32_t>(TCmp::st(f0 - TCmp::ld(h0))) |
                       (static_cast<uint32_t>(TCmp::st(f1 - TCmp::ld(h1))) << 16);
    }
#pragma unroll
    for (int pl = 0; pl < PL; ++pl) {
      *reinterpret_cast<u32x4 *>(Xhb + pl * plane_h + gr * Mp + gc) = o[pl];
      if (XT) *reinterpret_cast<u32x4 *>(&tile[pl][row][cv]) = o[pl];
    }
  }
  if (!XT) return;   // row layout only
  __syncthreads();
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int c = threadIdx.x & 63;
    const int k = (threadIdx.x >> 6) + 4 * h;
#pragma unroll
    for (int pl = 0; pl < PL; ++pl) {
      u32x4 o;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        o[q] = static_cast<uint32_t>(tile[pl][8 * k + 2 * q][c]) |
               (static_cast<uint32_t>(tile[pl][8 * k + 2 * q + 1][c]) << 16);
      *reinterpret_cast<u32x4 *>(XTb + pl * plane_t + (c0 + c) * Np + r0 + 8 * k) = o;
    }
  }
}

// ---------------------------------------------------------------------------
// row subset check
// ---------------------------------------------------------------------------
__global__ void check_rows_init(int32_t *result) { *result = 0; }

__global__ void __launch_bounds__(256)
check_rows(const int64_t *row_idx, int64_t k, int64_t n, int32_t *result) {
  __shared__ uint32_t seen[65536 / 32];
  const int64_t words = (n + 31) / 32;
  for (int64_t i = threadIdx.x; i < words; i += blockDim.x) seen[i] = 0u;
  __syncthreads();
  const int64_t *ri = row_idx + static_cast<int64_t>(blockIdx.x) * k;
  int bad = 0;
  for (int64_t i = threadIdx.x; i < k; i += blockDim.x) {
    const int64_t r = ri[i];
    if (r < 0 || r >= n) {
      bad = bad > 1 ? bad : 1;
      continue;
    }
    const uint32_t bit = 1u << (r & 31);
    const uint32_t old = atomicOr(&seen[r >> 5], bit);
    if (old & bit) bad = 2;
  }
  if (bad) atomicMax(result, bad);
}

// ---------------------------------------------------------------------------
// finite check of an output: *result = 1 if any checked element is Inf or NaN
// (plain stores of the same value from every lane that sees one; the host
// cleared *result first).  One wave per row, rows taken through row_idx when
// given (indices outside [0, rows) are skipped).
// ---------------------------------------------------------------------------
template <class E>
__global__ void __launch_bounds__(256)
check_finite(const void *A, int64_t rows, int64_t cols, const int64_t *row_idx, int64_t k,
             int32_t *result) {
  using S = typename E::S;
  const int64_t b = blockIdx.y;
  const int64_t sel = row_idx ? k : rows;
  const int lane = threadIdx.x & 63;
  bool bad = false;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6); i < sel;
       i += static_cast<int64_t>(gridDim.x) * 4) {
    const int64_t r = row_idx ? row_idx[b * k + i] : i;
    if (r < 0 || r >= rows) continue;
    const S *row = static_cast<const S *>(A) + (b * rows + r) * cols;
    for (int64_t j = lane; j < cols; j += 64) {
      // Inf or NaN: every exponent bit set (binary32 bits 30..23, bfloat16
      // bits 14..7, binary16 bits 14..10)
      if constexpr (E::code == DT_F32) bad |= (__float_as_uint(row[j]) & 0x7f800000u) == 0x7f800000u;
      else if constexpr (E::code == DT_BF16) bad |= (row[j] & 0x7f80u) == 0x7f80u;
      else bad |= (row[j] & 0x7c00u) == 0x7c00u;
    }
  }
  if (bad) *result = 1;
}

// ---------------------------------------------------------------------------
// Input path without a normalised copy (16-bit input in the compute type,
// whole tiles): the products read X itself and take 1/(||X||_F + eps) as a
// per-matrix factor in their epilogues, so only X^T is materialised.
// ---------------------------------------------------------------------------
// One 128x128 tile per workgroup: X^T tile through a padded LDS tile (16-byte
// loads and stores, all eight loads of a thread in flight together), and the
// tile's sum of squares (fp32 per thread over 64 elements, then a fixed-order
// fp64 combination).  The n x m matrix is either X_b itself (n_src = n) or,
// with row_idx, rows row_idx[b][0..n) of the n_src x m matrix X_b (a row
// outside X_b reads as zeros).
template <class T, bool GATHER>
__global__ void __launch_bounds__(256)
transpose_sumsq(const void *__restrict__ X, int64_t n, int64_t m, void *__restrict__ XT,
                void *__restrict__ Xcopy, double *partials, const int64_t *__restrict__ row_idx,
                int64_t n_src) {
  constexpr int TT = 128;                 // tile edge
  constexpr int PR = TT / 8;              // 16-byte pieces per tile row
  constexpr int NP = TT * PR / 256;       // pieces per thread
  const int b = blockIdx.z;
  const int64_t c0 = static_cast<int64_t>(blockIdx.x) * TT;
  const int64_t r0 = static_cast<int64_t>(blockIdx.y) * TT;
  __shared__ __attribute__((aligned(16))) uint16_t tile[TT][TT + 8];
  __shared__ double wsum[4];
  const uint16_t *Xb = static_cast<const uint16_t *>(X) + static_cast<int64_t>(b) * n_src * m;
  const int64_t *rib = GATHER ? row_idx + static_cast<int64_t>(b) * n : nullptr;
  uint16_t *XTb = static_cast<uint16_t *>(XT) + static_cast<int64_t>(b) * m * n;
  u32x4 in[NP];
#pragma unroll
  for (int h = 0; h < NP; ++h) {
    const int v = threadIdx.x + 256 * h;
    const int64_t r = r0 + v / PR;
    if constexpr (!GATHER) {
      in[h] = *reinterpret_cast<const u32x4 *>(Xb + r * m + c0 + (v % PR) * 8);
    } else {
      // a row index outside X_b reads as zeros: row 0 is loaded instead and
      // the value dropped, which keeps every load unconditional
      const int64_t src = rib[r];
      const bool ok = src >= 0 && src < n_src;
      const u32x4 x = *reinterpret_cast<const u32x4 *>(Xb + (ok ? src : 0) * m + c0 + (v % PR) * 8);
      in[h] = ok ? x : u32x4{0u, 0u, 0u, 0u};
    }
  }
  // optional row-major copy of the n x m matrix (read by later products in
  // place of the caller's X: a row subset, or X when it is also the output)
  if (Xcopy) {
    uint16_t *Xc = static_cast<uint16_t *>(Xcopy) + static_cast<int64_t>(b) * n * m;
#pragma unroll
    for (int h = 0; h < NP; ++h) {
      const int v = threadIdx.x + 256 * h;
      *reinterpret_cast<u32x4 *>(Xc + (r0 + v / PR) * m + c0 + (v % PR) * 8) = in[h];
    }
  }
  float sq = 0.0f;
#pragma unroll
  for (int h = 0; h < NP; ++h) {
    const int v = threadIdx.x + 256 * h;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float f0 = T::ld(static_cast<uint16_t>(in[h][q] & 0xffffu));
      const float f1 = T::ld(static_cast<uint16_t>(in[h][q] >> 16));
      sq += f0 * f0 + f1 * f1;
    }
    if (XT) *reinterpret_cast<u32x4 *>(&tile[v / PR][(v % PR) * 8]) = in[h];
  }
  double d = static_cast<double>(sq);
  for (int off = 32; off > 0; off >>= 1) d += __shfl_down(d, off, 64);
  if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = d;
  __syncthreads();
  if (threadIdx.x == 0) {
    const int64_t tile_id = static_cast<int64_t>(blockIdx.y) * gridDim.x + blockIdx.x;
    partials[static_cast<int64_t>(b) * gridDim.x * gridDim.y + tile_id] = ((wsum[0] + wsum[1]) + wsum[2]) + wsum[3];
  }
  if (!XT) return;   // sums of squares only
  // X^T row c0 + c takes the 8-row run 8 k .. 8 k + 7 of tile column c
#pragma unroll
  for (int h = 0; h < NP; ++h) {
    const int v = threadIdx.x + 256 * h;
    const int c = v % TT;
    const int k = v / TT;
    u32x4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      o[q] = static_cast<uint32_t>(tile[8 * k + 2 * q][c]) | (static_cast<uint32_t>(tile[8 * k + 2 * q + 1][c]) << 16);
    *reinterpret_cast<u32x4 *>(XTb + (c0 + c) * n + r0 + 8 * k) = o;
  }
}

// One workgroup per matrix: fixed-order sum of the partials, then the
// scale factors of the normalisation X / (||X||_F + eps).
__global__ void __launch_bounds__(256)
norm_finish(const double *partials, int64_t parts, double eps, float *inv, float *inv2) {
  const int b = blockIdx.x;
  __shared__ double wsum[4];
  double s = 0.0;
  for (int64_t i = threadIdx.x; i < parts; i += 256) s += partials[static_cast<int64_t>(b) * parts + i];
  for (int off = 32; off > 0; off >>= 1) s += __shfl_down(s, off, 64);
  if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    const double r = 1.0 / (sqrt(((wsum[0] + wsum[1]) + wsum[2]) + wsum[3]) + eps);
    inv[b] = static_cast<float>(r);
    inv2[b] = static_cast<float>(r * r);
  }
}

// ---------------------------------------------------------------------------
// Row selection of the Dion3 update ("Dion3: Full-Stack Orthogonal Updates",
// §6, Algorithm 4, selection step): the k rows of largest l1 norm
// ---------------------------------------------------------------------------
// Key of every row: sum_j |M_ij| in fp64, one wave per row, each lane over a
// fixed set of 16-byte pieces, then a fixed-order wave tree.  For 16-bit
// inputs whose values in a row span less than 2^31 in magnitude the sum is
// exact, so the keys do not depend on the summation order.
template <class TIn>
__global__ void __launch_bounds__(256)
row_l1(const void *M, int64_t n, int64_t m, double *keys) {
  using S = typename TIn::S;
  constexpr int VE = 16 / sizeof(S);
  const int b = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= n) return;
  const S *r = static_cast<const S *>(M) + (static_cast<int64_t>(b) * n + row) * m;
  double acc = 0.0;
  if ((m % VE) == 0 && (reinterpret_cast<uintptr_t>(M) & 15) == 0) {
    const uint4 *rv = reinterpret_cast<const uint4 *>(r);
    for (int64_t v = lane; v < m / VE; v += 64) {
      const uint4 u = rv[v];
      const S *e = reinterpret_cast<const S *>(&u);
#pragma unroll
      for (int q = 0; q < VE; ++q) acc += fabs(static_cast<double>(TIn::ld(e[q])));
    }
  } else {
    for (int64_t c = lane; c < m; c += 64) acc += fabs(static_cast<double>(TIn::ld(r[c])));
  }
  for (int off = 32; off > 0; off >>= 1) acc += __shfl_down(acc, off, 64);
  if (lane == 0) keys[static_cast<int64_t>(b) * n + row] = acc;
}

// Exclusive prefix sum over the 1024 threads of a workgroup (16 waves);
// *total receives the sum over all threads.
__device__ __forceinline__ int block_scan_excl(int v, int *total, int *wsum) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int w = 0; w < 16; ++w) {
      const int t = wsum[w];
      wsum[w] = run;
      run += t;
    }
    wsum[16] = run;
  }
  __syncthreads();
  const int r = wsum[wave] + x - v;
  *total = wsum[16];
  __syncthreads();
  return r;
}

// One workgroup per matrix.  The keys are non-negative doubles, so their bit
// patterns order like the values: an MSB-first radix select (8 bits per
// pass) finds the k-th largest key tau and how many keys equal to tau still
// belong to the top k; a pass over the rows in index order then takes every
// key above tau and the first of the keys equal to tau, writing the indices
// in ascending order (equal keys: the smaller index wins).
__global__ void __launch_bounds__(1024)
select_topk(const double *keys, int64_t n, int64_t k, int64_t *out) {
  const int b = blockIdx.x;
  const uint64_t *K = reinterpret_cast<const uint64_t *>(keys) + static_cast<int64_t>(b) * n;
  __shared__ uint32_t hist[256];
  __shared__ uint64_t s_prefix;
  __shared__ int64_t s_need;
  __shared__ int wsum[17];
  uint64_t prefix = 0, mask = 0;
  int64_t need = k;
  for (int pass = 0; pass < 8; ++pass) {
    const int shift = 56 - 8 * pass;
    if (threadIdx.x < 256) hist[threadIdx.x] = 0u;
    __syncthreads();
    for (int64_t i = threadIdx.x; i < n; i += 1024) {
      const uint64_t u = K[i];
      if ((u & mask) == prefix) atomicAdd(&hist[(u >> shift) & 255u], 1u);
    }
    __syncthreads();
    // the digit d of the k-th largest key: the keys in buckets above d
    // number fewer than `need`, and with bucket d at least `need` (an
    // exclusive scan over the buckets from 255 down gives every thread its
    // bucket's count above; the one thread whose bucket qualifies writes;
    // bucket 0 takes the rest)
    {
      const int d = 255 - static_cast<int>(threadIdx.x);
      const int h = threadIdx.x < 256 ? static_cast<int>(hist[d]) : 0;
      int total = 0;
      const int64_t above = block_scan_excl(h, &total, wsum);
      if (threadIdx.x < 256 && (d == 0 || above + h >= need) && above < need) {
        s_prefix = prefix | (static_cast<uint64_t>(d) << shift);
        s_need = need - above;
      }
    }
    __syncthreads();
    prefix = s_prefix;
    need = s_need;
    mask |= static_cast<uint64_t>(255) << shift;
  }
  const uint64_t tau = prefix;
  int64_t base = 0, eq_before = 0;
  int64_t *o = out + static_cast<int64_t>(b) * k;
  for (int64_t c0 = 0; c0 < n; c0 += 1024) {
    const int64_t i = c0 + threadIdx.x;
    const uint64_t u = i < n ? K[i] : 0;
    const int gt = (i < n && u > tau) ? 1 : 0;
    const int eq = (i < n && u == tau) ? 1 : 0;
    int eq_total = 0, take_total = 0;
    const int eq_rank = block_scan_excl(eq, &eq_total, wsum);
    const int take = (gt || (eq && eq_before + eq_rank < need)) ? 1 : 0;
    const int pos = block_scan_excl(take, &take_total, wsum);
    if (take && base + pos < k) o[base + pos] = i;
    base += take_total;
    eq_before += eq_total;
  }
}

// ---------------------------------------------------------------------------
// Dion3 update around the orthogonalisation ("Dion3: Full-Stack Orthogonal
// Updates", §6, Algorithm 4, with the optional NorMuon steps of §2.1, eq. (2))
// ---------------------------------------------------------------------------
// The momentum takes the gradient, M <- M + G (one fp32 addition per
// element, stored), and every row of the sum gets its l1 key sum_j |M_ij|
// and, when sumsq is given, its sum of squares sum_j M_ij^2 (both fp64;
// lane-strided 16-byte pieces, then the wave tree: a fixed order for a given
// shape).  One wave per row.
template <class TG>
__global__ void __launch_bounds__(256)
momentum_l1(float *M, const void *G, int64_t n, int64_t m, bool vec, double *keys, double *sumsq) {
  using SG = typename TG::S;
  const int b = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= n) return;
  const int64_t base = (static_cast<int64_t>(b) * n + row) * m;
  float *mr = M + base;
  const SG *gr = static_cast<const SG *>(G) + base;
  double acc = 0.0, sq = 0.0;
  if (vec) {
    // four elements per piece: 16 bytes of M, 16 (fp32) or 8 (16-bit) of G
    auto load = [&](int64_t v, float4 &mv, float *g) {
      mv = ld_once(reinterpret_cast<const float4 *>(mr) + v);
      if constexpr (sizeof(SG) == 4) {
        const float4 gv = ld_once(reinterpret_cast<const float4 *>(gr) + v);
        g[0] = gv.x; g[1] = gv.y; g[2] = gv.z; g[3] = gv.w;
      } else {
        const uint2 gv = ld_once(reinterpret_cast<const uint2 *>(gr) + v);
        g[0] = TG::ld(static_cast<SG>(gv.x & 0xffffu));
        g[1] = TG::ld(static_cast<SG>(gv.x >> 16));
        g[2] = TG::ld(static_cast<SG>(gv.y & 0xffffu));
        g[3] = TG::ld(static_cast<SG>(gv.y >> 16));
      }
    };
    auto finish = [&](int64_t v, float4 mv, const float *g) {
      mv.x += g[0];
      mv.y += g[1];
      mv.z += g[2];
      mv.w += g[3];
      st_once(reinterpret_cast<float4 *>(mr) + v, mv);
      acc += fabs(static_cast<double>(mv.x));
      acc += fabs(static_cast<double>(mv.y));
      acc += fabs(static_cast<double>(mv.z));
      acc += fabs(static_cast<double>(mv.w));
      sq += static_cast<double>(mv.x) * mv.x;
      sq += static_cast<double>(mv.y) * mv.y;
      sq += static_cast<double>(mv.z) * mv.z;
      sq += static_cast<double>(mv.w) * mv.w;
    };
    // kUnroll pieces per lane in flight: all their loads are issued before
    // the first store (the lane's pieces are summed in the same order)
    const int64_t nv = m / 4;
    int64_t v = lane;
    for (; v + 64 * (kUnroll - 1) < nv; v += 64 * kUnroll) {
      float4 mv[kUnroll];
      float g[kUnroll][4];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) load(v + 64 * u, mv[u], g[u]);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) finish(v + 64 * u, mv[u], g[u]);
    }
    for (; v < nv; v += 64) {
      float4 mv;
      float g[4];
      load(v, mv, g);
      finish(v, mv, g);
    }
  } else {
    for (int64_t c = lane; c < m; c += 64) {
      const float s = mr[c] + TG::ld(gr[c]);
      mr[c] = s;
      acc += fabs(static_cast<double>(s));
      sq += static_cast<double>(s) * s;
    }
  }
  for (int off = 32; off > 0; off >>= 1) {
    acc += __shfl_down(acc, off, 64);
    sq += __shfl_down(sq, off, 64);
  }
  if (lane == 0) {
    keys[static_cast<int64_t>(b) * n + row] = acc;
    if (sumsq) sumsq[static_cast<int64_t>(b) * n + row] = sq;
  }
}

// Norm partials of a row subset from known per-row sums of squares:
// partial p of matrix b adds rowsq[b][row_idx[b][r]] over the rows r in
// [p rpp, min((p + 1) rpp, k)), rpp = ceil(k / parts), in order (an index
// outside [0, n) adds nothing).  The scaled copy then sums the partials
// exactly as it sums those of a pass over the rows themselves.
__global__ void __launch_bounds__(256)
row_partials(const double *rowsq, const int64_t *row_idx, int64_t n, int64_t k, int parts,
             double *partials) {
  const int b = blockIdx.y;
  const int p = blockIdx.x * 256 + threadIdx.x;
  if (p >= parts) return;
  const int64_t rpp = (k + parts - 1) / parts;
  const int64_t r0 = p * rpp;
  const int64_t r1 = r0 + rpp < k ? r0 + rpp : k;
  const int64_t *ri = row_idx + static_cast<int64_t>(b) * k;
  const double *rs = rowsq + static_cast<int64_t>(b) * n;
  double acc = 0.0;
  for (int64_t r = r0; r < r1; ++r) {
    const int64_t row = ri[r];
    if (row >= 0 && row < n) acc += rs[row];
  }
  partials[static_cast<int64_t>(b) * parts + p] = acc;
}

// Sum of squares of every row of the k x m update O (fp32 values, fp64
// sums in a fixed order), one wave per row: the row means of O^2 that the
// NorMuon second moment takes, and the squared Frobenius norm of O.
__global__ void __launch_bounds__(256)
row_sumsq(const float *O, int64_t k, int64_t m, bool vec, double *rowsq) {
  const int b = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= k) return;
  const float *orow = O + (static_cast<int64_t>(b) * k + row) * m;
  double acc = 0.0;
  if (vec) {
    auto add = [&](const float4 &o) {
      acc += static_cast<double>(o.x) * o.x;
      acc += static_cast<double>(o.y) * o.y;
      acc += static_cast<double>(o.z) * o.z;
      acc += static_cast<double>(o.w) * o.w;
    };
    // kUnroll pieces per lane in flight, summed in the same order
    const int64_t nv = m / 4;
    int64_t v = lane;
    for (; v + 64 * (kUnroll - 1) < nv; v += 64 * kUnroll) {
      float4 o[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) o[u] = ld_once(reinterpret_cast<const float4 *>(orow) + v + 64 * u);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) add(o[u]);
    }
    for (; v < nv; v += 64) add(ld_once(reinterpret_cast<const float4 *>(orow) + v));
  } else {
    for (int64_t c = lane; c < m; c += 64) acc += static_cast<double>(orow[c]) * orow[c];
  }
  for (int off = 32; off > 0; off >>= 1) acc += __shfl_down(acc, off, 64);
  if (lane == 0) rowsq[static_cast<int64_t>(b) * k + row] = acc;
}

// Row factors of the update, one workgroup per matrix.  With NorMuon, for
// every selected row i (index S_i):
//   v_i <- beta2 v_i + (1 - beta2) mean_j O_ij^2      (stored, fp32 buffer)
//   s_i = 1 / (sqrt(v_i) + eps)
// and O_hat = diag(s) O is brought back to the Frobenius norm of O, so the
// factor of row i is g s_i with g = ||O||_F / ||O_hat||_F (g = 0 when O_hat
// is zero).  Without NorMuon every factor is 1.  fp64 throughout, with
// fixed-order reductions.
__global__ void __launch_bounds__(256)
normuon_factors(const double *rowsq, float *v, const int64_t *S, int64_t n, int64_t k, int64_t m,
                double beta2, double eps, int normuon, double *factor) {
  const int b = blockIdx.x;
  const double *rs = rowsq + static_cast<int64_t>(b) * k;
  const int64_t *Sb = S + static_cast<int64_t>(b) * k;
  double *f = factor + static_cast<int64_t>(b) * k;
  if (!normuon) {
    for (int64_t i = threadIdx.x; i < k; i += blockDim.x) f[i] = 1.0;
    return;
  }
  float *vb = v + static_cast<int64_t>(b) * n;
  double a = 0.0, h = 0.0;   // ||O||^2 and ||O_hat||^2, this thread's share
  for (int64_t i = threadIdx.x; i < k; i += blockDim.x) {
    const int64_t row = Sb[i];
    const double sq = rs[i];
    const double vi = beta2 * static_cast<double>(vb[row]) + (1.0 - beta2) * (sq / static_cast<double>(m));
    vb[row] = static_cast<float>(vi);
    const double s = 1.0 / (sqrt(vi) + eps);
    f[i] = s;
    a += sq;
    h += sq * s * s;
  }
  for (int off = 32; off > 0; off >>= 1) {
    a += __shfl_down(a, off, 64);
    h += __shfl_down(h, off, 64);
  }
  __shared__ double wa[4], wh[4];
  __shared__ double g_s;
  if ((threadIdx.x & 63) == 0) {
    wa[threadIdx.x >> 6] = a;
    wh[threadIdx.x >> 6] = h;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const double A = ((wa[0] + wa[1]) + wa[2]) + wa[3];
    const double H = ((wh[0] + wh[1]) + wh[2]) + wh[3];
    g_s = H > 0.0 ? sqrt(A / H) : 0.0;
  }
  __syncthreads();
  const double g = g_s;
  for (int64_t i = threadIdx.x; i < k; i += blockDim.x) f[i] *= g;
}

// Weight and momentum update, one workgroup per row of W:
//   W <- (1 - lr wd) W                on every row (skipped when wd = 0),
//   W[S_i] <- W[S_i] - lr f_i O_i     on the selected rows,
//   M[S_i] <- mu M[S_i]               (error feedback, selected rows only).
// The slot i of a row in the ascending index list S comes from a binary
// search.  fp32 arithmetic on the caller's fp32 buffers.
__global__ void __launch_bounds__(256)
dion3_update(float *W, float *M, const float *O, const int64_t *S, const double *factor, int64_t n,
             int64_t m, int64_t k, float decay, double lr, float mu, bool vec) {
  const int b = blockIdx.y;
  const int64_t row = blockIdx.x;
  const int64_t *Sb = S + static_cast<int64_t>(b) * k;
  int64_t lo = 0, hi = k;
  while (lo < hi) {
    const int64_t mid = (lo + hi) >> 1;
    if (Sb[mid] < row) lo = mid + 1;
    else hi = mid;
  }
  const int64_t slot = (lo < k && Sb[lo] == row) ? lo : -1;
  if (slot < 0 && decay == 1.0f) return;
  float *wr = W + (static_cast<int64_t>(b) * n + row) * m;
  const int64_t nv = m / 4;
  const int64_t step = blockDim.x;
  if (slot < 0) {
    if (vec) {
      auto scale = [&](int64_t v, float4 w) {
        w.x *= decay; w.y *= decay; w.z *= decay; w.w *= decay;
        st_once(reinterpret_cast<float4 *>(wr) + v, w);
      };
      // kUnroll pieces per thread in flight: loads first, then the stores
      int64_t v = threadIdx.x;
      for (; v + step * (kUnroll - 1) < nv; v += step * kUnroll) {
        float4 w[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) w[u] = ld_once(reinterpret_cast<const float4 *>(wr) + v + step * u);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) scale(v + step * u, w[u]);
      }
      for (; v < nv; v += step) scale(v, ld_once(reinterpret_cast<const float4 *>(wr) + v));
    } else {
      for (int64_t c = threadIdx.x; c < m; c += blockDim.x) wr[c] *= decay;
    }
    return;
  }
  const float c = static_cast<float>(lr * factor[static_cast<int64_t>(b) * k + slot]);
  const float *orow = O + (static_cast<int64_t>(b) * k + slot) * m;
  float *mr = M + (static_cast<int64_t>(b) * n + row) * m;
  if (vec) {
    auto update = [&](int64_t v, float4 w, const float4 &o, float4 mm) {
      w.x = fmaf(-c, o.x, decay * w.x);
      w.y = fmaf(-c, o.y, decay * w.y);
      w.z = fmaf(-c, o.z, decay * w.z);
      w.w = fmaf(-c, o.w, decay * w.w);
      mm.x *= mu; mm.y *= mu; mm.z *= mu; mm.w *= mu;
      st_once(reinterpret_cast<float4 *>(wr) + v, w);
      st_once(reinterpret_cast<float4 *>(mr) + v, mm);
    };
    int64_t v = threadIdx.x;
    for (; v + step * (kUnroll - 1) < nv; v += step * kUnroll) {
      float4 w[kUnroll], o[kUnroll], mm[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        w[u] = ld_once(reinterpret_cast<const float4 *>(wr) + v + step * u);
        o[u] = ld_once(reinterpret_cast<const float4 *>(orow) + v + step * u);
        mm[u] = ld_once(reinterpret_cast<const float4 *>(mr) + v + step * u);
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) update(v + step * u, w[u], o[u], mm[u]);
    }
    for (; v < nv; v += step)
      update(v, ld_once(reinterpret_cast<const float4 *>(wr) + v), ld_once(reinterpret_cast<const float4 *>(orow) + v),
             ld_once(reinterpret_cast<const float4 *>(mr) + v));
  } else {
    for (int64_t j = threadIdx.x; j < m; j += blockDim.x) {
      wr[j] = fmaf(-c, orow[j], decay * wr[j]);
      mr[j] *= mu;
    }
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
template <class E, int TILE, int PL = 1>
static hipError_t launch_gemm_t(int mode, const GemmParams &p, hipStream_t s) {
  const bool split1 = p.part_out != nullptr, split2 = p.part_in != nullptr;
  const int grid = p.tiles_per_mat * p.batch * (split1 ? p.k_parts : 1);
  if (grid <= 0) return hipSuccess;
  // a K split: symmetric results on the 256-edge 16-bit kernel, one pass at a time
  if (split1 || split2) {
    if (mode != MODE_SYM || TILE != 256 || PL != 1 || sizeof(typename E::S) != 2 || (split1 && split2) ||
        (split1 && (p.k_parts < 1 || p.K / 32 < p.k_parts)) || (split2 && (p.parts_in < 1 || p.K != 0)))
      return hipErrorInvalidValue;
    if constexpr (TILE == 256 && PL == 1 && sizeof(typename E::S) == 2) {
      constexpr int nt = WaveLayout<TILE>::THREADS;
      if (split1) gemm_nt<E, TILE, MODE_SYM, PL, 0, 1><<<grid, nt, 0, s>>>(p);
      else gemm_nt<E, TILE, MODE_SYM, PL, 0, 2><<<grid, nt, 0, s>>>(p);
      return hipGetLastError();
    }
  }
  constexpr int nt = WaveLayout<TILE>::THREADS;
  if constexpr (TILE == 256 && PL == 1) {
    if (p.b_kmajor && mode != MODE_SYM) {
      if (mode == MODE_GEN) gemm_nt<E, TILE, MODE_GEN, PL, 1><<<grid, nt, 0, s>>>(p);
      else gemm_nt<E, TILE, MODE_FINAL, PL, 1><<<grid, nt, 0, s>>>(p);
      return hipGetLastError();
    }
  }
  if (p.b_kmajor) return hipErrorInvalidValue;   // K-major B needs 256-edge 16-bit tiles
  switch (mode) {
    case MODE_SYM: gemm_nt<E, TILE, MODE_SYM, PL><<<grid, nt, 0, s>>>(p); break;
    case MODE_GEN: gemm_nt<E, TILE, MODE_GEN, PL><<<grid, nt, 0, s>>>(p); break;
    default: gemm_nt<E, TILE, MODE_FINAL, PL><<<grid, nt, 0, s>>>(p); break;
  }
  return hipGetLastError();
}

hipError_t launch_gemm(int dt, int tile, int mode, const GemmParams &p, hipStream_t s) {
  if (dt == DT_BF16) return tile == 256 ? launch_gemm_t<EBF16, 256>(mode, p, s) : launch_gemm_t<EBF16, 128>(mode, p, s);
  if (dt == DT_F16) return tile == 256 ? launch_gemm_t<EF16, 256>(mode, p, s) : launch_gemm_t<EF16, 128>(mode, p, s);
  if (dt == DT_BF16X3) return launch_gemm_t<EBF16, 128, 2>(mode, p, s);   // split planes: 128-edge tiles
  return launch_gemm_t<EF32, 128>(mode, p, s);   // fp32 always uses 128-edge tiles
}

const char *gemm_kernel_name(int dt, int tile, int mode, bool b_kmajor) {
  if (b_kmajor && tile == 256 && (dt == DT_BF16 || dt == DT_F16) && mode != MODE_SYM) {
    static const char *nn[2][2] = {{"gemm_nn<bf16,256,gen>", "gemm_nn<bf16,256,final>"},
                                   {"gemm_nn<f16,256,gen>", "gemm_nn<f16,256,final>"}};
    return nn[dt == DT_F16 ? 1 : 0][mode == MODE_GEN ? 0 : 1];
  }
  static const char *names[4][2][3] = {
      {{"gemm_nt<f32,128,sym>", "gemm_nt<f32,128,gen>", "gemm_nt<f32,128,final>"},
       {"gemm_nt<f32,128,sym>", "gemm_nt<f32,128,gen>", "gemm_nt<f32,128,final>"}},
      {{"gemm_nt<bf16,128,sym>", "gemm_nt<bf16,128,gen>", "gemm_nt<bf16,128,final>"},
       {"gemm_nt<bf16,256,sym>", "gemm_nt<bf16,256,gen>", "gemm_nt<bf16,256,final>"}},
      {{"gemm_nt<f16,128,sym>", "gemm_nt<f16,128,gen>", "gemm_nt<f16,128,final>"},
       {"gemm_nt<f16,256,sym>", "gemm_nt<f16,256,gen>", "gemm_nt<f16,256,final>"}},
      {{"gemm_nt<bf16x3,128,sym>", "gemm_nt<bf16x3,128,gen>", "gemm_nt<bf16x3,128,final>"},
       {"gemm_nt<bf16x3,128,sym>", "gemm_nt<bf16x3,128,gen>", "gemm_nt<bf16x3,128,final>"}}};
  return names[dt][tile == 256 ? 1 : 0][mode];
}

hipError_t launch_norm_partial(int io, const void *X, int64_t batch, int64_t n, int64_t m,
                               int64_t rows_eff, const int64_t *row_idx, int parts,
                               double *partials, hipStream_t s) {
  dim3 grid(parts, static_cast<unsigned>(batch));
  if (io == DT_BF16) norm_partial<EBF16><<<grid, 256, 0, s>>>(X, n, m, rows_eff, row_idx, parts, partials);
  else if (io == DT_F16) norm_partial<EF16><<<grid, 256, 0, s>>>(X, n, m, rows_eff, row_idx, parts, partials);
  else norm_partial<EF32><<<grid, 256, 0, s>>>(X, n, m, rows_eff, row_idx, parts, partials);
  return hipGetLastError();
}

template <class TIn>
static void st_dispatch(int cdt, dim3 grid, hipStream_t s, const void *X, int64_t n, int64_t m,
                        int64_t rows_eff, const int64_t *row_idx, const double *partials,
                        int parts, double eps, void *Xh, void *XT, int64_t Np, int64_t Mp,
                        int64_t ph, int64_t pt) {
  if (cdt == DT_BF16)
    scale_transpose<TIn, EBF16, 1><<<grid, 256, 0, s>>>(X, n, m, rows_eff, row_idx, partials, parts, eps, Xh, XT, Np, Mp, ph, pt);
  else if (cdt == DT_BF16X3)
    scale_transpose<TIn, EBF16, 2><<<grid, 256, 0, s>>>(X, n, m, rows_eff, row_idx, partials, parts, eps, Xh, XT, Np, Mp, ph, pt);
  else if (cdt == DT_F16)
    scale_transpose<TIn, EF16, 1><<<grid, 256, 0, s>>>(X, n, m, rows_eff, row_idx, partials, parts, eps, Xh, XT, Np, Mp, ph, pt);
  else
    scale_transpose<TIn, EF32, 1><<<grid, 256, 0, s>>>(X, n, m, rows_eff, row_idx, partials, parts, eps, Xh, XT, Np, Mp, ph, pt);
}

hipError_t launch_scale_transpose(int io, int cdt, const void *X, int64_t batch, int64_t n,
                                  int64_t m, int64_t rows_eff, const int64_t *row_idx,
                                  const double *partials, int parts, double eps, void *Xh,
                                  void *XT, int64_t Np, int64_t Mp, int64_t ph, int64_t pt,
                                  hipStream_t s) {
  dim3 grid(static_cast<unsigned>(Mp / 64), static_cast<unsigned>(Np / 64), static_cast<unsigned>(batch));
  if (io == DT_F32 && (cdt == DT_BF16 || cdt == DT_F16) && !XT && m % 4 == 0 && Mp % 4 == 0 &&
      (reinterpret_cast<uintptr_t>(X) & 15) == 0 && (reinterpret_cast<uintptr_t>(Xh) & 7) == 0) {
    const dim3 g(static_cast<unsigned>((Np + 3) / 4), static_cast<unsigned>(batch));
    const float *Xf = static_cast<const float *>(X);
    if (cdt == DT_BF16)
      scale_rows_f32<EBF16><<<g, 256, 0, s>>>(Xf, n, m, rows_eff, row_idx, partials, parts, eps, Xh, Np, Mp);
    else
      scale_rows_f32<EF16><<<g, 256, 0, s>>>(Xf, n, m, rows_eff, row_idx, partials, parts, eps, Xh, Np, Mp);
    return hipGetLastError();
  }
  const bool vec = (m % 8 == 0) && ((reinterpret_cast<uintptr_t>(X) & 15) == 0) && io != DT_F32 && cdt != DT_F32;
  if (vec) {
#define GNS_ST16(TI, TC, PL) \
  scale_transpose16<TI, TC, PL><<<grid, 256, 0, s>>>(X, n, m, rows_eff, row_idx, partials, parts, eps, Xh, XT, Np, Mp, ph, pt)
    if (io == DT_BF16) {
      if (cdt == DT_BF16) GNS_ST16(EBF16, EBF16, 1);
      else if (cdt == DT_BF16X3) GNS_ST16(EBF16, EBF16, 2);
      else GNS_ST16(EBF16, EF16, 1);
    } else {
      if (cdt == DT_BF16) GNS_ST16(EF16, EBF16, 1);
      else if (cdt == DT_BF16X3) GNS_ST16(EF16, EBF16, 2);
      else GNS_ST16(EF16, EF16, 1);
    }
#undef GNS_ST16
    return hipGetLastError();
  }
  if (io == DT_BF16) st_dispatch<EBF16>(cdt, grid, s, X, n, m, rows_eff, row_idx, partials, parts, eps, Xh, XT, Np, Mp, ph, pt);
  else if (io == DT_F16) st_dispatch<EF16>(cdt, grid, s, X, n, m, rows_eff, row_idx, partials, parts, eps, Xh, XT, Np, Mp, ph, pt);
  else st_dispatch<EF32>(cdt, grid, s, X, n, m, rows_eff, row_idx, partials, parts, eps, Xh, XT, Np, Mp, ph, pt);
  return hipGetLastError();
}

hipError_t launch_transpose_sumsq(int dt, const void *X, int64_t batch, int64_t n, int64_t m,
                                  void *XT, void *Xcopy, double *partials, const int64_t *row_idx,
                                  int64_t n_src, hipStream_t s) {
  dim3 grid(static_cast<unsigned>(m / 128), static_cast<unsigned>(n / 128), static_cast<unsigned>(batch));
  if (!row_idx) {
    if (dt == DT_BF16) transpose_sumsq<EBF16, false><<<grid, 256, 0, s>>>(X, n, m, XT, Xcopy, partials, nullptr, n);
    else transpose_sumsq<EF16, false><<<grid, 256, 0, s>>>(X, n, m, XT, Xcopy, partials, nullptr, n);
  } else {
    if (dt == DT_BF16) transpose_sumsq<EBF16, true><<<grid, 256, 0, s>>>(X, n, m, XT, Xcopy, partials, row_idx, n_src);
    else transpose_sumsq<EF16, true><<<grid, 256, 0, s>>>(X, n, m, XT, Xcopy, partials, row_idx, n_src);
  }
  return hipGetLastError();
}

hipError_t launch_check_finite(int dt, const void *A, int64_t batch, int64_t rows, int64_t cols,
                               const int64_t *row_idx, int64_t k, int32_t *result, hipStream_t s) {
  check_rows_init<<<1, 1, 0, s>>>(result);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || batch == 0) return e;
  const int64_t sel = row_idx ? k : rows;
  const int64_t gx = std::min<int64_t>((sel + 3) / 4, 65535);
  dim3 grid(static_cast<unsigned>(gx), static_cast<unsigned>(batch));
  if (dt == DT_F32) check_finite<EF32><<<grid, 256, 0, s>>>(A, rows, cols, row_idx, k, result);
  else if (dt == DT_BF16) check_finite<EBF16><<<grid, 256, 0, s>>>(A, rows, cols, row_idx, k, result);
  else check_finite<EF16><<<grid, 256, 0, s>>>(A, rows, cols, row_idx, k, result);
  return hipGetLastError();
}

hipError_t launch_norm_finish(const double *partials, int64_t batch, int64_t parts, double eps,
                              float *inv, float *inv2, hipStream_t s) {
  norm_finish<<<static_cast<unsigned>(batch), 256, 0, s>>>(partials, parts, eps, inv, inv2);
  return hipGetLastError();
}

hipError_t launch_select_rows_l1(int io, const void *M, int64_t batch, int64_t n, int64_t m,
                                 int64_t k, double *keys, int64_t *out, hipStream_t s) {
  dim3 grid(static_cast<unsigned>((n + 3) / 4), static_cast<unsigned>(batch));
  if (io == DT_BF16) row_l1<EBF16><<<grid, 256, 0, s>>>(M, n, m, keys);
  else if (io == DT_F16) row_l1<EF16><<<grid, 256, 0, s>>>(M, n, m, keys);
  else row_l1<EF32><<<grid, 256, 0, s>>>(M, n, m, keys);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  select_topk<<<static_cast<unsigned>(batch), 1024, 0, s>>>(keys, n, k, out);
  return hipGetLastError();
}

hipError_t launch_check_rows(const int64_t *row_idx, int64_t batch, int64_t k, int64_t n,
                             int32_t *result, hipStream_t s) {
  check_rows_init<<<1, 1, 0, s>>>(result);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  check_rows<<<static_cast<unsigned>(batch), 256, 0, s>>>(row_idx, k, n, result);
  return hipGetLastError();
}

hipError_t launch_momentum_l1(int grad_dtype, float *M, const void *G, int64_t batch, int64_t n,
                              int64_t m, double *keys, double *sumsq, hipStream_t s) {
  dim3 grid(static_cast<unsigned>((n + 3) / 4), static_cast<unsigned>(batch));
  const bool vec = (m % 4) == 0 && (reinterpret_cast<uintptr_t>(M) & 15) == 0 &&
                   (reinterpret_cast<uintptr_t>(G) & (grad_dtype == DT_F32 ? 15 : 7)) == 0;
  if (grad_dtype == DT_BF16) momentum_l1<EBF16><<<grid, 256, 0, s>>>(M, G, n, m, vec, keys, sumsq);
  else if (grad_dtype == DT_F16) momentum_l1<EF16><<<grid, 256, 0, s>>>(M, G, n, m, vec, keys, sumsq);
  else momentum_l1<EF32><<<grid, 256, 0, s>>>(M, G, n, m, vec, keys, sumsq);
  return hipGetLastError();
}

hipError_t launch_row_partials(const double *rowsq, const int64_t *row_idx, int64_t batch, int64_t n,
                               int64_t k, int parts, double *partials, hipStream_t s) {
  if (batch == 0 || parts < 1) return hipSuccess;
  dim3 grid(static_cast<unsigned>((parts + 255) / 256), static_cast<unsigned>(batch));
  row_partials<<<grid, 256, 0, s>>>(rowsq, row_idx, n, k, parts, partials);
  return hipGetLastError();
}

hipError_t launch_select_topk(const double *keys, int64_t batch, int64_t n, int64_t k, int64_t *out,
                              hipStream_t s) {
  select_topk<<<static_cast<unsigned>(batch), 1024, 0, s>>>(keys, n, k, out);
  return hipGetLastError();
}

hipError_t launch_normuon(const float *O, int64_t batch, int64_t k, int64_t m, float *v,
                          const int64_t *S, int64_t n, double beta2, double eps, int normuon,
                          double *rowsq, double *factor, hipStream_t s) {
  if (normuon) {
    dim3 grid(static_cast<unsigned>((k + 3) / 4), static_cast<unsigned>(batch));
    const bool vec = (m % 4) == 0 && (reinterpret_cast<uintptr_t>(O) & 15) == 0;
    row_sumsq<<<grid, 256, 0, s>>>(O, k, m, vec, rowsq);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  normuon_factors<<<static_cast<unsigned>(batch), 256, 0, s>>>(rowsq, v, S, n, k, m, beta2, eps, normuon,
                                                               factor);
  return hipGetLastError();
}

hipError_t launch_dion3_update(float *W, float *M, const float *O, const int64_t *S,
                               const double *factor, int64_t batch, int64_t n, int64_t m, int64_t k,
                               float decay, double lr, float mu, hipStream_t s) {
  dim3 grid(static_cast<unsigned>(n), static_cast<unsigned>(batch));
  const bool vec = (m % 4) == 0 && (reinterpret_cast<uintptr_t>(W) & 15) == 0 &&
                   (reinterpret_cast<uintptr_t>(M) & 15) == 0 && (reinterpret_cast<uintptr_t>(O) & 15) == 0;
  dion3_update<<<grid, 256, 0, s>>>(W, M, O, S, factor, n, m, k, decay, lr, mu, vec);
  return hipGetLastError();
}

}  // namespace gns

#ifdef GNS_TIMELINE
// Timeline build only: copies up to max_rec records (8 x uint64 each, see
// Timeline) to host memory dst, stores the number recorded since the last
// reset in *n_out, and with reset != 0 starts a new recording.  Returns 0, or
// the step that failed (1-3).
extern "C" int gns_timeline_read(void *dst, unsigned max_rec, unsigned *n_out, int reset) {
  unsigned n = 0;
  if (hipMemcpyFromSymbol(&n, HIP_SYMBOL(gns::g_timeline_n), sizeof(n)) != hipSuccess) return 1;
  *n_out = n;
  unsigned c = n < max_rec ? n : max_rec;
  if (c > gns::kTimelineMax) c = gns::kTimelineMax;
  if (c && dst && hipMemcpyFromSymbol(dst, HIP_SYMBOL(gns::g_timeline), size_t(c) * 64) != hipSuccess) return 2;
  if (reset) {
    const unsigned z = 0;
    if (hipMemcpyToSymbol(HIP_SYMBOL(gns::g_timeline_n), &z, sizeof(z)) != hipSuccess) return 3;
  }
  return 0;
}
#endif
