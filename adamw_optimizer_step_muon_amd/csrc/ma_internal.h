// Internal declarations shared by the library's translation units (not installed).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace ma {

// ---------------------------------------------------------------------------
// Vector types for gfx950 (64-wide wavefronts, MFMA bf16 operands of 8 values)
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// fp32 -> bf16, round to nearest even (NaN stays NaN).
__device__ __forceinline__ unsigned short f2bf(float f) {
  return __builtin_bit_cast(unsigned short, static_cast<__bf16>(f));
}
// fp32 -> fp16 (IEEE binary16), round to nearest even; fp16 -> fp32 (exact).
__device__ __forceinline__ unsigned short f2h(float f) {
  return __builtin_bit_cast(unsigned short, static_cast<_Float16>(f));
}
__device__ __forceinline__ float h2f(unsigned short h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, h));
}
__device__ __forceinline__ float bf2f(unsigned short h) {
  return __builtin_bit_cast(float, static_cast<unsigned int>(h) << 16);
}

// ---------------------------------------------------------------------------
// Workspace layout of one Muon bucket (bf16 buffers, tile-padded)
// ---------------------------------------------------------------------------
constexpr int kCastTile = 64;     // momentum/cast kernel tile

struct BucketPlan {
  int64_t K, A, B;
  bool transposed;
  int tile;  // square GEMM tile (128 or 256); m and n are padded to it
  int64_t m, n, m_pad, n_pad;
  int64_t nblk;  // momentum/cast tiles per matrix (one partial sum of U^2 each)
  // byte offsets inside the workspace: X ping-pong, R, P, per-tile fp64 sums of U^2,
  // per-matrix 1 / (||U|| + eps) (fp32) and power-of-two shift of X (int32)
  size_t off_x[2], off_r, off_p, off_part, off_inv, off_shift, bytes;
  // buckets with 256-tiles and a Gram side above 2048 also keep X^T (n_pad x m_pad),
  // which their combine reads
  bool keeps_xt;
  size_t off_xt[2];
  // Gram-space iteration (long side >= 3.5 x the Gram side, when asked for), on fp16
  // operands: X0 is converted in place to fp16 X0 * sx_k (sx_k = gs_sx but for norms
  // near eps); R ping-pong (stored as R * kGramSpaceRScale) in off_r / off_r2, the
  // accumulated polynomial Q in off_q[2], the product R P in off_t (m_pad x m_pad fp16
  // each); per matrix ||X0||, then the Gram's and the last product's factors, in off_gsc
  // (3 K floats)
  bool gram_space;
  float gs_sx;
  size_t off_r2, off_q[2], off_t, off_gsc;
};

// Plan of one bucket on the given GEMM tile (128 or 256), or on pick_tile's choice
// (tile 0); MA_NS_TILE, when set to 128 or 256, overrides either.
BucketPlan plan_bucket(int64_t K, int64_t A, int64_t B, int tile = 0, bool gram_space = false);
// Whether a bucket runs the Gram-space iteration under ns_mode: 1 asks for it on buckets
// whose long side is at least 3.5 times the Gram side (either orientation), when the
// coefficients keep the route inside fp16's range (gs_mode).
constexpr int64_t kGramSpaceAspectNum = 7, kGramSpaceAspectDen = 2;
bool wants_gram_space(int32_t ns_mode, int64_t A, int64_t B);
// Gram-space scales: R is stored times kGramSpaceRScale; X0 times gram_space_sx(m, n),
// the power of two nearest below sqrt(m n) (at most 2^14), so that the normalised
// X0 entries (|x| <= 1, about 1 / sqrt(m n) typically) sit in fp16's normal range.
constexpr float kGramSpaceRScale = 16384.0f;
float gram_space_sx(int64_t m, int64_t n);
// Whether GEMM launches holding `tri` lower-triangle and `comb` combine tiles of
// 256 x 256 fill the chip well enough for 256-tiles.
bool fills_256(int64_t tri, int64_t comb);
// 256 x 256 tiles of a bucket of K matrices with Gram side m and long side n: the
// lower triangle of the Gram products and the combine
int64_t tri_tiles_256(int64_t K, int64_t m);
int64_t comb_tiles_256(int64_t K, int64_t m, int64_t n);
// GEMM tile for a bucket of K matrices with Gram side m and long side n, alone
int pick_tile(int64_t K, int64_t m, int64_t n);
// Gram sides below this always run on 128-tiles
constexpr int64_t kMinGram256 = 512;
// Tuning override of the GEMM tile (MA_NS_TILE = 128 or 256), 0 when unset.
int forced_tile();

// ---------------------------------------------------------------------------
// Kernel launchers (return hipSuccess or the launch error)
// ---------------------------------------------------------------------------
struct NsCoeffs {
  float a, b, c;
};

// M <- mu M + G (when M != nullptr), U = G + mu M_new | M_new | G, cast to bf16 as the
// orientation copy S (Ap x Bp) and/or the transposed copy T (Bp x Ap) (either may be
// null), zero in the padding; per-tile sums of U^2.
hipError_t launch_muon_prep(const BucketPlan& p, const float* G, float* M, float mu,
                            int nesterov, double* partials, unsigned short* S,
                            unsigned short* T, hipStream_t s);
// inv[k] = 1 / (sqrt(sum of partials of matrix k) + eps), shift[k] = 0; for a norm
// outside [2^-32, 2^32], shift[k] = -e and inv[k] = 2^e / (norm + eps) (e its exponent)
// (x0norm, when given: ||X0|| = ||U|| / (||U|| + eps) per matrix)
hipError_t launch_norm_finalize(const BucketPlan& p, const double* partials, float eps,
                                float* inv, int* shift, hipStream_t s, float* x0norm = nullptr);
// S and T (m_pad x n_pad bf16 per matrix, either may be null) *= 2^shift[k] where
// shift[k] != 0, so that inv[k] * X is still X0 = U / (||U|| + eps)
hipError_t launch_rescale(const BucketPlan& p, unsigned short* S, unsigned short* T,
                          const int* shift, hipStream_t s);
// Gram-space route: S and T (bf16 U, m_pad x n_pad per matrix, either may be null) are
// replaced in place by fp16(U * inv[k] * sx_k), i.e. X0 * sx_k in fp16, sx_k = sx unless
// ||X0|| (x0norm) < 1/2, then sx times the power of two that brings it to [1/2, 1);
// gsc (2 K floats) receives the Gram's per-matrix factor 2^7 / sx_k and the last
// product's 1 / sx_k
hipError_t launch_to_f16(const BucketPlan& p, unsigned short* S, unsigned short* T,
                         const float* inv, const float* x0norm, float sx, float* gsc,
                         hipStream_t s);
// Newton-Schulz products over a group of up to kMaxGemmGroups buckets with the same
// tile, one launch per product for the whole group.
constexpr int kMaxGemmGroups = 4;
struct NsGroup {
  const BucketPlan* plan;
  unsigned short* X;    // current iterate, m_pad x n_pad per matrix
  unsigned short* Xn;   // next iterate (one-orientation buckets: the last iteration of
                        // a transposed bucket writes its transpose here)
  unsigned short* XT;   // X^T and the next X^T, n_pad x m_pad (keeps_xt buckets only)
  unsigned short* XTn;
  unsigned short* R;    // m_pad x m_pad
  unsigned short* P;
};
// One Newton-Schulz GEMM launch: its arguments are read by the kernel in place from the
// kernel-argument segment (see ns_gemm.hip), so the table must fit there.
enum Epi { kGram = 0, kPoly = 1, kCombine = 2 };
// Element types of a GEMM launch: bf16 operands and result (the printed iteration);
// fp16 operands and result (the Gram-space products); fp16 operands and a bf16 result
// (the Gram-space route's last product, which the update reads).
enum GemmTypes { kTyBf16 = 0, kTyF16 = 1, kTyF16ToBf16 = 2 };

struct GemmArgs {
  const unsigned short* A;
  const unsigned short* B;
  int64_t lda, ldb, strideA, strideB;
  int kdim;
  unsigned short* C;    // row-major target
  unsigned short* C2;   // transposed target (combine) or mirror target (gram/poly); the
                        // combine may leave either C or C2 null
  int64_t ldc, ldc2, strideC, strideC2;
  const unsigned short* aux;  // poly: R, source of the b R term (read transposed)
  int64_t ldaux, strideAux;
  float alpha, beta, diag;  // poly: P = alpha R + beta R R^T + diag I
  const float* scale;   // per-matrix factor or null: gram R *= scale^2, combine X' *= scale
  int tiles_m, tiles_n; // tile grid (triangular for gram/poly)
  int tiles_per_batch;
  int tiles_k;          // matrices in the group (host side: block count = tiles_k x tiles_per_batch)
  int band;             // tile rows per L2 band (tile order; 0: plain row-major triangle)
  int xcd_remap;        // block order across the XCDs (XcdOrder)
  int spread;           // 1: spread the next stage's DMAs over the first half-stage
  int symmetrize;       // gram with A != B: copy each diagonal tile's lower triangle up
  float post;           // gram / combine: constant factor on the result (0: none)
};

// Up to kMaxGroups buckets (same tile shape) share one launch: block b belongs to the
// group g with start[g] <= b' < start[g+1], b' the XCD-remapped block id.
struct GemmTable {
  GemmArgs g[kMaxGemmGroups];
  int start[kMaxGemmGroups + 1];
  int ngroups;
};
static_assert(sizeof(GemmTable) <= 2048, "GemmTable is passed whole as the kernel argument");
static_assert(offsetof(GemmTable, g) == 0, "the kernel reads the table at the segment start");

// Block order across the 8 XCDs (blocks go to them round-robin: bid % 8).
//   kXcdRoundRobin: logical id = block id;
//   kXcdRuns: each XCD takes a contiguous run of the logical ids, so the blocks one XCD
//     runs together are neighbouring tiles whose operand panels its L2 serves;
//   kXcdShared: the XCDs share each matrix: XCD x takes the x-th eighth of every
//     matrix's tiles (in the band order), matrix after matrix, so at any time all eight
//     work on the same matrix and the panels one XCD's L2 misses are likely in the
//     memory-side cache (MALL) from another's.  For matrices of many tiles (the
//     8192-wide Gram sides: 528 triangle tiles, 3584 combine tiles) that measured 5 %
//     less Newton-Schulz time than kXcdRuns; for matrices of a few dozen tiles, where
//     one XCD's run covers whole matrices, 5-7 % more.  A group then takes
//     8 * K * ceil(tiles_per_batch / 8) blocks (XCDs with one tile fewer per matrix
//     get padding blocks).
enum XcdOrder { kXcdRoundRobin = 0, kXcdRuns = 1, kXcdShared = 2 };

// blocks a group of K matrices of `tpb` tiles takes in the grid (a multiple of 8)
__host__ __device__ __forceinline__ int gemm_group_blocks(int tpb, int K, int xcd_order) {
  return xcd_order == kXcdShared ? 8 * K * ((tpb + 7) / 8) : (tpb * K + 7) & ~7;
}

// kXcdRuns: block id -> logical id so that each XCD's blocks are a contiguous run.
__host__ __device__ __forceinline__ int xcd_linear(int bid, int nblocks) {
  constexpr int kXcd = 8;
  const int q = nblocks / kXcd, r = nblocks % kXcd;
  const int xcd = bid % kXcd, local = bid / kXcd;
  return xcd < r ? xcd * (q + 1) + local : r * (q + 1) + (xcd - r) * q + local;
}

// The output tile block `bid` of a launch computes: its group gi, matrix `batch`, tile row
// ti and tile column tj; false for a padding block (which exits at once).  Groups start
// on multiples of 8 blocks, so a group's blocks keep the round-robin XCD pattern; inside
// a group the blocks are renumbered so each XCD owns a contiguous run of tiles, in bands
// of `band` row panels (the combine: column by column inside a band; the symmetric
// products: the lower triangle band by band); or, kXcdShared, each matrix's run is
// split among the eight XCDs.  Used by the kernel and by the host-side
// plan check, which enumerates every block of every launch.
__host__ __device__ __forceinline__ bool gemm_block_tile(const GemmTable& t, int epi, int bid,
                                                         int& gi, int64_t& batch, int& ti,
                                                         int& tj) {
  gi = 0;
#pragma unroll
  for (int i = 1; i < kMaxGemmGroups; ++i)
    if (i < t.ngroups && bid >= t.start[i]) gi = i;
  const GemmArgs& args = t.g[gi];
  const int g0 = t.start[gi];
  const int gcount = args.tiles_per_batch * args.tiles_k;
  const int raw = bid - g0;
  int lid;
  if (args.xcd_remap == kXcdShared) {
    // XCD x: tiles [x q + min(x, r), ... + per) of matrix 0, then of matrix 1, ...
    const int tpb = args.tiles_per_batch;
    const int q = tpb / 8, r = tpb % 8;
    const int x = raw % 8, local = raw / 8;
    const int per = q + (x < r ? 1 : 0);
    if (per == 0) return false;
    const int b = local / per;
    if (b >= args.tiles_k) return false;
    lid = b * tpb + x * q + (x < r ? x : r) + (local - b * per);
  } else {
    lid = args.xcd_remap == kXcdRuns ? xcd_linear(raw, (gcount + 7) & ~7) : raw;
    if (lid >= gcount) return false;
  }
  batch = lid / args.tiles_per_batch;
  const int tile = lid - static_cast<int>(batch) * args.tiles_per_batch;
  if (epi == kCombine) {
    // bands of `band` row panels; inside a band, column-major over tiles
    const int G = args.band;
    const int per_band = G * args.tiles_n;
    const int b = tile / per_band;
    const int first = b * G;
    const int rows = (args.tiles_m - first) < G ? (args.tiles_m - first) : G;
    const int in = tile - b * per_band;
    ti = first + in % rows;
    tj = in / rows;
  } else if (args.band > 0) {
    // lower triangle in bands of G tile rows [r0, r1); inside a band, column by column
    // (the r0 full-height columns, then the band's own triangle), so the blocks that
    // run together share G row panels and a few column panels
    const int G = args.band, T = args.tiles_m;
    int r0 = 0, u = tile;
    for (;;) {
      const int r1 = (r0 + G) < T ? (r0 + G) : T, h = r1 - r0;
      const int cnt = r0 * h + h * (h + 1) / 2;
      if (u < cnt) {
        if (u < r0 * h) {
          tj = u / h;
          ti = r0 + (u - tj * h);
        } else {
          int v = u - r0 * h, c = 0;
          while (v >= h - c) { v -= h - c; ++c; }
          tj = r0 + c;
          ti = tj + v;
        }
        break;
      }
      u -= cnt;
      r0 = r1;
    }
  } else {
    // lower-triangle enumeration: tile = ti (ti + 1) / 2 + tj, tj <= ti
    ti = static_cast<int>((__builtin_sqrtf(8.0f * tile + 1.0f) - 1.0f) * 0.5f);
    while ((ti + 1) * (ti + 2) / 2 <= tile) ++ti;
    while (ti * (ti + 1) / 2 > tile) --ti;
    tj = tile - ti * (ti + 1) / 2;
  }
  return true;
}

// Compiled GEMM configurations: 128 x 128 tiles; 256 x 256 reading X^T in the combine;
// 256 x 256 whose combine reads X (transposing LDS loads); 192 x 256 combine tiles.
enum TileCfg { kTileSmall = 0, kTileBig = 1, kTileBigX = 2, kTileMidX = 3 };
struct TileShape {
  int bm, bn, bk;
  bool combine_reads_x;  // the combine's B operand is X (k rows), not X^T
};

// The GEMM configuration of one Newton-Schulz product of a phase.  A field at its
// default (0, or -1 for spread) takes the library's rule for it.  Every configuration
// accumulates each output over the same k order, so results do not depend on it.
struct GemmChoice {
  int tile = 0;      // 128 or 256 (on a 256-padded phase), 192 (combine only)
  int band = 0;      // row panels per L2 band in the tile order (default 4)
  int spread = -1;   // 256-tiles: 1 spreads the next stage's DMAs over half a stage, 0
                     // issues them in one burst (default 1; 128-tiles always 0)
  int pipeline = 0;  // 256-tiles of the Gram, polynomial and X^T-reading combine:
                     // 1 = stages of k = 64 in a 3 + 2 ring, 2 = 4 stages of k = 32
                     // (default 1)
  int xcd = 0;       // 1 = contiguous runs per XCD, 2 = round-robin order, 3 = matrices
                     // shared by the XCDs (default: 3 for matrices of >= 512 tiles, else 1)
  bool operator==(const GemmChoice& o) const {
    return tile == o.tile && band == o.band && spread == o.spread && pipeline == o.pipeline &&
           xcd == o.xcd;
  }
  bool is_default() const { return *this == GemmChoice{}; }
};

// Dry run: while a recorder is installed on the calling thread, every launcher hands its
// launch to the recorder and returns hipSuccess without touching the GPU (the host-side
// plan check replays a step this way).
struct LaunchRecorder {
  virtual ~LaunchRecorder() = default;
  virtual void gemm(int epi, const TileShape& shape, const GemmTable& t) = 0;
  virtual void prep(const BucketPlan& p, const float* G, const float* M, const double* partials,
                    const unsigned short* S, const unsigned short* T) = 0;
  virtual void norm(const BucketPlan& p, const double* partials, const float* inv,
                    const int* shift, const float* x0norm) = 0;
  virtual void rescale(const BucketPlan& p, const unsigned short* S, const unsigned short* T,
                       const int* shift) = 0;
  virtual void to_f16(const BucketPlan& p, const unsigned short* S, const unsigned short* T,
                      const float* inv, const float* x0norm, const float* gsc) = 0;
  virtual void apply(const BucketPlan& p, const float* out, const unsigned short* O,
                     const float* oscale, int64_t ldo) = 0;
};
LaunchRecorder*& launch_recorder();

// GEMM configurations (GemmChoice): tile 0 takes the default for the phase; 128 or 256
// picks that tile (256 only on a 256-padded phase; the combine of a phase that keeps
// X^T always runs its own 256-tile configuration), and the combine also takes 192
// (192 x 256 tiles) where combine_192_ok holds for every bucket.
bool combine_192_ok(const BucketPlan& p);
// R = X X^T (lower-triangle tiles, mirrored); R *= scale[i][k]^2 where scale[i] is given
// (ty: GemmTypes; post: a constant factor on the result, 0 for none)
hipError_t launch_gram(const NsGroup* g, int n, const float* const* scale,
                       const GemmChoice& ch, hipStream_t s, int ty = kTyBf16, float post = 0.0f);
// P = a I + b R + c R R^T (lower-triangle tiles, mirrored)
hipError_t launch_poly(const NsGroup* g, int n, float a, float b, float c,
                       const GemmChoice& ch, hipStream_t s, int ty = kTyBf16);
// Xn = P X (times scale[i][k] where given), written row-major (and as X^T into
// XTn for keeps_xt buckets); with `last`, only in the orientation of the parameter
// (X^T when A > B: n_pad x m_pad, into XTn, or into Xn for one-orientation buckets)
hipError_t launch_combine(const NsGroup* g, int n, const float* const* scale, bool last,
                          const GemmChoice& ch, hipStream_t s, int ty = kTyBf16,
                          float post = 0.0f);
// One symmetric product per bucket: C = A B^T (= A B for symmetric B) on lower-triangle
// tiles, mirrored, all m_pad x m_pad; exact only when A B is symmetric (A and B
// polynomials in one matrix, as in the Gram-space iteration).  Tile as launch_poly's.
struct SymProd {
  const BucketPlan* plan;
  const unsigned short* A;
  const unsigned short* B;
  unsigned short* C;
};
hipError_t launch_sym(const SymProd* p, int n, const GemmChoice& ch, hipStream_t s,
                      int ty = kTyBf16);
// param <- param - lr*wd*mask*param - lr*scale*O with O = oscale[k] * (bf16 O) (oscale
// may be null: 1), row stride ldo
hipError_t launch_muon_apply(const BucketPlan& p, float* param, const unsigned short* O,
                             const float* oscale, int64_t ldo, float lr, float wd, float scale,
                             int cautious, hipStream_t s);
// out = oscale[k] * O as fp32 in the (K, A, B) orientation
hipError_t launch_ns_extract(const BucketPlan& p, float* out, const unsigned short* O,
                             const float* oscale, int64_t ldo, hipStream_t s);

struct AdamWConst {
  float lr, beta1, beta2, one_m_beta1, one_m_beta2, eps, wd, inv_bc1, inv_bc2;
  int decoupled, cautious;
};
hipError_t launch_adamw(float* p, const float* g, float* m, float* v, int64_t n,
                        const AdamWConst& c, hipStream_t s);
// Up to kMaxAdamWSegs tensors in one launch (ma_adamw_step_multi): segment i covers
// blocks [block_start[i], block_start[i + 1]) of the grid, adamw_multi_blocks(n[i]) of them
// (n[i] >= 1); vec[i] = 1 when its four pointers are 16-byte aligned.
constexpr int kMaxAdamWSegs = 48;
struct AdamWSegTable {
  float* p[kMaxAdamWSegs];
  const float* g[kMaxAdamWSegs];
  float* m[kMaxAdamWSegs];
  float* v[kMaxAdamWSegs];
  int64_t n[kMaxAdamWSegs];
  int64_t block_start[kMaxAdamWSegs + 1];
  int32_t vec[kMaxAdamWSegs];
  int32_t nseg;
  AdamWConst c;
};
int64_t adamw_multi_blocks(int64_t n);
// Reference stream: `reads` (1..4) fp32 arrays in, `writes` (0..3) out, n elements
// (n % 4 == 0, 16-byte aligned), the AdamW kernel's access pattern without its arithmetic.
hipError_t launch_stream_probe(const float* const* in, int reads, float* const* out, int writes,
                               int64_t n, hipStream_t s);
hipError_t launch_adamw_multi(const AdamWSegTable& t, hipStream_t s);

// Matrix-core reference loop (mfma_probe.hip): `blocks` blocks of 512 threads, each wave
// running `iters` rounds of 8 v_mfma_f32_32x32x16_bf16 on 16 fragments read once from
// `operands` (16 x 64 x 8 bf16, 16-byte aligned); out: blocks x 512 floats; clocks
// (may be null): 2 per block, s_memtime and s_memrealtime deltas.
hipError_t launch_mfma_probe(const void* operands, int blocks, int iters, float* out,
                             unsigned long long* clocks, hipStream_t s);

}  // namespace ma
