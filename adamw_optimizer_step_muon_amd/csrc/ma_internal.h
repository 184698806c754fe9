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
  // byte offsets inside the workspace
  size_t off_x[2], off_r, off_p, off_part, off_inv, bytes;
  // buckets with 256-tiles and a Gram side above 2048 also keep X^T (n_pad x m_pad),
  // which their combine reads
  bool keeps_xt;
  size_t off_xt[2];
  // Gram-space iteration (n >= 2 m, when asked for): R ping-pong in off_r / off_r2, the
  // accumulated polynomial Q in off_q[2], the product R P in off_t (m_pad x m_pad bf16)
  bool gram_space;
  size_t off_r2, off_q[2], off_t;
};

// Plan of one bucket on the given GEMM tile (128 or 256), or on pick_tile's choice
// (tile 0); MA_NS_TILE, when set to 128 or 256, overrides either.
BucketPlan plan_bucket(int64_t K, int64_t A, int64_t B, int tile = 0, bool gram_space = false);
// Whether a bucket runs the Gram-space iteration under ns_mode: 1 asks for it where the
// long side is at least twice the Gram side.
bool wants_gram_space(int32_t ns_mode, int64_t A, int64_t B);
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
                            int nesterov, float* partials, unsigned short* S,
                            unsigned short* T, hipStream_t s);
// inv[k] = 1 / (sqrt(sum of partials of matrix k) + eps)
hipError_t launch_norm_finalize(const BucketPlan& p, const float* partials, float eps,
                                float* inv, hipStream_t s);
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
// GEMM tiles: `tile` (and `tile_choice`) 0 takes the default for the phase; 128 or 256
// picks that tile (256 only on a 256-padded phase; the combine of a phase that keeps
// X^T always runs its own 256-tile configuration), and the combine also takes 192
// (192 x 256 tiles) where combine_192_ok holds for every bucket.  Every choice
// accumulates each output over the same k order, so results do not depend on it.
bool combine_192_ok(const BucketPlan& p);
// R = X X^T (lower-triangle tiles, mirrored); R *= scale[i][k]^2 where scale[i] is given
hipError_t launch_gram(const NsGroup* g, int n, const float* const* scale, int tile,
                       hipStream_t s);
// P = a I + b R + c R R^T (lower-triangle tiles, mirrored)
hipError_t launch_poly(const NsGroup* g, int n, float a, float b, float c, int tile_choice,
                       hipStream_t s);
// Xn = P X (times scale[i][k] where given), written row-major (and as X^T into
// XTn for keeps_xt buckets); with `last`, only in the orientation of the parameter
// (X^T when A > B: n_pad x m_pad, into XTn, or into Xn for one-orientation buckets)
hipError_t launch_combine(const NsGroup* g, int n, const float* const* scale, bool last,
                          int tile, hipStream_t s);
// One symmetric product per bucket: C = A B^T (= A B for symmetric B) on lower-triangle
// tiles, mirrored, all m_pad x m_pad; exact only when A B is symmetric (A and B
// polynomials in one matrix, as in the Gram-space iteration).  Tile as launch_poly's.
struct SymProd {
  const BucketPlan* plan;
  const unsigned short* A;
  const unsigned short* B;
  unsigned short* C;
};
hipError_t launch_sym(const SymProd* p, int n, int tile_choice, hipStream_t s);
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
hipError_t launch_adamw_multi(const AdamWSegTable& t, hipStream_t s);

}  // namespace ma
