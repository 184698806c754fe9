// Newton-Schulz matrix products on the gfx950 matrix cores (bf16 in, fp32 accumulate).
//
// One iteration of the quintic ("Optimizers: AdamW, Muon and the distributed
// optimizer", section "Muon: orthogonalising the update", newton_schulz listing) on
// an m x n bf16 matrix X (m <= n):
//
//   gram:     R  = X X^T               m x m, symmetric
//   poly:     P  = b R + c R R^T       m x m, symmetric (R R^T = R^2 as R = R^T)
//   combine:  X' = a X + P X           m x n
//
// Every product is C = A B^T with both operands stored row-major along the
// contraction index, which is what the MFMA operand layout wants:
//   gram     A = B = X  (contraction over n)
//   poly     A = B = R  (contraction over m)
//   combine  A = P, B = X^T (the library keeps X in both orientations; contraction m)
// Symmetric outputs are computed on lower-triangle tiles only and mirrored, halving
// the work of the two symmetric products ("DMuon: Efficient Distributed Muon Training
// with Near-Adam Overhead", section 2.2, symmetry exploitation); same-shape matrices
// are batched in one launch (same section, batching).
//
// Tiling: 128 x 128 output tile per 256-thread block (2 x 2 waves of 64 x 64), k-steps
// of 64, operands staged through LDS (double-buffered, XOR-swizzled 16-byte chunks so
// the 32 rows an MFMA fragment reads hit distinct banks), v_mfma_f32_32x32x16_bf16.
// All sizes are padded to the tile by the caller (zero padding is preserved by the
// iteration), so there are no bounds checks inside.
#include "ma_internal.h"

namespace ma {
namespace {

constexpr int BM = kTile;  // 128
constexpr int BN = kTile;
constexpr int BK = 64;
constexpr int kThreads = 256;
constexpr int WTM = 2;     // 32x32 MFMA tiles per wave along M
constexpr int WTN = 2;     // along N
constexpr int kChunksPerRow = BK / 8;  // 16-byte chunks per LDS row
constexpr int kLoadIters = (BM * kChunksPerRow) / kThreads;  // 4
constexpr int kTPad = 8;   // epilogue transpose tile padding (bf16 elements)

enum Epi { kGram = 0, kPoly = 1, kCombine = 2 };

struct GemmArgs {
  const unsigned short* A;
  const unsigned short* B;
  int64_t lda, ldb, strideA, strideB;
  int kdim;
  unsigned short* C;    // row-major target
  unsigned short* C2;   // transposed target (combine) or mirror target (gram/poly)
  int64_t ldc, ldc2, strideC, strideC2;
  const unsigned short* aux;  // poly: R; combine: X
  int64_t ldaux, strideAux;
  float alpha, beta;    // poly: b, c; combine: a, 1
  int tiles_m, tiles_n; // tile grid (triangular for gram/poly)
  int tiles_per_batch;
};

__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ (row & 7); }

template <int kEpi>
__global__ __launch_bounds__(kThreads, 2) void ns_gemm_kernel(GemmArgs args) {
  __shared__ __attribute__((aligned(16))) unsigned short smem[2 * 2 * BM * BK];
  unsigned short* As = smem;                 // [2][BM][BK]
  unsigned short* Bs = smem + 2 * BM * BK;   // [2][BN][BK]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1;
  const int wn = wave & 1;

  const int64_t batch = blockIdx.x / args.tiles_per_batch;
  const int tile = blockIdx.x - static_cast<int>(batch) * args.tiles_per_batch;
  int ti, tj;
  if (kEpi == kCombine) {
    ti = tile / args.tiles_n;
    tj = tile - ti * args.tiles_n;
  } else {
    // lower-triangle enumeration: tile = ti (ti + 1) / 2 + tj, tj <= ti
    ti = static_cast<int>((__builtin_sqrtf(8.0f * tile + 1.0f) - 1.0f) * 0.5f);
    while ((ti + 1) * (ti + 2) / 2 <= tile) ++ti;
    while (ti * (ti + 1) / 2 > tile) --ti;
    tj = tile - ti * (ti + 1) / 2;
  }
  const int64_t m0 = static_cast<int64_t>(ti) * BM;
  const int64_t n0 = static_cast<int64_t>(tj) * BN;

  const unsigned short* gA = args.A + batch * args.strideA + m0 * args.lda;
  const unsigned short* gB = args.B + batch * args.strideB + n0 * args.ldb;

  // global -> register prefetch mapping: thread covers rows (tid>>3)+32*i, chunk tid&7
  const int lrow = tid >> 3;
  const int lch = tid & 7;
  u32x4 ra[kLoadIters], rb[kLoadIters];

  auto load_global = [&](int kt) {
#pragma unroll
    for (int i = 0; i < kLoadIters; ++i) {
      const int r = lrow + 32 * i;
      ra[i] = *reinterpret_cast<const u32x4*>(gA + r * args.lda + kt * BK + lch * 8);
      rb[i] = *reinterpret_cast<const u32x4*>(gB + r * args.ldb + kt * BK + lch * 8);
    }
  };
  auto store_lds = [&](int buf) {
    unsigned short* as = As + buf * BM * BK;
    unsigned short* bs = Bs + buf * BN * BK;
#pragma unroll
    for (int i = 0; i < kLoadIters; ++i) {
      const int r = lrow + 32 * i;
      *reinterpret_cast<u32x4*>(as + r * BK + swz(r, lch) * 8) = ra[i];
      *reinterpret_cast<u32x4*>(bs + r * BK + swz(r, lch) * 8) = rb[i];
    }
  };

  f32x16 acc[WTM][WTN];
#pragma unroll
  for (int i = 0; i < WTM; ++i)
#pragma unroll
    for (int j = 0; j < WTN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int nk = args.kdim / BK;
  load_global(0);
  store_lds(0);
  __syncthreads();

  const int frow = lane & 31;   // fragment row (A) / column (B)
  const int fkh = lane >> 5;    // which 8-wide half of the 16-wide k slice

  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load_global(kt + 1);
    const unsigned short* as = As + buf * BM * BK;
    const unsigned short* bs = Bs + buf * BN * BK;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      bf16x8 af[WTM], bfr[WTN];
      const int ch = kk * 2 + fkh;
#pragma unroll
      for (int i = 0; i < WTM; ++i) {
        const int r = wm * (WTM * 32) + i * 32 + frow;
        af[i] = *reinterpret_cast<const bf16x8*>(as + r * BK + swz(r, ch) * 8);
      }
#pragma unroll
      for (int j = 0; j < WTN; ++j) {
        const int r = wn * (WTN * 32) + j * 32 + frow;
        bfr[j] = *reinterpret_cast<const bf16x8*>(bs + r * BK + swz(r, ch) * 8);
      }
#pragma unroll
      for (int i = 0; i < WTM; ++i)
#pragma unroll
        for (int j = 0; j < WTN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) store_lds(buf ^ 1);
    __syncthreads();
  }

  // ---------------- epilogue ----------------
  // MFMA 32x32 accumulator layout: lane holds column (lane & 31) of the tile and rows
  // 8*(r/4) + 4*(lane/32) + r%4 for r = 0..15.
  const bool mirror = (kEpi != kCombine) && (ti != tj);
  const bool need_t = (kEpi == kCombine) || mirror;
  unsigned short* Ts = smem;  // [BN][BM + kTPad], reused after the main loop
  unsigned short* C = args.C + batch * args.strideC;
  const unsigned short* aux =
      (kEpi == kGram) ? nullptr : args.aux + batch * args.strideAux;

#pragma unroll
  for (int i = 0; i < WTM; ++i) {
#pragma unroll
    for (int j = 0; j < WTN; ++j) {
      const int jl = wn * (WTN * 32) + j * 32 + (lane & 31);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        unsigned short h[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = q * 4 + e;
          const int il = wm * (WTM * 32) + i * 32 + 8 * q + 4 * fkh + e;
          float v = acc[i][j][r];
          const int64_t gi = m0 + il;
          const int64_t gj = n0 + jl;
          if (kEpi == kPoly) {
            v = args.alpha * bf2f(aux[gi * args.ldaux + gj]) + args.beta * v;
          } else if (kEpi == kCombine) {
            v = args.alpha * bf2f(aux[gi * args.ldaux + gj]) + v;
          }
          h[e] = f2bf(v);
          C[gi * args.ldc + gj] = h[e];
        }
        if (need_t) {
          const int il0 = wm * (WTM * 32) + i * 32 + 8 * q + 4 * fkh;
          u32x2 packed;
          packed[0] = static_cast<unsigned>(h[0]) | (static_cast<unsigned>(h[1]) << 16);
          packed[1] = static_cast<unsigned>(h[2]) | (static_cast<unsigned>(h[3]) << 16);
          // Ts is written only after every wave has left the main loop (the loop ends
          // with a barrier), so reusing the operand buffers is safe.
          *reinterpret_cast<u32x2*>(Ts + jl * (BM + kTPad) + il0) = packed;
        }
      }
    }
  }
  if (!need_t) return;
  __syncthreads();
  unsigned short* C2 = args.C2 + batch * args.strideC2;
  constexpr int kChunks = BN * (BM / 8);  // 16-byte chunks in the transposed tile
#pragma unroll
  for (int it = 0; it < kChunks / kThreads; ++it) {
    const int idx = tid + it * kThreads;
    const int row = idx / (BM / 8);  // local column j of the product
    const int ch = idx - row * (BM / 8);
    const u32x4 v = *reinterpret_cast<const u32x4*>(Ts + row * (BM + kTPad) + ch * 8);
    *reinterpret_cast<u32x4*>(C2 + (n0 + row) * args.ldc2 + m0 + ch * 8) = v;
  }
}

static_assert(2 * 2 * BM * BK >= BN * (BM + kTPad), "epilogue tile must fit the operand buffers");
static_assert(((BM + kTPad) * 2) % 16 == 0, "transpose tile rows must stay 16-byte aligned");

hipError_t launch(int epi, const GemmArgs& a, int64_t K, hipStream_t s) {
  const int64_t blocks = K * a.tiles_per_batch;
  if (blocks <= 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(blocks));
  switch (epi) {
    case kGram: hipLaunchKernelGGL((ns_gemm_kernel<kGram>), grid, dim3(kThreads), 0, s, a); break;
    case kPoly: hipLaunchKernelGGL((ns_gemm_kernel<kPoly>), grid, dim3(kThreads), 0, s, a); break;
    default: hipLaunchKernelGGL((ns_gemm_kernel<kCombine>), grid, dim3(kThreads), 0, s, a); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gram(const BucketPlan& p, const unsigned short* X, unsigned short* R,
                       hipStream_t s) {
  GemmArgs a{};
  const int T = static_cast<int>(p.m_pad / BM);
  a.A = X; a.B = X;
  a.lda = a.ldb = p.n_pad;
  a.strideA = a.strideB = p.m_pad * p.n_pad;
  a.kdim = static_cast<int>(p.n_pad);
  a.C = R; a.C2 = R;
  a.ldc = a.ldc2 = p.m_pad;
  a.strideC = a.strideC2 = p.m_pad * p.m_pad;
  a.tiles_m = a.tiles_n = T;
  a.tiles_per_batch = T * (T + 1) / 2;
  return launch(kGram, a, p.K, s);
}

hipError_t launch_poly(const BucketPlan& p, const unsigned short* R, unsigned short* P,
                       float b, float c, hipStream_t s) {
  GemmArgs a{};
  const int T = static_cast<int>(p.m_pad / BM);
  a.A = R; a.B = R;
  a.lda = a.ldb = p.m_pad;
  a.strideA = a.strideB = p.m_pad * p.m_pad;
  a.kdim = static_cast<int>(p.m_pad);
  a.C = P; a.C2 = P;
  a.ldc = a.ldc2 = p.m_pad;
  a.strideC = a.strideC2 = p.m_pad * p.m_pad;
  a.aux = R;
  a.ldaux = p.m_pad;
  a.strideAux = p.m_pad * p.m_pad;
  a.alpha = b; a.beta = c;
  a.tiles_m = a.tiles_n = T;
  a.tiles_per_batch = T * (T + 1) / 2;
  return launch(kPoly, a, p.K, s);
}

hipError_t launch_combine(const BucketPlan& p, const unsigned short* P,
                          const unsigned short* X, const unsigned short* XT, float alpha,
                          unsigned short* Xn, unsigned short* XTn, hipStream_t s) {
  GemmArgs a{};
  a.A = P; a.B = XT;
  a.lda = p.m_pad; a.ldb = p.m_pad;
  a.strideA = p.m_pad * p.m_pad;
  a.strideB = p.m_pad * p.n_pad;
  a.kdim = static_cast<int>(p.m_pad);
  a.C = Xn; a.C2 = XTn;
  a.ldc = p.n_pad; a.ldc2 = p.m_pad;
  a.strideC = a.strideC2 = p.m_pad * p.n_pad;
  a.aux = X;
  a.ldaux = p.n_pad;
  a.strideAux = p.m_pad * p.n_pad;
  a.alpha = alpha; a.beta = 1.0f;
  a.tiles_m = static_cast<int>(p.m_pad / BM);
  a.tiles_n = static_cast<int>(p.n_pad / BN);
  a.tiles_per_batch = a.tiles_m * a.tiles_n;
  return launch(kCombine, a, p.K, s);
}

}  // namespace ma
