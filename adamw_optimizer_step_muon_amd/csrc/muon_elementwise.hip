// Memory-bound stages of the Muon step around the Newton-Schulz iteration.
//
// "Optimizers: AdamW, Muon and the distributed optimizer", section "Muon:
// orthogonalising the update" (update steps 1-3 and the newton_schulz listing):
//   prep:      one pass per 64 x 64 tile: M <- mu M + G, U = G + mu M (Nesterov, new M)
//              or M; U in bf16 in the Gram-side orientation X (transposed when A > B,
//              through an LDS tile), and in the matrix's own orientation too when no
//              iteration runs; per-tile sums of U^2.  U is cast before it is normalised: the normalisation is a
//              scalar per matrix, applied by the first Newton-Schulz products
//              (R = inv^2 U U^T, X1 = inv (a U + P U)), which is X0 = inv U up to the
//              order of rounding, and saves a second pass over G and M.
//   finalize:  inv = 1 / (||U||_F + eps), one value per matrix, fixed summation order;
//              the tile sums are float64, so ||U|| is exact to rounding for any finite
//              fp32 U.  A matrix whose norm lies outside [2^-32, 2^32] has its bf16 copy
//              multiplied by 2^-e (e = the exponent of its norm: exact, a power of two)
//              and inv by 2^e, so the first Gram product accumulates values of order one
//              in fp32 (unscaled, its sums would overflow above ~1e19 or lose their
//              small terms below ~1e-19); inside the range nothing is rescaled.
//   apply:     P <- P - lr wd [mask] P - lr s O   ("dtensor-muon", "Features": the
//              cautious mask keeps the decay only where update and weight share a sign)
//
// Reductions are deterministic: every partial sum has a fixed owner and a fixed
// order, so a matrix's result does not depend on which bucket it is in.
#include <algorithm>

#include "ma_internal.h"

namespace ma {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ double wave_sum_d(double x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

__device__ __forceinline__ float nesterov_input(float g, float m_new, float mu, int nesterov) {
  return nesterov ? g + mu * m_new : m_new;
}

// grid (Bp/64, Ap/64, K).  Source A x B; S is the same orientation padded to Ap x Bp
// (row stride Bp), T the transpose padded to Bp x Ap (row stride Ap); zero padding.
// Either may be null (only the Gram-side orientation X is needed by the iteration).
// partials[k * tiles + tile] = sum of U^2 over the tile (fixed order).
template <bool kVec, bool kHasM>
__global__ __launch_bounds__(kThreads) void muon_prep_kernel(
    const float* __restrict__ G, float* __restrict__ M, float mu, int nesterov, int64_t A,
    int64_t B, int64_t Ap, int64_t Bp, unsigned short* __restrict__ S,
    unsigned short* __restrict__ T, double* __restrict__ partials) {
  constexpr int kT = kCastTile;
  __shared__ unsigned short tile[kT][kT + 4];
  __shared__ double red[kThreads / 64];
  const int64_t k = blockIdx.z;
  const int64_t a0 = static_cast<int64_t>(blockIdx.y) * kT;
  const int64_t b0 = static_cast<int64_t>(blockIdx.x) * kT;
  const float* g = G + k * A * B;
  float* mm = kHasM ? M + k * A * B : nullptr;
  unsigned short* s = S ? S + k * Ap * Bp : nullptr;
  unsigned short* t = T ? T + k * Ap * Bp : nullptr;
  const int c4 = (threadIdx.x & 15) * 4;
  double ss = 0.0;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = (threadIdx.x >> 4) + 16 * r;
    const int64_t a = a0 + row;
    const int64_t b = b0 + c4;
    float u[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (a < A) {
      if (kVec && b + 3 < B) {
        const f32x4 gv = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(g + a * B + b));
        if (kHasM) {
          f32x4* mp = reinterpret_cast<f32x4*>(mm + a * B + b);
          f32x4 mv = __builtin_nontemporal_load(mp);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            mv[e] = mu * mv[e] + gv[e];
            u[e] = nesterov_input(gv[e], mv[e], mu, nesterov);
          }
          __builtin_nontemporal_store(mv, mp);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) u[e] = gv[e];
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (b + e < B) {
            const float gv = g[a * B + b + e];
            if (kHasM) {
              const float mv = mu * mm[a * B + b + e] + gv;
              mm[a * B + b + e] = mv;
              u[e] = nesterov_input(gv, mv, mu, nesterov);
            } else {
              u[e] = gv;
            }
          }
        }
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) ss = __builtin_fma(static_cast<double>(u[e]), static_cast<double>(u[e]), ss);
    unsigned short h[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      h[e] = f2bf(u[e]);
      tile[row][c4 + e] = h[e];
    }
    u32x2 packed;
    packed[0] = static_cast<unsigned>(h[0]) | (static_cast<unsigned>(h[1]) << 16);
    packed[1] = static_cast<unsigned>(h[2]) | (static_cast<unsigned>(h[3]) << 16);
    if (s) *reinterpret_cast<u32x2*>(s + a * Bp + b) = packed;
  }
  ss = wave_sum_d(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  if (threadIdx.x == 0) {
    double tot = 0.0;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) tot += red[w];
    partials[k * gridDim.x * gridDim.y + blockIdx.y * gridDim.x + blockIdx.x] = tot;
  }
  if (!t) return;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int trow = (threadIdx.x >> 4) + 16 * r;  // local b
    u32x2 packed;
    packed[0] = static_cast<unsigned>(tile[c4 + 0][trow]) |
                (static_cast<unsigned>(tile[c4 + 1][trow]) << 16);
    packed[1] = static_cast<unsigned>(tile[c4 + 2][trow]) |
                (static_cast<unsigned>(tile[c4 + 3][trow]) << 16);
    *reinterpret_cast<u32x2*>(t + (b0 + trow) * Ap + a0 + c4) = packed;
  }
}

// grid (K); inv[k] = 1 / (sqrt(sum of matrix k's partials) + eps) and shift[k] = 0, or,
// for a finite nonzero norm outside [2^-32, 2^32] with exponent e (norm = f 2^e,
// 1 <= f < 2), inv[k] = 2^e / (norm + eps) and shift[k] = -e
__global__ __launch_bounds__(kThreads) void norm_finalize_kernel(
    const double* __restrict__ partials, int64_t nblk, float eps, float* __restrict__ inv,
    int* __restrict__ shift, float* __restrict__ x0norm) {
  const int64_t k = blockIdx.x;
  double acc = 0.0;
  for (int64_t i = threadIdx.x; i < nblk; i += kThreads) acc += partials[k * nblk + i];
  __shared__ double red[kThreads / 64];
  acc = wave_sum_d(acc);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    double t = 0.0;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) t += red[w];
    const double norm = __builtin_sqrt(t);
    double iv = 1.0 / (norm + static_cast<double>(eps));
    int sh = 0;
    if ((norm > 0.0 && norm < 0x1p-32) || (norm > 0x1p32 && norm <= 1.7976931348623157e308)) {
      // exponent of a normal double (every nonzero norm of fp32 values is one)
      const int e = static_cast<int>((__builtin_bit_cast(unsigned long long, norm) >> 52) & 0x7ff) - 1023;
      iv = __builtin_ldexp(iv, e);
      sh = -e;
    }
    inv[k] = static_cast<float>(iv);
    shift[k] = sh;
    // ||X0|| = ||U|| / (||U|| + eps): 1 up to eps / ||U||, smaller only for norms near eps
    if (x0norm) x0norm[k] = static_cast<float>(norm / (norm + static_cast<double>(eps)));
  }
}

// grid (nb, K): the `per` bf16 values of matrix k in X and in Y (either may be null) are
// multiplied by 2^shift[k] where shift[k] != 0 (exact, up to values that leave the
// normal range); per % 8 == 0
__global__ __launch_bounds__(kThreads) void rescale_kernel(unsigned short* __restrict__ X,
                                                           unsigned short* __restrict__ Y,
                                                           int64_t per, const int* __restrict__ shift) {
  const int64_t k = blockIdx.y;
  const int sh = shift[k];
  if (sh == 0) return;
  for (int b = 0; b < 2; ++b) {
    unsigned short* base = b == 0 ? X : Y;
    if (!base) continue;
    u32x4* q = reinterpret_cast<u32x4*>(base + k * per);
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; i < per / 8;
         i += static_cast<int64_t>(gridDim.x) * kThreads) {
      u32x4 v = q[i];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const unsigned lo = f2bf(__builtin_ldexpf(bf2f(static_cast<unsigned short>(v[e] & 0xffffu)), sh));
        const unsigned hi = f2bf(__builtin_ldexpf(bf2f(static_cast<unsigned short>(v[e] >> 16)), sh));
        v[e] = lo | (hi << 16);
      }
      q[i] = v;
    }
  }
}

// grid (nb, K): the `per` bf16 values of matrix k in X and in Y (either may be null) are
// replaced in place by fp16(value * inv[k] * sx_k): the normalised X0 of the Gram-space
// route times sx_k = sx * 2^-e, a power of two that puts its entries in fp16's range.
// e <= 0 is the exponent of ||X0|| (x0norm[k]) when that norm is below 1/2, which
// happens only when ||U|| is near eps; then X0 itself is small and its fp16 copy would
// otherwise lose its digits or flush to zero.  Block (0, k) also writes the factors the
// route's products apply: gsc[k] = 2^7 / sx_k (the Gram: R * 2^14 = (X0 sx_k)(X0 sx_k)^T
// gsc^2) and gsc[K + k] = 1 / sx_k (the last product: X = Q (X0 sx_k) / sx_k).
// per % 8 == 0
__global__ __launch_bounds__(kThreads) void to_f16_kernel(unsigned short* __restrict__ X,
                                                          unsigned short* __restrict__ Y,
                                                          int64_t per, const float* __restrict__ inv,
                                                          const float* __restrict__ x0norm,
                                                          float sx, float* __restrict__ gsc) {
  const int64_t k = blockIdx.y;
  float xn = x0norm[k], sxk = sx;
  for (int e = 0; xn > 0.0f && xn < 0.5f && e < 100; ++e) {
    xn *= 2.0f;
    sxk *= 2.0f;
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    gsc[k] = 128.0f / sxk;
    gsc[gridDim.y + k] = 1.0f / sxk;
  }
  const float f = inv[k] * sxk;
  for (int b = 0; b < 2; ++b) {
    unsigned short* base = b == 0 ? X : Y;
    if (!base) continue;
    u32x4* q = reinterpret_cast<u32x4*>(base + k * per);
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; i < per / 8;
         i += static_cast<int64_t>(gridDim.x) * kThreads) {
      u32x4 v = q[i];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const unsigned lo = f2h(bf2f(static_cast<unsigned short>(v[e] & 0xffffu)) * f);
        const unsigned hi = f2h(bf2f(static_cast<unsigned short>(v[e] >> 16)) * f);
        v[e] = lo | (hi << 16);
      }
      q[i] = v;
    }
  }
}

// Elementwise over (K, A, B), 4 consecutive columns per thread when B % 4 == 0.
// O (bf16) holds the orthogonalised matrix in the parameter's orientation with row
// stride ldo and per-matrix slab `slab`.
template <bool kVec, bool kExtract>
__global__ __launch_bounds__(kThreads) void muon_apply_kernel(
    float* __restrict__ P, const unsigned short* __restrict__ O, const float* __restrict__ oscale,
    int64_t A, int64_t B, int64_t ldo, int64_t slab, int64_t total, float lr_wd, float lr_scale,
    int cautious) {
  const int64_t e0 = (static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x) * (kVec ? 4 : 1);
  if (e0 >= total) return;
  const int64_t AB = A * B;
  const int64_t k = e0 / AB;
  const int64_t rem = e0 - k * AB;
  const int64_t a = rem / B;
  const int64_t b = rem - a * B;
  const unsigned short* o = O + k * slab + a * ldo + b;
  const float osc = oscale ? oscale[k] : 1.0f;
  if (kVec) {
    // single-use streams (O, the parameters) go through with non-temporal accesses
    const u32x2 ov = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(o));
    float of[4] = {osc * bf2f(ov[0] & 0xffffu), osc * bf2f(ov[0] >> 16),
                   osc * bf2f(ov[1] & 0xffffu), osc * bf2f(ov[1] >> 16)};
    f32x4* p4 = reinterpret_cast<f32x4*>(P + e0);
    f32x4 pv;
    if (!kExtract) pv = __builtin_nontemporal_load(p4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (kExtract) {
        pv[e] = of[e];
      } else {
        const float d = (cautious && !(of[e] * pv[e] > 0.0f)) ? 0.0f : lr_wd;
        pv[e] = pv[e] - d * pv[e] - lr_scale * of[e];
      }
    }
    __builtin_nontemporal_store(pv, p4);
  } else {
    const float of = osc * bf2f(*o);
    if (kExtract) {
      P[e0] = of;
    } else {
      const float pv = P[e0];
      const float d = (cautious && !(of * pv > 0.0f)) ? 0.0f : lr_wd;
      P[e0] = pv - d * pv - lr_scale * of;
    }
  }
}

bool aligned16(const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15u) == 0; }

}  // namespace

hipError_t launch_muon_prep(const BucketPlan& p, const float* G, float* M, float mu,
                            int nesterov, double* partials, unsigned short* S,
                            unsigned short* T, hipStream_t s) {
  if (LaunchRecorder* r = launch_recorder()) {
    r->prep(p, G, M, partials, S, T);
    return hipSuccess;
  }
  const int64_t Ap = p.transposed ? p.n_pad : p.m_pad;
  const int64_t Bp = p.transposed ? p.m_pad : p.n_pad;
  const bool vec = (p.B % 4 == 0) && aligned16(G) && (!M || aligned16(M));
  const dim3 grid(static_cast<unsigned>(Bp / kCastTile), static_cast<unsigned>(Ap / kCastTile),
                  static_cast<unsigned>(p.K));
  if (M) {
    if (vec)
      hipLaunchKernelGGL((muon_prep_kernel<true, true>), grid, dim3(kThreads), 0, s, G, M, mu,
                         nesterov, p.A, p.B, Ap, Bp, S, T, partials);
    else
      hipLaunchKernelGGL((muon_prep_kernel<false, true>), grid, dim3(kThreads), 0, s, G, M, mu,
                         nesterov, p.A, p.B, Ap, Bp, S, T, partials);
  } else {
    if (vec)
      hipLaunchKernelGGL((muon_prep_kernel<true, false>), grid, dim3(kThreads), 0, s, G, M, mu,
                         nesterov, p.A, p.B, Ap, Bp, S, T, partials);
    else
      hipLaunchKernelGGL((muon_prep_kernel<false, false>), grid, dim3(kThreads), 0, s, G, M, mu,
                         nesterov, p.A, p.B, Ap, Bp, S, T, partials);
  }
  return hipGetLastError();
}

hipError_t launch_norm_finalize(const BucketPlan& p, const double* partials, float eps,
                                float* inv, int* shift, hipStream_t s, float* x0norm) {
  if (LaunchRecorder* r = launch_recorder()) {
    r->norm(p, partials, inv, shift, x0norm);
    return hipSuccess;
  }
  hipLaunchKernelGGL(norm_finalize_kernel, dim3(static_cast<unsigned>(p.K)), dim3(kThreads), 0,
                     s, partials, p.nblk, eps, inv, shift, x0norm);
  return hipGetLastError();
}

hipError_t launch_to_f16(const BucketPlan& p, unsigned short* S, unsigned short* T,
                         const float* inv, const float* x0norm, float sx, float* gsc,
                         hipStream_t s) {
  if (LaunchRecorder* r = launch_recorder()) {
    r->to_f16(p, S, T, inv, x0norm, gsc);
    return hipSuccess;
  }
  // streams both copies once: enough blocks per matrix to fill the chip
  const int64_t per = p.m_pad * p.n_pad;
  const int64_t want = std::max<int64_t>(1, 2048 / std::max<int64_t>(p.K, 1));
  const int64_t nb = std::max<int64_t>(1, std::min<int64_t>(want, (per / 8 + kThreads - 1) / kThreads));
  hipLaunchKernelGGL(to_f16_kernel, dim3(static_cast<unsigned>(nb), static_cast<unsigned>(p.K)),
                     dim3(kThreads), 0, s, S, T, per, inv, x0norm, sx, gsc);
  return hipGetLastError();
}

hipError_t launch_rescale(const BucketPlan& p, unsigned short* S, unsigned short* T,
                          const int* shift, hipStream_t s) {
  if (LaunchRecorder* r = launch_recorder()) {
    r->rescale(p, S, T, shift);
    return hipSuccess;
  }
  // a few blocks per matrix: in-range matrices (the usual case) return at once
  const int64_t per = p.m_pad * p.n_pad;
  const int64_t nb = std::min<int64_t>(64, (per / 8 + kThreads - 1) / kThreads);
  hipLaunchKernelGGL(rescale_kernel, dim3(static_cast<unsigned>(nb), static_cast<unsigned>(p.K)),
                     dim3(kThreads), 0, s, S, T, per, shift);
  return hipGetLastError();
}

namespace {
hipError_t launch_apply_impl(const BucketPlan& p, float* param, const unsigned short* O,
                             const float* oscale, int64_t ldo, float lr_wd, float lr_scale,
                             int cautious, bool extract, hipStream_t s) {
  const int64_t total = p.K * p.A * p.B;
  if (total == 0) return hipSuccess;
  if (LaunchRecorder* r = launch_recorder()) {
    r->apply(p, param, O, oscale, ldo);
    return hipSuccess;
  }
  const int64_t slab = p.m_pad * p.n_pad;
  const bool vec = (p.B % 4 == 0) && aligned16(param) && (ldo % 4 == 0);
  const int64_t per_thread = vec ? 4 : 1;
  const int64_t threads = (total + per_thread - 1) / per_thread;
  const dim3 grid(static_cast<unsigned>((threads + kThreads - 1) / kThreads));
  if (vec) {
    if (extract)
      hipLaunchKernelGGL((muon_apply_kernel<true, true>), grid, dim3(kThreads), 0, s, param, O,
                         oscale, p.A, p.B, ldo, slab, total, lr_wd, lr_scale, cautious);
    else
      hipLaunchKernelGGL((muon_apply_kernel<true, false>), grid, dim3(kThreads), 0, s, param, O,
                         oscale, p.A, p.B, ldo, slab, total, lr_wd, lr_scale, cautious);
  } else {
    if (extract)
      hipLaunchKernelGGL((muon_apply_kernel<false, true>), grid, dim3(kThreads), 0, s, param, O,
                         oscale, p.A, p.B, ldo, slab, total, lr_wd, lr_scale, cautious);
    else
      hipLaunchKernelGGL((muon_apply_kernel<false, false>), grid, dim3(kThreads), 0, s, param, O,
                         oscale, p.A, p.B, ldo, slab, total, lr_wd, lr_scale, cautious);
  }
  return hipGetLastError();
}
}  // namespace

hipError_t launch_muon_apply(const BucketPlan& p, float* param, const unsigned short* O,
                             const float* oscale, int64_t ldo, float lr, float wd, float scale,
                             int cautious, hipStream_t s) {
  return launch_apply_impl(p, param, O, oscale, ldo, lr * wd, lr * scale, cautious, false, s);
}

hipError_t launch_ns_extract(const BucketPlan& p, float* out, const unsigned short* O,
                             const float* oscale, int64_t ldo, hipStream_t s) {
  return launch_apply_impl(p, out, O, oscale, ldo, 0.0f, 0.0f, 0, true, s);
}

}  // namespace ma
