// Memory-bound stages of the Muon step around the Newton-Schulz iteration.
//
// "Optimizers: AdamW, Muon and the distributed optimizer", section "Muon:
// orthogonalising the update" (update steps 1-3 and the newton_schulz listing):
//   prep:      M <- mu M + G, U = G + mu M (Nesterov, new M) or M; per-block sums of U^2
//   finalize:  inv = 1 / (||U||_F + eps), one value per matrix, fixed summation order
//   cast:      X0 = U * inv in bf16, written in the matrix's own orientation and
//              transposed (the Gram side is the short side: transposed when A > B)
//   apply:     P <- P - lr wd [mask] P - lr s O   ("dtensor-muon", "Features": the
//              cautious mask keeps the decay only where update and weight share a sign)
//
// Reductions are deterministic: every partial sum has a fixed owner and a fixed
// order, so a matrix's result does not depend on which bucket it is in.
#include "ma_internal.h"

namespace ma {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

__device__ __forceinline__ double wave_sum_d(double x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

__device__ __forceinline__ float nesterov_input(float g, float m_new, float mu, int nesterov) {
  return nesterov ? g + mu * m_new : m_new;
}

// grid (nblk, K); block b of matrix k covers elements [b*chunk, min((b+1)*chunk, AB))
template <bool kVec, bool kHasM>
__global__ __launch_bounds__(kThreads) void muon_prep_kernel(
    const float* __restrict__ G, float* __restrict__ M, float mu, int nesterov, int64_t AB,
    int64_t chunk, int64_t nblk, float* __restrict__ partials) {
  const int64_t k = blockIdx.y;
  const int64_t lo = static_cast<int64_t>(blockIdx.x) * chunk;
  const int64_t hi = lo + chunk < AB ? lo + chunk : AB;
  const float* g = G + k * AB;
  float* mm = kHasM ? M + k * AB : nullptr;
  float ss = 0.0f;
  if (kVec) {
    const f32x4* g4 = reinterpret_cast<const f32x4*>(g);
    f32x4* m4 = reinterpret_cast<f32x4*>(mm);
    for (int64_t i = lo / 4 + threadIdx.x; i < hi / 4; i += kThreads) {
      const f32x4 gv = __builtin_nontemporal_load(&g4[i]);
      f32x4 u;
      if (kHasM) {
        f32x4 mv = m4[i];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          mv[e] = mu * mv[e] + gv[e];
          u[e] = nesterov_input(gv[e], mv[e], mu, nesterov);
        }
        m4[i] = mv;
      } else {
        u = gv;
      }
      ss += u[0] * u[0] + u[1] * u[1] + u[2] * u[2] + u[3] * u[3];
    }
  } else {
    for (int64_t i = lo + threadIdx.x; i < hi; i += kThreads) {
      const float gv = g[i];
      float u = gv;
      if (kHasM) {
        const float mv = mu * mm[i] + gv;
        mm[i] = mv;
        u = nesterov_input(gv, mv, mu, nesterov);
      }
      ss += u * u;
    }
  }
  __shared__ float red[kThreads / 64];
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  if (threadIdx.x == 0) {
    float t = 0.0f;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) t += red[w];
    partials[k * nblk + blockIdx.x] = t;
  }
}

// grid (K); inv[k] = 1 / (sqrt(sum of matrix k's partials) + eps)
__global__ __launch_bounds__(kThreads) void norm_finalize_kernel(
    const float* __restrict__ partials, int64_t nblk, float eps, float* __restrict__ inv) {
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
    inv[k] = static_cast<float>(1.0 / (__builtin_sqrt(t) + static_cast<double>(eps)));
  }
}

// grid (Bp/64, Ap/64, K).  Source U is A x B; S is the same orientation padded to
// Ap x Bp (row stride Bp), T the transpose padded to Bp x Ap (row stride Ap).
template <bool kVec, bool kHasM>
__global__ __launch_bounds__(kThreads) void norm_cast_kernel(
    const float* __restrict__ G, const float* __restrict__ M, float mu, int nesterov,
    const float* __restrict__ inv, int64_t A, int64_t B, int64_t Ap, int64_t Bp,
    unsigned short* __restrict__ S, unsigned short* __restrict__ T) {
  constexpr int kT = kCastTile;
  __shared__ unsigned short tile[kT][kT + 4];
  const int64_t k = blockIdx.z;
  const int64_t a0 = static_cast<int64_t>(blockIdx.y) * kT;
  const int64_t b0 = static_cast<int64_t>(blockIdx.x) * kT;
  const float sc = inv[k];
  const float* g = G + k * A * B;
  const float* mm = kHasM ? M + k * A * B : nullptr;
  unsigned short* s = S + k * Ap * Bp;
  unsigned short* t = T + k * Ap * Bp;
  const int c4 = (threadIdx.x & 15) * 4;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = (threadIdx.x >> 4) + 16 * r;
    const int64_t a = a0 + row;
    const int64_t b = b0 + c4;
    float u[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (a < A) {
      if (kVec && b + 3 < B) {
        const f32x4 gv = *reinterpret_cast<const f32x4*>(g + a * B + b);
        f32x4 mv;
        if (kHasM) mv = *reinterpret_cast<const f32x4*>(mm + a * B + b);
#pragma unroll
        for (int e = 0; e < 4; ++e) u[e] = kHasM ? nesterov_input(gv[e], mv[e], mu, nesterov) : gv[e];
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (b + e < B) {
            const float gv = g[a * B + b + e];
            u[e] = kHasM ? nesterov_input(gv, mm[a * B + b + e], mu, nesterov) : gv;
          }
        }
      }
    }
    unsigned short h[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      h[e] = f2bf(u[e] * sc);
      tile[row][c4 + e] = h[e];
    }
    u32x2 packed;
    packed[0] = static_cast<unsigned>(h[0]) | (static_cast<unsigned>(h[1]) << 16);
    packed[1] = static_cast<unsigned>(h[2]) | (static_cast<unsigned>(h[3]) << 16);
    *reinterpret_cast<u32x2*>(s + a * Bp + b) = packed;
  }
  __syncthreads();
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

// Elementwise over (K, A, B), 4 consecutive columns per thread when B % 4 == 0.
// O (bf16) holds the orthogonalised matrix in the parameter's orientation with row
// stride ldo and per-matrix slab `slab`.
template <bool kVec, bool kExtract>
__global__ __launch_bounds__(kThreads) void muon_apply_kernel(
    float* __restrict__ P, const unsigned short* __restrict__ O, int64_t A, int64_t B,
    int64_t ldo, int64_t slab, int64_t total, float lr_wd, float lr_scale, int cautious) {
  const int64_t e0 = (static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x) * (kVec ? 4 : 1);
  if (e0 >= total) return;
  const int64_t AB = A * B;
  const int64_t k = e0 / AB;
  const int64_t rem = e0 - k * AB;
  const int64_t a = rem / B;
  const int64_t b = rem - a * B;
  const unsigned short* o = O + k * slab + a * ldo + b;
  if (kVec) {
    const u32x2 ov = *reinterpret_cast<const u32x2*>(o);
    float of[4] = {bf2f(ov[0] & 0xffffu), bf2f(ov[0] >> 16), bf2f(ov[1] & 0xffffu),
                   bf2f(ov[1] >> 16)};
    f32x4* p4 = reinterpret_cast<f32x4*>(P + e0);
    f32x4 pv;
    if (!kExtract) pv = *p4;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (kExtract) {
        pv[e] = of[e];
      } else {
        const float d = (cautious && !(of[e] * pv[e] > 0.0f)) ? 0.0f : lr_wd;
        pv[e] = pv[e] - d * pv[e] - lr_scale * of[e];
      }
    }
    *p4 = pv;
  } else {
    const float of = bf2f(*o);
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
                            int nesterov, float* partials, hipStream_t s) {
  const int64_t AB = p.A * p.B;
  const int64_t chunk = kPrepChunk;  // nblk = ceil(AB / kPrepChunk) blocks cover [0, AB)
  const bool vec = (AB % 4 == 0) && aligned16(G) && (!M || aligned16(M));
  const dim3 grid(static_cast<unsigned>(p.nblk), static_cast<unsigned>(p.K));
  if (M) {
    if (vec)
      hipLaunchKernelGGL((muon_prep_kernel<true, true>), grid, dim3(kThreads), 0, s, G, M, mu,
                         nesterov, AB, chunk, p.nblk, partials);
    else
      hipLaunchKernelGGL((muon_prep_kernel<false, true>), grid, dim3(kThreads), 0, s, G, M, mu,
                         nesterov, AB, chunk, p.nblk, partials);
  } else {
    if (vec)
      hipLaunchKernelGGL((muon_prep_kernel<true, false>), grid, dim3(kThreads), 0, s, G, M, mu,
                         nesterov, AB, chunk, p.nblk, partials);
    else
      hipLaunchKernelGGL((muon_prep_kernel<false, false>), grid, dim3(kThreads), 0, s, G, M, mu,
                         nesterov, AB, chunk, p.nblk, partials);
  }
  return hipGetLastError();
}

hipError_t launch_norm_finalize(const BucketPlan& p, const float* partials, float eps,
                                float* inv, hipStream_t s) {
  hipLaunchKernelGGL(norm_finalize_kernel, dim3(static_cast<unsigned>(p.K)), dim3(kThreads), 0,
                     s, partials, p.nblk, eps, inv);
  return hipGetLastError();
}

hipError_t launch_norm_cast(const BucketPlan& p, const float* G, const float* M, float mu,
                            int nesterov, const float* inv, unsigned short* S,
                            unsigned short* T, hipStream_t s) {
  const int64_t Ap = p.transposed ? p.n_pad : p.m_pad;
  const int64_t Bp = p.transposed ? p.m_pad : p.n_pad;
  const bool vec = (p.B % 4 == 0) && aligned16(G) && (!M || aligned16(M));
  const dim3 grid(static_cast<unsigned>(Bp / kCastTile), static_cast<unsigned>(Ap / kCastTile),
                  static_cast<unsigned>(p.K));
  if (M) {
    if (vec)
      hipLaunchKernelGGL((norm_cast_kernel<true, true>), grid, dim3(kThreads), 0, s, G, M, mu,
                         nesterov, inv, p.A, p.B, Ap, Bp, S, T);
    else
      hipLaunchKernelGGL((norm_cast_kernel<false, true>), grid, dim3(kThreads), 0, s, G, M, mu,
                         nesterov, inv, p.A, p.B, Ap, Bp, S, T);
  } else {
    if (vec)
      hipLaunchKernelGGL((norm_cast_kernel<true, false>), grid, dim3(kThreads), 0, s, G, M, mu,
                         nesterov, inv, p.A, p.B, Ap, Bp, S, T);
    else
      hipLaunchKernelGGL((norm_cast_kernel<false, false>), grid, dim3(kThreads), 0, s, G, M, mu,
                         nesterov, inv, p.A, p.B, Ap, Bp, S, T);
  }
  return hipGetLastError();
}

namespace {
hipError_t launch_apply_impl(const BucketPlan& p, float* param, const unsigned short* O,
                             int64_t ldo, float lr_wd, float lr_scale, int cautious,
                             bool extract, hipStream_t s) {
  const int64_t total = p.K * p.A * p.B;
  if (total == 0) return hipSuccess;
  const int64_t slab = p.m_pad * p.n_pad;
  const bool vec = (p.B % 4 == 0) && aligned16(param) && (ldo % 4 == 0);
  const int64_t per_thread = vec ? 4 : 1;
  const int64_t threads = (total + per_thread - 1) / per_thread;
  const dim3 grid(static_cast<unsigned>((threads + kThreads - 1) / kThreads));
  if (vec) {
    if (extract)
      hipLaunchKernelGGL((muon_apply_kernel<true, true>), grid, dim3(kThreads), 0, s, param, O,
                         p.A, p.B, ldo, slab, total, lr_wd, lr_scale, cautious);
    else
      hipLaunchKernelGGL((muon_apply_kernel<true, false>), grid, dim3(kThreads), 0, s, param, O,
                         p.A, p.B, ldo, slab, total, lr_wd, lr_scale, cautious);
  } else {
    if (extract)
      hipLaunchKernelGGL((muon_apply_kernel<false, true>), grid, dim3(kThreads), 0, s, param, O,
                         p.A, p.B, ldo, slab, total, lr_wd, lr_scale, cautious);
    else
      hipLaunchKernelGGL((muon_apply_kernel<false, false>), grid, dim3(kThreads), 0, s, param, O,
                         p.A, p.B, ldo, slab, total, lr_wd, lr_scale, cautious);
  }
  return hipGetLastError();
}
}  // namespace

hipError_t launch_muon_apply(const BucketPlan& p, float* param, const unsigned short* O,
                             int64_t ldo, float lr, float wd, float scale, int cautious,
                             hipStream_t s) {
  return launch_apply_impl(p, param, O, ldo, lr * wd, lr * scale, cautious, false, s);
}

hipError_t launch_ns_extract(const BucketPlan& p, float* out, const unsigned short* O,
                             int64_t ldo, hipStream_t s) {
  return launch_apply_impl(p, out, O, ldo, 0.0f, 0.0f, 0, true, s);
}

}  // namespace ma
