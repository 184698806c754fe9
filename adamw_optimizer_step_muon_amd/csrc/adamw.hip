// Fused elementwise AdamW step over one flat fp32 range.
//
// "Optimizers: AdamW, Muon and the distributed optimizer", section "AdamW: decoupled
// weight decay": moments m, v; update m / (sqrt(v) + eps) with the bias-corrected
// moments of torch's Adam/AdamW (the section's decay experiment runs those);
// decoupled decay w <- w - lr wd w, or L2 decay added to the gradient (coupled).
// "dtensor-muon", "Features": cautious decay, only where update and weight share
// a sign.
//
// One pass: 16 bytes read and 12 written per element (p, g, m, v in; p, m, v out),
// no other traffic.  Each thread moves kUnroll float4 groups with all loads issued
// before any arithmetic, so a wave keeps 4 x kUnroll x 1 KiB in flight.
#include "ma_internal.h"

namespace ma {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;

__device__ __forceinline__ void adamw_elem(float& p, float g, float& m, float& v,
                                           const AdamWConst& c) {
  if (!c.decoupled) g = g + c.wd * p;
  m = c.beta1 * m + c.one_m_beta1 * g;
  v = c.beta2 * v + c.one_m_beta2 * (g * g);
  const float mhat = m * c.inv_bc1;
  const float vhat = v * c.inv_bc2;
  const float upd = mhat / (__builtin_sqrtf(vhat) + c.eps);
  if (c.decoupled) {
    const float keep = 1.0f - c.lr * c.wd;
    p = p * ((c.cautious && !(upd * p > 0.0f)) ? 1.0f : keep);
  }
  p = p - c.lr * upd;
}

__global__ __launch_bounds__(kThreads) void adamw_vec_kernel(
    f32x4* __restrict__ p, const f32x4* __restrict__ g, f32x4* __restrict__ m,
    f32x4* __restrict__ v, int64_t n4, AdamWConst c) {
  const int64_t base = static_cast<int64_t>(blockIdx.x) * (kThreads * kUnroll) + threadIdx.x;
  f32x4 P[kUnroll], G[kUnroll], M[kUnroll], V[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const int64_t i = base + static_cast<int64_t>(u) * kThreads;
    if (i < n4) {
      P[u] = p[i];
      G[u] = __builtin_nontemporal_load(&g[i]);
      M[u] = m[i];
      V[u] = v[i];
    }
  }
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const int64_t i = base + static_cast<int64_t>(u) * kThreads;
    if (i < n4) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float pe = P[u][e], me = M[u][e], ve = V[u][e];
        adamw_elem(pe, G[u][e], me, ve, c);
        P[u][e] = pe;
        M[u][e] = me;
        V[u][e] = ve;
      }
      p[i] = P[u];
      m[i] = M[u];
      v[i] = V[u];
    }
  }
}

__global__ __launch_bounds__(kThreads) void adamw_scalar_kernel(
    float* __restrict__ p, const float* __restrict__ g, float* __restrict__ m,
    float* __restrict__ v, int64_t n, AdamWConst c) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (i >= n) return;
  float P = p[i], M = m[i], V = v[i];
  adamw_elem(P, g[i], M, V, c);
  p[i] = P;
  m[i] = M;
  v[i] = V;
}

bool aligned16(const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15u) == 0; }

}  // namespace

hipError_t launch_adamw(float* p, const float* g, float* m, float* v, int64_t n,
                        const AdamWConst& c, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  int64_t done = 0;
  if (aligned16(p) && aligned16(g) && aligned16(m) && aligned16(v)) {
    const int64_t n4 = n / 4;
    if (n4 > 0) {
      const int64_t per_block = static_cast<int64_t>(kThreads) * kUnroll;
      const int64_t blocks = (n4 + per_block - 1) / per_block;
      hipLaunchKernelGGL(adamw_vec_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads),
                         0, s, reinterpret_cast<f32x4*>(p), reinterpret_cast<const f32x4*>(g),
                         reinterpret_cast<f32x4*>(m), reinterpret_cast<f32x4*>(v), n4, c);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      done = n4 * 4;
    }
  }
  const int64_t rest = n - done;
  if (rest > 0) {
    const int64_t blocks = (rest + kThreads - 1) / kThreads;
    hipLaunchKernelGGL(adamw_scalar_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads),
                       0, s, p + done, g + done, m + done, v + done, rest, c);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace ma
