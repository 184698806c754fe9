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
#include <cstdlib>

#include "ma_internal.h"

namespace ma {
namespace {

constexpr int kThreads = 256;

// Decay variants, fixed per launch so the vector kernel's body has no branches.
enum DecayMode { kDecoupled = 0, kDecoupledCautious = 1, kCoupled = 2 };

// The multiply-adds are explicit (fmaf) and nothing else is contracted: every kernel
// (flat vector, flat scalar, multi-tensor) rounds the same operations, so an element's
// result does not depend on which kernel updated it (left to the compiler, p keep -
// lr upd was fused differently in different kernels).  g + wd p (coupled decay) keeps a
// single rounding, which matters where the two terms cancel.
template <int kMode>
__device__ __forceinline__ void adamw_elem_t(float& p, float g, float& m, float& v,
                                             const AdamWConst& c) {
#pragma clang fp contract(off)
  if (kMode == kCoupled) g = __builtin_fmaf(c.wd, p, g);
  m = __builtin_fmaf(c.beta1, m, c.one_m_beta1 * g);
  v = __builtin_fmaf(c.beta2, v, c.one_m_beta2 * (g * g));
  const float mhat = m * c.inv_bc1;
  const float vhat = v * c.inv_bc2;
  const float upd = mhat / (__builtin_sqrtf(vhat) + c.eps);
  if (kMode != kCoupled) {
    const float keep = 1.0f - c.lr * c.wd;
    p = p * ((kMode == kDecoupledCautious && !(upd * p > 0.0f)) ? 1.0f : keep);
  }
  p = __builtin_fmaf(-c.lr, upd, p);
}

__device__ __forceinline__ void adamw_elem(float& p, float g, float& m, float& v,
                                           const AdamWConst& c) {
  if (!c.decoupled) adamw_elem_t<kCoupled>(p, g, m, v, c);
  else if (c.cautious) adamw_elem_t<kDecoupledCautious>(p, g, m, v, c);
  else adamw_elem_t<kDecoupled>(p, g, m, v, c);
}

int decay_mode(const AdamWConst& c) {
  return !c.decoupled ? kCoupled : c.cautious ? kDecoupledCautious : kDecoupled;
}

// The streaming choice is a template parameter: selecting between a non-temporal and a
// plain access at run time lets the compiler merge the two into one plain access
// (the non-temporal hint is lost), which measured 8 % slower.
template <bool kNt, typename T>
__device__ __forceinline__ T ld(const T* q) {
  if constexpr (kNt) return __builtin_nontemporal_load(q);
  else return *q;
}
template <bool kNt, typename T>
__device__ __forceinline__ void st(T* q, T v) {
  if constexpr (kNt) __builtin_nontemporal_store(v, q);
  else *q = v;
}

// kU float4 groups per thread, all loads issued before any arithmetic; kNt: streaming
// (non-temporal) loads and stores for every array; kPersistent: a grid-stride loop
// over a grid sized to the chip instead of one block per kThreads * kU groups.
template <int kU, bool kNt, bool kPersistent, int kMode>
__global__ __launch_bounds__(kThreads) void adamw_vec_kernel(
    f32x4* __restrict__ p, const f32x4* __restrict__ g, f32x4* __restrict__ m,
    f32x4* __restrict__ v, int64_t n4, AdamWConst c) {
  const int64_t stride = kPersistent ? static_cast<int64_t>(gridDim.x) * (kThreads * kU) : 0;
  for (int64_t base = static_cast<int64_t>(blockIdx.x) * (kThreads * kU) + threadIdx.x;
       base < n4; base += stride) {
    f32x4 P[kU], G[kU], M[kU], V[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t i = base + static_cast<int64_t>(u) * kThreads;
      if (i < n4) {
        P[u] = ld<kNt>(&p[i]);
        G[u] = ld<true>(&g[i]);
        M[u] = ld<kNt>(&m[i]);
        V[u] = ld<kNt>(&v[i]);
      }
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t i = base + static_cast<int64_t>(u) * kThreads;
      if (i < n4) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float pe = P[u][e], me = M[u][e], ve = V[u][e];
          adamw_elem_t<kMode>(pe, G[u][e], me, ve, c);
          P[u][e] = pe;
          M[u][e] = me;
          V[u][e] = ve;
        }
        st<kNt>(&p[i], P[u]);
        st<kNt>(&m[i], M[u]);
        st<kNt>(&v[i], V[u]);
      }
    }
    if (!kPersistent) break;
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


template <int kU, bool kNt, bool kPersistent, int kMode>
hipError_t launch_vec_mode(float* p, const float* g, float* m, float* v, int64_t n4,
                           const AdamWConst& c, hipStream_t s) {
  const int64_t per_block = static_cast<int64_t>(kThreads) * kU;
  int64_t blocks = (n4 + per_block - 1) / per_block;
  if (kPersistent && blocks > 256 * 16) blocks = 256 * 16;
  hipLaunchKernelGGL((adamw_vec_kernel<kU, kNt, kPersistent, kMode>),
                     dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, s,
                     reinterpret_cast<f32x4*>(p), reinterpret_cast<const f32x4*>(g),
                     reinterpret_cast<f32x4*>(m), reinterpret_cast<f32x4*>(v), n4, c);
  return hipGetLastError();
}

template <int kU, bool kNt, bool kPersistent>
hipError_t launch_vec(float* p, const float* g, float* m, float* v, int64_t n4,
                      const AdamWConst& c, hipStream_t s) {
  switch (decay_mode(c)) {
    case kCoupled: return launch_vec_mode<kU, kNt, kPersistent, kCoupled>(p, g, m, v, n4, c, s);
    case kDecoupledCautious:
      return launch_vec_mode<kU, kNt, kPersistent, kDecoupledCautious>(p, g, m, v, n4, c, s);
    default: return launch_vec_mode<kU, kNt, kPersistent, kDecoupled>(p, g, m, v, n4, c, s);
  }
}

int adamw_variant() {
  static const int v = [] {
    const char* e = std::getenv("MA_ADAMW_VARIANT");  // tuning override
    return e ? std::atoi(e) : 0;
  }();
  return v;
}

// Many tensors in one launch: each block belongs to one segment of the table (read in
// place from the kernel-argument segment) and covers kMultiChunk of its elements, as
// float4 groups where the segment's four pointers are 16-byte aligned (the last block
// also takes the n % 4 tail) and element by element otherwise.  The same element
// function as the flat kernels, so every element's result is bitwise the same.
constexpr int kMultiGroups = 4;                               // float4 groups per thread
constexpr int kMultiChunk = kThreads * kMultiGroups * 4;      // elements per block

template <int kMode>
__global__ __launch_bounds__(kThreads) void adamw_multi_kernel(AdamWSegTable table) {
  const AdamWSegTable* kt = (const AdamWSegTable*)__builtin_amdgcn_kernarg_segment_ptr();
  (void)table;
  const int64_t b = blockIdx.x;
  int s = 0;
  for (int i = 1; i < kt->nseg; ++i)
    if (b >= kt->block_start[i]) s = i;
  const AdamWConst& c = kt->c;
  const int64_t n = kt->n[s];
  const int64_t lb = b - kt->block_start[s];
  float* p = kt->p[s];
  const float* g = kt->g[s];
  float* m = kt->m[s];
  float* v = kt->v[s];
  const int tid = threadIdx.x;
  if (kt->vec[s]) {
    const int64_t n4 = n / 4;
    f32x4* p4 = reinterpret_cast<f32x4*>(p);
    const f32x4* g4 = reinterpret_cast<const f32x4*>(g);
    f32x4* m4 = reinterpret_cast<f32x4*>(m);
    f32x4* v4 = reinterpret_cast<f32x4*>(v);
    const int64_t base = lb * (kThreads * kMultiGroups) + tid;
    f32x4 P[kMultiGroups], G[kMultiGroups], M[kMultiGroups], V[kMultiGroups];
#pragma unroll
    for (int u = 0; u < kMultiGroups; ++u) {
      const int64_t i = base + static_cast<int64_t>(u) * kThreads;
      if (i < n4) {
        P[u] = ld<true>(&p4[i]);
        G[u] = ld<true>(&g4[i]);
        M[u] = ld<true>(&m4[i]);
        V[u] = ld<true>(&v4[i]);
      }
    }
#pragma unroll
    for (int u = 0; u < kMultiGroups; ++u) {
      const int64_t i = base + static_cast<int64_t>(u) * kThreads;
      if (i < n4) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float pe = P[u][e], me = M[u][e], ve = V[u][e];
          adamw_elem_t<kMode>(pe, G[u][e], me, ve, c);
          P[u][e] = pe;
          M[u][e] = me;
          V[u][e] = ve;
        }
        st<true>(&p4[i], P[u]);
        st<true>(&m4[i], M[u]);
        st<true>(&v4[i], V[u]);
      }
    }
    // the n % 4 tail, in the segment's last block
    const int64_t tail0 = n4 * 4;
    if ((lb + 1) * kMultiChunk >= n && tid < n - tail0) {
      const int64_t i = tail0 + tid;
      float P1 = p[i], M1 = m[i], V1 = v[i];
      adamw_elem_t<kMode>(P1, g[i], M1, V1, c);
      p[i] = P1;
      m[i] = M1;
      v[i] = V1;
    }
  } else {
#pragma unroll
    for (int k = 0; k < kMultiChunk / kThreads; ++k) {
      const int64_t i = lb * kMultiChunk + static_cast<int64_t>(k) * kThreads + tid;
      if (i < n) {
        float P1 = p[i], M1 = m[i], V1 = v[i];
        adamw_elem_t<kMode>(P1, g[i], M1, V1, c);
        p[i] = P1;
        m[i] = M1;
        v[i] = V1;
      }
    }
  }
}

// Reference stream for the bandwidth ceiling of an access pattern: R fp32 arrays read,
// W written (out[j] = in[0] + ... + in[R-1] + j), float4 groups with the same
// non-temporal accesses and the same 4 groups per thread as adamw_vec_kernel, and no
// other arithmetic.
struct ProbePtrs {
  const f32x4* in[4];
  f32x4* out[3];
};

template <int R, int W>
__global__ __launch_bounds__(kThreads) void stream_probe_entry(ProbePtrs p, int64_t n4) {
  // the pointer table lives in the kernel arguments
  const f32x4* const* in = p.in;
  f32x4* const* out = p.out;
  const int64_t base = static_cast<int64_t>(blockIdx.x) * (kThreads * 4) + threadIdx.x;
  f32x4 acc[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int64_t i = base + static_cast<int64_t>(u) * kThreads;
    acc[u] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    if (i < n4) {
#pragma unroll
      for (int r = 0; r < R; ++r) acc[u] += __builtin_nontemporal_load(&in[r][i]);
    }
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int64_t i = base + static_cast<int64_t>(u) * kThreads;
    if (i < n4) {
#pragma unroll
      for (int w = 0; w < W; ++w) __builtin_nontemporal_store(acc[u] + static_cast<float>(w), &out[w][i]);
    }
  }
}

}  // namespace

hipError_t launch_stream_probe(const float* const* in, int reads, float* const* out, int writes,
                               int64_t n, hipStream_t s) {
  ProbePtrs p{};
  for (int r = 0; r < reads; ++r) p.in[r] = reinterpret_cast<const f32x4*>(in[r]);
  for (int w = 0; w < writes; ++w) p.out[w] = reinterpret_cast<f32x4*>(out[w]);
  const int64_t n4 = n / 4;
  const int64_t blocks = (n4 + kThreads * 4 - 1) / (kThreads * 4);
  if (blocks <= 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(blocks));
#define MA_PROBE(R, W)                                                                        \
  if (reads == R && writes == W) {                                                           \
    hipLaunchKernelGGL((stream_probe_entry<R, W>), grid, dim3(kThreads), 0, s, p, n4);     \
    return hipGetLastError();                                                                \
  }
  MA_PROBE(1, 0) MA_PROBE(2, 0) MA_PROBE(3, 0) MA_PROBE(4, 0)
  MA_PROBE(1, 1) MA_PROBE(2, 1) MA_PROBE(3, 1) MA_PROBE(4, 1)
  MA_PROBE(1, 2) MA_PROBE(2, 2) MA_PROBE(3, 2) MA_PROBE(4, 2)
  MA_PROBE(1, 3) MA_PROBE(2, 3) MA_PROBE(3, 3) MA_PROBE(4, 3)
#undef MA_PROBE
  return hipErrorInvalidValue;
}

int64_t adamw_multi_blocks(int64_t n) { return (n + kMultiChunk - 1) / kMultiChunk; }

hipError_t launch_adamw_multi(const AdamWSegTable& t, hipStream_t s) {
  const int64_t blocks = t.block_start[t.nseg];
  if (blocks <= 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(blocks));
  switch (decay_mode(t.c)) {
    case kCoupled: hipLaunchKernelGGL(adamw_multi_kernel<kCoupled>, grid, dim3(kThreads), 0, s, t); break;
    case kDecoupledCautious:
      hipLaunchKernelGGL(adamw_multi_kernel<kDecoupledCautious>, grid, dim3(kThreads), 0, s, t);
      break;
    default: hipLaunchKernelGGL(adamw_multi_kernel<kDecoupled>, grid, dim3(kThreads), 0, s, t); break;
  }
  return hipGetLastError();
}

hipError_t launch_adamw(float* p, const float* g, float* m, float* v, int64_t n,
                        const AdamWConst& c, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  int64_t done = 0;
  if (aligned16(p) && aligned16(g) && aligned16(m) && aligned16(v)) {
    const int64_t n4 = n / 4;
    if (n4 > 0) {
      hipError_t e;
      switch (adamw_variant()) {
        // default: 4 groups per thread, streaming loads and stores (at the copy ceiling)
        case 1: e = launch_vec<4, false, false>(p, g, m, v, n4, c, s); break;
        case 2: e = launch_vec<2, true, false>(p, g, m, v, n4, c, s); break;
        case 3: e = launch_vec<4, true, true>(p, g, m, v, n4, c, s); break;
        default: e = launch_vec<4, true, false>(p, g, m, v, n4, c, s); break;
      }
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
