// Matrix-core reference loop: the sustained bf16 MFMA rate of the part on given operand
// data, with no memory traffic inside the loop.
//
// The Newton-Schulz GEMMs are priced against the 2.5 PFLOP/s dense bf16 rating, which
// assumes the 2.4 GHz clock.  Under a sustained load of random-valued operands the part
// lowers its clock to stay within its power limit, so the rating is out of reach even
// for code that does nothing but MFMAs.  This loop measures that ceiling on the same
// instruction (v_mfma_f32_32x32x16_bf16) and occupancy (blocks of 8 waves, two per SIMD)
// as the GEMM kernel: each wave holds eight A and eight B fragments in registers and
// cycles through them, so consecutive MFMAs see different operands as in a GEMM, into
// four independent accumulators (the MFMA latency stays covered).  Thread 0 of each
// block also records the shader-clock counter (s_memtime) and the 100 MHz real-time
// counter (s_memrealtime) around the loop, so the caller can read the clock it ran at.
#include <hip/hip_runtime.h>

#include "ma_internal.h"

namespace ma {
namespace {

constexpr int kProbeThreads = 512;
constexpr int kProbeSets = 8;  // operand pairs cycled per wave

__global__ __launch_bounds__(kProbeThreads) void mfma_probe_kernel(
    const bf16x8* __restrict__ operands, int iters, float* __restrict__ out,
    unsigned long long* __restrict__ clocks) {
  const int lane = threadIdx.x & 63;
  bf16x8 a[kProbeSets], b[kProbeSets];
#pragma unroll
  for (int s = 0; s < kProbeSets; ++s) {
    a[s] = operands[(2 * s) * 64 + lane];
    b[s] = operands[(2 * s + 1) * 64 + lane];
  }
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  f32x16 acc[4] = {};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int r = 0; r < kProbeSets; ++r)
      acc[r & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[r], b[(r + 3) & 7], acc[r & 3], 0, 0, 0);
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  float sum = 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int e = 0; e < 16; ++e) sum += acc[q][e];
  out[static_cast<int64_t>(blockIdx.x) * kProbeThreads + threadIdx.x] = sum;
  if (clocks != nullptr && threadIdx.x == 0) {
    clocks[2 * static_cast<int64_t>(blockIdx.x)] = t1 - t0;
    clocks[2 * static_cast<int64_t>(blockIdx.x) + 1] = r1 - r0;
  }
}

}  // namespace

hipError_t launch_mfma_probe(const void* operands, int blocks, int iters, float* out,
                             unsigned long long* clocks, hipStream_t s) {
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kProbeThreads),
                     0, s, static_cast<const bf16x8*>(operands), iters, out, clocks);
  return hipGetLastError();
}

}  // namespace ma
