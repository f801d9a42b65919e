// peak.hip -- matrix-core throughput loops (see include/gdn_peak.h): the
// measured counterpart of the published dense peaks, for context beside the
// roofline fractions.  Eight independent accumulators per wave keep the
// matrix pipe busy across the instruction latency; operands stay in
// registers, so the loop touches no memory until the final store.
#include <hip/hip_runtime.h>

#include "gdn_peak.h"

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kAcc = 8;

__global__ __launch_bounds__(256) void mfma_bf16_loop(int iters, float* __restrict__ sink) {
  const int t = threadIdx.x;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(0.001f * (t + e));
    b[e] = (__bf16)(0.002f * (t - e));
  }
  f32x4 acc[kAcc];
#pragma unroll
  for (int i = 0; i < kAcc; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < kAcc; ++i) acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[i], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < kAcc; ++i) s += acc[i][0] + acc[i][1] + acc[i][2] + acc[i][3];
  sink[(size_t)blockIdx.x * blockDim.x + t] = s;
}

__global__ __launch_bounds__(256) void mfma_f32_loop(int iters, float* __restrict__ sink) {
  const int t = threadIdx.x;
  const float a = 0.001f * t, b = 0.002f * (t ^ 5);
  f32x4 acc[kAcc];
#pragma unroll
  for (int i = 0; i < kAcc; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < kAcc; ++i) acc[i] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc[i], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < kAcc; ++i) s += acc[i][0] + acc[i][1] + acc[i][2] + acc[i][3];
  sink[(size_t)blockIdx.x * blockDim.x + t] = s;
}

// Vector fp32: eight independent fused multiply-add chains per thread.  The
// library is built without packed fp32 instructions, so this measures the
// v_fma_f32 rate the kernels here can reach (half the published vector peak,
// which counts packed issue).
__global__ __launch_bounds__(256) void fma_f32_loop(int iters, float* __restrict__ sink) {
  const int t = threadIdx.x;
  const float a = 0.999f + 1e-6f * t, b = 1e-3f * (t & 7);
  float acc[kAcc];
#pragma unroll
  for (int i = 0; i < kAcc; ++i) acc[i] = 0.01f * (i + t);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < kAcc; ++i) acc[i] = __builtin_fmaf(acc[i], a, b);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < kAcc; ++i) s += acc[i];
  sink[(size_t)blockIdx.x * blockDim.x + t] = s;
}

// Streaming read: each thread sums 16-byte words at a grid stride (the last
// partial word is not read).  Unrolled eight deep so every wave keeps eight
// loads in flight.
__global__ __launch_bounds__(256) void read_loop(const uint4* __restrict__ buf, size_t words,
                                                 float* __restrict__ sink) {
  constexpr int U = 8;
  const size_t tid = (size_t)blockIdx.x * blockDim.x + threadIdx.x, stride = (size_t)gridDim.x * blockDim.x;
  unsigned acc = 0;
  size_t i = tid;
  for (; i + (U - 1) * stride < words; i += U * stride) {
    uint4 x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) x[u] = buf[i + u * stride];
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= x[u].x ^ x[u].y ^ x[u].z ^ x[u].w;
  }
  for (; i < words; i += stride) {
    const uint4 a = buf[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  sink[tid] = (float)(acc & 0xFFFF);
}

}  // namespace

extern "C" int gdn_peak_read(const void* buf, size_t bytes, int blocks, float* sink, void* stream) {
  if (!buf || !sink || blocks < 1 || ((size_t)buf & 15)) return -1;
  hipLaunchKernelGGL(read_loop, dim3(blocks), dim3(256), 0, (hipStream_t)stream, (const uint4*)buf, bytes / 16,
                     sink);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

extern "C" int gdn_peak_mfma_loop(int kind, int iters, int blocks, float* sink, void* stream) {
  if (kind < 0 || kind > 2 || iters < 1 || blocks < 1 || !sink) return -1;
  hipStream_t s = (hipStream_t)stream;
  if (kind == 0)
    hipLaunchKernelGGL(mfma_bf16_loop, dim3(blocks), dim3(256), 0, s, iters, sink);
  else if (kind == 1)
    hipLaunchKernelGGL(mfma_f32_loop, dim3(blocks), dim3(256), 0, s, iters, sink);
  else
    hipLaunchKernelGGL(fma_f32_loop, dim3(blocks), dim3(256), 0, s, iters, sink);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}
