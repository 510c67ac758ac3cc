// Achievable-peak probes for the roofline fractions: a register-resident
// bf16 matrix-instruction loop and a streaming copy.  Neither is on the
// decision path; the benchmark runs them in the same job as the path so that
// each kernel's fraction is stated against the datasheet and against what
// this GPU delivers.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace s1 {

namespace {

// Each wave keeps eight independent 32x32 accumulators and issues
// v_mfma_f32_32x32x16_bf16 on register operands only: 8 * iters
// instructions of 2 * 32 * 32 * 16 flop per wave.
__global__ void __launch_bounds__(256) mfma_peak_kernel(const uint4* __restrict__ seed, int iters,
                                                        float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const bf16x8 a = as_frag(seed[lane]), b = as_frag(seed[64 + lane]);
  floatx16 acc[8];
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[t][r] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int t = 0; t < 8; ++t) mfma32(acc[t], a, b);
  }
  float s = 0.f;
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[t][r];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// dst = src, 16 bytes per lane and access, four accesses in flight,
// non-temporal (streamed past the caches).
__global__ void __launch_bounds__(256) stream_copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                          long long n) {
  const long long stride = (long long)gridDim.x * blockDim.x;
  long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n; i += 4 * stride) {
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < 4; ++u) __builtin_nontemporal_store(v[u], dst + i + u * stride);
  }
  for (; i < n; i += stride) dst[i] = src[i];
}

// Reads src (same access pattern) and folds it with xor; a lane writes its
// value to sink only if it equals a fixed pattern, which keeps the loads
// from being elided without adding traffic.
__global__ void __launch_bounds__(256) stream_read_kernel(const u32x4* __restrict__ src, long long n,
                                                          u32x4* __restrict__ sink) {
  const long long stride = (long long)gridDim.x * blockDim.x;
  long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x;
  u32x4 acc = {0, 0, 0, 0};
  for (; i + 3 * stride < n; i += 4 * stride) {
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < 4; ++u) acc ^= v[u];
  }
  for (; i < n; i += stride) acc ^= src[i];
  if (acc.x == 0x9E3779B9u && acc.y == 0x7F4A7C15u) sink[threadIdx.x] = acc;
}

}  // namespace

hipError_t launch_mfma_peak(const void* seed, int blocks, int iters, float* out, hipStream_t s) {
  if (blocks <= 0 || iters <= 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(mfma_peak_kernel, dim3(blocks), dim3(256), 0, s, static_cast<const uint4*>(seed), iters, out);
  return hipGetLastError();
}

hipError_t launch_stream_copy(const void* src, void* dst, long long bytes, hipStream_t s) {
  if (bytes < 0 || bytes % 16) return hipErrorInvalidValue;
  if (bytes == 0) return hipSuccess;
  const long long n = bytes / 16;
  const int blocks = (int)std::min<long long>((n + 255) / 256, 8192);
  hipLaunchKernelGGL(stream_copy_kernel, dim3(blocks), dim3(256), 0, s, static_cast<const u32x4*>(src),
                     static_cast<u32x4*>(dst), n);
  return hipGetLastError();
}

hipError_t launch_stream_read(const void* src, long long bytes, void* sink, hipStream_t s) {
  if (bytes < 0 || bytes % 16) return hipErrorInvalidValue;
  if (bytes == 0) return hipSuccess;
  const long long n = bytes / 16;
  const int blocks = (int)std::min<long long>((n + 255) / 256, 8192);
  hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(256), 0, s, static_cast<const u32x4*>(src), n,
                     static_cast<u32x4*>(sink));
  return hipGetLastError();
}

}  // namespace s1
