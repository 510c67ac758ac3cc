// Small HBM-bound kernels: embedding gather, RMSNorm, LoRA merge at load,
// RoPE table, row gathers, and the decision readout.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace s1 {

namespace {

// ---------------------------------------------------------------- embed
// x[t] = E[ids[t]] as fp32 (tied embedding, RFC #114 section 3).
template <typename T>
__global__ void embed_kernel(const int32_t* __restrict__ ids, const T* __restrict__ E,
                             float* __restrict__ x, int d) {
  const int t = blockIdx.x;
  const T* src = E + (long long)ids[t] * d;
  float* dst = x + (long long)t * d;
  for (int i = threadIdx.x * 4; i < d; i += blockDim.x * 4) {
    float4 v;
    if constexpr (sizeof(T) == 2) {
      const uint2 u = *reinterpret_cast<const uint2*>(src + i);
      v = make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xFFFF0000u),
                      __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xFFFF0000u));
    } else {
      v = *reinterpret_cast<const float4*>(src + i);
    }
    *reinterpret_cast<float4*>(dst + i) = v;
  }
}

// -------------------------------------------------------------- rmsnorm
// out = x / sqrt(mean(x^2) + eps) * w, one workgroup of 256 threads per row;
// the row stays in registers between the sum of squares and the scaling
// (d <= 4 * 256 * RMS_MAXV).  w == NULL: no gain (it is folded into the next
// GEMM's weights) and rs[row] = 1 / sqrt(mean(x^2) + eps).
constexpr int RMS_MAXV = 16;
template <typename T>
__global__ void __launch_bounds__(256) rmsnorm_kernel(const float* __restrict__ x, const float* __restrict__ w,
                                                      T* __restrict__ out, int d, float eps,
                                                      float* __restrict__ rs) {
  __shared__ float red[4];
  const long long row = blockIdx.x;
  const float* xr = x + row * d;
  float4 v[RMS_MAXV];
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < RMS_MAXV; ++k) {
    const int c = (k * 256 + (int)threadIdx.x) * 4;
    if (c >= d) break;
    v[k] = *reinterpret_cast<const float4*>(xr + c);
    ss += v[k].x * v[k].x + v[k].y * v[k].y + v[k].z * v[k].z + v[k].w * v[k].w;
  }
  ss = block_sum<4>(ss, red);
  write_normed_row<T, 256, RMS_MAXV>(v, ss, d, eps, w, out + row * d, rs ? rs + row : nullptr);
}

// Embedding gather fused with the first layer's input RMSNorm: x[t] =
// E[ids[t]] (fp32) and xn[t] = RMSNorm(x[t]) * w, one workgroup of 256
// threads per row, the row in registers (the same arithmetic as
// rmsnorm_kernel on the gathered row, the deferred form when w == NULL).
template <typename T>
__global__ void __launch_bounds__(256) embed_norm_kernel(const int32_t* __restrict__ ids, const T* __restrict__ E,
                                                         float* __restrict__ x, int d, const float* __restrict__ w,
                                                         T* __restrict__ xn, float eps, float* __restrict__ rs) {
  __shared__ float red[4];
  const long long row = blockIdx.x;
  const T* src = E + (long long)ids[row] * d;
  float* dst = x + row * d;
  float4 v[RMS_MAXV];
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < RMS_MAXV; ++k) {
    const int c = (k * 256 + (int)threadIdx.x) * 4;
    if (c >= d) break;
    if constexpr (sizeof(T) == 2) {
      const uint2 u = *reinterpret_cast<const uint2*>(src + c);
      v[k] = make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xFFFF0000u),
                         __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xFFFF0000u));
    } else {
      v[k] = *reinterpret_cast<const float4*>(src + c);
    }
    *reinterpret_cast<float4*>(dst + c) = v[k];
    ss += v[k].x * v[k].x + v[k].y * v[k].y + v[k].z * v[k].z + v[k].w * v[k].w;
  }
  ss = block_sum<4>(ss, red);
  write_normed_row<T, 256, RMS_MAXV>(v, ss, d, eps, w, xn + row * d, rs ? rs + row : nullptr);
}

// ---------------------------------------------------------------- merge
// out[map(o)] = (W[o] + scale * (B[o] . A[:, i])) * gain[i] (gain optional);
// fp32 arithmetic, one rounding.
template <typename T>
__global__ void merge_kernel(const T* __restrict__ W, const T* __restrict__ A,
                             const T* __restrict__ B, T* __restrict__ out, int in_dim, int rank,
                             float scale, const int* __restrict__ row_map, const float* __restrict__ gain) {
  __shared__ float sb[64];
  const int o = blockIdx.x;
  if (A != nullptr && threadIdx.x < rank) sb[threadIdx.x] = to_f<T>(B[(long long)o * rank + threadIdx.x]);
  __syncthreads();
  const int dst = row_map ? row_map[o] : o;
  const T* wr = W + (long long)o * in_dim;
  T* orow = out + (long long)dst * in_dim;
  for (int i = blockIdx.y * blockDim.x + threadIdx.x; i < in_dim; i += gridDim.y * blockDim.x) {
    float v = to_f<T>(wr[i]);
    if (A != nullptr) {
      float ba = 0.f;
      for (int j = 0; j < rank; ++j) ba = fmaf(sb[j], to_f<T>(A[(long long)j * in_dim + i]), ba);
      v += scale * ba;
    }
    if (gain != nullptr) v *= gain[i];
    orow[i] = from_f<T>(v);
  }
}

template <typename T>
__global__ void to_f32_kernel(const T* __restrict__ in, float* __restrict__ out, long long n) {
  for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < n;
       i += (long long)gridDim.x * blockDim.x)
    out[i] = to_f<T>(in[i]);
}

// (cos, sin) of p * base^(-2i/hd), computed in double precision once at load.
__global__ void rope_table_kernel(float2* table, int max_pos, int half, double base, int hd) {
  const long long n = (long long)max_pos * half;
  for (long long k = blockIdx.x * (long long)blockDim.x + threadIdx.x; k < n;
       k += (long long)gridDim.x * blockDim.x) {
    const int p = (int)(k / half), i = (int)(k % half);
    const double ang = (double)p * pow(base, -2.0 * i / hd);
    table[k] = make_float2((float)cos(ang), (float)sin(ang));
  }
}

__global__ void gather_rows_kernel(const float* __restrict__ x, int d, const int32_t* rows,
                                   const int32_t* dsti, float* __restrict__ out) {
  const float* src = x + (long long)rows[blockIdx.x] * d;
  float* dst = out + (long long)(dsti ? dsti[blockIdx.x] : blockIdx.x) * d;
  for (int i = threadIdx.x; i < d; i += blockDim.x) dst[i] = src[i];
}

// -------------------------------------------------------------- readout
struct Decision {
  int32_t choice;
  float score, noul, answer_confidence, confidence, entropy_confidence;
};

// One workgroup per question: final RMSNorm of the marker row into LDS,
// one wave per option for the dot product with its tied-embedding row
// (cross-lane reduction), then softmax and answer fields on wave 0.
// (Cua-S1 issue, first plan comment: softmax over the option logits at one
// position; sys1rust README "Try it": the answer fields.)
// Dot product of eight bf16 values (one 16-byte chunk) with h[0..7] (fp32, LDS).
__device__ __forceinline__ float dot8_bf16(uint4 u, const float* h) {
  const float4 h0 = *reinterpret_cast<const float4*>(h), h1 = *reinterpret_cast<const float4*>(h + 4);
  return __uint_as_float(u.x << 16) * h0.x + __uint_as_float(u.x & 0xFFFF0000u) * h0.y +
         __uint_as_float(u.y << 16) * h0.z + __uint_as_float(u.y & 0xFFFF0000u) * h0.w +
         __uint_as_float(u.z << 16) * h1.x + __uint_as_float(u.z & 0xFFFF0000u) * h1.y +
         __uint_as_float(u.w << 16) * h1.z + __uint_as_float(u.w & 0xFFFF0000u) * h1.w;
}

template <typename T>
__global__ void __launch_bounds__(256)
readout_kernel(const float* __restrict__ x, int d, const float* __restrict__ w, float eps,
               const T* __restrict__ E, const int32_t* __restrict__ rows,
               const int32_t* __restrict__ offs, const int32_t* __restrict__ ids,
               const uint8_t* __restrict__ qt, float* __restrict__ probs,
               Decision* __restrict__ dec) {
  extern __shared__ float sm[];
  float* h = sm;            // [d]
  float* z = sm + d;        // [K]
  __shared__ float red[4];
  const int q = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* xr = x + (long long)rows[q] * d;
  float ss = 0.f;
  for (int i = tid * 4; i < d; i += 1024) {
    const float4 v = *reinterpret_cast<const float4*>(xr + i);
    ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
  }
  ss = wave_sum(ss);
  if (lane == 0) red[wave] = ss;
  __syncthreads();
  const float r = rsqrtf((red[0] + red[1] + red[2] + red[3]) / d + eps);
  for (int i = tid; i < d; i += 256) h[i] = xr[i] * r * w[i];
  __syncthreads();
  const int o0 = offs[q], K = offs[q + 1] - o0;
  for (int k = wave; k < K; k += 4) {
    const T* e = E + (long long)ids[o0 + k] * d;
    float acc = 0.f;
    if (sizeof(T) == 2 && d % 8 == 0) {
      // 16 bytes (8 values) per lane and load, four loads in flight
      int i = lane * 8;
      for (; i + 3 * 512 < d; i += 4 * 512) {
        uint4 u[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) u[t] = *reinterpret_cast<const uint4*>(e + i + t * 512);
#pragma unroll
        for (int t = 0; t < 4; ++t) acc += dot8_bf16(u[t], h + i + t * 512);
      }
      for (; i < d; i += 512) acc += dot8_bf16(*reinterpret_cast<const uint4*>(e + i), h + i);
    } else {
      for (int i = lane * 4; i < d; i += 256) {
        float4 ev;
        if constexpr (sizeof(T) == 2) {
          const uint2 u = *reinterpret_cast<const uint2*>(e + i);
          ev = make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xFFFF0000u),
                           __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xFFFF0000u));
        } else {
          ev = *reinterpret_cast<const float4*>(e + i);
        }
        acc += ev.x * h[i] + ev.y * h[i + 1] + ev.z * h[i + 2] + ev.w * h[i + 3];
      }
    }
    acc = wave_sum(acc);
    if (lane == 0) z[k] = acc;
  }
  __syncthreads();
  if (wave != 0) return;
  float m = -INFINITY;
  for (int k = lane; k < K; k += 64) m = fmaxf(m, z[k]);
  m = wave_max(m);
  float s = 0.f;
  for (int k = lane; k < K; k += 64) s += __expf(z[k] - m);
  s = wave_sum(s);
  const float inv = 1.f / s;
  float pmax = 0.f, sc = 0.f, ent = 0.f;
  for (int k = lane; k < K; k += 64) {
    const float p = __expf(z[k] - m) * inv;
    probs[o0 + k] = p;
    z[k] = p;
    pmax = fmaxf(pmax, p);
    sc += k * p;
    if (p > 0.f) ent -= p * __logf(p);
  }
  pmax = wave_max(pmax);
  sc = wave_sum(sc);
  ent = wave_sum(ent);
  int first = K;
  for (int k = lane; k < K; k += 64)
    if (z[k] == pmax) first = min(first, k);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) first = min(first, __shfl_xor(first, o, 64));
  if (lane == 0) {
    float ec = 1.f - ent / __logf((float)K);
    ec = fminf(1.f, fmaxf(0.f, ec));
    Decision dd;
    dd.choice = first;
    dd.score = sc;
    dd.noul = z[0];
    dd.answer_confidence = pmax;
    dd.entropy_confidence = ec;
    dd.confidence = (qt[q] == 2) ? pmax : ec;
    dec[q] = dd;
  }
}

inline int grid_for(long long n, int threads, int cap = 8192) {
  long long b = (n + threads - 1) / threads;
  return (int)std::max<long long>(1, std::min<long long>(b, cap));
}

}  // namespace

hipError_t launch_embed(bool bf16, const int32_t* ids, const void* E, float* x, int T, int d,
                        hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if (bf16)
    hipLaunchKernelGGL(embed_kernel<bf16_t>, dim3(T), dim3(256), 0, s, ids,
                       reinterpret_cast<const bf16_t*>(E), x, d);
  else
    hipLaunchKernelGGL(embed_kernel<float>, dim3(T), dim3(256), 0, s, ids,
                       reinterpret_cast<const float*>(E), x, d);
  return hipGetLastError();
}

hipError_t launch_embed_norm(bool bf16, const int32_t* ids, const void* E, float* x, int T, int d,
                            const float* w, void* xn, float eps, hipStream_t s, float* rs) {
  if (T <= 0) return hipSuccess;
  if (d % 4 || d > 4 * 256 * RMS_MAXV || (w == nullptr && rs == nullptr)) return hipErrorInvalidValue;
  if (bf16)
    hipLaunchKernelGGL(embed_norm_kernel<bf16_t>, dim3(T), dim3(256), 0, s, ids,
                       reinterpret_cast<const bf16_t*>(E), x, d, w, reinterpret_cast<bf16_t*>(xn), eps, rs);
  else
    hipLaunchKernelGGL(embed_norm_kernel<float>, dim3(T), dim3(256), 0, s, ids,
                       reinterpret_cast<const float*>(E), x, d, w, reinterpret_cast<float*>(xn), eps, rs);
  return hipGetLastError();
}

hipError_t launch_rmsnorm(bool bf16, const float* x, const float* w, void* out, int T, int d,
                          float eps, hipStream_t s, float* rs) {
  if (T <= 0) return hipSuccess;
  if (d % 4 || d > 4 * 256 * RMS_MAXV || (w == nullptr && rs == nullptr)) return hipErrorInvalidValue;
  if (bf16)
    hipLaunchKernelGGL(rmsnorm_kernel<bf16_t>, dim3(T), dim3(256), 0, s, x, w,
                       reinterpret_cast<bf16_t*>(out), d, eps, rs);
  else
    hipLaunchKernelGGL(rmsnorm_kernel<float>, dim3(T), dim3(256), 0, s, x, w,
                       reinterpret_cast<float*>(out), d, eps, rs);
  return hipGetLastError();
}

hipError_t launch_merge(bool bf16, const void* W, const void* A, const void* B, void* out,
                        int out_dim, int in_dim, int rank, float scale, const int* row_map,
                        hipStream_t s, const float* gain) {
  if (out_dim <= 0 || in_dim <= 0) return hipSuccess;
  if (A != nullptr && (rank <= 0 || rank > 64)) return hipErrorInvalidValue;
  const dim3 grid(out_dim, std::max(1, std::min(8, (in_dim + 1023) / 1024)));
  if (bf16)
    hipLaunchKernelGGL(merge_kernel<bf16_t>, grid, dim3(256), 0, s,
                       reinterpret_cast<const bf16_t*>(W), reinterpret_cast<const bf16_t*>(A),
                       reinterpret_cast<const bf16_t*>(B), reinterpret_cast<bf16_t*>(out), in_dim,
                       rank, scale, row_map, gain);
  else
    hipLaunchKernelGGL(merge_kernel<float>, grid, dim3(256), 0, s,
                       reinterpret_cast<const float*>(W), reinterpret_cast<const float*>(A),
                       reinterpret_cast<const float*>(B), reinterpret_cast<float*>(out), in_dim,
                       rank, scale, row_map, gain);
  return hipGetLastError();
}

hipError_t launch_to_f32(bool bf16, const void* in, float* out, long long n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (bf16)
    hipLaunchKernelGGL(to_f32_kernel<bf16_t>, dim3(grid_for(n, 256)), dim3(256), 0, s,
                       reinterpret_cast<const bf16_t*>(in), out, n);
  else
    hipLaunchKernelGGL(to_f32_kernel<float>, dim3(grid_for(n, 256)), dim3(256), 0, s,
                       reinterpret_cast<const float*>(in), out, n);
  return hipGetLastError();
}

hipError_t launch_rope_table(float2* table, int max_pos, int head_dim, double base,
                             hipStream_t s) {
  const long long n = (long long)max_pos * (head_dim / 2);
  hipLaunchKernelGGL(rope_table_kernel, dim3(grid_for(n, 256)), dim3(256), 0, s, table, max_pos,
                     head_dim / 2, base, head_dim);
  return hipGetLastError();
}

hipError_t launch_gather_rows(const float* x, int d, const int32_t* rows, const int32_t* dst,
                              int n_rows, float* out, hipStream_t s) {
  if (n_rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(gather_rows_kernel, dim3(n_rows), dim3(256), 0, s, x, d, rows, dst, out);
  return hipGetLastError();
}

hipError_t launch_readout(bool bf16, const float* x, int d, const float* w_final, float eps,
                          const void* E, int Q, const int32_t* rows, const int32_t* opt_offsets,
                          const int32_t* opt_ids, const uint8_t* q_type, float* probs,
                          void* decisions, int max_k, hipStream_t s) {
  if (Q <= 0) return hipSuccess;
  const size_t shm = (size_t)(d + max_k) * sizeof(float);
  if (bf16)
    hipLaunchKernelGGL(readout_kernel<bf16_t>, dim3(Q), dim3(256), shm, s, x, d, w_final, eps,
                       reinterpret_cast<const bf16_t*>(E), rows, opt_offsets, opt_ids, q_type,
                       probs, reinterpret_cast<Decision*>(decisions));
  else
    hipLaunchKernelGGL(readout_kernel<float>, dim3(Q), dim3(256), shm, s, x, d, w_final, eps,
                       reinterpret_cast<const float*>(E), rows, opt_offsets, opt_ids, q_type,
                       probs, reinterpret_cast<Decision*>(decisions));
  return hipGetLastError();
}

}  // namespace s1
