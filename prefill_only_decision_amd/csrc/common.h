// Device-side helpers shared by the HIP kernels of the library (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace s1 {

typedef uint16_t bf16_t;   // raw bfloat16 bit pattern
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf2f(bf16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Two floats -> two bf16 in one word (a low, b high) with the packed
// hardware conversion v_cvt_pk_bf16_f32: round to nearest, ties to even
// (inputs are finite).
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef float float2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t cvt2(float a, float b) {
  const float2v f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2v));
}

// float -> bfloat16, round to nearest, ties to even (inputs are finite).
__device__ __forceinline__ bf16_t f2bf(float f) { return static_cast<bf16_t>(cvt2(f, 0.f)); }

__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) { return cvt2(lo, hi); }

// Element conversions used by templated kernels (T = bf16_t or float).
template <typename T> __device__ __forceinline__ float to_f(T v);
template <> __device__ __forceinline__ float to_f<float>(float v) { return v; }
template <> __device__ __forceinline__ float to_f<bf16_t>(bf16_t v) { return bf2f(v); }
template <typename T> __device__ __forceinline__ T from_f(float v);
template <> __device__ __forceinline__ float from_f<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16_t from_f<bf16_t>(float v) { return f2bf(v); }

// Eight consecutive bf16 values <-> one 16-byte vector, as an MFMA operand.
__device__ __forceinline__ bf16x8 as_frag(uint4 u) { return __builtin_bit_cast(bf16x8, u); }
__device__ __forceinline__ bf16x8 frag_from_f(const float* v) {
  uint4 u;
  u.x = pack_bf2(v[0], v[1]);
  u.y = pack_bf2(v[2], v[3]);
  u.z = pack_bf2(v[4], v[5]);
  u.w = pack_bf2(v[6], v[7]);
  return as_frag(u);
}
__device__ __forceinline__ float lo_half(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_half(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Split eight floats into hi + lo bf16 operands with v = hi + lo up to
// 2^-16 relative: hi = rne(v), lo = rne(v - hi) (the difference is exact).
__device__ __forceinline__ void split_frag(const float* v, bf16x8& hi, bf16x8& lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    h[e] = cvt2(v[2 * e], v[2 * e + 1]);
    l[e] = cvt2(v[2 * e] - lo_half(h[e]), v[2 * e + 1] - hi_half(h[e]));
  }
  hi = as_frag(make_uint4(h[0], h[1], h[2], h[3]));
  lo = as_frag(make_uint4(l[0], l[1], l[2], l[3]));
}

// Two 8-byte halves (4 bf16 each) -> one operand.
__device__ __forceinline__ bf16x8 frag_from_halves(uint2 a, uint2 b) {
  return as_frag(make_uint4(a.x, a.y, b.x, b.y));
}

// D = A x B + C on a 32x32 tile.  bf16: K = 16, each lane holds A[m = l%32]
// [k = 8*(l/32) .. +7] and B[k = 8*(l/32) .. +7][n = l%32].  fp32: K = 2,
// lane holds A[l%32][l/32] and B[l/32][l%32].  The 16 accumulators of lane l
// hold C[row][l%32] with row = 8*(r/4) + 4*(l/32) + r%4.
__device__ __forceinline__ void mfma32(floatx16& c, bf16x8 a, bf16x8 b) {
  c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ void mfma32(floatx16& c, float a, float b) {
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ int acc_row(int r, int lane) {
  return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}

// Workgroups are dispatched round-robin over the 8 XCDs of the chip.  This
// bijection maps launch order to a tile order in which each XCD receives a
// contiguous run of tiles, so neighbouring tiles (sharing operand panels)
// share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int b, int nb) {
  const int q = nb >> 3, r = nb & 7, x = b & 7;
  return x * q + min(x, r) + (b >> 3);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
// Sum over a workgroup of NW waves (every thread gets the total).
template <int NW>
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int i = 0; i < NW; ++i) t += red[i];
  return t;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// RMSNorm of one row held as float4 pieces v[k] (columns 4 (k * NT + tid)
// ...): out = v * r * w with r = 1 / sqrt(ss / d + eps), ss the row's sum of
// squares.  With w == NULL (the gain folded into the next GEMM's weights):
// out = v * r and *rs = r.
template <typename T, int NT, int MAXV>
__device__ __forceinline__ void write_normed_row(const float4 (&v)[MAXV], float ss, int d, float eps,
                                                 const float* __restrict__ w, T* __restrict__ o,
                                                 float* __restrict__ rs = nullptr) {
  const float r = rsqrtf(ss / d + eps);
  if (w == nullptr) {
    if (threadIdx.x == 0) *rs = r;
#pragma unroll
    for (int k = 0; k < MAXV; ++k) {
      const int c = (k * NT + (int)threadIdx.x) * 4;
      if (c >= d) break;
      const float4 x = v[k];
      if constexpr (sizeof(T) == 2) {
        uint2 u;
        u.x = pack_bf2(x.x * r, x.y * r);
        u.y = pack_bf2(x.z * r, x.w * r);
        *reinterpret_cast<uint2*>(o + c) = u;
      } else {
        *reinterpret_cast<float4*>(o + c) = make_float4(x.x * r, x.y * r, x.z * r, x.w * r);
      }
    }
    return;
  }
#pragma unroll
  for (int k = 0; k < MAXV; ++k) {
    const int c = (k * NT + (int)threadIdx.x) * 4;
    if (c >= d) break;
    const float4 g = *reinterpret_cast<const float4*>(w + c);
    const float4 x = v[k];
    if constexpr (sizeof(T) == 2) {
      uint2 u;
      u.x = pack_bf2(x.x * r * g.x, x.y * r * g.y);
      u.y = pack_bf2(x.z * r * g.z, x.w * r * g.w);
      *reinterpret_cast<uint2*>(o + c) = u;
    } else {
      *reinterpret_cast<float4*>(o + c) = make_float4(x.x * r * g.x, x.y * r * g.y, x.z * r * g.z, x.w * r * g.w);
    }
  }
}

}  // namespace s1
