// Projection GEMMs of the hybrid decoder on CDNA4 matrix cores.
//
// C[M,N] = A[M,K] x W[N,K]^T: activations times [out, in] weights, both
// K-contiguous.  bf16 operands use v_mfma_f32_32x32x16_bf16 (fp32
// accumulation); the fp32 model uses v_mfma_f32_32x32x2f32 with the same
// tiling and epilogues.  A workgroup computes a BM x BN tile; 2 x 2 waves each
// own a (BM/2) x (BN/2) sub-tile made of 32 x 32 MFMA tiles.  K advances in
// tiles of 128 bytes per row (64 bf16 / 32 fp32), double-buffered in LDS with
// one barrier per K tile: the next tile's global loads are in flight while the
// current tile is multiplied.  LDS rows are padded by 16 bytes so that the 16
// lanes of one LDS read phase, which read 16 different rows at the same
// column, hit disjoint banks.
//
// Epilogues fuse the elementwise work that follows each projection
// (Cua-S1 4B 0.2 issue, timing comment: the remaining time was GEMMs plus
// about 2,000 small elementwise kernels per forward):
//   residual add, decay-gate log-sigmoid, SwiGLU, RoPE + KV-cache write.
// SwiGLU and RoPE need two columns of the same row in one lane; the weight
// rows are permuted at load so that the partner column sits exactly 32
// columns later, i.e. in the neighbouring MFMA tile at the same register.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace s1 {

namespace {

template <typename T> struct Frag;
template <> struct Frag<bf16_t> {
  typedef bf16x8 type;
  static constexpr int KE = 16;      // K per MFMA
  static constexpr int LANE_K = 8;   // K elements per lane
  __device__ static type load(const char* p) { return as_frag(*reinterpret_cast<const uint4*>(p)); }
};
template <> struct Frag<float> {
  typedef float type;
  static constexpr int KE = 2;
  static constexpr int LANE_K = 1;
  __device__ static type load(const char* p) { return *reinterpret_cast<const float*>(p); }
};

__device__ __forceinline__ float log_sigmoid(float z) {
  // log(1 / (1 + e^-z)) = -(max(-z, 0) + log1p(e^-|z|))
  return -(fmaxf(-z, 0.f) + log1pf(__expf(-fabsf(z))));
}
__device__ __forceinline__ float silu(float a) { return a / (1.f + __expf(-a)); }

template <typename T, int EPI, int TM, int TN>
__device__ __forceinline__ void epilogue(const GemmArgs& g, floatx16 (&acc)[TM][TN], int rm0,
                                         int cn0, int lane, int split_idx) {
  const int cl = lane & 31;
  if constexpr (EPI == EPI_SWIGLU || EPI == EPI_QKV) {
#pragma unroll
    for (int j = 0; j < TN; j += 2) {
      const int cb = cn0 + 32 * j;                    // multiple of 64
      if (cb >= g.N) continue;
#pragma unroll
      for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = rm0 + 32 * i + acc_row(r, lane);
          if (row >= g.M) continue;
          const float a1 = acc[i][j][r], a2 = acc[i][j + 1][r];
          if constexpr (EPI == EPI_SWIGLU) {
            const int f = (cb >> 1) + cl;
            if (f < g.n_valid)
              reinterpret_cast<T*>(g.out0)[(long long)row * g.ld0 + f] = from_f<T>(silu(a1) * a2);
          } else {
            if (cb < g.nsplit2) {
              // rotate-half pair (d, d + hd/2): permuted to columns (cb+cl, cb+32+cl)
              const int hc = cb % g.head_dim;
              const int dim = 32 * (hc >> 6) + cl;
              const float2 cs = g.rope[(long long)g.pos[row] * (g.head_dim >> 1) + dim];
              const float r1 = a1 * cs.x - a2 * cs.y;
              const float r2 = a2 * cs.x + a1 * cs.y;
              T* dst;
              long long off;
              if (cb < g.nsplit) {
                dst = reinterpret_cast<T*>(g.out0);
                off = (long long)row * g.ld0 + cb;
              } else {
                dst = reinterpret_cast<T*>(g.out1);
                off = (long long)row * g.ld1 + (cb - g.nsplit);
              }
              dst[off + cl] = from_f<T>(r1);
              dst[off + 32 + cl] = from_f<T>(r2);
            } else {
              T* dst = reinterpret_cast<T*>(g.out2);
              const long long off = (long long)row * g.ld2 + (cb - g.nsplit2);
              dst[off + cl] = from_f<T>(a1);
              if (cb + 32 < g.N) dst[off + 32 + cl] = from_f<T>(a2);
            }
          }
        }
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int col = cn0 + 32 * j + cl;
      if (col >= g.N) continue;
#pragma unroll
      for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = rm0 + 32 * i + acc_row(r, lane);
          if (row >= g.M) continue;
          const float v = acc[i][j][r];
          if constexpr (EPI == EPI_F32) {
            reinterpret_cast<float*>(g.out0)[(long long)row * g.ld0 + col] = v;
          } else if constexpr (EPI == EPI_RESID) {
            reinterpret_cast<float*>(g.out0)[(long long)row * g.ld0 + col] += v;
          } else if constexpr (EPI == EPI_PARTIAL) {
            reinterpret_cast<float*>(g.out0)[split_idx * g.split_stride + (long long)row * g.ld0 + col] = v;
          } else if constexpr (EPI == EPI_GATE) {
            if (col < g.nsplit)
              reinterpret_cast<T*>(g.out0)[(long long)row * g.ld0 + col] = from_f<T>(v);
            else
              reinterpret_cast<float*>(g.out1)[(long long)row * g.ld1 + (col - g.nsplit)] = log_sigmoid(v);
          }
        }
      }
    }
  }
}

template <typename T, int BM, int BN, int WM, int WN, int EPI>
__global__ void __launch_bounds__(WM * WN * 64)
gemm_kernel(GemmArgs g) {
  typedef Frag<T> F;
  constexpr int NT = WM * WN * 64;
  constexpr int ROWB = 128;                  // bytes of one K tile row
  constexpr int BK = ROWB / (int)sizeof(T);
  constexpr int PITCH = ROWB + 16;
  constexpr int CHR = ROWB / 16;             // 16-byte chunks per row
  constexpr int EPC = 16 / (int)sizeof(T);   // elements per chunk
  constexpr int A_CH = BM * CHR / NT;
  constexpr int B_CH = BN * CHR / NT;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int TM = WTM / 32, TN = WTN / 32;
  static_assert(A_CH * NT == BM * CHR && B_CH * NT == BN * CHR, "tile/thread mismatch");
  constexpr int STAGE = (BM + BN) * PITCH;
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int nbm = (g.M + BM - 1) / BM;
  const int t = xcd_remap(blockIdx.x, gridDim.x);
  const int m0 = (t % nbm) * BM, n0 = (t / nbm) * BN;
  const int kb = blockIdx.y * g.k_split;
  const int ke = min(g.K, kb + g.k_split);
  const int nk = ke > kb ? (ke - kb + BK - 1) / BK : 0;

  const char* Ab = reinterpret_cast<const char*>(g.A);
  const char* Wb = reinterpret_cast<const char*>(g.W);
  uint4 ra[A_CH], rb[B_CH];

  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      const int c = tid + i * NT, row = c / CHR, kk = k0 + (c % CHR) * EPC;
      const int gm = m0 + row;
      ra[i] = (gm < g.M && kk < ke)
                  ? *reinterpret_cast<const uint4*>(Ab + ((long long)gm * g.lda + kk) * sizeof(T))
                  : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
      const int c = tid + i * NT, row = c / CHR, kk = k0 + (c % CHR) * EPC;
      const int gn = n0 + row;
      rb[i] = (gn < g.N && kk < ke)
                  ? *reinterpret_cast<const uint4*>(Wb + ((long long)gn * g.ldw + kk) * sizeof(T))
                  : make_uint4(0, 0, 0, 0);
    }
  };
  auto lstore = [&](int buf) {
    char* sA = smem + buf * STAGE;
    char* sB = sA + BM * PITCH;
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      const int c = tid + i * NT;
      *reinterpret_cast<uint4*>(sA + (c / CHR) * PITCH + (c % CHR) * 16) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
      const int c = tid + i * NT;
      *reinterpret_cast<uint4*>(sB + (c / CHR) * PITCH + (c % CHR) * 16) = rb[i];
    }
  };

  floatx16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  if (nk > 0) {
    gload(kb);
    lstore(0);
  }
  __syncthreads();
  const int arow = wm * WTM + (lane & 31);
  const int brow = wn * WTN + (lane & 31);
  const int khalf = (lane >> 5) * F::LANE_K * (int)sizeof(T);
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload(kb + (kt + 1) * BK);
    const char* sA = smem + buf * STAGE;
    const char* sB = sA + BM * PITCH;
#pragma unroll
    for (int ks = 0; ks < BK / F::KE; ++ks) {
      const int koff = ks * F::KE * (int)sizeof(T) + khalf;
      typename F::type fa[TM], fb[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) fa[i] = F::load(sA + (arow + 32 * i) * PITCH + koff);
#pragma unroll
      for (int j = 0; j < TN; ++j) fb[j] = F::load(sB + (brow + 32 * j) * PITCH + koff);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) mfma32(acc[i][j], fa[i], fb[j]);
    }
    if (kt + 1 < nk) lstore(buf ^ 1);
    __syncthreads();
  }
  epilogue<T, EPI, TM, TN>(g, acc, m0 + wm * WTM, n0 + wn * WTN, lane, blockIdx.y);
}

// Sum of split-K partial slabs in a fixed order, then the epilogue.
template <bool RESID>
__global__ void splitk_reduce_kernel(const float* __restrict__ ws, int split, long long stride,
                                     float* __restrict__ out, int M, int N, int ld) {
  const long long n4 = (long long)M * (N >> 2);
  for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < n4;
       i += (long long)gridDim.x * blockDim.x) {
    const long long row = i / (N >> 2), c = (i % (N >> 2)) * 4;
    const long long src = row * N + c;
    float4 s = *reinterpret_cast<const float4*>(ws + src);
    for (int z = 1; z < split; ++z) {
      const float4 p = *reinterpret_cast<const float4*>(ws + z * stride + src);
      s.x += p.x; s.y += p.y; s.z += p.z; s.w += p.w;
    }
    float4* d = reinterpret_cast<float4*>(out + row * ld + c);
    if (RESID) {
      float4 o = *d;
      o.x += s.x; o.y += s.y; o.z += s.z; o.w += s.w;
      *d = o;
    } else {
      *d = s;
    }
  }
}

constexpr int BM_ = 128, BN_ = 128, WM_ = 2, WN_ = 2;

template <typename T, int EPI>
hipError_t run(const GemmArgs& a, int split, hipStream_t s) {
  const int nbm = (a.M + BM_ - 1) / BM_, nbn = (a.N + BN_ - 1) / BN_;
  dim3 grid(nbm * nbn, split);
  hipLaunchKernelGGL((gemm_kernel<T, BM_, BN_, WM_, WN_, EPI>), grid, dim3(WM_ * WN_ * 64), 0, s, a);
  return hipGetLastError();
}

template <typename T>
hipError_t dispatch(Epi epi, const GemmArgs& a, int split, float* ws, hipStream_t s) {
  if (split > 1) {
    if (epi != EPI_F32 && epi != EPI_RESID) return hipErrorInvalidValue;
    GemmArgs p = a;
    p.out0 = ws;
    p.ld0 = a.N;
    p.split_stride = (long long)a.M * a.N;
    hipError_t e = run<T, EPI_PARTIAL>(p, split, s);
    if (e != hipSuccess) return e;
    const long long n4 = (long long)a.M * (a.N / 4);
    const int blocks = (int)std::min<long long>((n4 + 255) / 256, 4096);
    if (epi == EPI_RESID)
      hipLaunchKernelGGL(splitk_reduce_kernel<true>, dim3(blocks), dim3(256), 0, s, ws, split,
                         p.split_stride, reinterpret_cast<float*>(a.out0), a.M, a.N, a.ld0);
    else
      hipLaunchKernelGGL(splitk_reduce_kernel<false>, dim3(blocks), dim3(256), 0, s, ws, split,
                         p.split_stride, reinterpret_cast<float*>(a.out0), a.M, a.N, a.ld0);
    return hipGetLastError();
  }
  switch (epi) {
    case EPI_F32: return run<T, EPI_F32>(a, 1, s);
    case EPI_RESID: return run<T, EPI_RESID>(a, 1, s);
    case EPI_GATE: return run<T, EPI_GATE>(a, 1, s);
    case EPI_SWIGLU: return run<T, EPI_SWIGLU>(a, 1, s);
    case EPI_QKV: return run<T, EPI_QKV>(a, 1, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int gemm_k_tile(bool bf16) { return bf16 ? 64 : 32; }

hipError_t launch_gemm(bool bf16, Epi epi, const GemmArgs& a, int split, float* ws,
                       hipStream_t s) {
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  GemmArgs g = a;
  const int bk = gemm_k_tile(bf16);
  if (split < 1) split = 1;
  // K range per split: a whole number of K tiles
  const int tiles = (a.K + bk - 1) / bk;
  if (split > tiles) split = tiles > 0 ? tiles : 1;
  g.k_split = ((tiles + split - 1) / split) * bk;
  split = (a.K + g.k_split - 1) / g.k_split;
  if (split < 1) split = 1;
  return bf16 ? dispatch<bf16_t>(epi, g, split, ws, s) : dispatch<float>(epi, g, split, ws, s);
}

}  // namespace s1
