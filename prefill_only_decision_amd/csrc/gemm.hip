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
#include <type_traits>

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

template <typename T, int BM, int BN, int WM, int WN>
struct GemmShape {
  static constexpr int NT = WM * WN * 64;
  static constexpr int ROWB = 128;                  // bytes of one K tile row
  static constexpr int BK = ROWB / (int)sizeof(T);
  static constexpr int PITCH = ROWB + 16;           // padded LDS row
  static constexpr int CHR = ROWB / 16;             // 16-byte chunks per row
  static constexpr int EPC = 16 / (int)sizeof(T);   // elements per chunk
  static constexpr int A_CH = BM * CHR / NT;        // chunks per thread
  static constexpr int B_CH = BN * CHR / NT;
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int TM = WTM / 32, TN = WTN / 32;
  static constexpr int STAGE = (BM + BN) * PITCH;   // LDS bytes per stage
  static_assert(A_CH * NT == BM * CHR && B_CH * NT == BN * CHR, "tile/thread mismatch");
};

template <int A_CH, int B_CH>
struct Stage {
  uint4 a[A_CH];
  uint4 b[B_CH];
};

struct TileCtx {
  const char* pa;     // this thread's first A chunk (row m0 + tid / CHR)
  const char* pw;     // this thread's first W chunk (row n0 + tid / CHR)
  long long sa, sw;   // bytes between the thread's successive chunks (uniform)
  int ra, rw;         // rows still valid below the thread's first chunk (A, W)
  int kc;             // this thread's K offset inside a K tile (elements)
  int ke;
};

// Loads of one K tile into registers.  GUARD zero-fills rows past M / N and
// columns past the end of the K range.
template <typename T, typename S, bool GUARD>
__device__ __forceinline__ void gload(Stage<S::A_CH, S::B_CH>& st, const TileCtx& c, int k0) {
  constexpr int RSTEP = S::NT / S::CHR;   // rows between a thread's chunks
  const long long ko = (long long)k0 * sizeof(T);
  const bool kok = !GUARD || k0 + c.kc < c.ke;
#pragma unroll
  for (int i = 0; i < S::A_CH; ++i) {
    const uint4* src = reinterpret_cast<const uint4*>(c.pa + i * c.sa + ko);
    st.a[i] = (!GUARD || (kok && i * RSTEP < c.ra)) ? *src : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < S::B_CH; ++i) {
    const uint4* src = reinterpret_cast<const uint4*>(c.pw + i * c.sw + ko);
    st.b[i] = (!GUARD || (kok && i * RSTEP < c.rw)) ? *src : make_uint4(0, 0, 0, 0);
  }
}

template <typename S, int BM>
__device__ __forceinline__ void lstore(const Stage<S::A_CH, S::B_CH>& st, char* stage, int tid) {
  char* sB = stage + BM * S::PITCH;
#pragma unroll
  for (int i = 0; i < S::A_CH; ++i) {
    const int q = tid + i * S::NT;
    *reinterpret_cast<uint4*>(stage + (q / S::CHR) * S::PITCH + (q % S::CHR) * 16) = st.a[i];
  }
#pragma unroll
  for (int i = 0; i < S::B_CH; ++i) {
    const int q = tid + i * S::NT;
    *reinterpret_cast<uint4*>(sB + (q / S::CHR) * S::PITCH + (q % S::CHR) * 16) = st.b[i];
  }
}

template <typename T, typename S, int BM>
__device__ __forceinline__ void compute(floatx16 (&acc)[S::TM][S::TN], const char* stage, int arow, int brow,
                                        int khalf) {
  typedef Frag<T> F;
  const char* sB = stage + BM * S::PITCH;
#pragma unroll
  for (int ks = 0; ks < S::BK / F::KE; ++ks) {
    const int koff = ks * F::KE * (int)sizeof(T) + khalf;
    typename F::type fa[S::TM], fb[S::TN];
#pragma unroll
    for (int i = 0; i < S::TM; ++i) fa[i] = F::load(stage + (arow + 32 * i) * S::PITCH + koff);
#pragma unroll
    for (int j = 0; j < S::TN; ++j) fb[j] = F::load(sB + (brow + 32 * j) * S::PITCH + koff);
#pragma unroll
    for (int i = 0; i < S::TM; ++i)
#pragma unroll
      for (int j = 0; j < S::TN; ++j) mfma32(acc[i][j], fa[i], fb[j]);
  }
}

// Two register stages alternate: the loads for K tile k+2 are issued while
// tile k is multiplied from LDS and tile k+1 waits in the other stage, so a
// load has two compute phases to arrive.  Interior tiles skip bounds checks.
template <typename T, typename S, int BM, bool GUARD>
__device__ __forceinline__ void mainloop(floatx16 (&acc)[S::TM][S::TN], const TileCtx& c, char* smem, int tid,
                                         int kb, int nk, int arow, int brow, int khalf) {
  Stage<S::A_CH, S::B_CH> st0, st1;
  if (nk <= 0) return;
  gload<T, S, GUARD>(st0, c, kb);
  lstore<S, BM>(st0, smem, tid);
  if (nk > 1) gload<T, S, GUARD>(st1, c, kb + S::BK);
  __syncthreads();
  for (int kt = 0; kt < nk; kt += 2) {
    if (kt + 2 < nk) gload<T, S, GUARD>(st0, c, kb + (kt + 2) * S::BK);
    compute<T, S, BM>(acc, smem, arow, brow, khalf);
    if (kt + 1 < nk) lstore<S, BM>(st1, smem + S::STAGE, tid);
    __syncthreads();
    if (kt + 1 >= nk) break;
    if (kt + 3 < nk) gload<T, S, GUARD>(st1, c, kb + (kt + 3) * S::BK);
    compute<T, S, BM>(acc, smem + S::STAGE, arow, brow, khalf);
    if (kt + 2 < nk) lstore<S, BM>(st0, smem, tid);
    __syncthreads();
  }
}

template <typename T, int BM, int BN, int WM, int WN, int EPI>
__global__ void __launch_bounds__(WM * WN * 64)
__attribute__((amdgpu_waves_per_eu(BM * BN <= 128 * 128 ? 2 : 1, 2)))
gemm_kernel(GemmArgs g) {
  typedef GemmShape<T, BM, BN, WM, WN> S;
  __shared__ __attribute__((aligned(16))) char smem[2 * S::STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int nbm = (g.M + BM - 1) / BM;
  const int t = xcd_remap(blockIdx.x, gridDim.x);
  const int m0 = (t % nbm) * BM, n0 = (t / nbm) * BN;
  const int kb = blockIdx.y * g.k_split;
  TileCtx c;
  c.ke = min(g.K, kb + g.k_split);
  c.kc = (tid % S::CHR) * S::EPC;
  const int r0 = tid / S::CHR;
  // rows past the end are clamped to a valid row; their loads are masked
  const int ra = min(m0 + r0, g.M - 1), rw = min(n0 + r0, g.N - 1);
  c.pa = reinterpret_cast<const char*>(g.A) + ((long long)ra * g.lda + c.kc) * sizeof(T);
  c.pw = reinterpret_cast<const char*>(g.W) + ((long long)rw * g.ldw + c.kc) * sizeof(T);
  constexpr int RSTEP = S::NT / S::CHR;
  c.sa = (long long)RSTEP * g.lda * sizeof(T);
  c.sw = (long long)RSTEP * g.ldw * sizeof(T);
  c.ra = g.M - (m0 + r0);
  c.rw = g.N - (n0 + r0);
  const int nk = c.ke > kb ? (c.ke - kb + S::BK - 1) / S::BK : 0;

  floatx16 acc[S::TM][S::TN];
#pragma unroll
  for (int i = 0; i < S::TM; ++i)
#pragma unroll
    for (int j = 0; j < S::TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int arow = wm * S::WTM + (lane & 31);
  const int brow = wn * S::WTN + (lane & 31);
  const int khalf = (lane >> 5) * Frag<T>::LANE_K * (int)sizeof(T);
  mainloop<T, S, BM, true>(acc, c, smem, tid, kb, nk, arow, brow, khalf);
  epilogue<T, EPI, S::TM, S::TN>(g, acc, m0 + wm * S::WTM, n0 + wn * S::WTN, lane, blockIdx.y);
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

template <int BM, int BN, int WM, int WN>
struct Tile {
  static constexpr int bm = BM, bn = BN, wm = WM, wn = WN;
};
// Tile shapes (rows x cols per workgroup, waves as rows x cols).  Config 0
// runs every epilogue; the others are compiled for the plain and split-K
// epilogues so that shapes can be compared on the same operands.
using Tile0 = Tile<128, 128, 2, 2>;
using Tile1 = Tile<128, 64, 2, 1>;
using Tile2 = Tile<256, 128, 2, 2>;
using Tile3 = Tile<128, 256, 2, 2>;
using Tile4 = Tile<256, 256, 2, 2>;
using Tile5 = Tile<64, 128, 1, 2>;
constexpr int N_TILE_CFG = 6;

template <typename T, typename TL, int EPI>
hipError_t run(const GemmArgs& a, int split, hipStream_t s) {
  const int nbm = (a.M + TL::bm - 1) / TL::bm, nbn = (a.N + TL::bn - 1) / TL::bn;
  dim3 grid(nbm * nbn, split);
  hipLaunchKernelGGL((gemm_kernel<T, TL::bm, TL::bn, TL::wm, TL::wn, EPI>), grid, dim3(TL::wm * TL::wn * 64), 0,
                     s, a);
  return hipGetLastError();
}

template <typename T, int EPI>
hipError_t run_cfg(const GemmArgs& a, int split, int cfg, hipStream_t s) {
  if constexpr (EPI == EPI_F32 || EPI == EPI_PARTIAL) {
    if constexpr (sizeof(T) == 2) {
      switch (cfg) {
        case 1: return run<T, Tile1, EPI>(a, split, s);
        case 2: return run<T, Tile2, EPI>(a, split, s);
        case 3: return run<T, Tile3, EPI>(a, split, s);
        case 4: return run<T, Tile4, EPI>(a, split, s);
        case 5: return run<T, Tile5, EPI>(a, split, s);
        default: break;
      }
    }
  }
  return run<T, Tile0, EPI>(a, split, s);
}

template <typename T>
hipError_t dispatch(Epi epi, const GemmArgs& a, int split, float* ws, int cfg, hipStream_t s) {
  if (split > 1) {
    if (epi != EPI_F32 && epi != EPI_RESID) return hipErrorInvalidValue;
    GemmArgs p = a;
    p.out0 = ws;
    p.ld0 = a.N;
    p.split_stride = (long long)a.M * a.N;
    hipError_t e = run_cfg<T, EPI_PARTIAL>(p, split, cfg, s);
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
    case EPI_F32: return run_cfg<T, EPI_F32>(a, 1, cfg, s);
    case EPI_RESID: return run<T, Tile0, EPI_RESID>(a, 1, s);
    case EPI_GATE: return run<T, Tile0, EPI_GATE>(a, 1, s);
    case EPI_SWIGLU: return run<T, Tile0, EPI_SWIGLU>(a, 1, s);
    case EPI_QKV: return run<T, Tile0, EPI_QKV>(a, 1, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int gemm_k_tile(bool bf16) { return bf16 ? 64 : 32; }

int gemm_tile_configs() { return N_TILE_CFG; }

hipError_t launch_gemm(bool bf16, Epi epi, const GemmArgs& a, int split, float* ws, hipStream_t s,
                       int cfg) {
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
  return bf16 ? dispatch<bf16_t>(epi, g, split, ws, cfg, s) : dispatch<float>(epi, g, split, ws, cfg, s);
}

}  // namespace s1
