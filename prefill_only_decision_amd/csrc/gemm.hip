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
#include <climits>
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
// silu(a) = a / (1 + e^-a), with the hardware reciprocal (1 ulp) in place of
// an IEEE division: the epilogues run once per output with one wave per
// SIMD, so their VALU time is not hidden.  e^-a = inf gives a * 0.
__device__ __forceinline__ float silu(float a) { return a * __builtin_amdgcn_rcpf(1.f + __expf(-a)); }

// The rotate-half pair (a1, a2) by (cos, sin), with the multiply-adds
// written out: left to contraction, kernels of different tiles could fuse
// different products and round a row differently.
__device__ __forceinline__ float rope_lo(float a1, float a2, float2 cs) { return fmaf(a1, cs.x, -(a2 * cs.y)); }
__device__ __forceinline__ float rope_hi(float a1, float a2, float2 cs) { return fmaf(a2, cs.x, a1 * cs.y); }

// Global-memory views of the epilogue's pointers: through the generic
// pointers of GemmArgs the compiler emits flat accesses, whose results it
// must wait for with vmcnt(0) and lgkmcnt(0) (flat operations may complete
// out of order), one element at a time.
template <typename T>
using gmem = __attribute__((address_space(1))) T;
template <typename T>
__device__ __forceinline__ gmem<T>* gptr(void* p) {
  return (gmem<T>*)p;
}
template <typename T>
__device__ __forceinline__ const gmem<T>* gptr(const void* p) {
  return (const gmem<T>*)p;
}

// ------------------------------------------- deferred RMSNorm (bf16 model)
// The pre-norm before a projection, x / rms(x) * gain, is split between the
// GEMM that updates the residual x and the GEMM that consumes it: the gain
// multiplies the consumer's weight columns (folded in at load), the consumer
// reads x rounded to bf16 and multiplies each accumulator row by 1 / rms of
// its row; the producer's epilogue writes that bf16 copy and the 1 / rms.
// No separate norm pass reads and writes the rows.
//
// The sum of squares of a row is taken in one fixed tree whatever the tile
// configuration (so a row's scale does not depend on the number of rows):
// each aligned block of 32 columns is summed as a butterfly (pairs of columns
// c, c ^ 16, then c ^ 8, ... c ^ 1), the blocks as a pairwise tree over
// aligned groups of 2^k blocks, missing blocks past N being zero.

// Exchange with lane ^ M inside each half-wave (ds_swizzle, bit mode).
template <int M>
__device__ __forceinline__ float swz_xor(float v) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x1F | (M << 10)));
}

// v[r]: one value per accumulator row r of a 32 x 32 MFMA tile, column lane &
// 31.  Sums each row over the 32 columns of its half-wave (reduce-scatter:
// each exchange halves the values a lane keeps) and returns in lanes 2q and
// 2q + 1 the sum for accumulator row r = q & 15 (row acc_row(r, lane)).
__device__ __forceinline__ float half_wave_row_sum(float (&v)[16], int lane) {
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const bool b = lane & 16;
    const float keep = b ? v[k + 8] : v[k], send = b ? v[k] : v[k + 8];
    v[k] = keep + swz_xor<16>(send);
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const bool b = lane & 8;
    const float keep = b ? v[k + 4] : v[k], send = b ? v[k] : v[k + 4];
    v[k] = keep + swz_xor<8>(send);
  }
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const bool b = lane & 4;
    const float keep = b ? v[k + 2] : v[k], send = b ? v[k] : v[k + 2];
    v[k] = keep + swz_xor<4>(send);
  }
  {
    const bool b = lane & 2;
    const float keep = b ? v[1] : v[0], send = b ? v[0] : v[1];
    v[0] = keep + swz_xor<2>(send);
  }
  return v[0] + swz_xor<1>(v[0]);
}

template <int N>
__device__ __forceinline__ float tree_sum(float (&v)[N]) {
#pragma unroll
  for (int w = 1; w < N; w *= 2)
#pragma unroll
    for (int u = 0; u + w < N; u += 2 * w) v[u] += v[u + w];
  return v[0];
}

// Residual epilogue: out0 (fp32) += the tile.  With the deferred norm
// (bf16, rs_out set) it also writes the updated rows rounded to bf16 and,
// per row and aligned group of TG = 2^k column blocks (TG the largest power
// of two dividing TN), the partial sum of squares, to
// ss_parts[(cn0 / 32 / TG + group) * ss_ld + row].  Each 32 x 32 tile's
// squares are summed while its values are in registers; no lane skips the
// exchanges (columns past N count as zero).
// Sums over the 32 columns of each half-wave for TN tiles at once, one
// exchange level for all tiles before the next (independent chains
// interleave); the same reduce-scatter as half_wave_row_sum.
template <int TN>
__device__ __forceinline__ void half_wave_row_sums(float (&v)[TN][16], float (&out)[TN], int lane) {
  const bool b16 = lane & 16, b8 = lane & 8, b4 = lane & 4, b2 = lane & 2;
#pragma unroll
  for (int k = 0; k < 8; ++k)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const float keep = b16 ? v[j][k + 8] : v[j][k], send = b16 ? v[j][k] : v[j][k + 8];
      v[j][k] = keep + swz_xor<16>(send);
    }
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const float keep = b8 ? v[j][k + 4] : v[j][k], send = b8 ? v[j][k] : v[j][k + 4];
      v[j][k] = keep + swz_xor<8>(send);
    }
#pragma unroll
  for (int k = 0; k < 2; ++k)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const float keep = b4 ? v[j][k + 2] : v[j][k], send = b4 ? v[j][k] : v[j][k + 2];
      v[j][k] = keep + swz_xor<4>(send);
    }
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const float keep = b2 ? v[j][1] : v[j][0], send = b2 ? v[j][0] : v[j][1];
    v[j][0] = keep + swz_xor<2>(send);
  }
#pragma unroll
  for (int j = 0; j < TN; ++j) out[j] = v[j][0] + swz_xor<1>(v[j][0]);
}

// Residual epilogue: out0 (fp32) += the tile.  The rows are addressed
// through a buffer resource over rows rm0 .. M - 1: loads past the end read
// zero and stores past it are dropped, so no access is predicated and a row
// block's loads (all its column tiles) are issued together before its stores.
// With the deferred norm (bf16, rs_out set) it also writes the updated rows
// rounded to bf16 (staged in LDS when `stage` is given) and, per row and
// aligned group of TG = 2^k column blocks (TG the largest power of two
// dividing TN), the partial sum of squares, to ss_parts[(cn0 / 32 / TG +
// group) * ss_ld + row]; columns past N count as zero.
template <typename T, int TM, int TN>
__device__ __forceinline__ void epilogue_resid(const GemmArgs& g, floatx16 (&acc)[TM][TN], int rm0, int cn0,
                                               int lane, char* stage = nullptr, int pitch = 0, int wr0 = 0,
                                               int wc0 = 0) {
  constexpr int TG = TN & -TN;
  const int cl = lane & 31;
  bool defer = false;
  if constexpr (sizeof(T) == 2) defer = g.rs_out != nullptr;
  const int nrow = max(0, g.M - rm0);
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
      static_cast<float*>(g.out0) + (long long)rm0 * g.ld0, (short)0, nrow * g.ld0 * 4, 0x00020000);
  // byte offsets: this lane's row and column parts (a column past N is sent
  // out of range)
  const int lrow = 4 * (lane >> 5) * g.ld0 * 4;
  int coff[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j) coff[j] = cn0 + 32 * j + cl < g.N ? lrow + (cn0 + 32 * j + cl) * 4 : INT_MIN;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int rb = rm0 + 32 * i;
    float v[TN][16];
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        v[j][r] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
            rx, coff[j] + (32 * i + 8 * (r >> 2) + (r & 3)) * g.ld0 * 4, 0, 0));
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        v[j][r] += acc[i][j][r];
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v[j][r]), rx,
                                              coff[j] + (32 * i + 8 * (r >> 2) + (r & 3)) * g.ld0 * 4, 0, 0);
      }
    if (defer) {
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int col = cn0 + 32 * j + cl;
        const bool cok = col < g.N;
        if (stage != nullptr) {   // the bf16 copy staged for whole-row 16-byte stores
#pragma unroll
          for (int r = 0; r < 16; ++r)
            *reinterpret_cast<bf16_t*>(stage + (wr0 + 32 * i + acc_row(r, lane)) * pitch +
                                       2 * (wc0 + 32 * j + cl)) = f2bf(v[j][r]);
        } else {
          gmem<bf16_t>* hb = gptr<bf16_t>(g.norm_out);
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = rb + acc_row(r, lane);
            if (cok && row < g.M) hb[(long long)row * g.N + col] = f2bf(v[j][r]);
          }
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) v[j][r] = cok ? __fmul_rn(v[j][r], v[j][r]) : 0.f;
      }
      float part[TN];
      half_wave_row_sums<TN>(v, part, lane);
      const int row = rb + acc_row((lane >> 1) & 15, lane);
#pragma unroll
      for (int q = 0; q < TN / TG; ++q) {
        float sg[TG];
#pragma unroll
        for (int u = 0; u < TG; ++u) sg[u] = part[q * TG + u];
        const float t = tree_sum(sg);
        // only groups with a column before N: their slots exist ([N / 32]
        // rows).  Device-scope stores (coherent across the XCDs' L2s): the
        // row block's last workgroup, possibly on another XCD, reads them.
        if ((lane & 1) == 0 && row < g.M && cn0 + 32 * TG * q < g.N)
          __hip_atomic_store(g.ss_parts + (long long)((cn0 >> 5) / TG + q) * g.ss_ld + row, t, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}

// After the epilogue of a residual tile with the deferred norm: the last
// workgroup to finish row block tm (one ticket per column tile) turns the
// block's partial sums into rs_out.  The partial sums travel as device-scope
// stores and loads (no cache of one XCD holds a stale copy); every wave waits
// for its own stores to complete before the workgroup barrier that precedes
// the ticket, so a workgroup's ticket is taken only after all its partial
// sums are visible.  Nothing waits on another workgroup.  The slots are
// summed as aligned 16-slot pairwise trees, then a pairwise tree over those:
// for any slot width this is the fixed tree above, zero-padded.  Every
// thread of the workgroup calls this (it has barriers).
template <int BM, int NT, int TG>
__device__ __forceinline__ void resid_norm_finish(const GemmArgs& g, int m0, int tm, int nbn) {
  __shared__ int s_last;
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's stores are complete
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned old = __hip_atomic_fetch_add(g.tickets + tm, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int last = old + 1 == (unsigned)nbn;
    if (last) __hip_atomic_store(g.tickets + tm, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);   // for the next launch
    s_last = last;
  }
  __syncthreads();
  if (!s_last) return;
  const int ns = (g.N + 32 * TG - 1) / (32 * TG);
  for (int t = threadIdx.x; t < BM; t += NT) {
    const int row = m0 + t;
    if (row >= g.M) break;
    float* p = g.ss_parts + row;
    // 16 groups of 16 slots; the groups' tree is built as a binary counter
    // (lv[k]: the pending left subtree of 2^k groups)
    float lv[4] = {0.f, 0.f, 0.f, 0.f}, total = 0.f;
#pragma unroll 1
    for (int q = 0; q < 16; ++q) {
      float v[16];
#pragma unroll
      for (int k = 0; k < 16; ++k) v[k] = 0.f;
      if (16 * q < ns) {
#pragma unroll
        for (int k = 0; k < 16; ++k)
          if (16 * q + k < ns)
            v[k] = __hip_atomic_load(p + (long long)(16 * q + k) * g.ss_ld, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      float x = tree_sum(v);
      if (q & 1) {
        x = lv[0] + x;
        if (q & 2) {
          x = lv[1] + x;
          if (q & 4) {
            x = lv[2] + x;
            if (q & 8) total = lv[3] + x;
            else lv[3] = x;
          } else {
            lv[2] = x;
          }
        } else {
          lv[1] = x;
        }
      } else {
        lv[0] = x;
      }
    }
    gptr<float>(g.rs_out)[row] = rsqrtf(total / g.N + g.norm_eps);
  }
}

// The residual epilogue of a BM x BN workgroup tile whose operand stages
// (smem_bytes) are free: with the deferred norm the bf16 copy of the updated
// rows goes through LDS and out as 16-byte chunks of whole rows (written
// from the accumulators every store would be 2 bytes per lane, half a cache
// line of two rows per wave store).  Every thread calls this.
template <int TM, int TN, int BM, int BN, int NT>
__device__ __forceinline__ void epilogue_resid_tile(const GemmArgs& g, floatx16 (&acc)[TM][TN], int m0, int n0,
                                                    int wr0, int wc0, int lane, char* smem, int smem_bytes) {
  constexpr int PP = BN * 2 + 16;
  const int pitch = BM * PP <= smem_bytes ? PP : BN * 2;
  const bool stage = g.rs_out != nullptr && g.N % 8 == 0 && BM * BN * 2 <= smem_bytes;
  if (stage) {
    __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) lgkmcnt(0): no operand DMA still lands in the stages
    __syncthreads();                      // every wave is done reading the stages
  }
  epilogue_resid<bf16_t, TM, TN>(g, acc, m0 + wr0, n0 + wc0, lane, stage ? smem : nullptr, pitch, wr0, wc0);
  if (!stage) return;
  __syncthreads();
  typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
  constexpr int CPR = BN / 8;
#pragma unroll 4
  for (int c = threadIdx.x; c < BM * CPR; c += NT) {
    const int rl = c / CPR, ch = c % CPR;
    const int row = m0 + rl, col = n0 + ch * 8;
    if (row >= g.M || col >= g.N) continue;
    *reinterpret_cast<gmem<u32x4v>*>(gptr<bf16_t>(g.norm_out) + (long long)row * g.N + col) =
        *reinterpret_cast<const u32x4v*>(smem + rl * pitch + ch * 16);
  }
}

// Consumer side: the scale of row m0 + tid (tid < BM; 1 without row_scale),
// loaded at kernel entry so that its latency hides under the operand loads,
// stored to LDS after the main loop; the epilogues multiply each accumulator
// by its row's scale where they read it (a separate pass over the
// accumulators costs the largest tiles registers).
// The load is issued whether or not there is a row scale (from the operand A
// when there is none, always in range: M rows of at least two bf16): a load
// on one path only leaves the compiler's wait counting at the main loop's
// head imprecise, and it then waits more inside the loop.
template <int BM>
__device__ __forceinline__ float row_scale_load(const GemmArgs& g, int m0) {
  const bool has = g.row_scale != nullptr;
  const float* p = has ? g.row_scale : static_cast<const float*>(g.A);
  const float v = gptr<float>(p)[min(m0 + min((int)threadIdx.x, BM - 1), g.M - 1)];
  return has ? v : 1.f;
}
template <int BM>
__device__ __forceinline__ const float* row_scale_store(float rsv, float* rsl) {
  if (threadIdx.x < BM) rsl[threadIdx.x] = rsv;
  __syncthreads();
  return rsl;
}
constexpr bool scaled_epi(int epi) { return epi == EPI_SWIGLU || epi == EPI_GATE || epi == EPI_QKV; }

// Loads an epilogue needs (the residual, positions, RoPE factors) are issued
// for a whole 32-row MFMA tile before its stores: a store to the output may
// alias a later load as far as the compiler knows, so element-by-element
// read-modify-write would wait for the memory latency once per element.
template <typename T, int EPI, int TM, int TN, bool RS = false>
__device__ __forceinline__ void epilogue(const GemmArgs& g, floatx16 (&acc)[TM][TN], int rm0,
                                         int cn0, int lane, int split_idx, const float* rsw = nullptr) {
  const int cl = lane & 31;
  // RS: the row scale of accumulator r of MFMA row block i (rsw: LDS, the
  // wave's first row); without it the factor is the constant 1 and folds away
  auto scl = [&](int i, int r) { return RS ? rsw[32 * i + acc_row(r, lane)] : 1.f; };
  if constexpr (EPI == EPI_RESID) {
    epilogue_resid<T, TM, TN>(g, acc, rm0, cn0, lane);
  } else if constexpr (EPI == EPI_SWIGLU || EPI == EPI_QKV) {
    static_assert(TN % 2 == 0, "pair epilogues need both MFMA tiles of a 64-column block in the wave");
#pragma unroll
    for (int j = 0; j < TN; j += 2) {
      const int cb = cn0 + 32 * j;                    // multiple of 64
      if (cb >= g.N) continue;
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int rb = rm0 + 32 * i;
        if constexpr (EPI == EPI_SWIGLU) {
          const int f = (cb >> 1) + cl;
          if (f >= g.n_valid) continue;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = rb + acc_row(r, lane);
            const float sc = scl(i, r);
            if (row < g.M)
              gptr<T>(g.out0)[(long long)row * g.ld0 + f] =
                  from_f<T>(silu(acc[i][j][r] * sc) * (acc[i][j + 1][r] * sc));
          }
        } else if (cb < g.nsplit2) {
          // rotate-half pair (d, d + hd/2): permuted to columns (cb+cl, cb+32+cl)
          const int hc = cb % g.head_dim;
          const int dim = 32 * (hc >> 6) + cl;
          float2 cs[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = min(rb + acc_row(r, lane), g.M - 1);
            const unsigned long long bits =
                gptr<unsigned long long>(g.rope)[(long long)gptr<int>(g.pos)[row] * (g.head_dim >> 1) + dim];
            cs[r] = __builtin_bit_cast(float2, bits);
          }
          gmem<T>* dst;
          long long base;
          int ld;
          if (cb < g.nsplit) {
            dst = gptr<T>(g.out0);
            base = cb;
            ld = g.ld0;
          } else {
            dst = gptr<T>(g.out1);
            base = cb - g.nsplit;
            ld = g.ld1;
          }
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = rb + acc_row(r, lane);
            if (row >= g.M) continue;
            const float sc = scl(i, r);
            const float a1 = acc[i][j][r] * sc, a2 = acc[i][j + 1][r] * sc;
            const long long off = (long long)row * ld + base;
            dst[off + cl] = from_f<T>(rope_lo(a1, a2, cs[r]));
            dst[off + 32 + cl] = from_f<T>(rope_hi(a1, a2, cs[r]));
          }
        } else {
          gmem<T>* dst = gptr<T>(g.out2);
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = rb + acc_row(r, lane);
            if (row >= g.M) continue;
            const long long off = (long long)row * g.ld2 + (cb - g.nsplit2);
            const float sc = scl(i, r);
            dst[off + cl] = from_f<T>(acc[i][j][r] * sc);
            if (cb + 32 < g.N) dst[off + 32 + cl] = from_f<T>(acc[i][j + 1][r] * sc);
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
        const int rb = rm0 + 32 * i;
        {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = rb + acc_row(r, lane);
            if (row >= g.M) continue;
            float v = acc[i][j][r];
            if constexpr (EPI == EPI_GATE) v *= scl(i, r);
            if constexpr (EPI == EPI_F32) {
              gptr<float>(g.out0)[(long long)row * g.ld0 + col] = v;
            } else if constexpr (EPI == EPI_PARTIAL) {
              gptr<float>(g.out0)[split_idx * g.split_stride + (long long)row * g.ld0 + col] = v;
            } else if constexpr (EPI == EPI_GATE) {
              // gate columns raw here, finished by the wave's loop below
              if (col < g.nsplit)
                gptr<T>(g.out0)[(long long)row * g.ld0 + col] = from_f<T>(v);
              else if (g.out2 == nullptr || col < g.nsplit2)
                gptr<float>(g.out1)[(long long)row * g.ld1 + (col - g.nsplit)] = v;
              else
                gptr<float>(g.out2)[(long long)row * g.ld1 + (col - g.nsplit2)] = v;
            }
          }
        }
      }
    }
  }
  if constexpr (EPI == EPI_GATE) {
    // the nonlinearity of the wave's gate columns, once per element in a
    // small loop (unrolled over every accumulator it costs the main loop of
    // the largest tiles registers); the wave's own raw stores are complete
    // after vmcnt(0)
    const int g0 = max(cn0, g.nsplit), ngc = min(cn0 + 32 * TN, g.N) - g0;
    if (ngc > 0) {
      __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
      for (int e = lane; e < 32 * TM * ngc; e += 64) {
        const int row = rm0 + e / ngc, col = g0 + e % ngc;
        if (row >= g.M) continue;
        const bool beta = g.out2 != nullptr && col >= g.nsplit2;
        gmem<float>* p = beta ? gptr<float>(g.out2) + (long long)row * g.ld1 + (col - g.nsplit2)
                              : gptr<float>(g.out1) + (long long)row * g.ld1 + (col - g.nsplit);
        const float v = *p;
        *p = beta ? 1.f / (1.f + __expf(-v)) : log_sigmoid(v);
      }
    }
  }
}

// bf16 outputs of the LA in-projection (q | k | v) and of the attention QKV
// projection (RoPE applied), staged through the workgroup's drained operand
// stages and written as 16-byte chunks of whole rows.  Written straight from
// the accumulators, every store is 2 bytes per lane and a wave's store
// covers half a cache line of two rows; at 16,925 rows that doubled the LA
// in-projection (1,192 against 592 us for the same tiles with 4-byte stores
// on MI355X).  The fp32 decay-gate columns (and write strengths) still go
// straight from the lanes.  Needs 16-byte aligned destinations (ld0, ld1,
// ld2, nsplit and nsplit2 multiples of 8); the caller checks.
template <int EPI, int TM, int TN, int BM, int BN, int NT, bool RS = false>
__device__ __forceinline__ void epilogue_staged(const GemmArgs& g, floatx16 (&acc)[TM][TN], int m0, int n0,
                                                int wr0, int wc0, int lane, char* smem, int smem_bytes,
                                                const float* rsl = nullptr) {
  constexpr int PP = BN * 2 + 16;
  const int pitch = BM * PP <= smem_bytes ? PP : BN * 2;   // pad the rows when the stages allow
  typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
  const int cl = lane & 31;
  __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) lgkmcnt(0): no operand DMA still lands in the stages
  __syncthreads();                      // every wave is done reading the stages
  auto put = [&](int rl, int cll, float v) {
    *reinterpret_cast<bf16_t*>(smem + rl * pitch + 2 * cll) = f2bf(v);
  };
  // RS: the row scale of tile-local row rl (LDS); otherwise the constant 1
  auto scl = [&](int rl) { return RS ? rsl[rl] : 1.f; };
  if constexpr (EPI == EPI_QKV) {
#pragma unroll
    for (int j = 0; j < TN; j += 2) {
      const int cbl = wc0 + 32 * j, cb = n0 + cbl;   // multiple of 64
      if (cb >= g.N) continue;
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int rbl = wr0 + 32 * i;
        if (cb < g.nsplit2) {
          const int hc = cb % g.head_dim;
          const int dim = 32 * (hc >> 6) + cl;
          float2 cs[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = min(m0 + rbl + acc_row(r, lane), g.M - 1);
            const unsigned long long bits =
                gptr<unsigned long long>(g.rope)[(long long)gptr<int>(g.pos)[row] * (g.head_dim >> 1) + dim];
            cs[r] = __builtin_bit_cast(float2, bits);
          }
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int rl = rbl + acc_row(r, lane);
            const float sc = scl(rl);
            const float a1 = acc[i][j][r] * sc, a2 = acc[i][j + 1][r] * sc;
            put(rl, cbl + cl, rope_lo(a1, a2, cs[r]));
            put(rl, cbl + 32 + cl, rope_hi(a1, a2, cs[r]));
          }
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int rl = rbl + acc_row(r, lane);
            const float sc = scl(rl);
            put(rl, cbl + cl, acc[i][j][r] * sc);
            put(rl, cbl + 32 + cl, acc[i][j + 1][r] * sc);
          }
        }
      }
    }
  } else {   // EPI_GATE
    // nsplit is a multiple of 32, so each 32-column block is all q|k|v
    // (staged as bf16) or all gate columns; the gate columns are written raw
    // here and finished by the small loop below: with the nonlinearity
    // unrolled over every accumulator the epilogue's code and registers
    // spilled into the main loop of the largest tiles
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int cbl = wc0 + 32 * j, cb = n0 + cbl;
      const int cll = cbl + cl, col = cb + cl;
      if (cb < g.nsplit) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int rl = wr0 + 32 * i + acc_row(r, lane);
            put(rl, cll, acc[i][j][r] * scl(rl));
          }
      } else if (col < g.N) {
        gmem<float>* dst = (g.out2 != nullptr && col >= g.nsplit2) ? gptr<float>(g.out2) + (col - g.nsplit2)
                                                                  : gptr<float>(g.out1) + (col - g.nsplit);
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = m0 + wr0 + 32 * i + acc_row(r, lane);
            if (row < g.M) dst[(long long)row * g.ld1] = acc[i][j][r] * scl(row - m0);
          }
      }
    }
  }
  __syncthreads();   // staged rows complete; raw gate values visible to the workgroup
  if constexpr (EPI == EPI_GATE) {
    if (n0 + BN > g.nsplit) {
      const int g0 = max(n0, g.nsplit), ngc = min(n0 + BN, g.N) - g0;
      for (int e = threadIdx.x; e < BM * ngc; e += NT) {
        const int row = m0 + e / ngc, col = g0 + e % ngc;
        if (row >= g.M) continue;
        const bool beta = g.out2 != nullptr && col >= g.nsplit2;
        gmem<float>* p = beta ? gptr<float>(g.out2) + (long long)row * g.ld1 + (col - g.nsplit2)
                              : gptr<float>(g.out1) + (long long)row * g.ld1 + (col - g.nsplit);
        const float v = *p;
        *p = beta ? 1.f / (1.f + __expf(-v)) : log_sigmoid(v);
      }
    }
  }
  constexpr int CPR = BN / 8;                     // 16-byte chunks per row
  const int lim = EPI == EPI_GATE ? min(g.N, g.nsplit) : g.N;
#pragma unroll 4
  for (int c = threadIdx.x; c < BM * CPR; c += NT) {
    const int rl = c / CPR, ch = c % CPR;
    const int row = m0 + rl, col = n0 + ch * 8;
    if (row >= g.M || col >= lim) continue;
    const u32x4v val = *reinterpret_cast<const u32x4v*>(smem + rl * pitch + ch * 16);
    gmem<bf16_t>* dst;
    if (EPI == EPI_GATE || col < g.nsplit)
      dst = gptr<bf16_t>(g.out0) + (long long)row * g.ld0 + col;
    else if (col < g.nsplit2)
      dst = gptr<bf16_t>(g.out1) + (long long)row * g.ld1 + (col - g.nsplit);
    else
      dst = gptr<bf16_t>(g.out2) + (long long)row * g.ld2 + (col - g.nsplit2);
    *reinterpret_cast<gmem<u32x4v>*>(dst) = val;
  }
}

// Whether a launch can use epilogue_staged (16-byte aligned destinations).
__host__ __device__ inline bool staged_ok(int epi, const GemmArgs& g) {
  if (epi == EPI_GATE) return g.ld0 % 8 == 0 && g.nsplit % 32 == 0;
  if (epi == EPI_QKV) return g.ld0 % 8 == 0 && g.ld1 % 8 == 0 && g.ld2 % 8 == 0 && g.nsplit % 8 == 0 &&
                             g.nsplit2 % 8 == 0 && g.N % 8 == 0;
  return false;
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

template <typename T, int BM, int BN, int WM, int WN, int EPI, bool RS = false>
__global__ void __launch_bounds__(WM * WN * 64)
__attribute__((amdgpu_waves_per_eu(BM * BN <= 128 * 128 ? 2 : 1, 2)))
gemm_kernel(GemmArgs g) {
  typedef GemmShape<T, BM, BN, WM, WN> S;
  static_assert(BM <= S::NT, "one row scale per thread");
  __shared__ __attribute__((aligned(16))) char smem[2 * S::STAGE];
  __shared__ float rsl[RS ? BM : 1];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int nbm = (g.M + BM - 1) / BM;
  const int t = xcd_remap(blockIdx.x, gridDim.x);
  const int m0 = (t % nbm) * BM, n0 = (t / nbm) * BN;
  const float rsv = RS ? row_scale_load<BM>(g, m0) : 1.f;
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
  if constexpr (RS)
    epilogue<T, EPI, S::TM, S::TN, true>(g, acc, m0 + wm * S::WTM, n0 + wn * S::WTN, lane, blockIdx.y,
                                         row_scale_store<BM>(rsv, rsl) + wm * S::WTM);
  else
    epilogue<T, EPI, S::TM, S::TN>(g, acc, m0 + wm * S::WTM, n0 + wn * S::WTN, lane, blockIdx.y);
  if constexpr (EPI == EPI_RESID && sizeof(T) == 2) {
    if (g.rs_out != nullptr) resid_norm_finish<BM, S::NT, (S::TN & -S::TN)>(g, m0, t % nbm, (g.N + BN - 1) / BN);
  }
}

// ------------------------------------------------------- bf16 LDS-DMA kernel
// Operand tiles travel from global memory straight into LDS
// (buffer_load_dwordx4 ... lds: lane l writes 16 bytes at M0 + 16 l), NS
// stages deep, one barrier per K tile.  An LDS row holds BK bf16 (RB bytes)
// without padding; 16-byte chunk c of row r is stored at chunk position
// c ^ ((r >> SH) & (CH - 1)), which spreads the 16 rows that one
// ds_read_b128 phase reads (same chunk, consecutive rows) over all 64 LDS
// banks.  Rows past M or N read as zero through the buffer range check, so
// no load is predicated.  The K range must be a whole number of K tiles.
template <int BM_, int BN_, int WM_, int WN_, int BK_, int NS_>
struct L3 {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, BK = BK_, NS = NS_;
  static constexpr int NWAVE = WM * WN, NT = NWAVE * 64;
  static constexpr int RB = BK * 2, CH = RB / 16, RPI = 1024 / RB;
  static constexpr int SH = RB >= 256 ? 0 : (RB == 128 ? 1 : 2);
  static constexpr int A_BYTES = BM * RB, STAGE = (BM + BN) * RB;
  static constexpr int A_INS = BM * RB / 1024 / NWAVE, B_INS = BN * RB / 1024 / NWAVE;
  static constexpr int INS = A_INS + B_INS;
  static constexpr int WTM = BM / WM, WTN = BN / WN, TM = WTM / 32, TN = WTN / 32;
  static constexpr int KS = BK / 16;
  // workgroups per CU the LDS allows (at most 2 are asked for)
  static constexpr int OCC = NS * STAGE * 2 <= 160 * 1024 ? 2 : 1;
  static_assert(A_INS * NWAVE * 1024 == BM * RB && B_INS * NWAVE * 1024 == BN * RB, "tile/wave mismatch");
  static_assert(NS >= 2 && NS * STAGE <= 160 * 1024, "LDS budget");
  static_assert(INS * (NS - 1) < 64, "vmcnt range");
  static_assert(KS % 2 == 0, "operand double buffer alternates per k-step");
};

typedef int int32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;

// Buffer resource over `bytes` bytes from `base` (raw buffer, no stride):
// offsets at or past `bytes` read as zero.
__device__ __forceinline__ int32x4 buffer_rsrc(const void* base, int bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  int32x4 r;
  // readfirstlane: the values are wave-uniform; saying so keeps them in
  // scalar registers, which the buffer instructions require
  r.x = __builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(a)));
  r.y = __builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(a >> 32) & 0xFFFFu));
  r.z = __builtin_amdgcn_readfirstlane(bytes);
  r.w = 0x00020000;
  return r;
}

// One 16-byte-per-lane load from a buffer straight into LDS: lane l's bytes
// land at lds + 16 l.  Written as inline assembly so that the compiler does
// not treat later LDS reads as dependent on it (it would wait for every
// outstanding load before each of them); completion is awaited explicitly
// with vmcnt before the barrier that publishes the stage.  m0 is written
// here and is used by nothing else in these kernels.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(int32x4 rsrc, uint32_t lds, int voff, int soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :: "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(rsrc),
                  "s"(__builtin_amdgcn_readfirstlane(soff)) : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ __forceinline__ uint32_t lds_addr(const char* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const lds_char*)p));
}

// As dma16, 4 bytes per lane (lane l's at lds + 4 l).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma4(int32x4 rsrc, uint32_t lds, int voff, int soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, %3 offen lds"
               :: "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(rsrc),
                  "s"(__builtin_amdgcn_readfirstlane(soff)) : "memory", "m0");
}
#pragma clang diagnostic pop

// The row scales of rows m0 .. m0 + BM - 1 into LDS by LDS-DMA at kernel
// entry, ahead of the operand loads: no register is held through the main
// loop for them.  Blocks of 64 rows go to waves in turn (the LDS array holds
// BM rounded up to 64: rows past the tile are loaded and not used); rows past
// M read zero.  row_scale_sync, after the main loop, waits for the wave's own
// DMA and meets the other waves.
constexpr int rsl_rows(int bm) { return (bm + 63) / 64 * 64; }
template <int BM, int NW = 4>
__device__ __forceinline__ void row_scale_dma(const GemmArgs& g, int m0, const float* rsl, int wave, int lane) {
  if (g.row_scale == nullptr) return;
  const int32x4 r = buffer_rsrc(g.row_scale + m0, (g.M - m0) * 4);
#pragma unroll
  for (int b = 0; b < rsl_rows(BM) / 64; b += NW)
    if (b + wave < rsl_rows(BM) / 64)
      dma4(r, lds_addr(reinterpret_cast<const char*>(rsl)) + (b + wave) * 256, ((b + wave) * 64 + lane) * 4, 0);
}
__device__ __forceinline__ const float* row_scale_sync(const float* rsl) {
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
  __syncthreads();
  return rsl;
}

// The epilogue's arguments, loaded into SGPRs at kernel entry.  Left to the
// compiler, these kernel-argument loads are placed just before the main loop
// and are still outstanding when it starts; the waitcnt pass then has to
// assume the worst at the loop head and waits for every LDS read there.
template <typename T>
__device__ __forceinline__ T pin_sgpr(T v) {
  asm volatile("" : "+s"(v));
  return v;
}
// The RoPE/KV epilogue needs the most arguments; pinned, they can leave too
// few scalar registers for the 128-bit buffer resource of the operand loads,
// so that epilogue reads its arguments where it uses them.
template <int EPI>
__device__ __forceinline__ GemmArgs pin_epilogue_args(const GemmArgs& g) {
  GemmArgs e = g;
  if constexpr (EPI == EPI_QKV || EPI == EPI_GATE) return e;
  e.M = pin_sgpr(g.M);
  e.N = pin_sgpr(g.N);
  e.out0 = pin_sgpr(g.out0);
  e.out1 = pin_sgpr(g.out1);
  e.out2 = pin_sgpr(g.out2);
  e.ld0 = pin_sgpr(g.ld0);
  e.ld1 = pin_sgpr(g.ld1);
  e.ld2 = pin_sgpr(g.ld2);
  e.nsplit = pin_sgpr(g.nsplit);
  e.nsplit2 = pin_sgpr(g.nsplit2);
  e.n_valid = pin_sgpr(g.n_valid);
  e.head_dim = pin_sgpr(g.head_dim);
  e.pos = pin_sgpr(g.pos);
  e.rope = pin_sgpr(g.rope);
  e.split_stride = pin_sgpr(g.split_stride);
  return e;
}

// s_waitcnt with vmcnt(vm), lgkmcnt(0), expcnt untouched.
template <int VM>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(VM >= 0 && VM < 64, "");
  __builtin_amdgcn_s_waitcnt((VM & 0xF) | (0x7 << 4) | ((VM >> 4) << 14));
}

// Tile index -> (tile row, tile column): column-major inside groups of GM
// tile rows, so that the tiles running at the same time on one XCD share a
// few A row blocks and W column blocks.
template <int GM>
__device__ __forceinline__ void tile_coords(int t, int nbm, int nbn, int& tm, int& tn) {
  const int group = GM * nbn;
  const int first = (t / group) * GM;
  const int gsz = min(nbm - first, GM);
  const int u = t - (t / group) * group;
  tm = first + u % gsz;
  tn = u / gsz;
}

template <typename S>
__device__ __forceinline__ int dma_voffset(int b, int lane, int ld) {
  const int r = b * S::RPI + lane / S::CH;
  const int c = (lane % S::CH) ^ ((r >> S::SH) & (S::CH - 1));
  return r * ld * 2 + c * 16;
}

template <typename S, int EPI, bool RS = false>
__global__ void __launch_bounds__(S::NT)
__attribute__((amdgpu_waves_per_eu(S::OCC, S::OCC)))
gemm_lds_kernel(GemmArgs g) {
  static_assert(S::BM <= S::NT, "one row scale per thread");
  __shared__ __attribute__((aligned(1024))) char smem[S::NS * S::STAGE];
  __shared__ __attribute__((aligned(16))) float rsl[RS ? rsl_rows(S::BM) : 1];
  const GemmArgs e = pin_epilogue_args<EPI>(g);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / S::WN, wn = wave % S::WN;
  const int nbm = (g.M + S::BM - 1) / S::BM, nbn = (g.N + S::BN - 1) / S::BN;
  int tm, tn;
  tile_coords<8>(xcd_remap(blockIdx.x, gridDim.x), nbm, nbn, tm, tn);
  const int m0 = tm * S::BM, n0 = tn * S::BN;
  if constexpr (RS) row_scale_dma<S::BM, S::NWAVE>(g, m0, rsl, wave, lane);
  const int kb = blockIdx.y * g.k_split;
  const int ke = min(g.K, kb + g.k_split);
  const int nk = ke > kb ? (ke - kb) / S::BK : 0;

  const char* abase = reinterpret_cast<const char*>(g.A) + (long long)m0 * g.lda * 2;
  const char* wbase = reinterpret_cast<const char*>(g.W) + (long long)n0 * g.ldw * 2;
  const int32x4 ra = buffer_rsrc(abase, (g.M - m0) * g.lda * 2);
  const int32x4 rw = buffer_rsrc(wbase, (g.N - n0) * g.ldw * 2);
  const uint32_t lds0 = lds_addr(smem);
  int va[S::A_INS], vw[S::B_INS];
#pragma unroll
  for (int i = 0; i < S::A_INS; ++i) va[i] = dma_voffset<S>(wave * S::A_INS + i, lane, g.lda);
#pragma unroll
  for (int i = 0; i < S::B_INS; ++i) vw[i] = dma_voffset<S>(wave * S::B_INS + i, lane, g.ldw);

  auto issue = [&](int kt) {
    const uint32_t st = lds0 + (kt % S::NS) * S::STAGE;
    const int so = (kb + kt * S::BK) * 2;
#pragma unroll
    for (int i = 0; i < S::A_INS; ++i) dma16(ra, st + (wave * S::A_INS + i) * 1024, va[i], so);
#pragma unroll
    for (int i = 0; i < S::B_INS; ++i) dma16(rw, st + S::A_BYTES + (wave * S::B_INS + i) * 1024, vw[i], so);
  };

  // per-lane LDS offsets of the MFMA operands for each k-step of a K tile
  const int l32 = lane & 31, h = lane >> 5;
  const int sw = (l32 >> S::SH) & (S::CH - 1);
  int oa[S::KS], ob[S::KS];
#pragma unroll
  for (int s = 0; s < S::KS; ++s) {
    const int pos = ((2 * s + h) ^ sw) * 16;
    oa[s] = (wm * S::WTM + l32) * S::RB + pos;
    ob[s] = S::A_BYTES + (wn * S::WTN + l32) * S::RB + pos;
  }

  floatx16 acc[S::TM][S::TN];
#pragma unroll
  for (int i = 0; i < S::TM; ++i)
#pragma unroll
    for (int j = 0; j < S::TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // All NS stages start full (tiles 0 .. NS-1); at the end of K tile kt its
  // stage is refilled with tile kt + NS.  Operands are read one k-step
  // ahead, and the barrier that publishes tile kt + 1 sits between the
  // reads for the last k-step of tile kt and that k-step's MFMAs, so the
  // matrix pipeline keeps running across it.
  bf16x8 fa[2][S::TM], fb[2][S::TN];
  auto read_ops = [&](int buf, const char* st, int s) {
#pragma unroll
    for (int i = 0; i < S::TM; ++i)
      fa[buf][i] = as_frag(*reinterpret_cast<const uint4*>(st + oa[s] + i * 32 * S::RB));
#pragma unroll
    for (int j = 0; j < S::TN; ++j)
      fb[buf][j] = as_frag(*reinterpret_cast<const uint4*>(st + ob[s] + j * 32 * S::RB));
  };
  // The host guarantees at least one K tile per split.
#pragma unroll
  for (int p = 0; p < S::NS; ++p)
    if (p < nk) issue(p);
  if (S::NS - 1 < nk) wait_vm_lgkm0<(S::NS - 1) * S::INS>();
  else wait_vm_lgkm0<0>();
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  read_ops(0, smem, 0);
  // nothing else (kernel-argument loads included) may be outstanding on
  // lgkmcnt when the loop is entered, or every iteration waits for all
  __builtin_amdgcn_s_waitcnt(0xC07F);
  // The last K tile is peeled so that the loop body is straight-line code
  // around the barrier: the compiler then sees the last k-step's operands
  // as complete (explicit lgkmcnt(0)) and does not hold its MFMAs until the
  // next tile's reads return.
  auto tile = [&](int kt, auto last_tag) {
    constexpr bool LAST = decltype(last_tag)::value;
    const char* st = smem + (kt % S::NS) * S::STAGE;
#pragma unroll
    for (int s = 0; s < S::KS; ++s) {
      // reads for the next k-step are issued before this k-step's MFMAs
      // (sched_barrier keeps the scheduler from sinking them)
      if (s + 1 < S::KS) {
        read_ops((s + 1) & 1, st, s + 1);
        __builtin_amdgcn_sched_barrier(0);
      } else if (!LAST) {
        // tile kt + 1 landed (own loads) and own reads of tile kt done
        if (kt + S::NS - 1 < nk) wait_vm_lgkm0<(S::NS - 2) * S::INS>();
        else wait_vm_lgkm0<0>();
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (kt + S::NS < nk) issue(kt + S::NS);
        read_ops((s + 1) & 1, smem + ((kt + 1) % S::NS) * S::STAGE, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int i = 0; i < S::TM; ++i)
#pragma unroll
        for (int j = 0; j < S::TN; ++j) mfma32(acc[i][j], fa[s & 1][i], fb[s & 1][j]);
    }
  };
  for (int kt = 0; kt + 1 < nk; ++kt) tile(kt, std::false_type{});
  if (nk > 0) tile(nk - 1, std::true_type{});
  if constexpr (EPI == EPI_GATE || EPI == EPI_QKV) {
    // bf16 q|k|v outputs: only the staged form is compiled here (the host
    // runs unaligned launches on the register-staged kernel); both forms in
    // one kernel cost registers and code in the main loop
    static_assert(S::BM * S::BN * 2 <= S::NS * S::STAGE, "the staged output tile must fit the operand stages");
    if constexpr (RS)
      epilogue_staged<EPI, S::TM, S::TN, S::BM, S::BN, S::NT, true>(e, acc, m0, n0, wm * S::WTM, wn * S::WTN, lane,
                                                                    smem, S::NS * S::STAGE, row_scale_sync(rsl));
    else
      epilogue_staged<EPI, S::TM, S::TN, S::BM, S::BN, S::NT>(e, acc, m0, n0, wm * S::WTM, wn * S::WTN, lane, smem,
                                                              S::NS * S::STAGE);
  } else if constexpr (EPI == EPI_RESID) {
    epilogue_resid_tile<S::TM, S::TN, S::BM, S::BN, S::NT>(e, acc, m0, n0, wm * S::WTM, wn * S::WTN, lane, smem,
                                                           S::NS * S::STAGE);
    if (g.rs_out != nullptr) resid_norm_finish<S::BM, S::NT, (S::TN & -S::TN)>(g, m0, tm, nbn);
  } else if constexpr (RS) {
    epilogue<bf16_t, EPI, S::TM, S::TN, true>(e, acc, m0 + wm * S::WTM, n0 + wn * S::WTN, lane, blockIdx.y,
                                              row_scale_sync(rsl) + wm * S::WTM);
  } else {
    epilogue<bf16_t, EPI, S::TM, S::TN>(e, acc, m0 + wm * S::WTM, n0 + wn * S::WTN, lane, blockIdx.y);
  }
}

// ------------------------------------------------- bf16 wide-wave kernel
// Every wave owns a TM x TN block of 32 x 32 MFMA tiles (128 x 128, or
// 64 x 192), which cuts the LDS bytes read per MFMA against 64 x 64 waves:
// 8 KB of operands feed 12 or 16 MFMAs.  Four waves, WM x WN, make the
// workgroup tile.  Operands travel global -> LDS as in the kernel above
// (same swizzle, same buffer range checks, same read-ahead and barrier
// placement).
template <int WM_, int WN_, int TM_, int TN_, int BK_, int NS_>
struct W4 {
  static constexpr int WM = WM_, WN = WN_, BK = BK_, NS = NS_;
  static constexpr int NWAVE = WM * WN, NT = NWAVE * 64;
  static constexpr int TM = TM_, TN = TN_, WTM = 32 * TM, WTN = 32 * TN;
  static constexpr int BM = WM * WTM, BN = WN * WTN;
  static constexpr int RB = BK * 2, CH = RB / 16, RPI = 1024 / RB;
  static constexpr int SH = RB >= 256 ? 0 : (RB == 128 ? 1 : 2);
  static constexpr int A_BYTES = BM * RB, STAGE = (BM + BN) * RB;
  static constexpr int A_INS = BM * RB / 1024 / NWAVE, B_INS = BN * RB / 1024 / NWAVE;
  static constexpr int INS = A_INS + B_INS;
  static constexpr int KS = BK / 16;
  static_assert(KS % 2 == 0, "operand double buffer alternates per k-step");
  static_assert(A_INS * NWAVE * 1024 == BM * RB && B_INS * NWAVE * 1024 == BN * RB, "tile/wave mismatch");
  static_assert(NS >= 2 && NS * STAGE <= 160 * 1024, "LDS budget");
  static_assert(INS * (NS - 1) < 64, "vmcnt range");
};

template <typename S, int EPI, bool RS = false>
__global__ void __launch_bounds__(S::NT) __attribute__((amdgpu_waves_per_eu(1, 1)))
gemm_wide_kernel(GemmArgs g) {
  static_assert(S::BM <= S::NT, "one row scale per thread");
  __shared__ __attribute__((aligned(1024))) char smem[S::NS * S::STAGE];
  __shared__ __attribute__((aligned(16))) float rsl[RS ? rsl_rows(S::BM) : 1];
  const GemmArgs e = pin_epilogue_args<EPI>(g);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / S::WN, wn = wave % S::WN;
  const int nbm = (g.M + S::BM - 1) / S::BM, nbn = (g.N + S::BN - 1) / S::BN;
  int tm, tn;
  tile_coords<8>(xcd_remap(blockIdx.x, gridDim.x), nbm, nbn, tm, tn);
  const int m0 = tm * S::BM, n0 = tn * S::BN;
  if constexpr (RS) row_scale_dma<S::BM, S::NWAVE>(g, m0, rsl, wave, lane);
  const int kb = blockIdx.y * g.k_split;
  const int ke = min(g.K, kb + g.k_split);
  const int nk = (ke - kb) / S::BK;   // >= 1: the host gives every split a K tile

  const char* abase = reinterpret_cast<const char*>(g.A) + (long long)m0 * g.lda * 2;
  const char* wbase = reinterpret_cast<const char*>(g.W) + (long long)n0 * g.ldw * 2;
  const int32x4 ra = buffer_rsrc(abase, (g.M - m0) * g.lda * 2);
  const int32x4 rw = buffer_rsrc(wbase, (g.N - n0) * g.ldw * 2);
  const uint32_t lds0 = lds_addr(smem);
  int va[S::A_INS], vw[S::B_INS];
#pragma unroll
  for (int i = 0; i < S::A_INS; ++i) va[i] = dma_voffset<S>(wave * S::A_INS + i, lane, g.lda);
#pragma unroll
  for (int i = 0; i < S::B_INS; ++i) vw[i] = dma_voffset<S>(wave * S::B_INS + i, lane, g.ldw);
  auto issue = [&](int kt) {
    const uint32_t st = lds0 + (kt % S::NS) * S::STAGE;
    const int so = (kb + kt * S::BK) * 2;
#pragma unroll
    for (int i = 0; i < S::A_INS; ++i) dma16(ra, st + (wave * S::A_INS + i) * 1024, va[i], so);
#pragma unroll
    for (int i = 0; i < S::B_INS; ++i) dma16(rw, st + S::A_BYTES + (wave * S::B_INS + i) * 1024, vw[i], so);
  };

  const int l32 = lane & 31, h = lane >> 5;
  const int sw = (l32 >> S::SH) & (S::CH - 1);
  int oa[S::KS], ob[S::KS];
#pragma unroll
  for (int u = 0; u < S::KS; ++u) {
    const int pos = ((2 * u + h) ^ sw) * 16;
    oa[u] = (wm * S::WTM + l32) * S::RB + pos;
    ob[u] = S::A_BYTES + (wn * S::WTN + l32) * S::RB + pos;
  }

  floatx16 acc[S::TM][S::TN];
#pragma unroll
  for (int i = 0; i < S::TM; ++i)
#pragma unroll
    for (int j = 0; j < S::TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  bf16x8 fa[2][S::TM], fb[2][S::TN];
  auto read_ops = [&](int buf, const char* st, int u) {
#pragma unroll
    for (int i = 0; i < S::TM; ++i) fa[buf][i] = as_frag(*reinterpret_cast<const uint4*>(st + oa[u] + i * 32 * S::RB));
#pragma unroll
    for (int j = 0; j < S::TN; ++j) fb[buf][j] = as_frag(*reinterpret_cast<const uint4*>(st + ob[u] + j * 32 * S::RB));
  };
#pragma unroll
  for (int p = 0; p < S::NS; ++p)
    if (p < nk) issue(p);
  if (S::NS - 1 < nk) wait_vm_lgkm0<(S::NS - 1) * S::INS>();
  else wait_vm_lgkm0<0>();
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  read_ops(0, smem, 0);
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): nothing outstanding entering the loop

  auto tile = [&](int kt, auto last_tag) {
    constexpr bool LAST = decltype(last_tag)::value;
    const char* st = smem + (kt % S::NS) * S::STAGE;
#pragma unroll
    for (int u = 0; u < S::KS; ++u) {
      if (u + 1 < S::KS) {
        read_ops((u + 1) & 1, st, u + 1);
        __builtin_amdgcn_sched_barrier(0);
      } else if (!LAST) {
        if (kt + S::NS - 1 < nk) wait_vm_lgkm0<(S::NS - 2) * S::INS>();
        else wait_vm_lgkm0<0>();
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (kt + S::NS < nk) issue(kt + S::NS);
        read_ops((u + 1) & 1, smem + ((kt + 1) % S::NS) * S::STAGE, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int i = 0; i < S::TM; ++i)
#pragma unroll
        for (int j = 0; j < S::TN; ++j) mfma32(acc[i][j], fa[u & 1][i], fb[u & 1][j]);
    }
  };
  for (int kt = 0; kt + 1 < nk; ++kt) tile(kt, std::false_type{});
  tile(nk - 1, std::true_type{});
  if constexpr (EPI == EPI_GATE || EPI == EPI_QKV) {
    // only the staged form, as in the LDS kernels (with both forms compiled
    // in, the gate epilogue spilled registers into the main loop of these
    // 256 x 256 tiles)
    static_assert(S::BM * S::BN * 2 <= S::NS * S::STAGE, "the staged output tile must fit the operand stages");
    if constexpr (RS)
      epilogue_staged<EPI, S::TM, S::TN, S::BM, S::BN, S::NT, true>(e, acc, m0, n0, wm * S::WTM, wn * S::WTN, lane,
                                                                    smem, S::NS * S::STAGE, row_scale_sync(rsl));
    else
      epilogue_staged<EPI, S::TM, S::TN, S::BM, S::BN, S::NT>(e, acc, m0, n0, wm * S::WTM, wn * S::WTN, lane, smem,
                                                              S::NS * S::STAGE);
  } else if constexpr (EPI == EPI_RESID) {
    epilogue_resid_tile<S::TM, S::TN, S::BM, S::BN, S::NT>(e, acc, m0, n0, wm * S::WTM, wn * S::WTN, lane, smem,
                                                           S::NS * S::STAGE);
    if (g.rs_out != nullptr) resid_norm_finish<S::BM, S::NT, (S::TN & -S::TN)>(g, m0, tm, nbn);
  } else if constexpr (RS) {
    epilogue<bf16_t, EPI, S::TM, S::TN, true>(e, acc, m0 + wm * S::WTM, n0 + wn * S::WTN, lane, blockIdx.y,
                                              row_scale_sync(rsl) + wm * S::WTM);
  } else {
    epilogue<bf16_t, EPI, S::TM, S::TN>(e, acc, m0 + wm * S::WTM, n0 + wn * S::WTN, lane, blockIdx.y);
  }
}

// ----------------------------------------------- bf16 weight-direct kernel
// For GEMMs of a few hundred rows the weights stream from HBM once while the
// activations stay in L2, and the launch is bound by the operand stream into
// each CU.  Measured on MI355X at the FFN gate/up shape, LDS-DMA staging of
// both operands (the kernels above) delivers about 33 GB/s per CU and this
// kernel about 42 GB/s, whatever the number of active CUs.
// Here the weight operand bypasses LDS: the weights are stored at load time
// in fragment order (for each 32-row block and each 16-element K step, the
// 64 lanes' 16-byte MFMA B operands as one contiguous 1 KB block), and each
// wave loads its own columns' fragments with coalesced 1 KB loads into a
// register ring DK K tiles deep.  Only the activation tile goes through LDS
// (LDS-DMA as above, NS stages of BM x 64).  The four waves split the
// columns: a wave owns all BM rows and 32 TN columns, so no weight byte is
// loaded twice in a workgroup.  Every load is issued unconditionally (tile
// indices past the end are clamped to the last tile), so the number of loads
// between an activation stage and its wait is fixed.
template <int TM_, int TN_, int NS_, int DK_>
struct WD {
  static constexpr int TM = TM_, TN = TN_, NS = NS_, DK = DK_;
  static constexpr int NWAVE = 4, NT = 256;
  static constexpr int BK = 64, RB = 128, CH = 8, RPI = 8, SH = 1;
  static constexpr int BM = 32 * TM, WTN = 32 * TN, BN = NWAVE * WTN;
  static constexpr int STAGE = BM * RB;
  static constexpr int A_INS = BM * RB / 1024 / NWAVE;   // activation DMA loads per K tile and wave
  static constexpr int KS = BK / 16;
  static constexpr int W_INS = KS * TN;                  // weight loads per K tile and wave
  // loads issued after the activation DMA of tile kt + 1 when tile kt waits for it
  static constexpr int VM_A = W_INS + (NS - 2) * (A_INS + W_INS);
  static constexpr int VM_PRO = (NS - 1) * A_INS + DK * W_INS;
  static_assert(A_INS * NWAVE * 1024 == BM * RB, "tile/wave mismatch");
  static_assert(NS >= 2 && NS * STAGE <= 160 * 1024, "LDS budget");
  static_assert(VM_A < 64 && VM_PRO < 64, "vmcnt range");
};

// SwiGLU over weights packed with gate/up interleaved in blocks of 16 rows:
// in each 32-column MFMA tile, lane column c < 16 holds gate feature f0 + c
// and lane c + 16 its up partner, for the same 16 rows.  For each pair of
// accumulator rows (2k, 2k + 1) one exchange between the two lanes gives the
// gate lane the up value of row 2k and the up lane the gate value of row
// 2k + 1, so that every lane computes one output.  The outputs are staged
// through LDS (free once the main loop has drained) and written as whole
// 16-byte chunks of each output row: a tile's BN / 2 features of one row are
// contiguous in the output.  Needs ld0 and n_valid multiples of 8 (the host
// checks) and the tile's first feature 16-byte aligned.
template <typename S, bool RS = false>
__device__ __forceinline__ void epilogue_swiglu16_lds(const GemmArgs& g, floatx16 (&acc)[S::TM][S::TN], int m0,
                                                      int n0, int wave, int lane, char* smem,
                                                      const float* rsl = nullptr) {
  constexpr int FT = S::BN / 2;                   // features per tile
  constexpr int PITCH = FT * 2 + 16;              // bytes per staged row
  constexpr int CPR = FT * 2 / 16;                // 16-byte chunks per row
  static_assert(S::BM * PITCH <= S::NS * S::STAGE, "staging must fit the operand stages");
  typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
  const int cl = lane & 31;
  const bool gate_lane = cl < 16;
  __syncthreads();                                // every wave is done reading the stages
#pragma unroll
  for (int j = 0; j < S::TN; ++j) {
    const int fl = wave * (S::WTN / 2) + 16 * j + (cl & 15);
#pragma unroll
    for (int i = 0; i < S::TM; ++i) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        // RS: each value times its row's scale (LDS); otherwise times the constant 1
        const float a0 = acc[i][j][2 * k] * (RS ? rsl[32 * i + acc_row(2 * k, lane)] : 1.f);
        const float a1 = acc[i][j][2 * k + 1] * (RS ? rsl[32 * i + acc_row(2 * k + 1, lane)] : 1.f);
        const float got = __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(gate_lane ? a1 : a0), 0x401F));
        const float gt = gate_lane ? a0 : got, up = gate_lane ? got : a1;
        const int rl = 32 * i + acc_row(2 * k + (gate_lane ? 0 : 1), lane);
        *reinterpret_cast<bf16_t*>(smem + rl * PITCH + 2 * fl) = f2bf(silu(gt) * up);
      }
    }
  }
  __syncthreads();
  const int f0 = n0 >> 1;
#pragma unroll 4
  for (int c = threadIdx.x; c < S::BM * CPR; c += S::NT) {
    const int rl = c / CPR, ch = c % CPR;
    const int row = m0 + rl, f = f0 + ch * 8;
    if (row < g.M && f < g.n_valid)
      *reinterpret_cast<gmem<u32x4v>*>(gptr<bf16_t>(g.out0) + (long long)row * g.ld0 + f) =
          *reinterpret_cast<const u32x4v*>(smem + rl * PITCH + ch * 16);
  }
}

template <typename S, int EPI, bool RS = false>
__global__ void __launch_bounds__(S::NT) __attribute__((amdgpu_waves_per_eu(1, 1)))
gemm_wd_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(1024))) char smem[S::NS * S::STAGE];
  __shared__ __attribute__((aligned(16))) float rsl[RS ? rsl_rows(S::BM) : 1];
  const GemmArgs e = pin_epilogue_args<EPI>(g);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nbm = (g.M + S::BM - 1) / S::BM, nbn = (g.N + S::BN - 1) / S::BN;
  int tm, tn;
  tile_coords<8>(xcd_remap(blockIdx.x, gridDim.x), nbm, nbn, tm, tn);
  const int m0 = tm * S::BM, n0 = tn * S::BN;
  if constexpr (RS) row_scale_dma<S::BM, S::NWAVE>(g, m0, rsl, wave, lane);
  const int nk = g.K / S::BK;   // >= 1: the host requires K to be a positive multiple of 64

  const char* abase = reinterpret_cast<const char*>(g.A) + (long long)m0 * g.lda * 2;
  const int32x4 ra = buffer_rsrc(abase, (g.M - m0) * g.lda * 2);
  const uint32_t lds0 = lds_addr(smem);
  int va[S::A_INS];
#pragma unroll
  for (int i = 0; i < S::A_INS; ++i) va[i] = dma_voffset<S>(wave * S::A_INS + i, lane, g.lda);
  auto issue_a = [&](int kt) {
    const uint32_t st = lds0 + (kt % S::NS) * S::STAGE;
    const int so = min(kt, nk - 1) * S::BK * 2;
#pragma unroll
    for (int i = 0; i < S::A_INS; ++i) dma16(ra, st + (wave * S::A_INS + i) * 1024, va[i], so);
  };

  // the wave's weight fragments: block row nb, K step ks at ((nb * ksteps + ks) * 64 + lane) * 16 bytes
  const int ksteps = g.K >> 4, nblk = (g.N + 31) >> 5;
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const gmem<u32x4>* wp[S::TN];
#pragma unroll
  for (int j = 0; j < S::TN; ++j) {
    const int nb = min((n0 + wave * S::WTN) / 32 + j, nblk - 1);
    wp[j] = gptr<u32x4>(g.W) + (long long)nb * ksteps * 64 + lane;
  }
  u32x4 wr[S::DK][S::KS][S::TN];
  auto issue_w = [&](int kt, int d) {
    const int t = min(kt, nk - 1);
#pragma unroll
    for (int u = 0; u < S::KS; ++u)
#pragma unroll
      for (int j = 0; j < S::TN; ++j) wr[d][u][j] = wp[j][(t * S::KS + u) * 64];
  };

  const int l32 = lane & 31, h = lane >> 5;
  const int sw = (l32 >> S::SH) & (S::CH - 1);
  int oa[S::KS];
#pragma unroll
  for (int u = 0; u < S::KS; ++u) oa[u] = l32 * S::RB + (((2 * u + h) ^ sw) * 16);

  floatx16 acc[S::TM][S::TN];
#pragma unroll
  for (int i = 0; i < S::TM; ++i)
#pragma unroll
    for (int j = 0; j < S::TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  bf16x8 fa[2][S::TM];
  auto read_ops = [&](int buf, const char* st, int u) {
#pragma unroll
    for (int i = 0; i < S::TM; ++i) fa[buf][i] = as_frag(*reinterpret_cast<const uint4*>(st + oa[u] + i * 32 * S::RB));
  };
#pragma unroll
  for (int p = 0; p < S::NS; ++p) issue_a(p);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int d = 0; d < S::DK; ++d) issue_w(d, d);
  __builtin_amdgcn_sched_barrier(0);
  wait_vm_lgkm0<S::VM_PRO>();
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  read_ops(0, smem, 0);
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): nothing outstanding entering the loop

  auto tile = [&](int kt, int d) {
    const char* st = smem + (kt % S::NS) * S::STAGE;
#pragma unroll
    for (int u = 0; u < S::KS; ++u) {
      if (u + 1 < S::KS) {
        read_ops((u + 1) & 1, st, u + 1);
        __builtin_amdgcn_sched_barrier(0);
      } else {
        // activation tile kt + 1 landed (own DMA) and own reads of tile kt done;
        // the barrier publishes the first and frees stage kt % NS for tile kt + NS
        wait_vm_lgkm0<S::VM_A>();
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        issue_a(kt + S::NS);
        read_ops((u + 1) & 1, smem + ((kt + 1) % S::NS) * S::STAGE, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int i = 0; i < S::TM; ++i)
#pragma unroll
        for (int j = 0; j < S::TN; ++j) mfma32(acc[i][j], fa[u & 1][i], __builtin_bit_cast(bf16x8, wr[d][u][j]));
    }
    __builtin_amdgcn_sched_barrier(0);
    issue_w(kt + S::DK, d);
    __builtin_amdgcn_sched_barrier(0);
  };
  // whole groups of DK tiles without conditions (the ring slot is static and
  // the compiler's load counts are the same on every path into the loop),
  // then the remaining tiles
  int kt0 = 0;
  for (; kt0 + S::DK <= nk; kt0 += S::DK) {
#pragma unroll
    for (int d = 0; d < S::DK; ++d) tile(kt0 + d, d);
  }
#pragma unroll
  for (int d = 0; d + 1 < S::DK; ++d)
    if (kt0 + d < nk) tile(kt0 + d, d);
  // no DMA may still be writing this workgroup's LDS when it exits
  __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) lgkmcnt(0)
  if constexpr (EPI == EPI_SWIGLU) {
    if constexpr (RS)
      epilogue_swiglu16_lds<S, true>(e, acc, m0, n0, wave, lane, smem, row_scale_sync(rsl));
    else
      epilogue_swiglu16_lds<S>(e, acc, m0, n0, wave, lane, smem);
  } else if constexpr (EPI == EPI_GATE || EPI == EPI_QKV) {
    if constexpr (RS)
      epilogue_staged<EPI, S::TM, S::TN, S::BM, S::BN, S::NT, true>(e, acc, m0, n0, 0, wave * S::WTN, lane, smem,
                                                                    S::NS * S::STAGE, row_scale_sync(rsl));
    else
      epilogue_staged<EPI, S::TM, S::TN, S::BM, S::BN, S::NT>(e, acc, m0, n0, 0, wave * S::WTN, lane, smem,
                                                              S::NS * S::STAGE);
  }
  else if constexpr (EPI == EPI_RESID) {
    epilogue_resid_tile<S::TM, S::TN, S::BM, S::BN, S::NT>(e, acc, m0, n0, 0, wave * S::WTN, lane, smem,
                                                           S::NS * S::STAGE);
    if (g.rs_out != nullptr) resid_norm_finish<S::BM, S::NT, (S::TN & -S::TN)>(g, m0, tm, nbn);
  } else
    epilogue<bf16_t, EPI, S::TM, S::TN>(e, acc, m0, n0 + wave * S::WTN, lane, 0);
}

// Fragment-order copy of a bf16 weight W[N, K] (row stride ld): 16-byte
// chunk ((nb * K/16 + ks) * 64 + l) holds row src(32 nb + l % 32), columns
// 16 ks + 8 (l / 32) .. + 7; rows at or past N are zero.  With gu16 the
// source rows are gate/up interleaved in blocks of 32 and the copy
// interleaves them in blocks of 16 (the weight-direct SwiGLU epilogue).
__global__ void frag_pack_kernel(const bf16_t* __restrict__ W, int N, int K, int ld, int gu16,
                                 uint4* __restrict__ out, long long nchunks) {
  const int ksteps = K >> 4;
  for (long long c = blockIdx.x * (long long)blockDim.x + threadIdx.x; c < nchunks;
       c += (long long)gridDim.x * blockDim.x) {
    const int l = (int)(c & 63);
    const long long rest = c >> 6;
    const int ks = (int)(rest % ksteps);
    const int n = (int)(rest / ksteps) * 32 + (l & 31);
    uint4 v = make_uint4(0, 0, 0, 0);
    if (n < N) {
      int src = n;
      if (gu16) {
        const int feat = (n >> 5) * 16 + (n & 15);
        src = (feat >> 5) * 64 + ((n & 16) ? 32 : 0) + (feat & 31);
      }
      v = *reinterpret_cast<const uint4*>(W + (long long)src * ld + ks * 16 + 8 * (l >> 5));
    }
    out[c] = v;
  }
}

template <typename S, int EPI>
hipError_t run_wd(const GemmArgs& a, hipStream_t s) {
  const int nbm = (a.M + S::BM - 1) / S::BM, nbn = (a.N + S::BN - 1) / S::BN;
  if constexpr (scaled_epi(EPI)) {
    if (a.row_scale != nullptr) {
      hipLaunchKernelGGL((gemm_wd_kernel<S, EPI, true>), dim3(nbm * nbn), dim3(S::NT), 0, s, a);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((gemm_wd_kernel<S, EPI>), dim3(nbm * nbn), dim3(S::NT), 0, s, a);
  return hipGetLastError();
}
using CfgWD1 = WD<4, 3, 4, 3>;   // 128 x 384, a wave 128 x 96, four activation stages, three weight tiles ahead
using CfgWD2 = WD<8, 2, 4, 3>;   // 256 x 256, a wave 256 x 64
using CfgWD3 = WD<6, 2, 4, 3>;   // 192 x 256, a wave 192 x 64
using CfgWD4 = WD<7, 2, 4, 3>;   // 224 x 256, a wave 224 x 64 (288 rows spill registers)

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

// Split-K reduction into a residual row, fused with the RMSNorm of the
// updated row (without the gain when w is NULL, the 1 / rms then also to
// rs): one workgroup per row, partial slabs summed in a fixed order.
constexpr int RN_MAXV = 16;   // N <= 4 * 256 * RN_MAXV
template <typename T, int MAXV>
__global__ void __launch_bounds__(256)
splitk_resid_norm_kernel(const float* __restrict__ ws, int split, long long stride, float* __restrict__ out,
                         int N, int ld, const float* __restrict__ w, T* __restrict__ nout, float eps,
                         float* __restrict__ rs) {
  __shared__ float red[4];
  const long long row = blockIdx.x;
  // every load of the row first (partials of up to SPLIT_MAX splits and the
  // residual), then the sums in split order: one memory round trip
  constexpr int SPLIT_MAX = 4;
  float4 part[MAXV][SPLIT_MAX], v[MAXV];
#pragma unroll
  for (int k = 0; k < MAXV; ++k) {
    const int c = (k * 256 + (int)threadIdx.x) * 4;
    if (c < N) {
      const long long src = row * N + c;
#pragma unroll
      for (int z = 0; z < SPLIT_MAX; ++z)
        if (z < split) part[k][z] = *reinterpret_cast<const float4*>(ws + z * stride + src);
      v[k] = *reinterpret_cast<const float4*>(out + row * ld + c);
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < MAXV; ++k) {
    const int c = (k * 256 + (int)threadIdx.x) * 4;
    if (c >= N) break;
    float4 t = part[k][0];
#pragma unroll
    for (int z = 1; z < SPLIT_MAX; ++z)
      if (z < split) {
        t.x += part[k][z].x; t.y += part[k][z].y; t.z += part[k][z].z; t.w += part[k][z].w;
      }
    float4 o = v[k];
    o.x += t.x; o.y += t.y; o.z += t.z; o.w += t.w;
    *reinterpret_cast<float4*>(out + row * ld + c) = o;
    v[k] = o;
    ss += o.x * o.x + o.y * o.y + o.z * o.z + o.w * o.w;
  }
  ss = block_sum<4>(ss, red);
  write_normed_row<T, 256, MAXV>(v, ss, N, eps, w, nout + row * N, rs ? rs + row : nullptr);
}

// the smallest row-register count that holds N columns (N <= 4 * 256 * RN_MAXV)
template <typename T>
hipError_t launch_splitk_resid_norm(const GemmArgs& a, const float* ws, int split, long long stride, hipStream_t s) {
  const int nv = (a.N + 1023) / 1024;
#define S1_RN(V)                                                                                              \
  hipLaunchKernelGGL((splitk_resid_norm_kernel<T, V>), dim3(a.M), dim3(256), 0, s, ws, split, stride,          \
                     reinterpret_cast<float*>(a.out0), a.N, a.ld0, a.norm_w, reinterpret_cast<T*>(a.norm_out),  \
                     a.norm_eps, a.rs_out)
  if (nv <= 2) S1_RN(2);
  else if (nv <= 3) S1_RN(3);
  else if (nv <= 5) S1_RN(5);
  else if (nv <= 8) S1_RN(8);
  else S1_RN(RN_MAXV);
#undef S1_RN
  return hipGetLastError();
}

// ----------------------------------------------- fp32 kernel for few tiles
// fp32 GEMMs whose 128 x 128 tiles would leave most of the chip idle (the
// small fp32 model at a few hundred rows).  A workgroup owns a 32 x 64
// output tile and its four waves take consecutive quarters of the 16-element
// K blocks of its K range.  Operands go from global memory straight into
// MFMA registers: a lane loads eight consecutive K elements of its A row and
// of its two W rows (two float4 each), and k-step j of a block contracts
// elements j (lanes 0-31) and 8 + j (lanes 32-63), the same permutation of
// K for both operands.  The next block's loads are issued before the current
// block's products.  Waves 1-3 leave their partial tiles in LDS, wave 0 adds
// them in wave order and runs the epilogue.  The K partition depends on K
// (and the split) only.
template <int EPI>
__global__ void __launch_bounds__(256) gemm_f32_ks_kernel(GemmArgs g) {
  __shared__ float red[3][32][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int cl = lane & 31, hi = lane >> 5;
  const int nbm = (g.M + 31) / 32;
  const int t = xcd_remap(blockIdx.x, gridDim.x);
  const int m0 = (t % nbm) * 32, n0 = (t / nbm) * 64;
  const int kbeg = blockIdx.y * g.k_split, kend = min(g.K, kbeg + g.k_split);
  const int nkb = kend > kbeg ? (kend - kbeg + 15) / 16 : 0;
  const int kb0 = (nkb * wave) / 4, kb1 = (nkb * (wave + 1)) / 4;
  const float* pa = static_cast<const float*>(g.A) + (long long)min(m0 + cl, g.M - 1) * g.lda + kbeg + 8 * hi;
  const float* pw0 = static_cast<const float*>(g.W) + (long long)min(n0 + cl, g.N - 1) * g.ldw + kbeg + 8 * hi;
  const float* pw1 = static_cast<const float*>(g.W) + (long long)min(n0 + 32 + cl, g.N - 1) * g.ldw + kbeg + 8 * hi;
  const int klim = kend - kbeg - 8 * hi;   // elements of this lane's half-block still inside the K range
  floatx16 acc[1][2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[0][j][r] = 0.f;
  // ops[0..1]: A, ops[2..3]: W rows n0 + cl, ops[4..5]: W rows n0 + 32 + cl
  auto load = [&](int kb, float4 (&ops)[6]) {
    const int k = kb * 16;
    const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const bool in = k + 4 * q + 4 <= klim;   // K % 4 == 0: a float4 is wholly in or out
      ops[q] = in ? *reinterpret_cast<const float4*>(pa + k + 4 * q) : z;
      ops[2 + q] = in ? *reinterpret_cast<const float4*>(pw0 + k + 4 * q) : z;
      ops[4 + q] = in ? *reinterpret_cast<const float4*>(pw1 + k + 4 * q) : z;
    }
  };
  auto el = [](const float4& v, int e) { return e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w; };
  float4 cur[6], nxt[6];
  if (kb0 < kb1) load(kb0, cur);
  for (int kb = kb0; kb < kb1; ++kb) {
    if (kb + 1 < kb1) load(kb + 1, nxt);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float a = el(cur[j >> 2], j & 3);
      mfma32(acc[0][0], a, el(cur[2 + (j >> 2)], j & 3));
      mfma32(acc[0][1], a, el(cur[4 + (j >> 2)], j & 3));
    }
#pragma unroll
    for (int q = 0; q < 6; ++q) cur[q] = nxt[q];
  }
  if (wave > 0) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) red[wave - 1][16 * j + r][lane] = acc[0][j][r];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int w = 0; w < 3; ++w)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[0][j][r] += red[w][16 * j + r][lane];
  epilogue<float, EPI, 1, 2>(g, acc, m0, n0, lane, blockIdx.y);
}

// Whether the fp32 few-tile kernel can run the launch (16-byte aligned
// operand rows, K a multiple of 4).
inline bool f32_ks_ok(const GemmArgs& a) {
  return a.K % 4 == 0 && a.lda % 4 == 0 && a.ldw % 4 == 0 && reinterpret_cast<uintptr_t>(a.A) % 16 == 0 &&
         reinterpret_cast<uintptr_t>(a.W) % 16 == 0;
}

template <int EPI>
hipError_t run_f32_ks(const GemmArgs& a, int split, hipStream_t s) {
  const int nbm = (a.M + 31) / 32, nbn = (a.N + 63) / 64;
  hipLaunchKernelGGL((gemm_f32_ks_kernel<EPI>), dim3(nbm * nbn, split), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <typename T, int EPI>
hipError_t run_reg(const GemmArgs& a, int split, hipStream_t s) {
  constexpr int BM = 128, BN = 128, WM = 2, WN = 2;
  const int nbm = (a.M + BM - 1) / BM, nbn = (a.N + BN - 1) / BN;
  if constexpr (scaled_epi(EPI) && sizeof(T) == 2) {
    if (a.row_scale != nullptr) {
      hipLaunchKernelGGL((gemm_kernel<T, BM, BN, WM, WN, EPI, true>), dim3(nbm * nbn, split), dim3(WM * WN * 64), 0,
                         s, a);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((gemm_kernel<T, BM, BN, WM, WN, EPI>), dim3(nbm * nbn, split), dim3(WM * WN * 64), 0, s, a);
  return hipGetLastError();
}

template <typename S, int EPI>
hipError_t run_lds(const GemmArgs& a, int split, hipStream_t s) {
  const int nbm = (a.M + S::BM - 1) / S::BM, nbn = (a.N + S::BN - 1) / S::BN;
  if constexpr (scaled_epi(EPI)) {
    if (a.row_scale != nullptr) {
      hipLaunchKernelGGL((gemm_lds_kernel<S, EPI, true>), dim3(nbm * nbn, split), dim3(S::NT), 0, s, a);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((gemm_lds_kernel<S, EPI>), dim3(nbm * nbn, split), dim3(S::NT), 0, s, a);
  return hipGetLastError();
}

template <typename S, int EPI>
hipError_t run_wide(const GemmArgs& a, int split, hipStream_t s) {
  const int nbm = (a.M + S::BM - 1) / S::BM, nbn = (a.N + S::BN - 1) / S::BN;
  if constexpr (scaled_epi(EPI)) {
    if (a.row_scale != nullptr) {
      hipLaunchKernelGGL((gemm_wide_kernel<S, EPI, true>), dim3(nbm * nbn, split), dim3(S::NT), 0, s, a);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((gemm_wide_kernel<S, EPI>), dim3(nbm * nbn, split), dim3(S::NT), 0, s, a);
  return hipGetLastError();
}

// Tile configurations.  0: register-staged 128 x 128 (every element type
// and shape); 1-5 (bf16, LDS-DMA): rows x cols, waves, K tile, stages.
using Cfg1 = L3<128, 128, 2, 2, 64, 3>;
using Cfg2 = L3<128, 128, 2, 2, 64, 2>;   // small enough for two workgroups per CU
using Cfg3 = L3<128, 64, 2, 2, 64, 4>;    // one 32-column MFMA tile per wave: no pair epilogues
using Cfg4 = L3<64, 128, 2, 2, 64, 4>;
using Cfg5 = W4<2, 2, 4, 4, 64, 2>;       // 256 x 256, 128 x 128 per wave
using Cfg6 = W4<4, 1, 2, 6, 64, 2>;       // 256 x 192, 64 x 192 per wave
constexpr int N_CFG = 7;

// The LDS-DMA kernels need 16-byte aligned rows, a K range made of whole
// 64-element tiles and operands whose byte offsets fit the 32-bit buffer
// offsets.
inline bool lds_ok(const GemmArgs& a) {
  const long long abytes = (long long)a.M * a.lda * 2, wbytes = (long long)a.N * a.ldw * 2;
  return a.lda % 8 == 0 && a.ldw % 8 == 0 && a.K % 64 == 0 && a.k_split % 64 == 0 &&
         abytes < (1LL << 31) && wbytes < (1LL << 31);
}

// Internal configuration: the fp32 few-tile kernel (chosen by shape only).
constexpr int CFG_F32_FEW = 64;

template <typename T, int EPI>
hipError_t run_cfg(const GemmArgs& a, int split, int cfg, hipStream_t s) {
  if constexpr (sizeof(T) == 4) {
    if (cfg == CFG_F32_FEW && f32_ks_ok(a)) return run_f32_ks<EPI>(a, split, s);
  }
  if constexpr (sizeof(T) == 2) {
    constexpr bool PAIR = EPI == EPI_SWIGLU || EPI == EPI_QKV;
    constexpr bool STAGED_ONLY = EPI == EPI_GATE || EPI == EPI_QKV;   // see the kernels' epilogues
    if (cfg > 0 && lds_ok(a) && (!STAGED_ONLY || a.staged)) {
      switch (cfg) {
        case 1: return run_lds<Cfg1, EPI>(a, split, s);
        case 2: return run_lds<Cfg2, EPI>(a, split, s);
        case 3:
          if constexpr (!PAIR) return run_lds<Cfg3, EPI>(a, split, s);
          break;
        case 4: return run_lds<Cfg4, EPI>(a, split, s);
        case 5: return run_wide<Cfg5, EPI>(a, split, s);
        case 6: return run_wide<Cfg6, EPI>(a, split, s);
        default: break;
      }
    }
  }
  return run_reg<T, EPI>(a, split, s);
}

template <typename T>
hipError_t dispatch(Epi epi, const GemmArgs& a, int split, float* ws, int cfg, hipStream_t s, int* normed) {
  if (split > 1) {
    if (epi != EPI_F32 && epi != EPI_RESID) return hipErrorInvalidValue;
    GemmArgs p = a;
    p.out0 = ws;
    p.ld0 = a.N;
    p.split_stride = (long long)a.M * a.N;
    hipError_t e = run_cfg<T, EPI_PARTIAL>(p, split, cfg, s);
    if (e != hipSuccess) return e;
    if (epi == EPI_RESID && (a.norm_w || a.rs_out) && a.N % 4 == 0 && a.N <= 4 * 256 * RN_MAXV && split <= 4) {
      if (normed) *normed = NORM_ROWS;   // the reduction has whole rows: normalised there (without the gain when deferred)
      return launch_splitk_resid_norm<T>(a, ws, split, p.split_stride, s);
    }
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
    case EPI_RESID:
      if (normed && a.rs_out) *normed = NORM_DEFERRED;   // the rows and their scales from the epilogue
      return run_cfg<T, EPI_RESID>(a, 1, cfg, s);
    case EPI_GATE:
    case EPI_QKV: {
      GemmArgs r = a;
      r.staged = sizeof(T) == 2 && cfg > 0 && staged_ok(epi, a) ? 1 : 0;
      return epi == EPI_GATE ? run_cfg<T, EPI_GATE>(r, 1, cfg, s) : run_cfg<T, EPI_QKV>(r, 1, cfg, s);
    }
    case EPI_SWIGLU: return run_cfg<T, EPI_SWIGLU>(a, 1, cfg, s);
    default: return hipErrorInvalidValue;
  }
}

// Configuration and K split chosen by shape (bf16), from timings of the 4B
// projection shapes at 512 and 2,048 rows on MI355X with weights not in
// cache (rotated through more than the 256 MB last-level cache, as in a
// forward pass):
//   from 1,024 rows, 256 x 256 tiles when there are 192 of them, with a K
//   split for long reductions that have fewer;
//   below that, 256 x 192 tiles for wide outputs (204 tiles for the FFN
//   gate/up at 512 rows against 152 of 256 x 256), 128 x 128 tiles with a
//   K split for long reductions, 128 x 128 (three stages; two workgroups
//   per CU when there are several waves of tiles) down to 192 tiles, and
//   narrower tiles below that.
void auto_plan(bool bf16, Epi epi, const GemmArgs& a, int max_split, int& cfg, int& split) {
  const long long t128 = (long long)((a.M + 127) / 128) * ((a.N + 127) / 128);
  const long long t256 = (long long)((a.M + 255) / 256) * ((a.N + 255) / 256);
  const bool can_split = max_split > 1 && (epi == EPI_F32 || epi == EPI_RESID);
  const bool long_k = a.K >= 6144 && can_split;
  split = 1;
  if (!bf16) {
    // fewer 128 x 128 tiles than CUs: 32 x 64 tiles with the K range split
    // over the four waves of a workgroup (and over workgroups up to about
    // one per CU for the fp32 outputs); the row-invariant mode asks for
    // configuration 0 explicitly
    const long long tf = (long long)((a.M + 31) / 32) * ((a.N + 63) / 64);
    if (t128 < 256) {
      cfg = CFG_F32_FEW;
      if (can_split)
        while (split < max_split && tf * (split + 1) <= 256 && a.K / (64 * (split + 1)) >= 2) ++split;
      return;
    }
    cfg = 0;
    if (can_split)
      while (split < max_split && t128 * (split + 1) <= 320 && a.K / (32 * (split + 1)) >= 4) ++split;
    return;
  }
  auto split_for = [&](long long tiles, long long target) {
    int sp = 1;
    while (sp < max_split && tiles * sp < target) ++sp;
    return sp;
  };
  if (a.M >= 1024) {
    if (t256 >= 192) {
      cfg = 5;
    } else if (long_k) {
      cfg = 5;
      split = split_for(t256, 192);
    } else {
      cfg = t128 >= 300 ? 2 : 1;
    }
  } else if (t128 >= 384) {
    cfg = 6;
  } else if (long_k) {
    cfg = 1;
    split = split_for(t128, 240);
  } else if (t128 >= 192) {
    cfg = 1;
  } else if (can_split && a.K >= 2048 && t128 < 128) {
    // few output tiles (the d-wide out-projection at 512 rows: 80): a K split
    // fills the chip, and the reduction runs fused with the residual add and
    // the next RMSNorm in place of a separate norm (20 + 7 -> ~17 us)
    cfg = 1;
    split = split_for(t128, 240);
  } else {
    cfg = (epi == EPI_SWIGLU || epi == EPI_QKV) ? 4 : 3;
  }
}

}  // namespace

int gemm_k_tile(bool bf16) { return bf16 ? 64 : 32; }

// The residual epilogue addresses out0 through a 32-bit buffer range.
bool resid_rows_ok(Epi epi, const GemmArgs& a) {
  return epi != EPI_RESID || (long long)a.M * a.ld0 * 4 < (1LL << 31);
}

// Arguments of the deferred RMSNorm (bf16 only): the row scale on the
// scaled epilogues; on EPI_RESID the bf16 copy, the scale output and, for
// the form without a K split, the partial sums (at most 256 slots of 32
// columns per row, rows a multiple of 32 apart) and the tickets.
bool deferred_norm_ok(bool bf16, Epi epi, const GemmArgs& a) {
  if (a.row_scale && (!bf16 || !(epi == EPI_SWIGLU || epi == EPI_GATE || epi == EPI_QKV))) return false;
  if (a.rs_out == nullptr) return true;
  return bf16 && epi == EPI_RESID && a.norm_out && a.ss_parts && a.tickets && a.N <= 256 * 32 &&
         a.ss_ld >= a.M && a.ss_ld % 32 == 0;
}

int gemm_tile_configs() { return N_CFG; }

hipError_t launch_gemm(bool bf16, Epi epi, const GemmArgs& a, int split, float* ws, hipStream_t s,
                       int cfg, int* normed) {
  if (normed) *normed = NORM_NONE;
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  if (!deferred_norm_ok(bf16, epi, a) || !resid_rows_ok(epi, a)) return hipErrorInvalidValue;
  GemmArgs g = a;
  if (split < 1) split = 1;
  if (cfg < 0) auto_plan(bf16, epi, a, ws ? split : 1, cfg, split);
  const int bk = gemm_k_tile(bf16);
  // K range per split: a whole number of K tiles
  const int tiles = (a.K + bk - 1) / bk;
  if (split > tiles) split = tiles > 0 ? tiles : 1;
  g.k_split = ((tiles + split - 1) / split) * bk;
  split = (a.K + g.k_split - 1) / g.k_split;
  if (split < 1) split = 1;
  return bf16 ? dispatch<bf16_t>(epi, g, split, ws, cfg, s, normed)
              : dispatch<float>(epi, g, split, ws, cfg, s, normed);
}

size_t frag_bytes(int N, int K) { return (size_t)((N + 31) / 32) * 32 * K * 2; }

hipError_t launch_frag_pack(const void* W, int N, int K, int ld, bool gu16, void* out, hipStream_t s) {
  if (N <= 0 || K <= 0 || K % 16 || ld % 8) return hipErrorInvalidValue;
  const long long nchunks = (long long)((N + 31) / 32) * (K / 16) * 64;
  const int blocks = (int)std::min<long long>((nchunks + 255) / 256, 8192);
  hipLaunchKernelGGL(frag_pack_kernel, dim3(blocks), dim3(256), 0, s, static_cast<const bf16_t*>(W), N, K, ld,
                     gu16 ? 1 : 0, static_cast<uint4*>(out), nchunks);
  return hipGetLastError();
}

bool gemm_wd_ok(Epi epi, const GemmArgs& a) {
  const long long abytes = (long long)a.M * a.lda * 2;
  return (epi == EPI_F32 || epi == EPI_RESID || (epi == EPI_SWIGLU && a.ld0 % 8 == 0 && a.n_valid % 8 == 0) ||
          ((epi == EPI_GATE || epi == EPI_QKV) && staged_ok(epi, a))) &&
         a.K >= 64 && a.K % 64 == 0 && a.lda % 8 == 0 && abytes < (1LL << 31);
}

template <typename S>
hipError_t run_wd_epi(Epi epi, const GemmArgs& a, hipStream_t s) {
  switch (epi) {
    case EPI_F32: return run_wd<S, EPI_F32>(a, s);
    case EPI_RESID: return run_wd<S, EPI_RESID>(a, s);
    case EPI_SWIGLU: return run_wd<S, EPI_SWIGLU>(a, s);
    case EPI_GATE:
    case EPI_QKV:
      // bf16 q|k|v outputs staged through the activation stages: the
      // 256 x 256 tile only (the 128 x 384 tile's stages are too small)
      if constexpr (S::BM * S::BN * 2 <= S::NS * S::STAGE)
        return epi == EPI_GATE ? run_wd<S, EPI_GATE>(a, s) : run_wd<S, EPI_QKV>(a, s);
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

namespace {
int wd_dims(int tile, int& bn) {
  switch (tile) {
    case 2: bn = CfgWD2::BN; return CfgWD2::BM;
    case 3: bn = CfgWD3::BN; return CfgWD3::BM;
    case 4: bn = CfgWD4::BN; return CfgWD4::BM;
    default: bn = CfgWD1::BN; return CfgWD1::BM;
  }
}
}  // namespace

int gemm_wd_tiles(int tile, int M, int N) {
  int bn = 0;
  const int bm = wd_dims(tile, bn);
  return ((M + bm - 1) / bm) * ((N + bn - 1) / bn);
}

int gemm_wd_panel(int tile) {
  int bn = 0;
  const int bm = wd_dims(tile, bn);
  return bm + bn;
}

hipError_t launch_gemm_wd(Epi epi, const GemmArgs& a, int tile, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  if (!gemm_wd_ok(epi, a) || !deferred_norm_ok(true, epi, a) || !resid_rows_ok(epi, a) || tile < 1 || tile > 4)
    return hipErrorInvalidValue;
  if (tile == 3) {   // built for the SwiGLU and fp32 epilogues
    if (epi == EPI_SWIGLU) return run_wd<CfgWD3, EPI_SWIGLU>(a, s);
    if (epi == EPI_F32) return run_wd<CfgWD3, EPI_F32>(a, s);
    return hipErrorInvalidValue;
  }
  if (tile == 4) return run_wd_epi<CfgWD4>(epi, a, s);
  return tile == 2 ? run_wd_epi<CfgWD2>(epi, a, s) : run_wd_epi<CfgWD1>(epi, a, s);
}

}  // namespace s1
