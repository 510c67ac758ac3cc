// Full-vocabulary token log-probabilities and their normalisation across the
// candidates of a question (RFC #114 "Native Rust/CUDA support for
// OmniJev-4B v1.1", section 4, note under the semantics table: the language-
// model features use log-probabilities over the whole vocabulary, computed in
// bounded chunks; comment "Plan: native OmniJev-4B v1.1": the log-softmax
// runs over every row of the tied embedding, logits in fp32).
//
// Steps, all on the stream given:
//   1. feat_norm: gather the distinct rows the targets read, final RMSNorm
//      (fp32), and for bf16 models split each normalised value into a bf16
//      pair hi + lo (hi = rne(v), lo = rne(v - hi), |v - hi - lo| <= 2^-17 |v|).
//   2. vocab_lse: the hot kernel.  Every workgroup owns 128 consecutive
//      vocabulary rows (32 per wave), streams them once from HBM and forms
//      their logits against all rows of the group on MFMA (E x hi + E x lo,
//      fp32 accumulation), then reduces them to one (max, sum exp(z - max))
//      pair per row: no logit is written.  The normalised rows are staged
//      through LDS chunk by chunk and shared by the four waves.
//   3. lse_merge: per row, the partial pairs of every vocabulary block merged
//      in a fixed order, lse = m + log s (deterministic).
//   4. target_logp: one wave per target, z = hn . E[token] in fp32, logp =
//      z - lse.
//   5. cand_norm: one thread per question group, candidate score = sum of
//      its targets' logp, then score - logsumexp over the group.
#include "common.h"
#include "kernels.h"

#include <algorithm>
#include <utility>

namespace s1 {
namespace {

constexpr int VL_WAVES = 4;                 // waves per workgroup
constexpr int VL_ROWS = 32 * VL_WAVES;      // vocabulary rows per workgroup
constexpr int VL_KC = 128;                  // k per staged chunk

// 1. One workgroup per padded row; rows >= R are zero (so padded columns
// contribute logits of 0 that the caller never reads).  Four consecutive
// values per thread and step (d % 4 == 0).
template <bool SPLIT>
__global__ void __launch_bounds__(256)
feat_norm_kernel(const float* __restrict__ x, int d, const int32_t* __restrict__ rows, int R,
                 const float* __restrict__ w, float eps, float* __restrict__ hn,
                 bf16_t* __restrict__ hi, bf16_t* __restrict__ lo) {
  __shared__ float red[4];
  const int r = blockIdx.x;
  const long long o = (long long)r * d;
  if (r >= R) {
    for (int i = 4 * threadIdx.x; i < d; i += 1024) {
      *reinterpret_cast<float4*>(hn + o + i) = make_float4(0.f, 0.f, 0.f, 0.f);
      if constexpr (SPLIT) {
        *reinterpret_cast<uint2*>(hi + o + i) = make_uint2(0, 0);
        *reinterpret_cast<uint2*>(lo + o + i) = make_uint2(0, 0);
      }
    }
    return;
  }
  const float* xr = x + (long long)rows[r] * d;
  float ss = 0.f;
  for (int i = 4 * threadIdx.x; i < d; i += 1024) {
    const float4 v = *reinterpret_cast<const float4*>(xr + i);
    ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
  }
  const float rs = rsqrtf(block_sum<4>(ss, red) / d + eps);
  for (int i = 4 * threadIdx.x; i < d; i += 1024) {
    const float4 v = *reinterpret_cast<const float4*>(xr + i);
    const float4 g = *reinterpret_cast<const float4*>(w + i);
    const float e[4] = {v.x * rs * g.x, v.y * rs * g.y, v.z * rs * g.z, v.w * rs * g.w};
    *reinterpret_cast<float4*>(hn + o + i) = make_float4(e[0], e[1], e[2], e[3]);
    if constexpr (SPLIT) {
      bf16_t hb[4], lb[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        hb[k] = f2bf(e[k]);
        lb[k] = f2bf(e[k] - bf2f(hb[k]));
      }
      *reinterpret_cast<uint2*>(hi + o + i) = make_uint2(hb[0] | (uint32_t)hb[1] << 16, hb[2] | (uint32_t)hb[3] << 16);
      *reinterpret_cast<uint2*>(lo + o + i) = make_uint2(lb[0] | (uint32_t)lb[1] << 16, lb[2] | (uint32_t)lb[3] << 16);
    }
  }
}

// Merge of two (max, sum exp(z - max)) pairs; an empty pair has s = 0.
__device__ __forceinline__ float2 lse_pair(float2 a, float2 b) {
  if (a.y == 0.f) return b;
  if (b.y == 0.f) return a;
  const float m = fmaxf(a.x, b.x);
  return make_float2(m, a.y * __expf(a.x - m) + b.y * __expf(b.x - m));
}

// 2. Vocabulary log-sum-exp partials, bf16 tied embedding.
//
// Workgroup b owns vocabulary rows [128 b, 128 b + 128), wave w the 32 rows
// from 128 b + 32 w (one MFMA row tile), and NT tiles of 32 normalised rows
// (columns col0 .. col0 + 32 NT - 1).  The kernel is bound by streaming E
// from HBM, and HBM only delivers its bandwidth with a few hundred KB of
// loads in flight per CU; so the vocabulary rows stream through a ring of D
// register buffers per lane (D - 1 chunks of KC k-values in flight while one
// is multiplied), and the normalised rows -- identical for all waves --
// through a ring of D LDS buffers filled by buffer-to-LDS DMA, issued
// together with the vocabulary chunk of the same k range.
//
// Vector-memory completions are counted in issue order (vmcnt), so every
// chunk's loads (E into registers, hn into LDS) are issued as one group and
// a wait for "all but the last D - 2 groups" covers exactly the chunk about to
// be used.  Both kinds of load are written as inline assembly: a
// compiler-visible LDS DMA makes the compiler wait for every outstanding load
// before any LDS read, which would empty the ring.  The compiler does not
// know that these registers are written after the instruction issues, so
// every load's destination must stay live until a wait that covers it: each
// chunk's wait names the chunk's registers as operands (nothing that reads
// them moves before it), every step issues a group unconditionally (chunks
// past the end load from beyond the buffer's range, which reads zeros
// without touching memory, so no register merges a loaded and a kept value),
// and the final wait names every ring register, so none is reused while a
// load past the end is still in flight.
//
// k order: the contraction may visit k in any order as long as both operands
// use the same one.  Lane l (half h = l / 32) feeds MFMA step j with the
// eight vocabulary values at k = 16 j + 8 h of the chunk, and the B operand
// of lane l at step j is hn[col][16 j + 8 h ..].  Each LDS chunk holds, per
// normalised row, 2 U 16-byte slots (U = KC / 8 of hi, then U of lo), slot s
// stored at s ^ (row & 15): the 16 lanes of a ds_read_b128 phase (16 rows,
// one slot) then hit 16 distinct 16-byte bank groups.
typedef int int32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;

// Raw buffer resource over `bytes` bytes from base; offsets at or past
// `bytes` read as zero.  The fields are wave-uniform (readfirstlane keeps
// them in the scalar registers the buffer instructions take).
__device__ __forceinline__ int32x4 raw_rsrc(const void* base, int bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  int32x4 r;
  r.x = __builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(a)));
  r.y = __builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(a >> 32) & 0xFFFFu));
  r.z = __builtin_amdgcn_readfirstlane(bytes);
  r.w = 0x00020000;
  return r;
}

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// 16 bytes per lane from the buffer into LDS at lds + 16 * lane.
__device__ __forceinline__ void vl_dma16(int32x4 rsrc, uint32_t lds, int voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :: "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(rsrc) : "memory", "m0");
}
// 16 bytes per lane into registers; complete only after a vl_wait.
__device__ __forceinline__ u32x4 vl_load16(int32x4 rsrc, int voff) {
  u32x4 v;
  asm volatile("buffer_load_dwordx4 %0, %1, %2, 0 offen" : "=v"(v) : "v"(voff), "s"(rsrc) : "memory");
  return v;
}
#pragma clang diagnostic pop

// Wait until at most VM vector-memory loads are outstanding; the J
// registers of the chunk are tied to the wait.
template <int VM, int J>
__device__ __forceinline__ void vl_wait(u32x4 (&a)[J]) {
  static_assert(VM >= 0 && VM < 64, "vmcnt range");
  if constexpr (J == 8)
    asm volatile("s_waitcnt vmcnt(%8)" : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(a[4]),
                 "+v"(a[5]), "+v"(a[6]), "+v"(a[7]) : "n"(VM) : "memory");
  else if constexpr (J == 4)
    asm volatile("s_waitcnt vmcnt(%4)" : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]) : "n"(VM) : "memory");
  else
    static_assert(J == 8 || J == 4, "chunk register count");
}

// Marks the J registers as read and written here (no instruction).
template <int J>
__device__ __forceinline__ void vl_keep(u32x4 (&a)[J]) {
  if constexpr (J == 8)
    asm volatile("" : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(a[4]), "+v"(a[5]), "+v"(a[6]),
                 "+v"(a[7]));
  else
    asm volatile("" : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]));
}

template <int NT, int KC, int D>
__global__ void __launch_bounds__(256, 2)
vocab_lse_bf16_kernel(const bf16_t* __restrict__ E, int V, int d, const bf16_t* __restrict__ hi, int lo_delta,
                      int col0, float2* __restrict__ part) {
  constexpr int U = KC / 8, J = KC / 16, NR = 32 * NT;
  constexpr int ROWB = 32 * U;            // LDS bytes per normalised row and chunk (hi + lo)
  constexpr int CHB = NR * ROWB;          // LDS bytes per chunk
  constexpr int IPW = CHB / 4096;         // 1 KB DMA instructions per wave and chunk
  static_assert(IPW >= 1 && CHB % 4096 == 0 && 2 * U >= 16, "chunk layout");
  static_assert(D >= 3, "ring depth");
  __shared__ __attribute__((aligned(16))) char ring[D][CHB];
  __shared__ float2 red[VL_WAVES][NR];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5;
  const int vb = blockIdx.x * VL_ROWS;
  const int v0 = vb + wave * 32;
  // this workgroup's vocabulary rows; rows past V read as zero
  const int32x4 ra = raw_rsrc(E + (long long)vb * d, (int)(min(V - vb, VL_ROWS) * (long long)d * 2));
  const int a_base = (wave * 32 + (lane & 31)) * d * 2;
  // hi rows col0 .. col0 + NR - 1, lo rows lo_delta bytes further on
  const bf16_t* hb = hi + (long long)col0 * d;
  const int32x4 rb = raw_rsrc(hb, lo_delta + NR * d * 2);
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const lds_char*)&ring[0][0]));
  int b_off[IPW];
#pragma unroll
  for (int i = 0; i < IPW; ++i) {
    const int byte = 1024 * (wave * IPW + i) + 16 * lane;   // where this lane's DMA lands in the chunk
    const int row = byte / ROWB;
    const int hu = ((byte % ROWB) / 16) ^ (row & 15);       // (half, unit) kept in that slot
    b_off[i] = (hu / U) * lo_delta + (row * d + 8 * (hu % U)) * 2;
  }
  const int nk = d / KC;
  floatx16 acc[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[n][r] = 0.f;
  u32x4 a[D][J];

  auto issue = [&](int c, auto qc) {
    constexpr int q = decltype(qc)::value;
    const int koff = c < nk ? c * KC * 2 : 0x40000000;
#pragma unroll
    for (int i = 0; i < IPW; ++i) vl_dma16(rb, lds0 + q * CHB + 1024 * (wave * IPW + i), b_off[i] + koff);
#pragma unroll
    for (int j = 0; j < J; ++j) a[q][j] = vl_load16(ra, a_base + koff + 2 * (16 * j + 8 * h));
  };
  auto compute = [&](auto qc) {
    constexpr int q = decltype(qc)::value;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const bf16x8 av = __builtin_bit_cast(bf16x8, a[q][j]);
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        const int row = 32 * n + (lane & 31);
        const char* p = &ring[q][0] + row * ROWB;
        const int unit = 2 * j + h;
        mfma32(acc[n], av, as_frag(*reinterpret_cast<const uint4*>(p + 16 * (unit ^ (row & 15)))));
        mfma32(acc[n], av, as_frag(*reinterpret_cast<const uint4*>(p + 16 * ((U + unit) ^ (row & 15)))));
      }
    }
  };
  [&]<int... Q>(std::integer_sequence<int, Q...>) {
    (issue(Q, std::integral_constant<int, Q>{}), ...);
  }(std::make_integer_sequence<int, D - 1>{});
  for (int c0 = 0; c0 < nk; c0 += D) {
    [&]<int... Q>(std::integer_sequence<int, Q...>) {
      auto step = [&](auto qc) {
        constexpr int q = decltype(qc)::value;
        const int c = c0 + q;
        if (c < nk) {
          vl_wait<(D - 2) * (IPW + J), J>(a[q]);   // chunk c: its E registers and this wave's DMA
          __syncthreads();                         // every wave's DMA of chunk c; slot (c - 1) % D free
          issue(c + D - 1, std::integral_constant<int, (q + D - 1) % D>{});
          compute(qc);
        }
      };
      (step(std::integral_constant<int, Q>{}), ...);
    }(std::make_integer_sequence<int, D>{});
  }
  // drain the loads past the end (no wave leaves with a DMA into LDS in
  // flight) with every ring register live across the wait
  vl_wait<0, J>(a[0]);
  [&]<int... Q>(std::integer_sequence<int, Q...>) {
    (vl_keep(a[Q]), ...);
  }(std::make_integer_sequence<int, D>{});

  // per column: max and sum of exp over this wave's 32 vocabulary rows
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    float m = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (v0 + acc_row(r, lane) < V) m = fmaxf(m, acc[n][r]);
    m = fmaxf(m, __shfl_xor(m, 32, 64));
    float s = 0.f;
    if (m != -INFINITY) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (v0 + acc_row(r, lane) < V) s += __expf(acc[n][r] - m);
    }
    s += __shfl_xor(s, 32, 64);
    if (lane < 32) red[wave][32 * n + lane] = make_float2(m, s);
  }
  __syncthreads();
  if (tid < NR) {
    float2 t = red[0][tid];
#pragma unroll
    for (int w = 1; w < VL_WAVES; ++w) t = lse_pair(t, red[w][tid]);
    part[(long long)(col0 + tid) * gridDim.x + blockIdx.x] = t;
  }
}

// 2'. The same partials for fp32 models: thread t of block b owns vocabulary
// row 256 b + t and loops over the rows (fp32 dot products; these models are
// small).
__global__ void __launch_bounds__(256)
vocab_lse_f32_kernel(const float* __restrict__ E, int V, int d, const float* __restrict__ hn, int R,
                     float2* __restrict__ part) {
  __shared__ float2 red[4];
  const int v = blockIdx.x * 256 + threadIdx.x, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float* e = E + (long long)min(v, V - 1) * d;
  for (int r = 0; r < R; ++r) {
    const float* h = hn + (long long)r * d;
    float z = 0.f;
    for (int i = 0; i < d; i += 4) {
      const float4 a = *reinterpret_cast<const float4*>(e + i);
      const float4 b = *reinterpret_cast<const float4*>(h + i);
      z += a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w;
    }
    float2 t = v < V ? make_float2(z, 1.f) : make_float2(0.f, 0.f);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      float2 u;
      u.x = __shfl_xor(t.x, o, 64);
      u.y = __shfl_xor(t.y, o, 64);
      t = lse_pair(t, u);
    }
    if (lane == 0) red[wave] = t;
    __syncthreads();
    if (threadIdx.x == 0) {
      float2 s = red[0];
      for (int w = 1; w < 4; ++w) s = lse_pair(s, red[w]);
      part[(long long)r * gridDim.x + blockIdx.x] = s;
    }
    __syncthreads();
  }
}

// 3. One workgroup per row: merge the row's nb partial pairs (contiguous).
// Thread t folds blocks t, t + 256, ... in order, then a fixed butterfly and
// a fixed cross-wave order finish; the result does not depend on timing.
__global__ void __launch_bounds__(256)
lse_merge_kernel(const float2* __restrict__ part, int nb, float* __restrict__ lse) {
  __shared__ float2 red[4];
  const int r = blockIdx.x, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float2* pr = part + (long long)r * nb;
  float2 t = make_float2(0.f, 0.f);
  for (int b = threadIdx.x; b < nb; b += 256) t = lse_pair(t, pr[b]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    float2 u;
    u.x = __shfl_xor(t.x, o, 64);
    u.y = __shfl_xor(t.y, o, 64);
    t = lse_pair(t, u);
  }
  if (lane == 0) red[wave] = t;
  __syncthreads();
  if (threadIdx.x == 0) {
    float2 s = red[0];
    for (int w = 1; w < 4; ++w) s = lse_pair(s, red[w]);
    lse[r] = s.x + __logf(s.y);
  }
}

// 4. One wave per target.
template <typename T>
__global__ void __launch_bounds__(256)
target_logp_kernel(const float* __restrict__ hn, int d, const T* __restrict__ E,
                   const int32_t* __restrict__ t_ri, const int32_t* __restrict__ t_tok, int n,
                   const float* __restrict__ lse, float* __restrict__ logp) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (t >= n) return;
  const int ri = t_ri[t];
  const float* h = hn + (long long)ri * d;
  const T* e = E + (long long)t_tok[t] * d;
  float z = 0.f;
  for (int i = lane * 4; i < d; i += 256) {
    float4 ev;
    if constexpr (sizeof(T) == 2) {
      const uint2 u = *reinterpret_cast<const uint2*>(e + i);
      ev = make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xFFFF0000u),
                       __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xFFFF0000u));
    } else {
      ev = *reinterpret_cast<const float4*>(e + i);
    }
    const float4 hv = *reinterpret_cast<const float4*>(h + i);
    z += ev.x * hv.x + ev.y * hv.y + ev.z * hv.z + ev.w * hv.w;
  }
  z = wave_sum(z);
  if (lane == 0) logp[t] = z - lse[ri];
}

// 5. One thread per group: each member candidate's score (sum of its
// targets' logp, in target order), then score - logsumexp over the group.
__global__ void __launch_bounds__(256)
cand_norm_kernel(const float* __restrict__ logp, const int32_t* __restrict__ cand_off,
                 const int32_t* __restrict__ grp_off, const int32_t* __restrict__ grp_cands, int G,
                 float* __restrict__ cand_lp, float* __restrict__ cand_norm) {
  const int g = blockIdx.x * 256 + threadIdx.x;
  if (g >= G) return;
  const int c0 = grp_off[g], c1 = grp_off[g + 1];
  float m = -INFINITY;
  for (int i = c0; i < c1; ++i) {
    const int c = grp_cands[i];
    float s = 0.f;
    for (int t = cand_off[c]; t < cand_off[c + 1]; ++t) s += logp[t];
    cand_lp[c] = s;
    m = fmaxf(m, s);
  }
  float se = 0.f;
  for (int i = c0; i < c1; ++i) se += __expf(cand_lp[grp_cands[i]] - m);
  const float l = m + __logf(se);
  for (int i = c0; i < c1; ++i) {
    const int c = grp_cands[i];
    cand_norm[c] = cand_lp[c] - l;
  }
}

}  // namespace

FeatWs feat_ws_layout(bool bf16, int R, int V, int d) {
  FeatWs w;
  w.Rp = std::max(32, (R + 31) / 32 * 32);
  w.nb = bf16 ? (V + VL_ROWS - 1) / VL_ROWS : (V + 255) / 256;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += (bytes + 255) / 256 * 256;
    return o;
  };
  w.hn = take((size_t)w.Rp * d * 4);
  w.hi = bf16 ? take((size_t)w.Rp * d * 2) : 0;
  w.lo = bf16 ? take((size_t)w.Rp * d * 2) : 0;
  w.part = take((size_t)w.nb * w.Rp * 8);
  w.lse = take((size_t)w.Rp * 4);
  w.bytes = off;
  return w;
}

bool feat_shape_ok(bool bf16, int d) {
  return bf16 ? (d >= VL_KC && d % VL_KC == 0) : (d >= 4 && d % 4 == 0);
}

hipError_t launch_vocab_lse(bool bf16, const void* E, int V, int d, int R, void* ws, hipStream_t s) {
  const FeatWs w = feat_ws_layout(bf16, R, V, d);
  char* base = static_cast<char*>(ws);
  auto* part = reinterpret_cast<float2*>(base + w.part);
  if (bf16) {
    const auto* hi = reinterpret_cast<const bf16_t*>(base + w.hi);
    const int lo_delta = (int)(w.lo - w.hi);
    for (int c0 = 0; c0 < w.Rp; c0 += 64) {
      if (w.Rp - c0 >= 64)
        hipLaunchKernelGGL((vocab_lse_bf16_kernel<2, 64, 4>), dim3(w.nb), dim3(256), 0, s,
                           reinterpret_cast<const bf16_t*>(E), V, d, hi, lo_delta, c0, part);
      else
        hipLaunchKernelGGL((vocab_lse_bf16_kernel<1, 128, 4>), dim3(w.nb), dim3(256), 0, s,
                           reinterpret_cast<const bf16_t*>(E), V, d, hi, lo_delta, c0, part);
    }
  } else {
    hipLaunchKernelGGL(vocab_lse_f32_kernel, dim3(w.nb), dim3(256), 0, s, reinterpret_cast<const float*>(E), V,
                       d, reinterpret_cast<const float*>(base + w.hn), R, part);
  }
  return hipGetLastError();
}

hipError_t launch_lse_merge(bool bf16, int V, int d, int R, void* ws, hipStream_t s) {
  const FeatWs w = feat_ws_layout(bf16, R, V, d);
  char* base = static_cast<char*>(ws);
  hipLaunchKernelGGL(lse_merge_kernel, dim3(R), dim3(256), 0, s, reinterpret_cast<const float2*>(base + w.part),
                     w.nb, reinterpret_cast<float*>(base + w.lse));
  return hipGetLastError();
}

hipError_t launch_feat_norm(bool bf16, const float* x, int d, const int32_t* rows, int R, const float* w_final,
                            float eps, int V, void* ws, hipStream_t s) {
  const FeatWs w = feat_ws_layout(bf16, R, V, d);
  char* base = static_cast<char*>(ws);
  if (bf16)
    hipLaunchKernelGGL(feat_norm_kernel<true>, dim3(w.Rp), dim3(256), 0, s, x, d, rows, R, w_final, eps,
                       reinterpret_cast<float*>(base + w.hn), reinterpret_cast<bf16_t*>(base + w.hi),
                       reinterpret_cast<bf16_t*>(base + w.lo));
  else
    hipLaunchKernelGGL(feat_norm_kernel<false>, dim3(w.Rp), dim3(256), 0, s, x, d, rows, R, w_final, eps,
                       reinterpret_cast<float*>(base + w.hn), nullptr, nullptr);
  return hipGetLastError();
}

hipError_t launch_feat_targets(bool bf16, int d, const void* E, int V, const FeatArgs& f, float* logp,
                               float* cand_lp, float* cand_norm, void* ws, hipStream_t s) {
  if (f.n_targets <= 0) return hipSuccess;
  const FeatWs w = feat_ws_layout(bf16, f.R, V, d);
  char* base = static_cast<char*>(ws);
  const auto* hn = reinterpret_cast<const float*>(base + w.hn);
  const auto* lse = reinterpret_cast<const float*>(base + w.lse);
  const dim3 g((f.n_targets + 3) / 4);
  if (bf16)
    hipLaunchKernelGGL(target_logp_kernel<bf16_t>, g, dim3(256), 0, s, hn, d,
                       reinterpret_cast<const bf16_t*>(E), f.t_ri, f.t_tok, f.n_targets, lse, logp);
  else
    hipLaunchKernelGGL(target_logp_kernel<float>, g, dim3(256), 0, s, hn, d, reinterpret_cast<const float*>(E),
                       f.t_ri, f.t_tok, f.n_targets, lse, logp);
  if (f.n_groups > 0)
    hipLaunchKernelGGL(cand_norm_kernel, dim3((f.n_groups + 255) / 256), dim3(256), 0, s, logp, f.cand_off,
                       f.grp_off, f.grp_cands, f.n_groups, cand_lp, cand_norm);
  return hipGetLastError();
}

hipError_t launch_features(bool bf16, const float* x, int d, const float* w_final, float eps, const void* E,
                           int V, const FeatArgs& f, float* logp, float* cand_lp, float* cand_norm, void* ws,
                           hipStream_t s) {
  if (f.n_targets <= 0 || f.R <= 0) return hipSuccess;
  hipError_t e = launch_feat_norm(bf16, x, d, f.rows, f.R, w_final, eps, V, ws, s);
  if (e == hipSuccess) e = launch_vocab_lse(bf16, E, V, d, f.R, ws, s);
  if (e == hipSuccess) e = launch_lse_merge(bf16, V, d, f.R, ws, s);
  if (e == hipSuccess) e = launch_feat_targets(bf16, d, E, V, f, logp, cand_lp, cand_norm, ws, s);
  return e;
}

}  // namespace s1
