// Gated DeltaNet scan (Yang, Kautz, Hatamizadeh, "Gated Delta Networks:
// Improving Mamba2 with Delta Rule", ICLR 2025): per (token, head)
//   S_t = g_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T,  o_t = S_t^T q_t,
// with a [dk, dv] = [128, 128] fp32 state (RFC #114 section 5: FP32 recurrent
// state; a branch starts from its prefix's final state).
//
// Chunks of C = 64 tokens in the WY form (Yang et al., "Parallelizing Linear
// Transformers with the Delta Rule over Sequence Length", NeurIPS 2024, with
// the gate): writing S_t = g_t S_{t-1} + k_t u_t^T, inside a chunk that starts
// from S0, with gamma_t = prod_{j<=t} g_j (chunk-local),
//   (I + L) U = diag(beta) V - diag(beta gamma) K S0,
//       L[t][i] = beta_t (gamma_t / gamma_i) k_t . k_i  (i < t),
//   O  = diag(gamma) Q S0 + (Q K^T . M) U,   M[t][i] = gamma_t / gamma_i (i <= t),
//   S' = gamma_C S0 + (K . gamma_C / gamma)^T U.
// U = Ut - W S0 with W = (I + L)^-1 diag(beta gamma) K and
// Ut = (I + L)^-1 diag(beta) V, which do not depend on S0:
//   gdn_prep_kernel   every (chunk, head) in parallel: K K^T on MFMA, L, and
//                     W | Ut by forward substitution (one column per thread);
//   gdn_scan_kernel   every (sequence, head) in order over its chunks: the
//                     state stays in accumulator registers; U, O and S' on
//                     MFMA.
// Operands formed inside the kernels (W, U, decayed scores, the state,
// decayed keys) are fp32 values split into bf16 hi + lo parts; products of
// two such operands take three MFMAs (hi.hi + hi.lo + lo.hi), products with
// a bf16 input two, so the kernels add little beyond fp32 rounding to their
// bf16 q, k, v.
#include "common.h"
#include "kernels.h"

namespace s1 {
namespace {

constexpr int C = 64, DK = 128, DV = 128;
constexpr int QP = DK * 2 + 16;    // bytes per Q / K row in LDS
constexpr int TP = C * 2 + 16;     // bytes per decayed K^T row (hi or lo) in LDS
constexpr int WP = DK * 4 + 16;    // bytes per W row (fp32) in LDS
constexpr int XW = DK + DV;        // columns of W | Ut

// -------------------------------------------------------------- prepare
// One workgroup (4 waves) per (chunk, head).  X = W | Ut, [C][XW] fp32.
__global__ void __launch_bounds__(256)
gdn_prep_kernel(const bf16_t* __restrict__ k, const bf16_t* __restrict__ v, int ldqkv,
                const float* __restrict__ lg, const float* __restrict__ beta, int ldg,
                const ScanSeq* __restrict__ chunks, float* __restrict__ wu, int H) {
  __shared__ __attribute__((aligned(16))) char sK[C * QP];
  __shared__ float sL[C][C + 1];
  __shared__ float sG[C], sB[C];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hi = lane >> 5, cl = lane & 31;
  const int ch = blockIdx.x, h = blockIdx.y;
  const ScanSeq cq = chunks[ch];
  const int n = cq.len;
  const long long base = cq.row0;
  if (wave == 0) {
    float G = lane < n ? lg[(base + lane) * ldg + h] : 0.f;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float t = __shfl_up(G, off, 64);
      if (lane >= off) G += t;
    }
    sG[lane] = G;
    sB[lane] = lane < n ? beta[(base + lane) * ldg + h] : 0.f;
  }
  // rows past the chunk's end are loaded from its last row (in bounds) and
  // replaced by zeros: the loads carry no branch and issue back to back
  {
    uint4 kv[C * 16 / 256];
#pragma unroll
    for (int i = 0; i < C * 16 / 256; ++i) {
      const int c = tid + 256 * i, s = c >> 4, q8 = c & 15;
      kv[i] = *reinterpret_cast<const uint4*>(k + (base + min(s, n - 1)) * ldqkv + h * DK + q8 * 8);
    }
#pragma unroll
    for (int i = 0; i < C * 16 / 256; ++i) {
      const int c = tid + 256 * i, s = c >> 4, q8 = c & 15;
      *reinterpret_cast<uint4*>(sK + s * QP + q8 * 16) = s < n ? kv[i] : make_uint4(0, 0, 0, 0);
    }
  }
  __syncthreads();
  // K K^T: wave w computes the 32 x 32 tile (w / 2, w % 2); exact products
  // of bf16 inputs, fp32 accumulation
  {
    const int ti = wave >> 1, tj = wave & 1;
    floatx16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
    const char* ar = sK + (32 * ti + cl) * QP + 16 * hi;
    const char* br = sK + (32 * tj + cl) * QP + 16 * hi;
#pragma unroll
    for (int ks = 0; ks < DK / 16; ++ks)
      mfma32(acc, as_frag(*reinterpret_cast<const uint4*>(ar + 32 * ks)),
             as_frag(*reinterpret_cast<const uint4*>(br + 32 * ks)));
    // acc[r] = (K K^T)[32 ti + acc_row(r)][32 tj + cl]: L[t][i], t = row, i = column
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int t = 32 * ti + acc_row(r, lane), i = 32 * tj + cl;
      sL[t][i] = i < t ? sB[t] * __expf(sG[t] - sG[i]) * acc[r] : 0.f;
    }
  }
  __syncthreads();
  // forward substitution, one column j of W | Ut per thread:
  //   X_t = rhs_t - sum_{i<t} L[t][i] X_i,
  //   rhs_t = beta_t gamma_t k_t[j] (j < DK), beta_t v_t[j - DK] (j >= DK)
  const int j = tid;
  float x[C];
  if (j < DK) {
#pragma unroll
    for (int t = 0; t < C; ++t)
      x[t] = sB[t] * __expf(sG[t]) * bf2f(*reinterpret_cast<const bf16_t*>(sK + t * QP + 2 * j));
  } else {
    // sB is zero past the chunk's end; those rows read the last row in bounds
    const bf16_t* vc = v + base * ldqkv + (long long)h * DV + (j - DK);
#pragma unroll
    for (int t = 0; t < C; ++t) x[t] = bf2f(vc[(long long)min(t, n - 1) * ldqkv]);
#pragma unroll
    for (int t = 0; t < C; ++t) x[t] *= sB[t];
  }
  // four partial sums per row shorten the dependent chain
#pragma unroll
  for (int t = 1; t < C; ++t) {
    float a0 = x[t], a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
    for (int i = 0; i < t; i += 4) {
      a0 -= sL[t][i] * x[i];
      if (i + 1 < t) a1 -= sL[t][i + 1] * x[i + 1];
      if (i + 2 < t) a2 -= sL[t][i + 2] * x[i + 2];
      if (i + 3 < t) a3 -= sL[t][i + 3] * x[i + 3];
    }
    x[t] = (a0 + a1) + (a2 + a3);
  }
  float* out = wu + ((long long)ch * H + h) * C * XW;
#pragma unroll
  for (int t = 0; t < C; ++t) out[t * XW + j] = x[t];
}

// Conversions with the packed hardware instruction (v_cvt_pk_bf16_f32,
// round to nearest even, as f2bf for finite values).
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef float float2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t cvt2(float a, float b) {
  const float2v f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2v));
}
// v = hi + lo with hi = rne(v), lo = rne(v - hi).
__device__ __forceinline__ void split8(const float* v, bf16x8& h, bf16x8& l) {
  uint32_t hw[4], lw[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    hw[e] = cvt2(v[2 * e], v[2 * e + 1]);
    lw[e] = cvt2(v[2 * e] - __uint_as_float(hw[e] << 16), v[2 * e + 1] - __uint_as_float(hw[e] & 0xFFFF0000u));
  }
  h = as_frag(make_uint4(hw[0], hw[1], hw[2], hw[3]));
  l = as_frag(make_uint4(lw[0], lw[1], lw[2], lw[3]));
}
// The same for the negated values.
__device__ __forceinline__ void split_neg(const float* v, bf16x8& h, bf16x8& l) {
  float nv[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) nv[e] = -v[e];
  split8(nv, h, l);
}

// ------------------------------------------------------------------ scan
// One workgroup of 4 waves per (sequence, head); wave w owns value columns
// 32 w .. 32 w + 31.  The state accumulator S[a][r] = S[32 a + acc_row(r)][32 w
// + cl] is the B operand of Q S0 and W S0 with the contraction index permuted
// as acc_row (Q and W are read with that permutation); U's accumulator
// layout U[tt][r] = U[32 tt + acc_row(r)][32 w + cl] is likewise the B
// operand of the token contractions (scores and decayed K^T are read with
// the permutation).
__global__ void __launch_bounds__(256)
gdn_scan_kernel(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, int ldqkv,
                const float* __restrict__ lg, int ldg, const float* __restrict__ wu,
                bf16_t* __restrict__ o, int ldo, const GdnSeq* __restrict__ seqs,
                float* __restrict__ states, int H) {
  __shared__ __attribute__((aligned(16))) char sQ[C * QP];
  __shared__ __attribute__((aligned(16))) char sK[C * QP];
  __shared__ __attribute__((aligned(16))) char sKt[DK * TP];   // decayed K^T, hi
  __shared__ __attribute__((aligned(16))) char sKl[DK * TP];   // decayed K^T, lo
  __shared__ __attribute__((aligned(16))) char sW[C * WP];     // W rows, fp32
  __shared__ float sG[C];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hi = lane >> 5, cl = lane & 31;
  const int seq = blockIdx.x, h = blockIdx.y;
  const GdnSeq sq = seqs[seq];
  const int dv0 = wave * 32;

  floatx16 S[DK / 32];
#pragma unroll
  for (int a = 0; a < DK / 32; ++a)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      S[a][r] = sq.s_in >= 0
                    ? states[(((long long)sq.s_in * H + h) * DK + 32 * a + acc_row(r, lane)) * DV + dv0 + cl]
                    : 0.f;

  for (int c0 = 0, ci = sq.c0; c0 < sq.len; c0 += C, ++ci) {
    const int n = min(C, sq.len - c0);
    const long long base = (long long)sq.row0 + c0;
    const float* X = wu + ((long long)ci * H + h) * C * XW;
    float G = lane < n ? lg[(base + lane) * ldg + h] : 0.f;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float t = __shfl_up(G, off, 64);
      if (lane >= off) G += t;
    }
    const float Glast = __shfl(G, 63, 64);
    const float wK = __expf(Glast - G);

    __syncthreads();
    if (wave == 0) sG[lane] = G;
    // every global load of the chunk first (rows past its end read its last
    // row, in bounds, and are replaced by zeros), then the LDS stores
    uint4 qv[C * 16 / 256], kav[C * 8 / 256], kbv[C * 8 / 256];
    float4 wv4[C * (DK / 4) / 256];
#pragma unroll
    for (int i = 0; i < C * 16 / 256; ++i) {
      const int c = tid + 256 * i, s = c >> 4, q8 = c & 15;
      qv[i] = *reinterpret_cast<const uint4*>(q + (base + min(s, n - 1)) * ldqkv + h * DK + q8 * 8);
    }
#pragma unroll
    for (int i = 0; i < C * 8 / 256; ++i) {
      const int c = tid + 256 * i, p = c >> 4, q8 = c & 15;
      kav[i] = *reinterpret_cast<const uint4*>(k + (base + min(2 * p, n - 1)) * ldqkv + h * DK + q8 * 8);
      kbv[i] = *reinterpret_cast<const uint4*>(k + (base + min(2 * p + 1, n - 1)) * ldqkv + h * DK + q8 * 8);
    }
#pragma unroll
    for (int i = 0; i < C * (DK / 4) / 256; ++i) {
      const int c = tid + 256 * i, t = c / (DK / 4), q4 = c % (DK / 4);
      wv4[i] = *reinterpret_cast<const float4*>(X + t * XW + 4 * q4);
    }
#pragma unroll
    for (int i = 0; i < C * 16 / 256; ++i) {
      const int c = tid + 256 * i, s = c >> 4, q8 = c & 15;
      *reinterpret_cast<uint4*>(sQ + s * QP + q8 * 16) = s < n ? qv[i] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < C * (DK / 4) / 256; ++i) {
      const int c = tid + 256 * i, t = c / (DK / 4), q4 = c % (DK / 4);
      *reinterpret_cast<float4*>(sW + t * WP + q4 * 16) = wv4[i];
    }
#pragma unroll
    for (int i = 0; i < C * 8 / 256; ++i) {
      const int c = tid + 256 * i, p = c >> 4, q8 = c & 15, s0 = 2 * p, s1 = s0 + 1;
      const uint4 ka = s0 < n ? kav[i] : make_uint4(0, 0, 0, 0);
      const uint4 kb = s1 < n ? kbv[i] : make_uint4(0, 0, 0, 0);
      *reinterpret_cast<uint4*>(sK + s0 * QP + q8 * 16) = ka;
      *reinterpret_cast<uint4*>(sK + s1 * QP + q8 * 16) = kb;
      const float w0 = __shfl(wK, s0, 64), w1 = __shfl(wK, s1, 64);
      const uint32_t av[4] = {ka.x, ka.y, ka.z, ka.w}, bv[4] = {kb.x, kb.y, kb.z, kb.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int d0 = q8 * 8 + 2 * e;
        const float x00 = __uint_as_float(av[e] << 16) * w0, x01 = __uint_as_float(bv[e] << 16) * w1;
        const float x10 = __uint_as_float(av[e] & 0xFFFF0000u) * w0, x11 = __uint_as_float(bv[e] & 0xFFFF0000u) * w1;
        const uint32_t h0 = cvt2(x00, x01), h1 = cvt2(x10, x11);
        *reinterpret_cast<uint32_t*>(sKt + d0 * TP + 4 * p) = h0;
        *reinterpret_cast<uint32_t*>(sKt + (d0 + 1) * TP + 4 * p) = h1;
        *reinterpret_cast<uint32_t*>(sKl + d0 * TP + 4 * p) =
            cvt2(x00 - __uint_as_float(h0 << 16), x01 - __uint_as_float(h0 & 0xFFFF0000u));
        *reinterpret_cast<uint32_t*>(sKl + (d0 + 1) * TP + 4 * p) =
            cvt2(x10 - __uint_as_float(h1 << 16), x11 - __uint_as_float(h1 & 0xFFFF0000u));
      }
    }
    __syncthreads();

    // state operand, split once for W S0 and Q S0
    bf16x8 shi[DK / 32][2], slo[DK / 32][2];
#pragma unroll
    for (int a = 0; a < DK / 32; ++a)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        float sv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) sv[e] = S[a][8 * hf + e];
        split8(sv, shi[a][hf], slo[a][hf]);
      }

    // (1) U = Ut - W S0 for both token tiles
    floatx16 U[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        U[tt][r] = X[(32 * tt + acc_row(r, lane)) * XW + DK + dv0 + cl];
#pragma unroll
      for (int a = 0; a < DK / 32; ++a)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const float* wr = reinterpret_cast<const float*>(sW + (32 * tt + cl) * WP) + 32 * a + 16 * hf + 4 * hi;
          const float4 w0 = *reinterpret_cast<const float4*>(wr);
          const float4 w1 = *reinterpret_cast<const float4*>(wr + 8);
          const float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
          bf16x8 whi, wlo;
          split_neg(wv, whi, wlo);
          mfma32(U[tt], whi, shi[a][hf]);
          mfma32(U[tt], whi, slo[a][hf]);
          mfma32(U[tt], wlo, shi[a][hf]);
        }
    }

    // (2) scores A^T[s][t] = k_s . q_t for s-tile st <= t-tile tt, masked and
    // decayed by exp(G_t - G_s)
    floatx16 At[3];   // (0,0), (0,1), (1,1)
#pragma unroll
    for (int x = 0; x < 3; ++x) {
      const int st = x == 2 ? 1 : 0, tt = x == 0 ? 0 : 1;
#pragma unroll
      for (int r = 0; r < 16; ++r) At[x][r] = 0.f;
      const char* kr = sK + (32 * st + cl) * QP + 16 * hi;
      const char* qr = sQ + (32 * tt + cl) * QP + 16 * hi;
#pragma unroll
      for (int ks = 0; ks < DK / 16; ++ks)
        mfma32(At[x], as_frag(*reinterpret_cast<const uint4*>(kr + 32 * ks)),
               as_frag(*reinterpret_cast<const uint4*>(qr + 32 * ks)));
      const int t = 32 * tt + cl;
      const float Gt = sG[t];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int s = 32 * st + acc_row(r, lane);
        At[x][r] = s <= t ? At[x][r] * __expf(Gt - sG[s]) : 0.f;
      }
    }

    // U operand, hi / lo, shared by (3) and (4)
    bf16x8 uhi[2][2], ulo[2][2];
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        float uv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) uv[e] = U[st][8 * hf + e];
        split8(uv, uhi[st][hf], ulo[st][hf]);
      }

    // (3) O = (A . D) U + exp(G_t) Q S0
    floatx16 O1[2], O2[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        O1[tt][r] = 0.f;
        O2[tt][r] = 0.f;
      }
#pragma unroll
    for (int a = 0; a < DK / 32; ++a)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          const char* qp = sQ + (32 * tt + cl) * QP + (32 * a + 16 * hf + 4 * hi) * 2;
          const bf16x8 qf = frag_from_halves(*reinterpret_cast<const uint2*>(qp),
                                             *reinterpret_cast<const uint2*>(qp + 16));
          mfma32(O2[tt], qf, shi[a][hf]);
          mfma32(O2[tt], qf, slo[a][hf]);
        }
#pragma unroll
    for (int x = 0; x < 3; ++x) {
      const int st = x == 2 ? 1 : 0, tt = x == 0 ? 0 : 1;
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        float av[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) av[e] = At[x][8 * hf + e];
        bf16x8 ahi, alo;
        split8(av, ahi, alo);
        mfma32(O1[tt], ahi, uhi[st][hf]);
        mfma32(O1[tt], ahi, ulo[st][hf]);
        mfma32(O1[tt], alo, uhi[st][hf]);
      }
    }
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int t = 32 * tt + acc_row(r, lane);
        if (t < n) o[(base + t) * ldo + (long long)h * DV + dv0 + cl] = f2bf(O1[tt][r] + __expf(sG[t]) * O2[tt][r]);
      }

    // (4) S' = exp(G_last) S0 + (K . w)^T U, the token index permuted as
    // acc_row on both operands
    const float dec = __expf(Glast);
#pragma unroll
    for (int a = 0; a < DK / 32; ++a) {
#pragma unroll
      for (int r = 0; r < 16; ++r) S[a][r] *= dec;
      const char* kt = sKt + (32 * a + cl) * TP;
      const char* kl = sKl + (32 * a + cl) * TP;
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const int off = (32 * st + 16 * hf + 4 * hi) * 2;
          const bf16x8 khi = frag_from_halves(*reinterpret_cast<const uint2*>(kt + off),
                                              *reinterpret_cast<const uint2*>(kt + off + 16));
          const bf16x8 klo = frag_from_halves(*reinterpret_cast<const uint2*>(kl + off),
                                              *reinterpret_cast<const uint2*>(kl + off + 16));
          mfma32(S[a], khi, uhi[st][hf]);
          mfma32(S[a], khi, ulo[st][hf]);
          mfma32(S[a], klo, uhi[st][hf]);
        }
    }
  }

  if (sq.s_out >= 0) {
#pragma unroll
    for (int a = 0; a < DK / 32; ++a)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        states[(((long long)sq.s_out * H + h) * DK + 32 * a + acc_row(r, lane)) * DV + dv0 + cl] = S[a][r];
  }
}

// ----------------------------------------------------------- convolution
// Grid (channel blocks of 256 eight-channel groups, row blocks of CONV_ROWS
// rows of the pass). Thread t of channel block b handles group 256 b + t for
// the block's rows, with the group's taps held in registers; the 16 groups of
// one head are 16 consecutive threads, which reduce the head's sum of squares
// among themselves.
constexpr int CONV_ROWS = 4;

__global__ void __launch_bounds__(256)
gdn_conv_kernel(const bf16_t* __restrict__ x, bf16_t* __restrict__ y, int ld, const float* __restrict__ w,
                int H, int r0, int T, const int32_t* __restrict__ row_seq, const GdnSeq* __restrict__ seqs,
                bf16_t* __restrict__ hist, float qscale) {
  const int Cc = 3 * H * DK, NG = Cc / 8, QKG = 2 * H * DK / 8;
  const int g = blockIdx.x * 256 + (int)threadIdx.x;
  if (g >= NG) return;              // NG is a multiple of 16: whole 16-thread head groups leave together
  const int c0 = 8 * g;
  float4 tap[8];                    // taps of channels c0 .. c0 + 7
#pragma unroll
  for (int e = 0; e < 8; ++e) tap[e] = *reinterpret_cast<const float4*>(w + (long long)(c0 + e) * 4);
  const bool qk = g < QKG;
  const float nscale = g < QKG / 2 ? qscale : 1.f;
  for (int rr = 0; rr < CONV_ROWS; ++rr) {
    const int pr = blockIdx.y * CONV_ROWS + rr;     // row within the pass
    if (pr >= T) break;
    const int r = r0 + pr;
    const GdnSeq sq = seqs[row_seq[pr]];
    const int t = r - sq.row0;
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int tt = t - 3 + j;
      uint4 u = make_uint4(0, 0, 0, 0);
      if (tt >= 0)
        u = *reinterpret_cast<const uint4*>(x + (long long)(sq.row0 + tt) * ld + c0);
      else if (sq.s_in >= 0)
        u = *reinterpret_cast<const uint4*>(hist + ((long long)sq.s_in * 3 + (3 + tt)) * Cc + c0);
      const uint32_t uv[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float4 ta = tap[2 * e], tb = tap[2 * e + 1];
        const float wa = j == 0 ? ta.x : j == 1 ? ta.y : j == 2 ? ta.z : ta.w;
        const float wb = j == 0 ? tb.x : j == 1 ? tb.y : j == 2 ? tb.z : tb.w;
        acc[2 * e] += wa * __uint_as_float(uv[e] << 16);
        acc[2 * e + 1] += wb * __uint_as_float(uv[e] & 0xFFFF0000u);
      }
    }
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      acc[e] = acc[e] / (1.f + __expf(-acc[e]));
      ss += acc[e] * acc[e];
    }
    if (qk) {                       // q or k: L2 norm over the head's 16 groups
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) ss += __shfl_xor(ss, off, 64);
      const float sc = rsqrtf(ss + 1e-6f) * nscale;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] *= sc;
    }
    uint4 o;
    o.x = pack_bf2(acc[0], acc[1]);
    o.y = pack_bf2(acc[2], acc[3]);
    o.z = pack_bf2(acc[4], acc[5]);
    o.w = pack_bf2(acc[6], acc[7]);
    *reinterpret_cast<uint4*>(y + (long long)r * ld + c0) = o;
    if (sq.s_out >= 0) {
      // the sequence's last three pre-convolution rows (zeros before its start)
      const int hrow = t - (sq.len - 3);
      if (hrow >= 0)
        *reinterpret_cast<uint4*>(hist + ((long long)sq.s_out * 3 + hrow) * Cc + c0) =
            *reinterpret_cast<const uint4*>(x + (long long)r * ld + c0);
      if (t == 0)
        for (int z = 0; z < 3 - sq.len; ++z)
          *reinterpret_cast<uint4*>(hist + ((long long)sq.s_out * 3 + z) * Cc + c0) = make_uint4(0, 0, 0, 0);
    }
  }
}

}  // namespace

hipError_t launch_gdn_conv(const void* x, void* y, int ld, const float* w, int H, int r0, int T,
                           const int32_t* row_seq, const GdnSeq* seqs, void* hist, float qscale, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  const int NG = 3 * H * DK / 8;
  hipLaunchKernelGGL(gdn_conv_kernel, dim3((NG + 255) / 256, (T + CONV_ROWS - 1) / CONV_ROWS), dim3(256), 0, s,
                     reinterpret_cast<const bf16_t*>(x), reinterpret_cast<bf16_t*>(y), ld, w, H, r0, T, row_seq,
                     seqs, reinterpret_cast<bf16_t*>(hist), qscale);
  return hipGetLastError();
}

size_t gdn_ws_bytes(int n_chunks, int H) { return (size_t)n_chunks * H * C * XW * sizeof(float); }

hipError_t launch_gdn_scan(const void* q, const void* k, const void* v, int ld_qkv, const float* log_g,
                           const float* beta, int ld_g, void* o, int ld_o, const ScanSeq* chunks, int n_chunks,
                           const GdnSeq* seqs, int n_seqs, float* states, int H, float* ws, hipStream_t s) {
  if (n_seqs <= 0 || H <= 0 || n_chunks <= 0) return hipSuccess;
  hipLaunchKernelGGL(gdn_prep_kernel, dim3(n_chunks, H), dim3(256), 0, s, reinterpret_cast<const bf16_t*>(k),
                     reinterpret_cast<const bf16_t*>(v), ld_qkv, log_g, beta, ld_g, chunks, ws, H);
  hipLaunchKernelGGL(gdn_scan_kernel, dim3(n_seqs, H), dim3(256), 0, s, reinterpret_cast<const bf16_t*>(q),
                     reinterpret_cast<const bf16_t*>(k), ld_qkv, log_g, ld_g, ws, reinterpret_cast<bf16_t*>(o),
                     ld_o, seqs, states, H);
  return hipGetLastError();
}

}  // namespace s1
