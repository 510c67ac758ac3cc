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
//   O  = diag(gamma) Q S0 + A U,   A[t][i] = (gamma_t / gamma_i) q_t . k_i (i <= t),
//   S' = gamma_C S0 + Kd^T U,      Kd = K . gamma_C / gamma.
// With W = (I + L)^-1 diag(beta gamma) K and Ut = (I + L)^-1 diag(beta) V,
// U = Ut - W S0, so every chunk is an affine map of its initial state:
//   S' = M S0 + B,      M = gamma_C I - Kd^T W,          B = Kd^T Ut,
//   O  = Qt S0 + Ol,    Qt = diag(gamma) Q - A W,        Ol = A Ut.
//   gdn_chunk_kernel  every (chunk, head) in parallel: L and A on MFMA, W | Ut
//                     by forward substitution (one column per thread), then M,
//                     B, Qt and Ol on MFMA, written in the register layouts
//                     the state kernel consumes;
//   gdn_state_kernel  every (sequence, head, 32 value columns) in order over
//                     its chunks: the state stays in accumulator registers,
//                     O = Qt S + Ol and S <- M S + B, two MFMA products per
//                     chunk and no other arithmetic.
// Operands formed inside the kernels (W, Ut, A, decayed keys, M, Qt, the
// state) are fp32 values split into bf16 hi + lo parts; products of two such
// operands take three MFMAs (hi.hi + hi.lo + lo.hi), so the kernels add
// little beyond fp32 rounding to their bf16 q, k, v.
#include "common.h"
#include "kernels.h"

namespace s1 {
namespace {

constexpr int C = 64, DK = 128, DV = 128;
constexpr int QP = DK * 2 + 16;    // bytes per Q / K row in LDS (bf16)
constexpr int LP = C + 4;          // floats per L row in LDS
constexpr int RP = C * 2 + 16;     // bytes per row of a [.][C] bf16 operand in LDS
// Workspace of one (chunk, head), in 16-byte units:
//   M   A operands of M S: [row tile 4][k tile 4][half 2][hi, lo][lane 64]
//   B   accumulator tiles of B: [row tile 4][value tile 4][lane 64][16 floats]
//   Qt  A operands of Qt S: [token tile 2][k tile 4][half 2][hi, lo][lane 64]
//   Ol  accumulator tiles of Ol: [token tile 2][value tile 4][lane 64][16 floats]
constexpr int WS_M = 4 * 4 * 2 * 2 * 64, WS_B = 4 * 4 * 64 * 4, WS_Q = 2 * 4 * 2 * 2 * 64, WS_O = 2 * 4 * 64 * 4;
constexpr int WS_CH = WS_M + WS_B + WS_Q + WS_O;

// v = hi + lo with hi = rne(v), lo = rne(v - hi), as two 16-byte operands.
__device__ __forceinline__ void split8(const float* v, uint4& h, uint4& l) {
  uint32_t hw[4], lw[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    hw[e] = cvt2(v[2 * e], v[2 * e + 1]);
    lw[e] = cvt2(v[2 * e] - lo_half(hw[e]), v[2 * e + 1] - hi_half(hw[e]));
  }
  h = make_uint4(hw[0], hw[1], hw[2], hw[3]);
  l = make_uint4(lw[0], lw[1], lw[2], lw[3]);
}
__device__ __forceinline__ bf16x8 lds16(const char* p) { return as_frag(*reinterpret_cast<const uint4*>(p)); }
// c += a b in split precision (hi.hi + hi.lo + lo.hi)
__device__ __forceinline__ void mfma3(floatx16& c, bf16x8 ah, bf16x8 al, bf16x8 bh, bf16x8 bl) {
  mfma32(c, ah, bh);
  mfma32(c, ah, bl);
  mfma32(c, al, bh);
}

// ---------------------------------------------------------------- chunk
// One workgroup (4 waves) per (chunk, head).
__global__ void __launch_bounds__(256)
gdn_chunk_kernel(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
                 int ldqkv, const float* __restrict__ lg, const float* __restrict__ beta, int ldg,
                 const ScanSeq* __restrict__ chunks, uint4* __restrict__ ws, int H) {
  __shared__ __attribute__((aligned(16))) char sQ[C * QP];
  // K and L first; after the solve, the rows of W^T | Ut^T (hi, then lo)
  __shared__ __attribute__((aligned(16))) char sR[2 * (DK + DV) * RP];
  __shared__ __attribute__((aligned(16))) char sA[2 * C * RP];     // A [t][i], hi then lo
  __shared__ __attribute__((aligned(16))) char sKT[2 * DK * RP];   // Kd^T [d][t], hi then lo
  __shared__ float sG[C], sB[C];
  char* const sK = sR;
  float* const sL = reinterpret_cast<float*>(sR + C * QP);
  char* const sXh = sR;
  char* const sXl = sR + (DK + DV) * RP;
  char* const sAh = sA;
  char* const sAl = sA + C * RP;
  char* const sKh = sKT;
  char* const sKl = sKT + DK * RP;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hi = lane >> 5, cl = lane & 31;
  const int ch = blockIdx.x, h = blockIdx.y;
  const ScanSeq cq = chunks[ch];
  const int n = cq.len;
  const long long base = cq.row0;

  // every wave: cumulative log gate, lane = token (zero increments past the end)
  float G = lane < n ? lg[(base + lane) * ldg + h] : 0.f;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float t = __shfl_up(G, off, 64);
    if (lane >= off) G += t;
  }
  const float Glast = __shfl(G, 63, 64);
  const float wK = __expf(Glast - G);
  if (wave == 0) {
    sG[lane] = G;
    sB[lane] = lane < n ? beta[(base + lane) * ldg + h] : 0.f;
  }
  // Q and K rows (rows past the end read the last row, in bounds, and are
  // replaced by zeros), and the decayed keys transposed, hi / lo
  {
    uint4 qv[C * 16 / 256], kav[C * 8 / 256], kbv[C * 8 / 256];
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
    for (int i = 0; i < C * 16 / 256; ++i) {
      const int c = tid + 256 * i, s = c >> 4, q8 = c & 15;
      *reinterpret_cast<uint4*>(sQ + s * QP + q8 * 16) = s < n ? qv[i] : make_uint4(0, 0, 0, 0);
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
        const float x00 = lo_half(av[e]) * w0, x01 = lo_half(bv[e]) * w1;
        const float x10 = hi_half(av[e]) * w0, x11 = hi_half(bv[e]) * w1;
        const uint32_t h0 = cvt2(x00, x01), h1 = cvt2(x10, x11);
        *reinterpret_cast<uint32_t*>(sKh + d0 * RP + 4 * p) = h0;
        *reinterpret_cast<uint32_t*>(sKh + (d0 + 1) * RP + 4 * p) = h1;
        *reinterpret_cast<uint32_t*>(sKl + d0 * RP + 4 * p) = cvt2(x00 - lo_half(h0), x01 - hi_half(h0));
        *reinterpret_cast<uint32_t*>(sKl + (d0 + 1) * RP + 4 * p) = cvt2(x10 - lo_half(h1), x11 - hi_half(h1));
      }
    }
  }
  __syncthreads();

  // K K^T and Q K^T: wave w takes the 32 x 32 tile (w / 2, w % 2) of both;
  // exact products of bf16 inputs, fp32 accumulation
  {
    const int ti = wave >> 1, tj = wave & 1;
    floatx16 accL, accA;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      accL[r] = 0.f;
      accA[r] = 0.f;
    }
    const char* kr = sK + (32 * ti + cl) * QP + 16 * hi;
    const char* qr = sQ + (32 * ti + cl) * QP + 16 * hi;
    const char* br = sK + (32 * tj + cl) * QP + 16 * hi;
    // (the tile above the diagonal of Q K^T is formed too and masked below)
#pragma unroll
    for (int ks = 0; ks < DK / 16; ++ks) {
      const bf16x8 bf = lds16(br + 32 * ks);
      mfma32(accL, lds16(kr + 32 * ks), bf);
      mfma32(accA, lds16(qr + 32 * ks), bf);
    }
    // acc[r] = X[32 ti + acc_row(r)][32 tj + cl]: row t, column i
    const float Gi = sG[32 * tj + cl];
    float Gt[16], Bt[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      Gt[r] = sG[32 * ti + acc_row(r, lane)];
      Bt[r] = sB[32 * ti + acc_row(r, lane)];
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int t = 32 * ti + acc_row(r, lane), i = 32 * tj + cl;
      const float dcy = __expf(Gt[r] - Gi);   // may overflow above the diagonal, where it is not used
      sL[t * LP + i] = i < t ? Bt[r] * dcy * accL[r] : 0.f;
      const float a = i <= t ? dcy * accA[r] : 0.f;
      const uint32_t ah = cvt2(a, 0.f);
      const uint32_t al = cvt2(a - lo_half(ah), 0.f);
      *reinterpret_cast<bf16_t*>(sAh + t * RP + 2 * i) = (bf16_t)(ah & 0xFFFFu);
      *reinterpret_cast<bf16_t*>(sAl + t * RP + 2 * i) = (bf16_t)(al & 0xFFFFu);
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
  // Row t of L is read from LDS (a broadcast: every thread reads the same
  // words) while row t - 1 is applied, so the reads' latency is hidden; four
  // partial sums per row shorten the dependent chain.
  float4 Lr[2][C / 4];
  Lr[1][0] = *reinterpret_cast<const float4*>(sL + 1 * LP);
#pragma unroll
  for (int t = 1; t < C; ++t) {
    float4* const cur = Lr[t & 1];
    float4* const nxt = Lr[(t + 1) & 1];
    if (t + 1 < C) {
#pragma unroll
      for (int q4 = 0; q4 < (t + 4) / 4; ++q4) nxt[q4] = *reinterpret_cast<const float4*>(sL + (t + 1) * LP + 4 * q4);
    }
    __builtin_amdgcn_sched_barrier(0);
    float a0 = x[t], a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
    for (int i = 0; i < t; i += 4) {
      const float4 c = cur[i / 4];
      a0 -= c.x * x[i];
      if (i + 1 < t) a1 -= c.y * x[i + 1];
      if (i + 2 < t) a2 -= c.z * x[i + 2];
      if (i + 3 < t) a3 -= c.w * x[i + 3];
    }
    x[t] = (a0 + a1) + (a2 + a3);
  }
  __syncthreads();   // K and L are no longer read: their space takes W^T | Ut^T
#pragma unroll
  for (int t8 = 0; t8 < C / 8; ++t8) {
    uint4 xh, xl;
    split8(x + 8 * t8, xh, xl);
    *reinterpret_cast<uint4*>(sXh + j * RP + 16 * t8) = xh;
    *reinterpret_cast<uint4*>(sXl + j * RP + 16 * t8) = xl;
  }
  __syncthreads();

  uint4* const wsc = ws + ((long long)ch * H + h) * WS_CH;
  const float gC = __expf(Glast);
  // M^T = gamma_C I - W^T Kd (tiles (wave, ti)) and P = W^T A^T (tiles
  // (wave, tt)); the accumulator of M^T tile (j, i) holds, per lane, the A
  // operand of M S for row tile i, k tile j, which is how it is stored
  {
    floatx16 accM[4], accP[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
#pragma unroll
      for (int u = 0; u < 4; ++u) accM[u][r] = 0.f;
      accP[0][r] = 0.f;
      accP[1][r] = 0.f;
    }
#pragma unroll
    for (int ks = 0; ks < C / 16; ++ks) {
      const int off = 32 * ks + 16 * hi;
      const int wr = (32 * wave + cl) * RP + off;
      const bf16x8 wh = lds16(sXh + wr), wl = lds16(sXl + wr);
#pragma unroll
      for (int ti = 0; ti < 4; ++ti) {
        const int kr = (32 * ti + cl) * RP + off;
        mfma3(accM[ti], wh, wl, lds16(sKh + kr), lds16(sKl + kr));
      }
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const int ar = (32 * tt + cl) * RP + off;
        mfma3(accP[tt], wh, wl, lds16(sAh + ar), lds16(sAl + ar));
      }
    }
#pragma unroll
    for (int ti = 0; ti < 4; ++ti)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        float mv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int jj = 32 * wave + acc_row(8 * hf + e, lane), ii = 32 * ti + cl;
          mv[e] = (jj == ii ? gC : 0.f) - accM[ti][8 * hf + e];
        }
        uint4 mh, ml;
        split8(mv, mh, ml);
        uint4* dst = wsc + (((ti * 4 + wave) * 2 + hf) * 2) * 64 + lane;
        dst[0] = mh;
        dst[64] = ml;
      }
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        float qv[8];
        const int t = 32 * tt + cl;
        const float gt = __expf(sG[t]);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int jj = 32 * wave + acc_row(8 * hf + e, lane);
          qv[e] = gt * bf2f(*reinterpret_cast<const bf16_t*>(sQ + t * QP + 2 * jj)) - accP[tt][8 * hf + e];
        }
        uint4 qh, ql;
        split8(qv, qh, ql);
        uint4* dst = wsc + WS_M + WS_B + (((tt * 4 + wave) * 2 + hf) * 2) * 64 + lane;
        dst[0] = qh;
        dst[64] = ql;
      }
  }
  // B = Kd^T Ut (tiles (wave, value tile)) and Ol = A Ut (tiles (wave / 2,
  // value tiles 2 (wave % 2) + 0, 1)), stored as accumulator tiles
  {
    floatx16 accB[4], accO[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
#pragma unroll
      for (int u = 0; u < 4; ++u) accB[u][r] = 0.f;
      accO[0][r] = 0.f;
      accO[1][r] = 0.f;
    }
    const int tt = wave >> 1;
#pragma unroll
    for (int ks = 0; ks < C / 16; ++ks) {
      const int off = 32 * ks + 16 * hi;
      const int kr = (32 * wave + cl) * RP + off, ar = (32 * tt + cl) * RP + off;
      const bf16x8 kh = lds16(sKh + kr), kl = lds16(sKl + kr);
      const bf16x8 ah = lds16(sAh + ar), al = lds16(sAl + ar);
#pragma unroll
      for (int vt = 0; vt < 4; ++vt) {
        const int ur = (DK + 32 * vt + cl) * RP + off;
        const bf16x8 uh = lds16(sXh + ur), ul = lds16(sXl + ur);
        mfma3(accB[vt], kh, kl, uh, ul);
        if ((vt >> 1) == (wave & 1)) mfma3(accO[vt & 1], ah, al, uh, ul);
      }
    }
    float4* const wB = reinterpret_cast<float4*>(wsc + WS_M);
    float4* const wO = reinterpret_cast<float4*>(wsc + WS_M + WS_B + WS_Q);
#pragma unroll
    for (int vt = 0; vt < 4; ++vt)
#pragma unroll
      for (int f = 0; f < 4; ++f)
        wB[((wave * 4 + vt) * 64 + lane) * 4 + f] =
            make_float4(accB[vt][4 * f], accB[vt][4 * f + 1], accB[vt][4 * f + 2], accB[vt][4 * f + 3]);
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int f = 0; f < 4; ++f)
        wO[((tt * 4 + 2 * (wave & 1) + u) * 64 + lane) * 4 + f] =
            make_float4(accO[u][4 * f], accO[u][4 * f + 1], accO[u][4 * f + 2], accO[u][4 * f + 3]);
  }
}

// ---------------------------------------------------------------- state
// One workgroup of 6 waves per (sequence, head, value tile of 32 columns).
// Waves 0..3 own row tile w of the state, S_w = S[32 w .. 32 w + 31][32 vt
// .. 32 vt + 31], and form M_w S + B_w; waves 4 and 5 form the output rows
// 32 (w - 4) .. + 31 as Qt S + Ol.  Both are one 32 x 32 accumulator tile
// with 16 A operands from the chunk kernel; the state is exchanged through
// LDS each chunk as B operands (hi / lo, contraction index permuted as
// acc_row, as the chunk kernel wrote M and Qt), double-buffered so that one
// barrier per chunk suffices.  The operands of the next chunk, which do not
// depend on the state, are loaded while the current one is computed.
constexpr int ST_WAVES = 6;

__global__ void __launch_bounds__(64 * ST_WAVES)
gdn_state_kernel(const uint4* __restrict__ ws, bf16_t* __restrict__ o, int ldo, const GdnSeq* __restrict__ seqs,
                 float* __restrict__ states, int H) {
  __shared__ uint4 sS[2][DK / 32][2][2][64];   // [buffer][row tile][half][hi, lo][lane]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, cl = lane & 31;
  const int h = blockIdx.y, vt = blockIdx.z;
  const GdnSeq sq = seqs[blockIdx.x];
  const int v0 = 32 * vt;
  if (sq.len <= 0) return;
  const bool srow = wave < 4;

  floatx16 acc;
  if (srow) {
#pragma unroll
    for (int r = 0; r < 16; ++r)
      acc[r] = sq.s_in >= 0
                   ? states[(((long long)sq.s_in * H + h) * DK + 32 * wave + acc_row(r, lane)) * DV + v0 + cl]
                   : 0.f;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      float sv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) sv[e] = acc[8 * hf + e];
      split8(sv, sS[0][wave][hf][0][lane], sS[0][wave][hf][1][lane]);
    }
  }

  // this wave's 16 A operands [k tile][half][hi, lo] and accumulator start
  auto load = [&](int ci, uint4* af, float4* cf) {
    const uint4* const wsc = ws + ((long long)ci * H + h) * WS_CH;
    const uint4* const A = srow ? wsc + wave * 16 * 64 : wsc + WS_M + WS_B + (wave - 4) * 16 * 64;
    const float4* const Cs =
        srow ? reinterpret_cast<const float4*>(wsc + WS_M) + ((wave * 4 + vt) * 64 + lane) * 4
             : reinterpret_cast<const float4*>(wsc + WS_M + WS_B + WS_Q) + (((wave - 4) * 4 + vt) * 64 + lane) * 4;
#pragma unroll
    for (int i = 0; i < 16; ++i) af[i] = A[i * 64 + lane];
#pragma unroll
    for (int f = 0; f < 4; ++f) cf[f] = Cs[f];
  };
  uint4 ca[16];
  float4 cc[4];
  load(sq.c0, ca, cc);
  __syncthreads();

  int buf = 0;
  for (int c0 = 0, ci = sq.c0; c0 < sq.len; c0 += C, ++ci) {
    const int n = min(C, sq.len - c0);
    const long long base = (long long)sq.row0 + c0;
    uint4 na[16];
    float4 nc[4];
    load(c0 + C < sq.len ? ci + 1 : ci, na, nc);
    __builtin_amdgcn_sched_barrier(0);   // keep these loads ahead of the products

#pragma unroll
    for (int f = 0; f < 4; ++f) {
      acc[4 * f] = cc[f].x;
      acc[4 * f + 1] = cc[f].y;
      acc[4 * f + 2] = cc[f].z;
      acc[4 * f + 3] = cc[f].w;
    }
#pragma unroll
    for (int ai = 0; ai < DK / 32; ++ai)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int i = (ai * 2 + hf) * 2;
        mfma3(acc, as_frag(ca[i]), as_frag(ca[i + 1]), as_frag(sS[buf][ai][hf][0][lane]),
              as_frag(sS[buf][ai][hf][1][lane]));
      }
    if (srow) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        float sv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) sv[e] = acc[8 * hf + e];
        split8(sv, sS[buf ^ 1][wave][hf][0][lane], sS[buf ^ 1][wave][hf][1][lane]);
      }
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int t = 32 * (wave - 4) + acc_row(r, lane);
        if (t < n) o[(base + t) * ldo + (long long)h * DV + v0 + cl] = f2bf(acc[r]);
      }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) ca[i] = na[i];
#pragma unroll
    for (int f = 0; f < 4; ++f) cc[f] = nc[f];
    buf ^= 1;
    __syncthreads();
  }

  if (srow && sq.s_out >= 0) {
#pragma unroll
    for (int r = 0; r < 16; ++r)
      states[(((long long)sq.s_out * H + h) * DK + 32 * wave + acc_row(r, lane)) * DV + v0 + cl] = acc[r];
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

size_t gdn_ws_bytes(int n_chunks, int H) { return (size_t)n_chunks * H * WS_CH * sizeof(uint4); }

hipError_t launch_gdn_scan(const void* q, const void* k, const void* v, int ld_qkv, const float* log_g,
                           const float* beta, int ld_g, void* o, int ld_o, const ScanSeq* chunks, int n_chunks,
                           const GdnSeq* seqs, int n_seqs, float* states, int H, float* ws, hipStream_t s) {
  if (n_seqs <= 0 || H <= 0 || n_chunks <= 0) return hipSuccess;
  uint4* const w = reinterpret_cast<uint4*>(ws);
  hipLaunchKernelGGL(gdn_chunk_kernel, dim3(n_chunks, H), dim3(256), 0, s, reinterpret_cast<const bf16_t*>(q),
                     reinterpret_cast<const bf16_t*>(k), reinterpret_cast<const bf16_t*>(v), ld_qkv, log_g, beta, ld_g,
                     chunks, w, H);
  hipLaunchKernelGGL(gdn_state_kernel, dim3(n_seqs, H, DV / 32), dim3(64 * ST_WAVES), 0, s, w,
                     reinterpret_cast<bf16_t*>(o),
                     ld_o, seqs, states, H);
  return hipGetLastError();
}

}  // namespace s1
