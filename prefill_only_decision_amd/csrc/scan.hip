// Chunked gated linear-attention scan (the recurrence S_t = g_t S_{t-1} +
// k_t v_t^T, o_t = S_t^T q_t, one scalar gate per token and head; the pages
// name Gated DeltaNet without printing its equations, and this is the stated
// stand-in).  The state stays fp32 (RFC #114 section 5: FP32 recurrent state;
// a branch starts from its prefix's final state).
//
// Chunks of C = 64 tokens are processed in order; inside a chunk, with
// G_t = sum_{r <= t} log g_r (chunk-local),
//   O = (QK^T . D) V + diag(exp G) Q S0,   D[t][s] = exp(G_t - G_s) for s <= t
//   S = exp(G_last) S0 + (K . exp(G_last - G))^T V
// Decays are always exponentials of differences, never ratios of products.
// All four products run on v_mfma_f32_32x32x16_bf16 with fp32 accumulation;
// the state lives in accumulator registers across chunks.  q, k, v arrive as
// bf16; the operands formed inside the kernel (decayed scores, the state,
// decayed keys) are split into hi + lo bf16 parts and multiplied twice, so
// the scan adds no rounding beyond fp32 accumulation to its bf16 inputs.  A wave owns 32
// value columns of one head; NW waves share the chunk's Q, K, K^T and V^T
// tiles in LDS.  The intra-chunk score tile is computed as K Q^T so that its
// accumulator layout is directly the A operand of (QK^T . D) V, and the state
// accumulator layout is directly the B operand of Q S0: both use the same
// permutation of the contraction index, which Q and V^T are read with.
#include "common.h"
#include "kernels.h"

namespace s1 {

namespace {

constexpr int C = 64, DK = 128, DV = 128;
constexpr int QP = DK * 2 + 16;   // bytes per Q / K row in LDS
constexpr int TP = C * 2 + 16;    // bytes per K^T / V^T row in LDS

// Byte offset of K^T / V^T row d in LDS: 16 bytes of padding after every 16
// rows.  The transposing stores of one instruction hit rows 8 apart (one
// element pair of many 16-byte load chunks), which without it share a bank;
// the reads of the products take 16 consecutive rows at a time, which the
// padding leaves at the same relative addresses.
__device__ __forceinline__ int trow(int d) { return d * TP + (d >> 4) * 16; }
constexpr int trows_bytes(int rows) { return rows * TP + (rows / 16) * 16; }

// Raw buffer over `bytes` bytes from `base`: loads at or past the end read
// zero and stores there are dropped (the range check covers the per-lane
// offset, which is where every offset that needs checking goes).  Buffer
// addressing keeps the per-lane offsets in 32-bit registers computed once
// and the per-access constants in scalar offsets.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}
__device__ __forceinline__ uint4 ld16(rsrc_t r, int voff) {
  const auto x = __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0);
  return make_uint4(x[0], x[1], x[2], x[3]);
}
__device__ __forceinline__ float ldf(rsrc_t r, int voff, int soff) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
}
__device__ __forceinline__ void stf(float x, rsrc_t r, int voff, int soff) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), r, voff, soff, 0);
}

// MODE_FULL: the recurrence over whole sequences.  MODE_SUMMARY: one chunk
// per entry from a zero state; writes only the chunk's state contribution and
// its total log-decay.  MODE_OUTPUT: one chunk per entry from the state
// entering it; writes only the outputs.  MODE_FOLD: MODE_OUTPUT that first
// forms its entering state from the contributions of its sequence's earlier
// chunks (S <- exp(gamma) S + dS in chunk order, the same operations as
// chunk_state_scan_kernel), and whose last chunk writes the sequence's final
// state: two launches in place of three for short sequences.
enum { MODE_FULL = 0, MODE_SUMMARY = 1, MODE_OUTPUT = 2, MODE_FOLD = 3 };

template <int NW, int MODE>
__global__ void __launch_bounds__(NW * 64)
scan_bf16_kernel(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                 const bf16_t* __restrict__ v, int ldqkv, const float* __restrict__ lg, int ldg,
                 bf16_t* __restrict__ o, int ldo, const ScanSeq* __restrict__ seqs,
                 float* __restrict__ states, int H, float* __restrict__ gamma,
                 const ChunkSeq* __restrict__ cseqs, int n_cseqs, float* __restrict__ seq_states) {
  constexpr int NT = NW * 64;
  constexpr int DVG = 32 * NW;        // value columns per workgroup
  constexpr int NDVG = DV / DVG;      // workgroups per (sequence, head)
  __shared__ __attribute__((aligned(16))) char sQ[C * QP];
  __shared__ __attribute__((aligned(16))) char sK[C * QP];
  __shared__ __attribute__((aligned(16))) char sKt[trows_bytes(DK)];     // decayed K^T, hi part
  __shared__ __attribute__((aligned(16))) char sKl[trows_bytes(DK)];     // decayed K^T, lo part
  __shared__ __attribute__((aligned(16))) char sVt[trows_bytes(DVG)];
  __shared__ float sG[C], sEG[C];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hi = lane >> 5, cl = lane & 31;
  // The chunk modes take their (chunk, head) in head-major order through
  // the XCD remap, so that each XCD runs a contiguous run of heads: the
  // chunk states a head's summary workgroups write are read by its fold
  // workgroups on the same XCD, out of that XCD's L2.
  int bx = blockIdx.x, by = blockIdx.y;
  if constexpr (MODE != MODE_FULL) {
    const int t = xcd_remap(blockIdx.x + gridDim.x * blockIdx.y, gridDim.x * gridDim.y);
    by = t / gridDim.x;
    bx = t - by * gridDim.x;
  }
  const int seq = bx / NDVG, dvg = bx % NDVG, h = by;
  const ScanSeq sq = seqs[seq];
  const int dvw = dvg * DVG;          // first value column of the workgroup
  const int dv0 = dvw + wave * 32;    // first value column of this wave

  // Each chunk's global loads, through buffers that end at the chunk's last
  // row: rows past it read zero.  Four-wave workgroups issue them right
  // after the previous chunk's LDS stores, so that they are in flight while
  // that chunk is multiplied; with fewer waves each thread holds too many of
  // them to keep them across the products.  The first chunk's loads are
  // issued before the entering state is read (the output modes' only chunk:
  // its loads overlap the state loads).
  constexpr bool PREFETCH = NW == 4 || MODE == MODE_OUTPUT || MODE == MODE_FOLD;
  constexpr int QI = C * 16 / NT, KI = C * 8 / NT, VI = (C / 2) * (DVG / 8) / NT;
  uint4 qv[MODE != MODE_SUMMARY ? QI : 1], kav[KI], kbv[KI], vav[VI], vbv[VI];
  const int ldb = ldqkv * 2;          // bytes per q/k/v row
  int qo[MODE != MODE_SUMMARY ? QI : 1], ko[KI], vo[VI];   // chunk-relative byte offsets (rows 2p for k, v)
#pragma unroll
  for (int i = 0; i < QI; ++i) {
    const int c = tid + NT * i;
    if constexpr (MODE != MODE_SUMMARY) qo[i] = (c >> 4) * ldb + (h * DK + (c & 15) * 8) * 2;
  }
#pragma unroll
  for (int i = 0; i < KI; ++i) {
    const int c = tid + NT * i;
    ko[i] = 2 * (c >> 4) * ldb + (h * DK + (c & 15) * 8) * 2;
  }
#pragma unroll
  for (int i = 0; i < VI; ++i) {
    const int c = tid + NT * i;
    vo[i] = 2 * (c / (DVG / 8)) * ldb + (h * DV + dvw + (c % (DVG / 8)) * 8) * 2;
  }
  float lgv = 0.f;
  auto load_chunk = [&](int cc) {
    const int nn = min(C, sq.len - cc);   // >= 1
    const long long bb = (long long)sq.row0 + cc;
    lgv = ldf(make_rsrc(lg + bb * ldg, nn * ldg * 4), (lane * ldg + h) * 4, 0);
    if constexpr (MODE != MODE_SUMMARY) {
      const rsrc_t rq = make_rsrc(q + bb * ldqkv, nn * ldb);
#pragma unroll
      for (int i = 0; i < QI; ++i) qv[i] = ld16(rq, qo[i]);
    }
    const rsrc_t rk = make_rsrc(k + bb * ldqkv, nn * ldb);
#pragma unroll
    for (int i = 0; i < KI; ++i) {
      kav[i] = ld16(rk, ko[i]);
      kbv[i] = ld16(rk, ko[i] + ldb);
    }
    const rsrc_t rv = make_rsrc(v + bb * ldqkv, nn * ldb);
#pragma unroll
    for (int i = 0; i < VI; ++i) {
      vav[i] = ld16(rv, vo[i]);
      vbv[i] = ld16(rv, vo[i] + ldb);
    }
  };
  if (PREFETCH && sq.len > 0) load_chunk(0);

  floatx16 S[DK / 32];                // S[a][r] = S[32a + acc_row(r)][dv0 + cl]
  // state slabs [DK][DV] fp32 per (slot, head): lane part of the offset, and
  // the constant part of element (a, r)
  const int st_lane = (4 * hi * DV + dv0 + cl) * 4;
  auto st_soff = [](int a, int r) { return (32 * a + 8 * (r >> 2) + (r & 3)) * DV * 4; };
  // chunk slots (the chunk-parallel modes' `states`) hold the state in the
  // accumulator order instead: [32-column block][a][r / 4][lane][r % 4], so
  // that a lane's four consecutive accumulators are one 16-byte access
  const int fr_lane = ((dv0 / 32) * (DK / 32) * 4 * 256 + lane * 4) * 4;
  auto fr_soff = [](int a, int rq) { return (a * 4 + rq) * 1024; };
  auto ld_frag = [&](rsrc_t rs, floatx16 (&X)[DK / 32]) {
    uint4 u[DK / 32][4];
#pragma unroll
    for (int a = 0; a < DK / 32; ++a)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const auto x = __builtin_amdgcn_raw_buffer_load_b128(rs, fr_lane, fr_soff(a, rq), 0);
        u[a][rq] = make_uint4(x[0], x[1], x[2], x[3]);
      }
#pragma unroll
    for (int a = 0; a < DK / 32; ++a)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        X[a][4 * rq] = __uint_as_float(u[a][rq].x);
        X[a][4 * rq + 1] = __uint_as_float(u[a][rq].y);
        X[a][4 * rq + 2] = __uint_as_float(u[a][rq].z);
        X[a][4 * rq + 3] = __uint_as_float(u[a][rq].w);
      }
  };
  auto slab = [&](const float* base, long long slot) { return make_rsrc(base + (slot * H + h) * DK * DV, DK * DV * 4); };
  ChunkSeq cs{0, 0, -1, -1};
  if constexpr (MODE == MODE_FOLD) {
    // this chunk's sequence: the last entry whose first chunk is at or before it
    int lo = 0, hi2 = n_cseqs - 1;
    while (lo < hi2) {
      const int mid = (lo + hi2 + 1) >> 1;
      if (cseqs[mid].c0 <= seq) lo = mid;
      else hi2 = mid - 1;
    }
    cs = cseqs[lo];
    if (cs.s_in >= 0) {
      const rsrc_t rs = slab(seq_states, cs.s_in);
#pragma unroll
      for (int a = 0; a < DK / 32; ++a)
#pragma unroll
        for (int r = 0; r < 16; ++r) S[a][r] = ldf(rs, st_lane, st_soff(a, r));
    } else {
#pragma unroll
      for (int a = 0; a < DK / 32; ++a)
#pragma unroll
        for (int r = 0; r < 16; ++r) S[a][r] = 0.f;
    }
    // the next predecessor's contribution is loaded while the current one is added
    floatx16 dA[DK / 32], dB[DK / 32];
    if (cs.c0 < seq) ld_frag(slab(states, cs.c0), dA);
    for (int c = cs.c0; c < seq; ++c) {
      const float g = __expf(gamma[(long long)c * H + h]);
      if (c + 1 < seq) ld_frag(slab(states, c + 1), dB);
#pragma unroll
      for (int a = 0; a < DK / 32; ++a)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          S[a][r] = fmaf(g, S[a][r], dA[a][r]);
          dA[a][r] = dB[a][r];
        }
    }
  } else if (MODE == MODE_OUTPUT) {
    ld_frag(slab(states, sq.s_in), S);   // the state entering the chunk
  } else if (MODE == MODE_FULL && sq.s_in >= 0) {
    const rsrc_t rs = slab(states, sq.s_in);
#pragma unroll
    for (int a = 0; a < DK / 32; ++a)
#pragma unroll
      for (int r = 0; r < 16; ++r) S[a][r] = ldf(rs, st_lane, st_soff(a, r));
  } else {
#pragma unroll
    for (int a = 0; a < DK / 32; ++a)
#pragma unroll
      for (int r = 0; r < 16; ++r) S[a][r] = 0.f;
  }


  for (int c0 = 0; c0 < sq.len; c0 += C) {
    if constexpr (!PREFETCH) load_chunk(c0);
    const int n = min(C, sq.len - c0);
    const long long base = (long long)sq.row0 + c0;
    // chunk-local cumulative log-gate, redundantly in every wave
    float G = lgv;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float t = __shfl_up(G, off, 64);
      if (lane >= off) G += t;
    }
    const float Glast = __shfl(G, 63, 64);
    const float wK = __expf(Glast - G);   // decay from token `lane` to the chunk end

    __syncthreads();                      // previous chunk's reads of LDS are done
    if (wave == 0) {
      sG[lane] = G;
      sEG[lane] = __expf(G);
    }
    if (MODE == MODE_SUMMARY && tid == 0 && dvg == 0) gamma[(long long)seq * H + h] = Glast;
    // Q rows: straight copy
    if constexpr (MODE != MODE_SUMMARY) {
#pragma unroll
      for (int i = 0; i < QI; ++i) {
        const int c = tid + NT * i, s = c >> 4, ch = c & 15;
        *reinterpret_cast<uint4*>(sQ + s * QP + ch * 16) = qv[i];
      }
    }
    // K rows (row-major copy) and K^T scaled by the decay to the chunk end
#pragma unroll
    for (int i = 0; i < KI; ++i) {
      const int c = tid + NT * i, p = c >> 4, ch = c & 15, s0 = 2 * p, s1 = s0 + 1;
      const uint4 ka = kav[i], kb = kbv[i];
      *reinterpret_cast<uint4*>(sK + s0 * QP + ch * 16) = ka;
      *reinterpret_cast<uint4*>(sK + s1 * QP + ch * 16) = kb;
      if constexpr (MODE != MODE_OUTPUT && MODE != MODE_FOLD) {
        const float w0 = __shfl(wK, s0, 64), w1 = __shfl(wK, s1, 64);
        const uint32_t a[4] = {ka.x, ka.y, ka.z, ka.w}, b[4] = {kb.x, kb.y, kb.z, kb.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int d0 = ch * 8 + 2 * e;
          // element d0 of tokens s0, s1 and element d0 + 1 of both
          const float x00 = lo_half(a[e]) * w0, x01 = lo_half(b[e]) * w1;
          const float x10 = hi_half(a[e]) * w0, x11 = hi_half(b[e]) * w1;
          const uint32_t h0 = cvt2(x00, x01), h1 = cvt2(x10, x11);
          const int r0 = trow(d0) + 4 * p, r1 = trow(d0 + 1) + 4 * p;
          *reinterpret_cast<uint32_t*>(sKt + r0) = h0;
          *reinterpret_cast<uint32_t*>(sKt + r1) = h1;
          *reinterpret_cast<uint32_t*>(sKl + r0) = cvt2(x00 - lo_half(h0), x01 - hi_half(h0));
          *reinterpret_cast<uint32_t*>(sKl + r1) = cvt2(x10 - lo_half(h1), x11 - hi_half(h1));
        }
      }
    }
    // V^T for this workgroup's value columns
#pragma unroll
    for (int i = 0; i < VI; ++i) {
      const int c = tid + NT * i, p = c / (DVG / 8), ch = c % (DVG / 8), s0 = 2 * p, s1 = s0 + 1;
      const uint4 va = vav[i], vb = vbv[i];
      const uint32_t a[4] = {va.x, va.y, va.z, va.w}, b[4] = {vb.x, vb.y, vb.z, vb.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int d0 = ch * 8 + 2 * e;
        *reinterpret_cast<uint32_t*>(sVt + trow(d0) + 4 * p) = (a[e] & 0xFFFFu) | (b[e] << 16);
        *reinterpret_cast<uint32_t*>(sVt + trow(d0 + 1) + 4 * p) = (a[e] >> 16) | (b[e] & 0xFFFF0000u);
      }
    }
    if (PREFETCH && c0 + C < sq.len) load_chunk(c0 + C);
    __syncthreads();

    const char* vrow = sVt + trow(wave * 32 + cl);
    if constexpr (MODE != MODE_SUMMARY) {
    // (a) score tiles A^T[s][t] = k_s . q_t for s-tile st <= t-tile tt
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
    }
    // causal mask and decay exp(G_t - G_s), s <= t
    const float Gt0 = sG[cl], Gt1 = sG[32 + cl];
#pragma unroll
    for (int x = 0; x < 3; ++x) {
      const int st = x == 2 ? 1 : 0, tt = x == 0 ? 0 : 1;
      const int t = 32 * tt + cl;
      const float Gt = tt ? Gt1 : Gt0;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int s = 32 * st + acc_row(r, lane);
        At[x][r] = s <= t ? At[x][r] * __expf(Gt - sG[s]) : 0.f;
      }
    }

    // (b) O = (A . D) V + exp(G_t) Q S0 for both t-tiles
    floatx16 O1[2], O2[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        O1[tt][r] = 0.f;
        O2[tt][r] = 0.f;
      }
    // Q S0: the state accumulator layout is the B operand, with the
    // contraction index permuted as acc_row; Q is read with that permutation
#pragma unroll
    for (int a = 0; a < DK / 32; ++a)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        float sv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) sv[e] = S[a][8 * hf + e];
        bf16x8 shi, slo;
        split_frag(sv, shi, slo);
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          const char* qp = sQ + (32 * tt + cl) * QP + (32 * a + 16 * hf + 4 * hi) * 2;
          const bf16x8 qf = frag_from_halves(*reinterpret_cast<const uint2*>(qp),
                                             *reinterpret_cast<const uint2*>(qp + 16));
          mfma32(O2[tt], qf, shi);
          mfma32(O2[tt], qf, slo);
        }
      }
    // (A . D) V: the score accumulator layout is the A operand
#pragma unroll
    for (int x = 0; x < 3; ++x) {
      const int st = x == 2 ? 1 : 0, tt = x == 0 ? 0 : 1;
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        float av[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) av[e] = At[x][8 * hf + e];
        bf16x8 ahi, alo;
        split_frag(av, ahi, alo);
        const char* vp = vrow + (32 * st + 16 * hf + 4 * hi) * 2;
        const bf16x8 vf = frag_from_halves(*reinterpret_cast<const uint2*>(vp),
                                           *reinterpret_cast<const uint2*>(vp + 16));
        mfma32(O1[tt], ahi, vf);
        mfma32(O1[tt], alo, vf);
      }
    }
    {
      // rows at or past n are dropped by the buffer's range check
      const rsrc_t ro = make_rsrc(o + base * ldo, n * ldo * 2);
      const int olane = (4 * hi * ldo + h * DV + dv0 + cl) * 2;
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int t = 32 * tt + acc_row(r, lane);
          const float val = O1[tt][r] + sEG[t] * O2[tt][r];
          __builtin_amdgcn_raw_buffer_store_b16(f2bf(val), ro, olane + (32 * tt + 8 * (r >> 2) + (r & 3)) * ldo * 2,
                                                0, 0);
        }
    }

    }  // MODE != MODE_SUMMARY
    if constexpr (MODE != MODE_OUTPUT && MODE != MODE_FOLD) {
    // (c) S = exp(G_last) S + (K . w)^T V
    const float dec = __expf(Glast);
#pragma unroll
    for (int a = 0; a < DK / 32; ++a) {
#pragma unroll
      for (int r = 0; r < 16; ++r) S[a][r] *= dec;
      const char* kt = sKt + trow(32 * a + cl) + 16 * hi;
      const char* kl = sKl + trow(32 * a + cl) + 16 * hi;
      const char* vt = vrow + 16 * hi;
#pragma unroll
      for (int ks = 0; ks < C / 16; ++ks) {
        const bf16x8 vf = as_frag(*reinterpret_cast<const uint4*>(vt + 32 * ks));
        mfma32(S[a], as_frag(*reinterpret_cast<const uint4*>(kt + 32 * ks)), vf);
        mfma32(S[a], as_frag(*reinterpret_cast<const uint4*>(kl + 32 * ks)), vf);
      }
    }
    }  // MODE != MODE_OUTPUT
  }

  if constexpr (MODE == MODE_FOLD) {
    if (seq == cs.c0 + cs.nc - 1 && cs.s_out >= 0) {   // the sequence's final state
      const float g = __expf(gamma[(long long)seq * H + h]);
      floatx16 dS[DK / 32];
      ld_frag(slab(states, seq), dS);
      const rsrc_t rs = slab(seq_states, cs.s_out);
#pragma unroll
      for (int a = 0; a < DK / 32; ++a)
#pragma unroll
        for (int r = 0; r < 16; ++r) stf(fmaf(g, S[a][r], dS[a][r]), rs, st_lane, st_soff(a, r));
    }
  } else if (MODE == MODE_SUMMARY) {   // the chunk's contribution, in accumulator order
    const rsrc_t rs = slab(states, sq.s_out);
#pragma unroll
    for (int a = 0; a < DK / 32; ++a)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const uint4 u = make_uint4(__float_as_uint(S[a][4 * rq]), __float_as_uint(S[a][4 * rq + 1]),
                                   __float_as_uint(S[a][4 * rq + 2]), __float_as_uint(S[a][4 * rq + 3]));
        __builtin_amdgcn_raw_buffer_store_b128(
            __builtin_bit_cast(decltype(__builtin_amdgcn_raw_buffer_load_b128(rs, 0, 0, 0)), u), rs, fr_lane,
            fr_soff(a, rq), 0);
      }
  } else if (MODE == MODE_FULL && sq.s_out >= 0) {
    const rsrc_t rs = slab(states, sq.s_out);
#pragma unroll
    for (int a = 0; a < DK / 32; ++a)
#pragma unroll
      for (int r = 0; r < 16; ++r) stf(S[a][r], rs, st_lane, st_soff(a, r));
  }
}

// fp32 path (small models): the chunked form of the recurrence.  One
// workgroup per (sequence, head) walks the sequence in chunks of 32 tokens;
// thread t owns value column t % DV and state rows t / DV + IST u of the
// fp32 state.  Per chunk, with G_t the chunk-local cumulative log gate:
//   A[t][s] = (q_t . k_s) exp(G_t - G_s) for s <= t      (LDS)
//   O[t] = A V + exp(G_t) q_t S0                           (q_t S0 summed over the IST threads of a column)
//   S0 <- exp(G_last) S0 + sum_s exp(G_last - G_s) k_s v_s^T
// Every decay is the exponential of a difference, at most 1.
template <int DK, int DV>
__global__ void __launch_bounds__(256)
scan_f32_kernel(const float* __restrict__ q, const float* __restrict__ k,
                const float* __restrict__ v, int ldqkv, const float* __restrict__ lg, int ldg,
                float* __restrict__ o, int ldo, const ScanSeq* __restrict__ seqs,
                float* __restrict__ states, int H) {
  constexpr int CC = 32;
  constexpr int IST = 256 / DV, NI = DK / IST;
  constexpr int QF = CC * DK / 4 / 256, VF = CC * DV / 4 / 256;   // float4 loads per thread
  static_assert(QF >= 1 && VF >= 1 && QF * 1024 == CC * DK && VF * 1024 == CC * DV, "chunk / thread mismatch");
  __shared__ __attribute__((aligned(16))) float sQ[CC][DK + 4];
  __shared__ __attribute__((aligned(16))) float sK[CC][DK + 4];
  __shared__ __attribute__((aligned(16))) float sV[CC][DV + 4];
  __shared__ float sA[CC][CC + 1];
  __shared__ float sQS[IST][CC][DV + 1];
  __shared__ float sG[CC], sEG[CC], sW[CC];
  const int tid = threadIdx.x, seq = blockIdx.x, h = blockIdx.y;
  const ScanSeq sq = seqs[seq];
  const int col = tid % DV, i0 = tid / DV;
  float S[NI];
#pragma unroll
  for (int u = 0; u < NI; ++u)
    S[u] = sq.s_in >= 0 ? states[(((long long)sq.s_in * H + h) * DK + i0 + u * IST) * DV + col] : 0.f;
  // the chunk's q, k, v and log gates are loaded into registers one chunk
  // ahead (rows past the sequence read its last row and are zeroed at the
  // LDS stores)
  float4 qv[QF], kv[QF], vv[VF];
  float lgv = 0.f;
  auto load_chunk = [&](int c0) {
    const int n = min(CC, sq.len - c0);
    const long long base = (long long)sq.row0 + c0;
#pragma unroll
    for (int x = 0; x < QF; ++x) {
      const int e = tid + 256 * x, t = e / (DK / 4), d4 = (e % (DK / 4)) * 4;
      const long long row = base + min(t, n - 1);
      qv[x] = *reinterpret_cast<const float4*>(q + row * ldqkv + h * DK + d4);
      kv[x] = *reinterpret_cast<const float4*>(k + row * ldqkv + h * DK + d4);
    }
#pragma unroll
    for (int x = 0; x < VF; ++x) {
      const int e = tid + 256 * x, t = e / (DV / 4), d4 = (e % (DV / 4)) * 4;
      vv[x] = *reinterpret_cast<const float4*>(v + (base + min(t, n - 1)) * ldqkv + h * DV + d4);
    }
    lgv = tid < n ? lg[(base + tid) * ldg + h] : 0.f;
  };
  if (sq.len > 0) load_chunk(0);
  for (int c0 = 0; c0 < sq.len; c0 += CC) {
    const int n = min(CC, sq.len - c0);
    const long long base = (long long)sq.row0 + c0;
    __syncthreads();   // the previous chunk's reads of LDS are done
    const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int x = 0; x < QF; ++x) {
      const int e = tid + 256 * x, t = e / (DK / 4), d4 = (e % (DK / 4)) * 4;
      *reinterpret_cast<float4*>(&sQ[t][d4]) = t < n ? qv[x] : z;
      *reinterpret_cast<float4*>(&sK[t][d4]) = t < n ? kv[x] : z;
    }
#pragma unroll
    for (int x = 0; x < VF; ++x) {
      const int e = tid + 256 * x, t = e / (DV / 4), d4 = (e % (DV / 4)) * 4;
      *reinterpret_cast<float4*>(&sV[t][d4]) = t < n ? vv[x] : z;
    }
    if (tid < 64) {   // wave 0: cumulative log gate, its exponential, the decay to the chunk end
      float g = lgv;
#pragma unroll
      for (int off = 1; off < CC; off <<= 1) {
        const float t = __shfl_up(g, off, 64);
        if (tid >= off) g += t;
      }
      const float gl = __shfl(g, n - 1, 64);
      if (tid < CC) {
        sG[tid] = g;
        sEG[tid] = __expf(g);
        sW[tid] = tid < n ? __expf(gl - g) : 0.f;
      }
    }
    if (c0 + CC < sq.len) load_chunk(c0 + CC);
    __syncthreads();
    // decayed scores of the chunk, s <= t
    for (int e = tid; e < CC * CC; e += 256) {
      const int t = e / CC, s2 = e % CC;
      float a = 0.f;
      if (s2 <= t && t < n) {
#pragma unroll
        for (int d = 0; d < DK; d += 4) {
          const float4 x = *reinterpret_cast<const float4*>(&sQ[t][d]);
          const float4 y = *reinterpret_cast<const float4*>(&sK[s2][d]);
          a = fmaf(x.x, y.x, fmaf(x.y, y.y, fmaf(x.z, y.z, fmaf(x.w, y.w, a))));
        }
        a *= __expf(sG[t] - sG[s2]);
      }
      sA[t][s2] = a;
    }
    // q_t S0 over this thread's state rows
    for (int t = 0; t < n; ++t) {
      float part = 0.f;
#pragma unroll
      for (int u = 0; u < NI; ++u) part = fmaf(sQ[t][i0 + u * IST], S[u], part);
      sQS[i0][t][col] = part;
    }
    __syncthreads();
    for (int t = i0; t < n; t += IST) {
      float inter = 0.f;
#pragma unroll
      for (int x = 0; x < IST; ++x) inter += sQS[x][t][col];
      float intra = 0.f;
      for (int s2 = 0; s2 <= t; ++s2) intra = fmaf(sA[t][s2], sV[s2][col], intra);
      o[(base + t) * ldo + h * DV + col] = intra + sEG[t] * inter;
    }
    // the state leaving the chunk
    const float dec = __expf(sG[n - 1]);
#pragma unroll
    for (int u = 0; u < NI; ++u) S[u] *= dec;
    for (int s2 = 0; s2 < n; ++s2) {
      const float wv = sW[s2] * sV[s2][col];
#pragma unroll
      for (int u = 0; u < NI; ++u) S[u] = fmaf(sK[s2][i0 + u * IST], wv, S[u]);
    }
  }
  if (sq.s_out >= 0) {
#pragma unroll
    for (int u = 0; u < NI; ++u)
      states[(((long long)sq.s_out * H + h) * DK + i0 + u * IST) * DV + col] = S[u];
  }
}

// fp32 path for short sequences (at most QMAX tokens): the chunked form with
// the whole sequence as one chunk, so that no workgroup waits for another.
// A workgroup owns 32 query rows [b, b + n) of one (sequence, head):
//   o_t = sum_{s <= t} (q_t . k_s) exp(G_t - G_s) v_s + exp(G_t) q_t S0,
// over key blocks of 32 staged in LDS.  The log-gate sums are taken from b:
// R(x) = G_x - G_b, forward over the rows and backward over the earlier
// keys, so the exponent G_t - G_s = R(t) - R(s) is formed from short sums
// where the decay is not negligible.  One more workgroup per (sequence,
// head) writes the final state, S = exp(G_last) S0 + sum_s exp(G_last - G_s)
// k_s v_s^T, with the sums taken backward from the last token.  Initial and
// final states must be different slots.
constexpr int QMAX = 512;

// R(x) for x = -1 .. b + n - 1 into r[x + 1] (r holds lg_x at x + 1 on entry,
// anything at 0): backward sums from b, forward sums from b.  256 threads.
__device__ __forceinline__ void log_gate_sums(float* r, int b, int n, float* red) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // backward: u_i = lg_{b - i}, i = 0..b; R(b - 1 - i) = -(u_0 + .. + u_i)
  const int i0 = 2 * tid;
  const float u0 = i0 <= b ? r[b - i0 + 1] : 0.f, u1 = i0 + 1 <= b ? r[b - i0] : 0.f;
  // forward (wave 0): R(b + i) = lg_{b+1} + .. + lg_{b+i}
  float f = (wave == 0 && lane >= 1 && lane < n) ? r[b + lane + 1] : 0.f;
  float t = u0 + u1;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float x = __shfl_up(t, off, 64);
    if (lane >= off) t += x;
  }
  if (lane == 63) red[wave] = t;
  if (wave == 0) {
#pragma unroll
    for (int off = 1; off < 32; off <<= 1) {
      const float x = __shfl_up(f, off, 64);
      if (lane >= off) f += x;
    }
  }
  __syncthreads();   // every entry of r has been read
  float base = 0.f;
  for (int w = 0; w < wave; ++w) base += red[w];
  const float p1 = base + t, p0 = p1 - u1;   // inclusive sums through u_{i0 + 1}, u_{i0}
  if (i0 <= b) r[b - i0] = -p0;
  if (i0 + 1 <= b) r[b - i0 - 1] = -p1;
  if (wave == 0 && lane < n) r[b + lane + 1] = f;
  __syncthreads();
}

template <int DK, int DV>
__global__ void __launch_bounds__(256)
scan_f32_whole_kernel(const float* __restrict__ q, const float* __restrict__ k,
                      const float* __restrict__ v, int ldqkv, const float* __restrict__ lg, int ldg,
                      float* __restrict__ o, int ldo, const ScanSeq* __restrict__ seqs,
                      float* __restrict__ states, int H, int nqb) {
  constexpr int QB = 32, KB = 32, CPT = DV / 8;   // columns per thread (rows x column groups = 32 x 8)
  __shared__ __attribute__((aligned(16))) float sQ[QB][DK + 4];
  __shared__ __attribute__((aligned(16))) float sK[KB][DK + 4];
  __shared__ __attribute__((aligned(16))) float sV[KB][DV + 4];
  __shared__ float sA[QB][KB + 1];
  __shared__ float sR[QMAX + 1];
  __shared__ float red[4];
  const int tid = threadIdx.x, h = blockIdx.y;
  const int seq = blockIdx.x / (nqb + 1), j = blockIdx.x % (nqb + 1);
  const ScanSeq sq = seqs[seq];
  const int L = sq.len, nq = (L + QB - 1) / QB;
  const long long qoff = (long long)h * DK, voff = (long long)h * DV;
  const long long sbase = (long long)h * DK * DV;
  if (j < nq) {
    const int b = j * QB, n = min(QB, L - b), span = b + n;   // keys 0 .. span - 1
    for (int x = tid; x < span; x += 256) sR[x + 1] = lg[(long long)(sq.row0 + x) * ldg + h];
    for (int e = tid; e < QB * DK / 4; e += 256) {
      const int t = e / (DK / 4), d4 = (e % (DK / 4)) * 4;
      *reinterpret_cast<float4*>(&sQ[t][d4]) =
          t < n ? *reinterpret_cast<const float4*>(q + (long long)(sq.row0 + b + t) * ldqkv + qoff + d4)
                : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    __syncthreads();
    log_gate_sums(sR, b, n, red);
    const int t = tid >> 3, cg = tid & 7;   // query row t, columns 8 u + cg ... (scores), cg * CPT .. (outputs)
    const float Rt = sR[min(b + t, span - 1) + 1];
    float acc[CPT];
#pragma unroll
    for (int c = 0; c < CPT; ++c) acc[c] = 0.f;
    for (int s0 = 0; s0 < span; s0 += KB) {
      const int nk = min(KB, span - s0);
      __syncthreads();   // the previous key block's reads are done
      for (int e = tid; e < KB * DK / 4; e += 256) {
        const int r = e / (DK / 4), d4 = (e % (DK / 4)) * 4;
        *reinterpret_cast<float4*>(&sK[r][d4]) =
            r < nk ? *reinterpret_cast<const float4*>(k + (long long)(sq.row0 + s0 + r) * ldqkv + qoff + d4)
                   : make_float4(0.f, 0.f, 0.f, 0.f);
      }
      for (int e = tid; e < KB * DV / 4; e += 256) {
        const int r = e / (DV / 4), d4 = (e % (DV / 4)) * 4;
        *reinterpret_cast<float4*>(&sV[r][d4]) =
            r < nk ? *reinterpret_cast<const float4*>(v + (long long)(sq.row0 + s0 + r) * ldqkv + voff + d4)
                   : make_float4(0.f, 0.f, 0.f, 0.f);
      }
      __syncthreads();
      // decayed scores of row t against keys 8 u + cg
      float sc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
      for (int d = 0; d < DK; d += 4) {
        const float4 x = *reinterpret_cast<const float4*>(&sQ[t][d]);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float4 y = *reinterpret_cast<const float4*>(&sK[8 * u + cg][d]);
          sc[u] = fmaf(x.x, y.x, fmaf(x.y, y.y, fmaf(x.z, y.z, fmaf(x.w, y.w, sc[u]))));
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int sl = 8 * u + cg, sa = s0 + sl;
        sA[t][sl] = (sl < nk && sa <= b + t && t < n) ? sc[u] * __expf(Rt - sR[sa + 1]) : 0.f;
      }
      __syncthreads();
#pragma unroll 4
      for (int sl = 0; sl < KB; ++sl) {
        const float a = sA[t][sl];
#pragma unroll
        for (int c = 0; c < CPT; c += 4) {
          const float4 y = *reinterpret_cast<const float4*>(&sV[sl][cg * CPT + c]);
          acc[c] = fmaf(a, y.x, acc[c]);
          acc[c + 1] = fmaf(a, y.y, acc[c + 1]);
          acc[c + 2] = fmaf(a, y.z, acc[c + 2]);
          acc[c + 3] = fmaf(a, y.w, acc[c + 3]);
        }
      }
    }
    if (sq.s_in >= 0) {   // exp(G_t) q_t S0, S0 staged 32 rows at a time in sK's place
      float qs[CPT];
#pragma unroll
      for (int c = 0; c < CPT; ++c) qs[c] = 0.f;
      const float* S0 = states + (long long)sq.s_in * H * DK * DV + sbase;
      for (int k0 = 0; k0 < DK; k0 += KB) {
        __syncthreads();
        for (int e = tid; e < KB * DV / 4; e += 256) {
          const int r = e / (DV / 4), d4 = (e % (DV / 4)) * 4;
          *reinterpret_cast<float4*>(&sV[r][d4]) = *reinterpret_cast<const float4*>(S0 + (long long)(k0 + r) * DV + d4);
        }
        __syncthreads();
#pragma unroll 4
        for (int r = 0; r < KB; ++r) {
          const float a = sQ[t][k0 + r];
#pragma unroll
          for (int c = 0; c < CPT; c += 4) {
            const float4 y = *reinterpret_cast<const float4*>(&sV[r][cg * CPT + c]);
            qs[c] = fmaf(a, y.x, qs[c]);
            qs[c + 1] = fmaf(a, y.y, qs[c + 1]);
            qs[c + 2] = fmaf(a, y.z, qs[c + 2]);
            qs[c + 3] = fmaf(a, y.w, qs[c + 3]);
          }
        }
      }
      const float e0 = __expf(Rt - sR[0]);
#pragma unroll
      for (int c = 0; c < CPT; ++c) acc[c] = fmaf(e0, qs[c], acc[c]);
    }
    if (t < n) {
      float* orow = o + (long long)(sq.row0 + b + t) * ldo + voff + cg * CPT;
#pragma unroll
      for (int c = 0; c < CPT; ++c) orow[c] = acc[c];
    }
  } else if (j == nqb && sq.s_out >= 0) {
    // final state: thread (row group rg, column group cg) owns rows rg + RG m
    constexpr int NCG = DV / 8, RG = 256 / NCG, RPT = DK / RG;
    const int rg = tid / NCG, cg = tid % NCG;
    const int b = L - 1;   // sums backward from the last token (b = -1: no tokens)
    for (int x = tid; x < L; x += 256) sR[x + 1] = lg[(long long)(sq.row0 + x) * ldg + h];
    __syncthreads();
    if (L > 0) log_gate_sums(sR, b, 1, red);
    else if (tid == 0) sR[0] = 0.f;
    __syncthreads();
    float acc[RPT][8];
#pragma unroll
    for (int m = 0; m < RPT; ++m)
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[m][c] = 0.f;
    for (int s0 = 0; s0 < L; s0 += KB) {
      const int nk = min(KB, L - s0);
      __syncthreads();
      for (int e = tid; e < KB * DK / 4; e += 256) {
        const int r = e / (DK / 4), d4 = (e % (DK / 4)) * 4;
        float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
        if (r < nk) {
          // decay from token s0 + r to the end: exp(G_last - G_s) = exp(-R(s))
          const float w = __expf(-sR[s0 + r + 1]);
          x = *reinterpret_cast<const float4*>(k + (long long)(sq.row0 + s0 + r) * ldqkv + qoff + d4);
          x.x *= w; x.y *= w; x.z *= w; x.w *= w;
        }
        *reinterpret_cast<float4*>(&sK[r][d4]) = x;
      }
      for (int e = tid; e < KB * DV / 4; e += 256) {
        const int r = e / (DV / 4), d4 = (e % (DV / 4)) * 4;
        *reinterpret_cast<float4*>(&sV[r][d4]) =
            r < nk ? *reinterpret_cast<const float4*>(v + (long long)(sq.row0 + s0 + r) * ldqkv + voff + d4)
                   : make_float4(0.f, 0.f, 0.f, 0.f);
      }
      __syncthreads();
#pragma unroll 2
      for (int r = 0; r < KB; ++r) {
        const float4 y0 = *reinterpret_cast<const float4*>(&sV[r][cg * 8]);
        const float4 y1 = *reinterpret_cast<const float4*>(&sV[r][cg * 8 + 4]);
#pragma unroll
        for (int m = 0; m < RPT; ++m) {
          const float a = sK[r][rg + RG * m];
          acc[m][0] = fmaf(a, y0.x, acc[m][0]);
          acc[m][1] = fmaf(a, y0.y, acc[m][1]);
          acc[m][2] = fmaf(a, y0.z, acc[m][2]);
          acc[m][3] = fmaf(a, y0.w, acc[m][3]);
          acc[m][4] = fmaf(a, y1.x, acc[m][4]);
          acc[m][5] = fmaf(a, y1.y, acc[m][5]);
          acc[m][6] = fmaf(a, y1.z, acc[m][6]);
          acc[m][7] = fmaf(a, y1.w, acc[m][7]);
        }
      }
    }
    const float e0 = __expf(-sR[0]);   // exp(G_last): the decay of the initial state
    const float* S0 = sq.s_in >= 0 ? states + (long long)sq.s_in * H * DK * DV + sbase : nullptr;
    float* S1 = states + (long long)sq.s_out * H * DK * DV + sbase;
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
      const long long rowo = (long long)(rg + RG * m) * DV + cg * 8;
#pragma unroll
      for (int c = 0; c < 8; ++c) S1[rowo + c] = S0 ? fmaf(e0, S0[rowo + c], acc[m][c]) : acc[m][c];
    }
  }
}

// Scan of chunk states across the chunks of each sequence, elementwise over
// the [dk, dv] state: S_enter[c] = exp(gamma[c-1]) S_enter[c-1] + dS[c-1],
// starting from the sequence's initial state.  cstates holds dS[c] on entry
// and S_enter[c] on exit, in the accumulator order of the chunk kernels; the
// initial and final states are in the sequence slots' row-major order.
__global__ void __launch_bounds__(256)
chunk_state_scan_kernel(const ChunkSeq* __restrict__ cseqs, const float* __restrict__ gamma,
                        float* __restrict__ cstates, float* __restrict__ states, int H) {
  const int sidx = blockIdx.y / H, h = blockIdx.y % H;
  const ChunkSeq cs = cseqs[sidx];
  constexpr int E = DK * DV;
  const int e = blockIdx.x * 256 + threadIdx.x;   // index in the chunk slots' accumulator order
  // the same element in the sequence states' row-major order
  const int r3 = e & 3, lane = (e >> 2) & 63, rq = (e >> 8) & 3, a = (e >> 10) & 3, cb = e >> 12;
  const int rm = (32 * a + 8 * rq + 4 * (lane >> 5) + r3) * DV + 32 * cb + (lane & 31);
  float sv = cs.s_in >= 0 ? states[((long long)cs.s_in * H + h) * E + rm] : 0.f;
  // eight chunks at a time: their loads are issued together, then the
  // recurrence steps through them in order
  constexpr int G8 = 8;
  const int cend = cs.c0 + cs.nc;
  for (int c0 = cs.c0; c0 < cend; c0 += G8) {
    float d[G8], gm[G8];
#pragma unroll
    for (int i = 0; i < G8; ++i) {
      const int c = min(c0 + i, cend - 1);
      d[i] = cstates[((long long)c * H + h) * E + e];
      gm[i] = gamma[(long long)c * H + h];
    }
#pragma unroll
    for (int i = 0; i < G8; ++i) {
      if (c0 + i < cend) {
        cstates[((long long)(c0 + i) * H + h) * E + e] = sv;
        sv = fmaf(__expf(gm[i]), sv, d[i]);
      }
    }
  }
  if (cs.s_out >= 0) states[((long long)cs.s_out * H + h) * E + rm] = sv;
}

template <int MODE>
hipError_t launch_mode(const bf16_t* qq, const bf16_t* kk, const bf16_t* vv, int ld_qkv, const float* log_g,
                       int ld_g, bf16_t* oo, int ld_o, const ScanSeq* seqs, int n_seqs, float* states, int H,
                       float* gamma, int nw, hipStream_t s, const ChunkSeq* cseqs = nullptr, int n_cseqs = 0,
                       float* seq_states = nullptr) {
  if (nw == 4)
    hipLaunchKernelGGL((scan_bf16_kernel<4, MODE>), dim3(n_seqs * 1, H), dim3(256), 0, s, qq, kk, vv, ld_qkv,
                       log_g, ld_g, oo, ld_o, seqs, states, H, gamma, cseqs, n_cseqs, seq_states);
  else if (nw == 2)
    hipLaunchKernelGGL((scan_bf16_kernel<2, MODE>), dim3(n_seqs * 2, H), dim3(128), 0, s, qq, kk, vv, ld_qkv,
                       log_g, ld_g, oo, ld_o, seqs, states, H, gamma, cseqs, n_cseqs, seq_states);
  else
    hipLaunchKernelGGL((scan_bf16_kernel<1, MODE>), dim3(n_seqs * 4, H), dim3(64), 0, s, qq, kk, vv, ld_qkv,
                       log_g, ld_g, oo, ld_o, seqs, states, H, gamma, cseqs, n_cseqs, seq_states);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_scan_chunked(const void* q, const void* k, const void* v, int ld_qkv, const float* log_g,
                               int ld_g, void* o, int ld_o, const ScanSeq* chunks, int n_chunks,
                               const ChunkSeq* cseqs, int n_cseqs, float* cstates, float* gamma,
                               float* states, int H, hipStream_t s, int max_nc) {
  if (n_chunks <= 0 || H <= 0) return hipSuccess;
  const auto* qq = reinterpret_cast<const bf16_t*>(q);
  const auto* kk = reinterpret_cast<const bf16_t*>(k);
  const auto* vv = reinterpret_cast<const bf16_t*>(v);
  auto* oo = reinterpret_cast<bf16_t*>(o);
  // one wave per 32 value columns; the waves of a workgroup share the
  // chunk's Q / K / K^T tiles.  Four waves per (chunk, head) when there are
  // enough (chunk, head) pairs to fill the chip; below that two workgroups of
  // two waves each (8 chunks x 16 heads: 29.8 against 31.0 us per layer for
  // the three launches; one-wave workgroups, which each stage the tiles,
  // 35.1 us)
  const int nw = (long long)n_chunks * H >= 256 ? 4 : 2;
  hipError_t e = launch_mode<MODE_SUMMARY>(qq, kk, vv, ld_qkv, log_g, ld_g, oo, ld_o, chunks, n_chunks, cstates,
                                           H, gamma, nw, s);
  if (e != hipSuccess) return e;
  // sequences of up to FOLD_MAX chunks: each output workgroup folds its
  // predecessors' contributions itself (up to FOLD_MAX - 1 state slices read
  // per workgroup) in place of a separate scan over the chunk states
  constexpr int FOLD_MAX = 16;
  if (max_nc <= FOLD_MAX)
    return launch_mode<MODE_FOLD>(qq, kk, vv, ld_qkv, log_g, ld_g, oo, ld_o, chunks, n_chunks, cstates, H, gamma,
                                  nw, s, cseqs, n_cseqs, states);
  hipLaunchKernelGGL(chunk_state_scan_kernel, dim3(DK * DV / 256, n_cseqs * H), dim3(256), 0, s, cseqs, gamma,
                     cstates, states, H);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_mode<MODE_OUTPUT>(qq, kk, vv, ld_qkv, log_g, ld_g, oo, ld_o, chunks, n_chunks, cstates, H,
                                  gamma, nw, s);
}

hipError_t launch_scan(bool bf16, const void* q, const void* k, const void* v, int ld_qkv,
                       const float* log_g, int ld_g, void* o, int ld_o, const ScanSeq* seqs,
                       int n_seqs, float* states, int H, int dk, int dv, hipStream_t s, int max_len) {
  if (n_seqs <= 0 || H <= 0) return hipSuccess;
  if (bf16) {
    if (dk != DK || dv != DV) return hipErrorInvalidValue;
    const long long chains = (long long)n_seqs * H;
    const auto* qq = reinterpret_cast<const bf16_t*>(q);
    const auto* kk = reinterpret_cast<const bf16_t*>(k);
    const auto* vv = reinterpret_cast<const bf16_t*>(v);
    auto* oo = reinterpret_cast<bf16_t*>(o);
    return launch_mode<MODE_FULL>(qq, kk, vv, ld_qkv, log_g, ld_g, oo, ld_o, seqs, n_seqs, states, H, nullptr,
                                  chains >= 256 ? 4 : (chains >= 128 ? 2 : 1), s);
  } else {
    const auto* qq = reinterpret_cast<const float*>(q);
    const auto* kk = reinterpret_cast<const float*>(k);
    const auto* vv = reinterpret_cast<const float*>(v);
    auto* oo = reinterpret_cast<float*>(o);
    if (max_len <= QMAX && ld_qkv % 4 == 0) {
      const int nqb = (max_len + 31) / 32;
      const dim3 grid(n_seqs * (nqb + 1), H);
#define S1_WHOLE(DKV, DVV)                                                                                   \
  hipLaunchKernelGGL((scan_f32_whole_kernel<DKV, DVV>), grid, dim3(256), 0, s, qq, kk, vv, ld_qkv, log_g, ld_g, \
                     oo, ld_o, seqs, states, H, nqb)
      if (dk == 64 && dv == 64) S1_WHOLE(64, 64);
      else if (dk == 128 && dv == 128) S1_WHOLE(128, 128);
      else if (dk == 128 && dv == 64) S1_WHOLE(128, 64);
      else if (dk == 64 && dv == 128) S1_WHOLE(64, 128);
      else return hipErrorInvalidValue;
#undef S1_WHOLE
      return hipGetLastError();
    }
    if (dk == 64 && dv == 64)
      hipLaunchKernelGGL((scan_f32_kernel<64, 64>), dim3(n_seqs, H), dim3(256), 0, s, qq, kk, vv, ld_qkv, log_g,
                         ld_g, oo, ld_o, seqs, states, H);
    else if (dk == 128 && dv == 128)
      hipLaunchKernelGGL((scan_f32_kernel<128, 128>), dim3(n_seqs, H), dim3(256), 0, s, qq, kk, vv, ld_qkv, log_g,
                         ld_g, oo, ld_o, seqs, states, H);
    else if (dk == 128 && dv == 64)
      hipLaunchKernelGGL((scan_f32_kernel<128, 64>), dim3(n_seqs, H), dim3(256), 0, s, qq, kk, vv, ld_qkv, log_g,
                         ld_g, oo, ld_o, seqs, states, H);
    else if (dk == 64 && dv == 128)
      hipLaunchKernelGGL((scan_f32_kernel<64, 128>), dim3(n_seqs, H), dim3(256), 0, s, qq, kk, vv, ld_qkv, log_g,
                         ld_g, oo, ld_o, seqs, states, H);
    else
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace s1
