// Causal flash-attention prefill over packed sequences, grouped KV heads,
// optional prefix keys (branches continue from a prefix's key/value cache;
// RFC #114 section 5: every branch starts from the prefix snapshot).
//
// bf16, head dim 128.  A workgroup owns 32 NWQ queries of one sequence and
// one query head; each of its NWQ waves owns 32 queries (the decoder uses
// NWQ = 4).  Keys and values stream through LDS in blocks of 64 (K
// row-major, V transposed), shared by the waves; the next block's loads are
// in flight in registers while the current block is computed.  Per block each wave computes S^T = K Q^T on the matrix cores (keys
// on the M side, queries on the N side, so every lane owns one query and the
// online softmax is a per-lane scalar recurrence); the probabilities stay in
// registers and feed O^T += V^T P^T directly: the accumulator layout of S^T
// is a permutation of the key index that the B operand of the second product
// accepts as-is, provided V^T is read with the same key permutation.  Running
// max and sum are fp32; exp2 with log2(e) folded into the scale, applied in
// one multiply-add per score; the reference max moves only when a block
// raises it by more than 2^8 (no rescale of O in most blocks).
//
// Split keys: a workgroup may cover only a piece [k_lo, k_hi) of its
// queries' keys (pieces cut at fixed key positions, so a query's pieces do
// not depend on the other sequences) and then writes its running max, sum
// and unnormalised O; attn_combine_kernel merges a row's pieces in piece
// order.  This lets short requests fill the chip, and lets the branches of a
// prefix read the prefix keys once for all their queries (RFC #114 section 5:
// every branch attends to the same immutable prefix snapshot).
#include <algorithm>
#include <climits>

#include "common.h"
#include "kernels.h"

namespace s1 {

namespace {

constexpr int HD = 128, BKV = 64;
constexpr int KPITCH = HD * 2 + 16;   // bytes per K row in LDS
constexpr int VPITCH = BKV * 2 + 8;   // bytes per V^T row in LDS
constexpr int OPITCH = HD * 2 + 16;   // bytes per output row in LDS
// V^T row d sits at d * VPITCH plus 16 bytes per 32 rows before it: the
// transposing stores of one instruction hit rows 8 apart, which the padding
// spreads over the banks; a read takes 32 consecutive rows of one group.
constexpr int vt_row(int d) { return d * VPITCH + (d >> 5) * 16; }
constexpr int LDS_BYTES = BKV * KPITCH + HD * VPITCH + (HD / 32) * 16;
static_assert(4 * 32 * OPITCH <= LDS_BYTES, "output staging must fit");

// Four-wave workgroups are held to two waves per SIMD (all accumulators in
// VGPRs, no spills): two workgroups share a CU, so one's barriers and block
// staging overlap the other's products.
template <int NWQ>
__global__ void __launch_bounds__(NWQ * 64) __attribute__((amdgpu_waves_per_eu(NWQ == 4 ? 2 : 1, 2)))
attn_bf16_kernel(const bf16_t* __restrict__ q, int ldq, const bf16_t* __restrict__ k,
                 const bf16_t* __restrict__ v, int ldkv, bf16_t* __restrict__ o, int ldo,
                 const AttnSeq* __restrict__ seqs, const AttnBlock* __restrict__ blocks, int Hq,
                 int Hkv, float scale_log2, const int32_t* __restrict__ row_slot, int row_base,
                 float* __restrict__ pO, float2* __restrict__ pML) {
  constexpr int BQ = 32 * NWQ, NT = 64 * NWQ;
  __shared__ __attribute__((aligned(16))) char smem[LDS_BYTES];
  char* sK = smem;
  char* sVt = smem + BKV * KPITCH;
  // the heads of one block are adjacent in launch order (blocks come
  // heaviest first, so the whole launch runs longest work first)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = blockIdx.x % Hq;
  const int kvh = h / (Hq / Hkv);
  const AttnBlock blk = blocks[blockIdx.x / Hq];
  const AttnSeq sq = seqs[blk.seq];
  const int n_pre = sq.kv_pre_len, n_kv = n_pre + sq.len;
  const int k_lo = blk.k_lo, k_hi = min(blk.k_hi, n_kv);
  const int qw0 = blk.q0 + wave * 32;
  const bool wave_active = qw0 < sq.len;
  const int kv_end = min(k_hi, n_pre + min(blk.q0 + BQ, sq.len));   // keys any query of the WG sees
  const int wave_kv_end = min(k_hi, n_pre + min(qw0 + 32, sq.len));  // keys this wave sees
  const int qi = qw0 + (lane & 31);
  const int hi = lane >> 5;

  bf16x8 qf[HD / 16];
  {
    const int qr = sq.q_row0 + min(qi, sq.len - 1);
    const bf16_t* qp = q + (long long)qr * ldq + h * HD + 8 * hi;
#pragma unroll
    for (int ks = 0; ks < HD / 16; ++ks) qf[ks] = as_frag(*reinterpret_cast<const uint4*>(qp + 16 * ks));
  }
  floatx16 oacc[HD / 32];
#pragma unroll
  for (int dt = 0; dt < HD / 32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  // the K / V block of keys j0 .. j0 + 63 is loaded into registers one block
  // ahead and written to LDS (V transposed) after the previous block's reads
  constexpr int KIT = BKV * 16 / NT, VIT = BKV * 8 / NT;
  uint4 kreg[KIT], vreg[VIT][2];
  auto kv_row = [&](int j) {
    return j < n_pre ? (long long)sq.kv_pre_row0 + j : (long long)sq.kv_row0 + (j - n_pre);
  };
  auto load_block = [&](int j0) {
#pragma unroll
    for (int it = 0; it < KIT; ++it) {
      const int c = tid + it * NT, key = c >> 4, ch = c & 15;
      const int j = j0 + key;
      kreg[it] = j < n_kv ? *reinterpret_cast<const uint4*>(k + kv_row(j) * ldkv + kvh * HD + ch * 8)
                          : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int it = 0; it < VIT; ++it) {
      const int c = tid + it * NT, kp = c >> 4, ch = c & 15;
      const int ja = j0 + 2 * kp, jb = ja + 1;
      vreg[it][0] = ja < n_kv ? *reinterpret_cast<const uint4*>(v + kv_row(ja) * ldkv + kvh * HD + ch * 8)
                              : make_uint4(0, 0, 0, 0);
      vreg[it][1] = jb < n_kv ? *reinterpret_cast<const uint4*>(v + kv_row(jb) * ldkv + kvh * HD + ch * 8)
                              : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_block = [&]() {
#pragma unroll
    for (int it = 0; it < KIT; ++it) {
      const int c = tid + it * NT, key = c >> 4, ch = c & 15;
      *reinterpret_cast<uint4*>(sK + key * KPITCH + ch * 16) = kreg[it];
    }
#pragma unroll
    for (int it = 0; it < VIT; ++it) {
      const int c = tid + it * NT, kp = c >> 4, ch = c & 15;
      const uint4 va = vreg[it][0], vb = vreg[it][1];
      const uint32_t a[4] = {va.x, va.y, va.z, va.w}, b[4] = {vb.x, vb.y, vb.z, vb.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int d0 = ch * 8 + 2 * e;
        *reinterpret_cast<uint32_t*>(sVt + vt_row(d0) + 4 * kp) = (a[e] & 0xFFFFu) | (b[e] << 16);
        *reinterpret_cast<uint32_t*>(sVt + vt_row(d0 + 1) + 4 * kp) = (a[e] >> 16) | (b[e] & 0xFFFF0000u);
      }
    }
  };
  if (kv_end > k_lo) load_block(k_lo);
  for (int j0 = k_lo; j0 < kv_end; j0 += BKV) {
    __syncthreads();   // the previous block's LDS reads are done
    store_block();
    if (j0 + BKV < kv_end) load_block(j0 + BKV);
    __syncthreads();
    if (!wave_active || j0 >= wave_kv_end) continue;

    floatx16 s[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[t][r] = 0.f;
      const char* kr = sK + (32 * t + (lane & 31)) * KPITCH + 16 * hi;
#pragma unroll
      for (int ks = 0; ks < HD / 16; ++ks)
        mfma32(s[t], as_frag(*reinterpret_cast<const uint4*>(kr + 32 * ks)), qf[ks]);
    }
    // raw scores; keys a query must not see become -inf.  A block that every
    // query of the wave sees whole (the causal cut and the piece end both lie
    // past it) skips the mask: the values are the same either way.
    float mx = -INFINITY;
    if (j0 + BKV <= n_pre + qw0 + 1 && j0 + BKV <= k_hi) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[t][r]);
    } else {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = j0 + 32 * t + acc_row(r, lane);
          const bool vis = (j <= n_pre + qi) && (j < k_hi);
          s[t][r] = vis ? s[t][r] : -INFINITY;
          mx = fmaxf(mx, s[t][r]);
        }
    }
    // the block's largest scaled score (rounding is monotonic, so this is
    // the largest of the scaled scores); both halves of the wave hold the
    // same queries
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * scale_log2;
    // Lazy rescaling: the reference point m_run moves only when the block's
    // maximum exceeds it by more than 2^8, so p = 2^(s - m_run) <= 256 and
    // the running sums stay exact relative to their reference.  A query that
    // has seen no key of this piece yet keeps (m, l, O) = (-inf, 0, 0).  The
    // rescale runs for the whole wave when any of its queries needs it;
    // others multiply by exactly 1.
    const bool grow = mx > m_run + 8.f;
    if (__ballot(grow) != 0) {
      const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - mx) : 1.f;
      m_run = grow ? mx : m_run;
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < HD / 32; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
    }
    const float m_use = m_run == -INFINITY ? 0.f : m_run;
    float ps = 0.f;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[t][r], scale_log2, -m_use));
        s[t][r] = p;
        ps += p;
      }
    l_run += ps;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int e0 = 8 * hf;
        const bf16x8 pf = as_frag(make_uint4(cvt2(s[t][e0], s[t][e0 + 1]), cvt2(s[t][e0 + 2], s[t][e0 + 3]),
                                             cvt2(s[t][e0 + 4], s[t][e0 + 5]), cvt2(s[t][e0 + 6], s[t][e0 + 7])));
        const int kb = (32 * t + 16 * hf + 4 * hi) * 2;
#pragma unroll
        for (int dt = 0; dt < HD / 32; ++dt) {
          const char* vr = sVt + vt_row(32 * dt + (lane & 31)) + kb;
          const bf16x8 vf = frag_from_halves(*reinterpret_cast<const uint2*>(vr),
                                             *reinterpret_cast<const uint2*>(vr + 16));
          mfma32(oacc[dt], vf, pf);
        }
      }
    }
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  if (blk.part >= 0) {   // one piece of the keys: (max, sum, unnormalised O) to its slot
    const int qq = qw0 + (lane & 31);
    if (!wave_active || qq >= sq.len) return;
    const int row = sq.q_row0 + qq;
    const long long slot = (long long)(row_slot[row - row_base] + blk.part) * Hq + h;
    float* dst = pO + slot * HD;
#pragma unroll
    for (int dt = 0; dt < HD / 32; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<float4*>(dst + 32 * dt + 8 * g + 4 * hi) =
            make_float4(oacc[dt][4 * g], oacc[dt][4 * g + 1], oacc[dt][4 * g + 2], oacc[dt][4 * g + 3]);
    if (hi == 0) pML[slot] = make_float2(m_run, l_tot);
    return;
  }
  // normalise and stage O through LDS for coalesced row stores
  __syncthreads();
  const float inv = 1.f / l_tot;
  char* so = smem + wave * 32 * OPITCH;
#pragma unroll
  for (int dt = 0; dt < HD / 32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int d = 32 * dt + acc_row(r, lane);
      *reinterpret_cast<bf16_t*>(so + (lane & 31) * OPITCH + 2 * d) = f2bf(oacc[dt][r] * inv);
    }
  __syncthreads();
  if (!wave_active) return;
  // 32 rows x 16 chunks per wave
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    const int c = lane + it * 64, row = c >> 4, ch = c & 15;
    const int qq = qw0 + row;
    if (qq < sq.len)
      *reinterpret_cast<uint4*>(o + (long long)(sq.q_row0 + qq) * ldo + h * HD + ch * 8) =
          *reinterpret_cast<const uint4*>(so + row * OPITCH + ch * 16);
  }
}

// Merge a row's key pieces: with M the largest piece max, o = sum_p
// 2^(m_p - M) O_p / sum_p 2^(m_p - M) l_p, pieces in order (a piece that saw
// no key has m = -inf and weight 0).  One wave per (row, head), two output
// columns per lane.
__global__ void __launch_bounds__(256)
attn_combine_kernel(const int32_t* __restrict__ rows, int n_rows, const int32_t* __restrict__ row_slot,
                    const int32_t* __restrict__ row_np, int row_base, const float* __restrict__ pO,
                    const float2* __restrict__ pML, bf16_t* __restrict__ o, int ldo, int Hq) {
  const int lane = threadIdx.x & 63;
  const long long gw = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (gw >= (long long)n_rows * Hq) return;
  const int ri = (int)(gw / Hq), h = (int)(gw % Hq);
  const int row = rows[ri];
  const int base = row_slot[row - row_base], np = row_np[row - row_base];
  float M = -INFINITY;
  for (int pc = 0; pc < np; ++pc) M = fmaxf(M, pML[(long long)(base + pc) * Hq + h].x);
  float L = 0.f, a0 = 0.f, a1 = 0.f;
  for (int pc = 0; pc < np; ++pc) {
    const long long slot = (long long)(base + pc) * Hq + h;
    const float2 ml = pML[slot];
    const float w = ml.x == -INFINITY ? 0.f : exp2f(ml.x - M);
    const float2 val = *reinterpret_cast<const float2*>(pO + slot * HD + 2 * lane);
    L += w * ml.y;
    a0 += w * val.x;
    a1 += w * val.y;
  }
  const float inv = 1.f / L;
  *reinterpret_cast<uint32_t*>(o + (long long)row * ldo + h * HD + 2 * lane) = pack_bf2(a0 * inv, a1 * inv);
}

// fp32 path (small models).  A workgroup owns 16 queries of one head and
// 16 threads share a query: four quarters of its head dimensions times four
// key groups.  Keys and values stream through LDS in blocks of 64; key group
// g takes keys g, g + 4, ... of each block (so that the causal cut leaves
// the groups balanced) and keeps its own running maximum, sum and output
// quarter, with scores from partial dot products summed across the four
// dimension quarters.  The four groups are merged at the end with lane
// exchanges.  Sixteen threads per query (not four) give the few queries of
// a small request four times as many waves.
constexpr int BQ32 = 16, BK32 = 64;
template <int HD32>
__global__ void __launch_bounds__(256)
attn_f32_kernel(const float* __restrict__ q, int ldq, const float* __restrict__ k,
                const float* __restrict__ v, int ldkv, float* __restrict__ o, int ldo,
                const AttnSeq* __restrict__ seqs, const AttnBlock* __restrict__ blocks, int Hq,
                int Hkv, float scale_log2) {
  constexpr int QD = HD32 / 4;                  // dimensions per thread
  constexpr int KP = HD32 + 4;                  // LDS row pitch (floats)
  constexpr int KPG = BK32 / 4;                 // keys per group and block
  __shared__ __attribute__((aligned(16))) float sK[BK32 * KP];
  __shared__ __attribute__((aligned(16))) float sV[BK32 * KP];
  const int tid = threadIdx.x, h = blockIdx.y, kvh = h / (Hq / Hkv);
  const int qloc = tid >> 4, kg = (tid >> 2) & 3, sub = tid & 3;
  const AttnBlock blk = blocks[blockIdx.x];
  const AttnSeq sq = seqs[blk.seq];
  const int n_pre = sq.kv_pre_len, n_kv = n_pre + sq.len;
  const int qi = blk.q0 + qloc;
  const bool active = qi < sq.len;
  const int kv_end = n_pre + min(blk.q0 + BQ32, sq.len);
  float qr[QD], acc[QD];
  {
    const float* qp = q + (long long)(sq.q_row0 + min(qi, sq.len - 1)) * ldq + h * HD32 + sub * QD;
#pragma unroll
    for (int d = 0; d < QD; d += 4) {
      const float4 t = *reinterpret_cast<const float4*>(qp + d);
      qr[d] = t.x; qr[d + 1] = t.y; qr[d + 2] = t.z; qr[d + 3] = t.w;
    }
  }
#pragma unroll
  for (int d = 0; d < QD; ++d) acc[d] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  for (int j0 = 0; j0 < kv_end; j0 += BK32) {
    __syncthreads();   // the previous block's reads are done
    constexpr int F4 = BK32 * HD32 / 4;
    for (int c = tid; c < F4; c += 256) {
      const int key = c / (HD32 / 4), d4 = (c % (HD32 / 4)) * 4;
      const int j = j0 + key;
      float4 kv4 = make_float4(0.f, 0.f, 0.f, 0.f), vv4 = kv4;
      if (j < n_kv) {
        const long long row = j < n_pre ? (long long)sq.kv_pre_row0 + j : (long long)sq.kv_row0 + (j - n_pre);
        kv4 = *reinterpret_cast<const float4*>(k + row * ldkv + kvh * HD32 + d4);
        vv4 = *reinterpret_cast<const float4*>(v + row * ldkv + kvh * HD32 + d4);
      }
      *reinterpret_cast<float4*>(sK + key * KP + d4) = kv4;
      *reinterpret_cast<float4*>(sV + key * KP + d4) = vv4;
    }
    __syncthreads();
    float sc[KPG];
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < KPG; ++i) {
      const int kk = kg + 4 * i;
      const float* kr = sK + kk * KP + sub * QD;
      float part = 0.f;
#pragma unroll
      for (int d = 0; d < QD; ++d) part = fmaf(qr[d], kr[d], part);
      part += __shfl_xor(part, 1, 64);
      part += __shfl_xor(part, 2, 64);
      const int j = j0 + kk;
      const float val = (j <= n_pre + qi && j < n_kv) ? part * scale_log2 : -INFINITY;
      sc[i] = val;
      mx = fmaxf(mx, val);
    }
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);
    l_run *= alpha;
#pragma unroll
    for (int d = 0; d < QD; ++d) acc[d] *= alpha;
#pragma unroll
    for (int i = 0; i < KPG; ++i) {
      const float p = exp2f(sc[i] - m_use);
      l_run += p;
      const float* vr = sV + (kg + 4 * i) * KP + sub * QD;
#pragma unroll
      for (int d = 0; d < QD; ++d) acc[d] = fmaf(p, vr[d], acc[d]);
    }
    m_run = m_new;
  }
  // merge the four key groups (lanes 4 and 8 apart)
  float m_all = fmaxf(m_run, __shfl_xor(m_run, 4, 64));
  m_all = fmaxf(m_all, __shfl_xor(m_all, 8, 64));
  const float f = m_run == -INFINITY ? 0.f : exp2f(m_run - m_all);
  float l = l_run * f;
  l += __shfl_xor(l, 4, 64);
  l += __shfl_xor(l, 8, 64);
#pragma unroll
  for (int d = 0; d < QD; ++d) {
    float a = acc[d] * f;
    a += __shfl_xor(a, 4, 64);
    a += __shfl_xor(a, 8, 64);
    acc[d] = a;
  }
  if (!active || kg != 0) return;
  const float inv = 1.f / l;
  float* op = o + (long long)(sq.q_row0 + qi) * ldo + h * HD32 + sub * QD;
#pragma unroll
  for (int d = 0; d < QD; d += 4)
    *reinterpret_cast<float4*>(op + d) = make_float4(acc[d] * inv, acc[d + 1] * inv, acc[d + 2] * inv, acc[d + 3] * inv);
}

}  // namespace

bool attn_block_rows_valid(bool bf16, int rows) {
  return bf16 ? (rows == 32 || rows == 64 || rows == 128) : rows == BQ32;
}

int attn_block_rows(bool bf16, const int* lens, int n, int Hq) {
  (void)lens;
  (void)n;
  (void)Hq;
  // 128 queries per workgroup: measured faster than 32 at 512 tokens and 16
  // heads (64 vs 256 workgroups), where staging, not parallelism, bounds
  return bf16 ? 128 : BQ32;
}

namespace {

int cdiv(int a, int b) { return (a + b - 1) / b; }

// The pieces [lo, hi) of the keys [k0, k_end), cut at multiples of piece.
template <typename F>
int for_pieces(int k0, int k_end, int piece, F f) {
  int n = 0;
  for (int lo = k0; lo < k_end;) {
    const int hi = std::min(k_end, (lo / piece + 1) * piece);
    f(lo, hi, n++);
    lo = hi;
  }
  return n;
}

}  // namespace

void plan_attention(const AttnSeq* in, int n, int row_base, int n_rows, int Hq, int bq, int piece, int n_cu,
                    AttnPlanHost* out) {
  AttnPlanHost& P = *out;
  P = AttnPlanHost();
  P.seqs.assign(in, in + n);
  P.row_slot.assign(std::max(n_rows, 0), -1);
  P.row_np.assign(std::max(n_rows, 0), 1);
  if (piece < 0) {
    // key blocks (64 keys) per workgroup chain without a split, and their sum
    long long total = 0;
    int longest = 0;
    bool prefix = false;
    for (int i = 0; i < n; ++i) {
      prefix |= in[i].kv_pre_len > 0 && in[i].len > 0;
      for (int q0 = 0; q0 < in[i].len; q0 += bq) {
        const int kb = cdiv(in[i].kv_pre_len + std::min(q0 + bq, in[i].len), 64);
        total += kb;
        longest = std::max(longest, kb);
      }
    }
    total *= Hq;
    const long long target = std::max<long long>(2, (total + 2LL * n_cu - 1) / (2LL * n_cu));
    if (longest <= target && !prefix) {
      piece = 0;
    } else {
      long long pb = 2;
      while (pb * 2 <= target) pb *= 2;
      piece = (int)(64 * pb);
    }
  }
  P.piece = piece;
  auto assign_rows = [&](int row0, int nq, int np) {
    for (int r = row0; r < row0 + nq; ++r) {
      P.row_slot[r - row_base] = P.slots;
      P.row_np[r - row_base] = np;
      P.slots += np;
      P.comb_rows.push_back(r);
    }
  };
  for (int i = 0; i < n;) {
    const AttnSeq& a = in[i];
    if (piece > 0 && a.kv_pre_len > 0 && a.len > 0) {
      // the run of sequences continuing this prefix with contiguous query rows
      int j = i, rows = a.len;
      while (j + 1 < n && in[j + 1].kv_pre_len == a.kv_pre_len && in[j + 1].kv_pre_row0 == a.kv_pre_row0 &&
             in[j + 1].q_row0 == in[j].q_row0 + in[j].len && in[j + 1].len > 0) {
        ++j;
        rows += in[j].len;
      }
      const int Pn = a.kv_pre_len;
      const int npre = cdiv(Pn, piece);
      const int g = (int)P.seqs.size();
      P.seqs.push_back({a.q_row0, rows, a.q_row0, a.kv_pre_row0, Pn});
      for (int q0 = 0; q0 < rows; q0 += bq)
        for_pieces(0, Pn, piece, [&](int lo, int hi, int ord) { P.blocks.push_back({g, q0, lo, hi, ord}); });
      for (int k = i; k <= j; ++k)
        for (int q0 = 0; q0 < in[k].len; q0 += bq) {
          const int nq = std::min(bq, in[k].len - q0);
          const int nown = for_pieces(Pn, Pn + q0 + nq, piece, [&](int lo, int hi, int ord) {
            P.blocks.push_back({k, q0, lo, hi, npre + ord});
          });
          assign_rows(in[k].q_row0 + q0, nq, npre + nown);
        }
      i = j + 1;
      continue;
    }
    for (int q0 = 0; q0 < a.len; q0 += bq) {
      const int nq = std::min(bq, a.len - q0);
      const int k_end = a.kv_pre_len + q0 + nq;
      if (piece <= 0 || k_end <= piece) {
        P.blocks.push_back({i, q0, 0, a.kv_pre_len + a.len, -1});
        continue;
      }
      const int np = for_pieces(0, k_end, piece, [&](int lo, int hi, int ord) {
        P.blocks.push_back({i, q0, lo, hi, ord});
      });
      assign_rows(a.q_row0 + q0, nq, np);
    }
    ++i;
  }
  // heaviest workgroups first (the 64-key blocks each sweeps), so that the
  // long causal blocks do not start last and leave CUs idle at the end
  auto cost = [&](const AttnBlock& b) {
    const AttnSeq& q = P.seqs[b.seq];
    const int end = std::min(b.k_hi, q.kv_pre_len + std::min(b.q0 + bq, q.len));
    return end > b.k_lo ? cdiv(end - b.k_lo, 64) : 0;
  };
  std::stable_sort(P.blocks.begin(), P.blocks.end(),
                   [&](const AttnBlock& x, const AttnBlock& y) { return cost(x) > cost(y); });
}

hipError_t launch_attention(bool bf16, const void* q, int ld_q, const void* k, const void* v,
                            int ld_kv, void* o, int ld_o, const AttnSeq* seqs,
                            const AttnBlock* blocks, int n_blocks, int Hq, int Hkv, int hd, int block_rows,
                            const AttnPartials& part, hipStream_t s) {
  if (n_blocks <= 0) return hipSuccess;
  if (Hkv <= 0 || Hq % Hkv != 0 || !attn_block_rows_valid(bf16, block_rows)) return hipErrorInvalidValue;
  if ((long long)n_blocks * Hq > INT_MAX) return hipErrorInvalidValue;
  if (bf16) {
    const dim3 grid(n_blocks * Hq);   // block-major, heads adjacent
    if (hd != HD) return hipErrorInvalidValue;
    const float sl2 = 1.4426950408889634f / sqrtf((float)hd);
    const auto* qq = reinterpret_cast<const bf16_t*>(q);
    const auto* kk = reinterpret_cast<const bf16_t*>(k);
    const auto* vv = reinterpret_cast<const bf16_t*>(v);
    auto* oo = reinterpret_cast<bf16_t*>(o);
    if (block_rows == 128)
      hipLaunchKernelGGL(attn_bf16_kernel<4>, grid, dim3(256), 0, s, qq, ld_q, kk, vv, ld_kv, oo, ld_o, seqs,
                         blocks, Hq, Hkv, sl2, part.row_slot, part.row_base, part.pO, part.pML);
    else if (block_rows == 64)
      hipLaunchKernelGGL(attn_bf16_kernel<2>, grid, dim3(128), 0, s, qq, ld_q, kk, vv, ld_kv, oo, ld_o, seqs,
                         blocks, Hq, Hkv, sl2, part.row_slot, part.row_base, part.pO, part.pML);
    else
      hipLaunchKernelGGL(attn_bf16_kernel<1>, grid, dim3(64), 0, s, qq, ld_q, kk, vv, ld_kv, oo, ld_o, seqs,
                         blocks, Hq, Hkv, sl2, part.row_slot, part.row_base, part.pO, part.pML);
  } else {
    const dim3 grid(n_blocks, Hq);
    const float sl2 = 1.4426950408889634f / sqrtf((float)hd);
    const auto* qq = reinterpret_cast<const float*>(q);
    const auto* kk = reinterpret_cast<const float*>(k);
    const auto* vv = reinterpret_cast<const float*>(v);
    auto* oo = reinterpret_cast<float*>(o);
    if (hd == 64)
      hipLaunchKernelGGL(attn_f32_kernel<64>, grid, dim3(256), 0, s, qq, ld_q, kk, vv, ld_kv, oo, ld_o, seqs, blocks,
                         Hq, Hkv, sl2);
    else if (hd == 128)
      hipLaunchKernelGGL(attn_f32_kernel<128>, grid, dim3(256), 0, s, qq, ld_q, kk, vv, ld_kv, oo, ld_o, seqs,
                         blocks, Hq, Hkv, sl2);
    else
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_attn_combine(const int32_t* rows, int n_rows, const AttnPartials& part, void* o, int ld_o,
                               int Hq, hipStream_t s) {
  if (n_rows <= 0) return hipSuccess;
  const long long waves = (long long)n_rows * Hq;
  hipLaunchKernelGGL(attn_combine_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, s, rows, n_rows,
                     part.row_slot, part.row_np, part.row_base, part.pO, part.pML, reinterpret_cast<bf16_t*>(o),
                     ld_o, Hq);
  return hipGetLastError();
}

}  // namespace s1
