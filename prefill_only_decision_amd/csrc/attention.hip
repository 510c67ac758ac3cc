// Causal flash-attention prefill over packed sequences, grouped KV heads,
// optional prefix keys (branches continue from a prefix's key/value cache;
// RFC #114 section 5: every branch starts from the prefix snapshot).
//
// bf16, head dim 128.  A workgroup owns 128 queries of one sequence and one
// query head; each of its 4 waves owns 32 queries.  Keys and values stream
// through LDS in blocks of 64 (K row-major, V transposed), shared by the 4
// waves.  Per block each wave computes S^T = K Q^T on the matrix cores (keys
// on the M side, queries on the N side, so every lane owns one query and the
// online softmax is a per-lane scalar recurrence); the probabilities stay in
// registers and feed O^T += V^T P^T directly: the accumulator layout of S^T
// is a permutation of the key index that the B operand of the second product
// accepts as-is, provided V^T is read with the same key permutation.  Running
// max and sum are fp32; exp2 with log2(e) folded into the scale.
#include "common.h"
#include "kernels.h"

namespace s1 {

namespace {

constexpr int HD = 128, BQ = 128, BKV = 64;
constexpr int KPITCH = HD * 2 + 16;   // bytes per K row in LDS
constexpr int VPITCH = BKV * 2 + 8;   // bytes per V^T row in LDS
constexpr int OPITCH = HD * 2 + 16;   // bytes per output row in LDS
constexpr int LDS_BYTES = BKV * KPITCH + HD * VPITCH;
static_assert(4 * 32 * OPITCH <= LDS_BYTES, "output staging must fit");

__global__ void __launch_bounds__(256)
attn_bf16_kernel(const bf16_t* __restrict__ q, int ldq, const bf16_t* __restrict__ k,
                 const bf16_t* __restrict__ v, int ldkv, bf16_t* __restrict__ o, int ldo,
                 const AttnSeq* __restrict__ seqs, const AttnBlock* __restrict__ blocks, int Hq,
                 int Hkv, float scale_log2) {
  __shared__ __attribute__((aligned(16))) char smem[LDS_BYTES];
  char* sK = smem;
  char* sVt = smem + BKV * KPITCH;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = blockIdx.y;
  const int kvh = h / (Hq / Hkv);
  const AttnBlock blk = blocks[blockIdx.x];
  const AttnSeq sq = seqs[blk.seq];
  const int n_pre = sq.kv_pre_len, n_kv = n_pre + sq.len;
  const int qw0 = blk.q0 + wave * 32;
  const bool wave_active = qw0 < sq.len;
  const int kv_end = n_pre + min(blk.q0 + BQ, sq.len);          // keys any query of the WG sees
  const int wave_kv_end = n_pre + min(qw0 + 32, sq.len);         // keys this wave sees
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

  for (int j0 = 0; j0 < kv_end; j0 += BKV) {
    __syncthreads();
    // K block: 64 keys x 16 chunks of 16 bytes
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int c = tid + it * 256, key = c >> 4, ch = c & 15;
      const int j = j0 + key;
      uint4 val = make_uint4(0, 0, 0, 0);
      if (j < n_kv) {
        const long long row = j < n_pre ? (long long)sq.kv_pre_row0 + j : (long long)sq.kv_row0 + (j - n_pre);
        val = *reinterpret_cast<const uint4*>(k + row * ldkv + kvh * HD + ch * 8);
      }
      *reinterpret_cast<uint4*>(sK + key * KPITCH + ch * 16) = val;
    }
    // V block, transposed: pairs of keys x 16 chunks
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int c = tid + it * 256, kp = c >> 4, ch = c & 15;
      const int ja = j0 + 2 * kp, jb = ja + 1;
      uint4 va = make_uint4(0, 0, 0, 0), vb = make_uint4(0, 0, 0, 0);
      if (ja < n_kv) {
        const long long row = ja < n_pre ? (long long)sq.kv_pre_row0 + ja : (long long)sq.kv_row0 + (ja - n_pre);
        va = *reinterpret_cast<const uint4*>(v + row * ldkv + kvh * HD + ch * 8);
      }
      if (jb < n_kv) {
        const long long row = jb < n_pre ? (long long)sq.kv_pre_row0 + jb : (long long)sq.kv_row0 + (jb - n_pre);
        vb = *reinterpret_cast<const uint4*>(v + row * ldkv + kvh * HD + ch * 8);
      }
      const uint32_t a[4] = {va.x, va.y, va.z, va.w}, b[4] = {vb.x, vb.y, vb.z, vb.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int d0 = ch * 8 + 2 * e;
        *reinterpret_cast<uint32_t*>(sVt + d0 * VPITCH + 4 * kp) = (a[e] & 0xFFFFu) | (b[e] << 16);
        *reinterpret_cast<uint32_t*>(sVt + (d0 + 1) * VPITCH + 4 * kp) = (a[e] >> 16) | (b[e] & 0xFFFF0000u);
      }
    }
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
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = j0 + 32 * t + acc_row(r, lane);
        const bool vis = (j <= n_pre + qi) && (j < n_kv);
        const float val = vis ? s[t][r] * scale_log2 : -INFINITY;
        s[t][r] = val;
        mx = fmaxf(mx, val);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = exp2f(m_run - m_new);
    float ps = 0.f;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = exp2f(s[t][r] - m_new);
        s[t][r] = p;
        ps += p;
      }
    l_run = l_run * alpha + ps;
    m_run = m_new;
#pragma unroll
    for (int dt = 0; dt < HD / 32; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        float pv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) pv[e] = s[t][8 * hf + e];
        const bf16x8 pf = frag_from_f(pv);
        const int kb = (32 * t + 16 * hf + 4 * hi) * 2;
#pragma unroll
        for (int dt = 0; dt < HD / 32; ++dt) {
          const char* vr = sVt + (32 * dt + (lane & 31)) * VPITCH + kb;
          const bf16x8 vf = frag_from_halves(*reinterpret_cast<const uint2*>(vr),
                                             *reinterpret_cast<const uint2*>(vr + 16));
          mfma32(oacc[dt], vf, pf);
        }
      }
    }
  }

  // normalise and stage O through LDS for coalesced row stores
  __syncthreads();
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
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

// fp32 path (small models): one wave per query, online softmax over keys,
// lanes over the head dimension (hd <= 128).
constexpr int BQ32 = 64;
__global__ void __launch_bounds__(256)
attn_f32_kernel(const float* __restrict__ q, int ldq, const float* __restrict__ k,
                const float* __restrict__ v, int ldkv, float* __restrict__ o, int ldo,
                const AttnSeq* __restrict__ seqs, const AttnBlock* __restrict__ blocks, int Hq,
                int Hkv, int hd, float scale) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, h = blockIdx.y;
  const int kvh = h / (Hq / Hkv);
  const AttnBlock blk = blocks[blockIdx.x];
  const AttnSeq sq = seqs[blk.seq];
  const int n_pre = sq.kv_pre_len;
  const int qend = min(blk.q0 + BQ32, sq.len);
  for (int qi = blk.q0 + wave; qi < qend; qi += 4) {
    const float* qp = q + (long long)(sq.q_row0 + qi) * ldq + h * hd;
    const float q0 = lane < hd ? qp[lane] : 0.f;
    const float q1 = lane + 64 < hd ? qp[lane + 64] : 0.f;
    float m = -INFINITY, l = 0.f, a0 = 0.f, a1 = 0.f;
    const int nvis = n_pre + qi + 1;
    for (int j = 0; j < nvis; ++j) {
      const long long row = j < n_pre ? (long long)sq.kv_pre_row0 + j : (long long)sq.kv_row0 + (j - n_pre);
      const float* kp = k + row * ldkv + kvh * hd;
      const float* vp = v + row * ldkv + kvh * hd;
      const float k0 = lane < hd ? kp[lane] : 0.f, k1 = lane + 64 < hd ? kp[lane + 64] : 0.f;
      const float sc = wave_sum(q0 * k0 + q1 * k1) * scale;
      const float mn = fmaxf(m, sc);
      const float al = __expf(m - mn), p = __expf(sc - mn);
      l = l * al + p;
      a0 = a0 * al + p * (lane < hd ? vp[lane] : 0.f);
      a1 = a1 * al + p * (lane + 64 < hd ? vp[lane + 64] : 0.f);
      m = mn;
    }
    float* op = o + (long long)(sq.q_row0 + qi) * ldo + h * hd;
    if (lane < hd) op[lane] = a0 / l;
    if (lane + 64 < hd) op[lane + 64] = a1 / l;
  }
}

}  // namespace

int attn_block_rows(bool bf16) { return bf16 ? BQ : BQ32; }

hipError_t launch_attention(bool bf16, const void* q, int ld_q, const void* k, const void* v,
                            int ld_kv, void* o, int ld_o, const AttnSeq* seqs,
                            const AttnBlock* blocks, int n_blocks, int Hq, int Hkv, int hd,
                            hipStream_t s) {
  if (n_blocks <= 0) return hipSuccess;
  if (Hkv <= 0 || Hq % Hkv != 0) return hipErrorInvalidValue;
  const dim3 grid(n_blocks, Hq);
  if (bf16) {
    if (hd != HD) return hipErrorInvalidValue;
    const float sl2 = 1.4426950408889634f / sqrtf((float)hd);
    hipLaunchKernelGGL(attn_bf16_kernel, grid, dim3(256), 0, s,
                       reinterpret_cast<const bf16_t*>(q), ld_q, reinterpret_cast<const bf16_t*>(k),
                       reinterpret_cast<const bf16_t*>(v), ld_kv, reinterpret_cast<bf16_t*>(o), ld_o,
                       seqs, blocks, Hq, Hkv, sl2);
  } else {
    if (hd > 128) return hipErrorInvalidValue;
    hipLaunchKernelGGL(attn_f32_kernel, grid, dim3(256), 0, s, reinterpret_cast<const float*>(q),
                       ld_q, reinterpret_cast<const float*>(k), reinterpret_cast<const float*>(v),
                       ld_kv, reinterpret_cast<float*>(o), ld_o, seqs, blocks, Hq, Hkv, hd,
                       1.f / sqrtf((float)hd));
  }
  return hipGetLastError();
}

}  // namespace s1
