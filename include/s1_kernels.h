/*
 * s1_kernels.h -- per-kernel entry points of the prefill-only decision
 * library, for parity tests and micro-benchmarks.
 *
 * Every function enqueues one kernel family on hip_stream (NULL: the null
 * stream) and returns without synchronising, except s1k_la_scan and
 * s1k_attention, which copy their host metadata to temporary device memory
 * and synchronise the stream before returning.  All array arguments are device
 * pointers unless marked "host".  dtype is s1_dtype (S1_F32 or S1_BF16) and
 * selects the element type of the arrays marked "elem" (bf16 arrays hold raw
 * bfloat16 bit patterns).  Returns S1_OK, S1_EINVAL for shapes the kernel does
 * not support, or S1_EDEVICE if the launch failed.  Shapes are checked on the
 * host before launch; the caller guarantees that every buffer holds the
 * stated number of elements.
 */
#ifndef S1_KERNELS_H
#define S1_KERNELS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* C[M,N] (fp32, row stride N) = A[M,K] (elem, row stride K) x W[N,K]^T
 * (elem, row stride K): the projection GEMM with a plain fp32 epilogue, tile
 * configuration chosen by shape as in the decoder.  split_k >= 1 is the
 * largest K split allowed: split partial tiles are summed in a fixed order
 * (deterministic).  bf16 needs K % 8 == 0, fp32 K % 4 == 0.  Projection
 * GEMMs of the decoder (RFC #114, section 1: the language-model projections;
 * the Cua-S1 issue, "mostly GEMMs" comment). */
int s1k_gemm(int32_t dtype, const void* A, const void* W, float* C, int32_t M, int32_t N,
             int32_t K, int32_t split_k, void* hip_stream);

/* s1k_gemm with an explicit tile configuration, 0 <= tile_cfg <
 * s1k_gemm_tile_configs(), and exactly split_k K splits (fewer when K has
 * fewer K tiles).  0 is the register-staged kernel (any element type and
 * shape); 1..6 are the bf16 LDS-DMA kernels (128x128 three stages,
 * 128x128 two stages, 128x64, 64x128, 256x256, 256x192), used when
 * K % 64 == 0 and falling back to 0 otherwise.  Invalid arguments return
 * S1_EINVAL. */
int s1k_gemm_cfg(int32_t dtype, const void* A, const void* W, float* C, int32_t M, int32_t N,
                 int32_t K, int32_t split_k, int32_t tile_cfg, void* hip_stream);

/* s1k_gemm for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same kernels and results, with the split-K partial sums in a file-scope
 * device array of S1K_NOALLOC_SCRATCH_BYTES per GPU (held until the process
 * ends) instead of a per-call workspace; it calls no allocator.  S1_EINVAL
 * when split_k * M * N * 4 exceeds that size.  Every call on one GPU shares
 * its array: calls that overlap on one GPU (other streams, other threads)
 * race and must be serialised by the caller. */
#define S1K_NOALLOC_SCRATCH_BYTES (32u << 20)
int s1k_gemm_noalloc(int32_t dtype, const void* A, const void* W, float* C, int32_t M, int32_t N,
                     int32_t K, int32_t split_k, void* hip_stream);

/* Residual projection with the statistics of the RMSNorm that follows it
 * (pre-norm blocks of the Qwen3.5-family backbone the System1-Omni README
 * names; RFC #114 section 3, RMSNorm before each mixer and FFN), bf16:
 * x[M,N] (fp32, in/out, device) += A[M,K] W[N,K]^T (A, W bf16, device);
 * rs[M] (fp32, device) = 1 / sqrt(mean(x_row^2) + eps); hb[M,N] (bf16,
 * device) = the updated x rounded to bf16 (*form = 2, the launch ran without
 * a K split: the projection that consumes the norm multiplies its
 * accumulator rows by rs) or x * rs rounded to bf16 (*form = 1, a K split's
 * reduction, which holds whole rows).  Either way the norm gain is folded
 * into the consuming weight columns, so that no separate norm pass reads the
 * rows.  form: host int, may be NULL.
 * tile_cfg: -1 (configuration and split chosen by shape, at most split_k) or
 * as s1k_gemm_cfg (exactly split_k K splits, K % 64 == 0 and N % 4 == 0 when
 * split_k > 1).  Without a K split a row's sum of squares is taken in one
 * fixed order whatever tile_cfg and M, so rs is bitwise the same for a row
 * in any such launch.  N <= 8192, K % 8 == 0.  Allocates its workspace per
 * call.  S1_EINVAL on other arguments. */
int s1k_gemm_resid_norm(const void* A, const void* W, float* x, int32_t M, int32_t N, int32_t K,
                        int32_t split_k, int32_t tile_cfg, float eps, void* hb, float* rs, int32_t* form,
                        void* hip_stream);

/* Number of GEMM tile configurations (host-only, no device work). */
int s1k_gemm_tile_configs(void);

/* Achievable-peak probes (not on the decision path; they state each
 * kernel's roofline fraction against what the GPU in use delivers, beside
 * the datasheet figures).  s1k_mfma_peak: `blocks` workgroups of four
 * waves; each wave issues 8 * iters bf16 32x32x16 matrix instructions on
 * register operands (2 * 32 * 32 * 16 flop each) built from seed (device,
 * 2048 bytes, any bf16 bit patterns); out (device, blocks * 256 floats)
 * receives per-lane sums so the work is not elided.  s1k_stream_copy: dst =
 * src over `bytes` (a multiple of 16; device buffers of that size, not
 * overlapping), 16-byte non-temporal accesses.  s1k_stream_read: reads
 * `bytes` (a multiple of 16) of src with the same accesses; sink (device,
 * 4096 bytes) is written only when a lane's xor of what it read equals a
 * fixed pattern. */
int s1k_mfma_peak(const void* seed, int32_t blocks, int32_t iters, float* out, void* hip_stream);
int s1k_stream_copy(const void* src, void* dst, int64_t bytes, void* hip_stream);
int s1k_stream_read(const void* src, int64_t bytes, void* sink, void* hip_stream);

/* Bytes of the fragment-order copy of a bf16 weight W[N,K] (rows padded to
 * a multiple of 32); 0 for unsupported shapes (N < 1, K not a positive
 * multiple of 16).  Host-only. */
int64_t s1k_frag_bytes(int32_t N, int32_t K);

/* out (bf16, s1k_frag_bytes(N, K) bytes, caller-allocated device memory) =
 * W[N,K] (bf16, row stride K) in fragment order: for each block of 32 rows
 * nb and each step of 16 columns ks, one contiguous 1 KB block whose 16-byte
 * chunk l holds row 32 nb + l % 32, columns 16 ks + 8 (l / 32) .. + 7 (the
 * B operand of lane l of a 32x32x16 matrix instruction); rows past N are
 * zero.  gate_up16 != 0 (N a multiple of 64) takes W as FFN gate/up rows
 * interleaved in blocks of 32 ([32 gate | 32 up] per 64 rows, as the
 * decoder stores them) and packs them interleaved in blocks of 16, the
 * layout the SwiGLU epilogue of s1k_gemm_wfrag reads.  The weight layout of
 * the projection GEMMs (RFC #114, section 1; the Cua-S1 issue, "mostly
 * GEMMs" comment). */
int s1k_frag_pack(const void* W, int32_t N, int32_t K, int32_t gate_up16, void* out, void* hip_stream);

/* The weight-direct GEMM: A[M,K] (bf16, row stride K) times the packed
 * weight Wfrag (s1k_frag_pack) transposed.  swiglu = 0: out fp32 [M,N] =
 * A W^T.  swiglu != 0 (Wfrag packed with gate_up16, N a multiple of 64):
 * out bf16 [M, N/2][f] = silu(gate_f) * up_f, the FFN gate/up projection with
 * its SwiGLU (RFC #114 section 1; SwiGLU FFN of the Qwen3.5-family
 * backbone).  K must be a positive multiple of 64.  tile 1: workgroup tiles
 * of 128 rows x 384 columns; tile 2: 256 x 256; tile 3: 192 x 256; tile
 * 4: 224 x 256 (other values: S1_EINVAL).
 * Accumulation order over K is the same as s1k_gemm's without a K split
 * (results are bitwise equal). */
int s1k_gemm_wfrag(const void* A, const void* Wfrag, void* out, int32_t M, int32_t N, int32_t K,
                   int32_t swiglu, int32_t tile, void* hip_stream);

/* out[T,d] (elem) = x / sqrt(mean(x^2) + eps) * w for each row of x[T,d]
 * (fp32); w[d] fp32.  RMSNorm before each mixer and FFN (pre-norm blocks of
 * the Qwen3.5-family backbone the System1-Omni README names). */
int s1k_rmsnorm(int32_t dtype, const float* x, const float* w, void* out, int32_t T,
                int32_t d, float eps, void* hip_stream);

/* x[T,d] (fp32) = E[ids[t]] (E elem [V,d]); ids int32 in [0, V) (checked by
 * the caller).  Tied input embedding (RFC #114 section 3: input/output
 * embedding tying is preserved). */
int s1k_embed(int32_t dtype, const int32_t* ids, const void* E, float* x, int32_t T,
              int32_t d, void* hip_stream);

/* out[out_dim,in_dim] (elem) = W + scale * B A, computed in fp32 and rounded
 * once (round to nearest even for bf16); W elem [out_dim,in_dim], A elem
 * [rank,in_dim], B elem [out_dim,rank].  A or B NULL: plain copy of W.
 * LoRA merge at load (RFC #114 section 3). */
int s1k_lora_merge(int32_t dtype, const void* W, const void* A, const void* B, void* out,
                   int32_t out_dim, int32_t in_dim, int32_t rank, float scale, void* hip_stream);

/* Gated linear-attention scan over packed sequences:
 *   S_t = g_t S_{t-1} + k_t v_t^T,  o_t = S_t^T q_t   per (sequence, head)
 * q, k (elem, [T, H, dk] at row stride ld_qkv elements), v (elem, [T, H, dv]
 * at row stride ld_qkv), log_g (fp32 [T, H], natural log of the gate),
 * o (elem [T, H*dv]).  cu_seqlens (host, n_seqs + 1).  s_init (fp32
 * [n_seqs, H, dk, dv] or NULL = zero start) and s_final (same shape or NULL)
 * hold each sequence's initial and final state.  bf16 needs dk = dv = 128;
 * fp32 needs dk, dv in {64, 128}.  The recurrent state stays fp32 (RFC #114
 * section 5: FP32 recurrent state). */
int s1k_la_scan(int32_t dtype, const void* q, const void* k, const void* v, int32_t ld_qkv,
                const float* log_g, void* o, int32_t T, int32_t H, int32_t dk, int32_t dv,
                int32_t n_seqs, const int32_t* cu_seqlens, const float* s_init,
                float* s_final, void* hip_stream);

/* The same scan (bf16, dk = dv = 128) in its chunk-parallel form, used when a
 * request has few (sequence, head) chains: every 64-token chunk's state
 * contribution in parallel, an elementwise scan of chunk states across
 * chunks, then every chunk's outputs in parallel from the state entering it.
 * Arguments as s1k_la_scan (bf16 implied).  Synchronises the stream. */
int s1k_la_scan_chunked(const void* q, const void* k, const void* v, int32_t ld_qkv,
                        const float* log_g, void* o, int32_t T, int32_t H, int32_t n_seqs,
                        const int32_t* cu_seqlens, const float* s_init, float* s_final,
                        void* hip_stream);

/* Gated DeltaNet scan (Yang, Kautz, Hatamizadeh, "Gated Delta Networks",
 * ICLR 2025; RFC #114 section 5 for the fp32 state) over packed sequences,
 * bf16, dk = dv = 128:
 *   S_t = g_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T,  o_t = S_t^T q_t,
 * in 64-token chunks in the WY form.  q, k, v elem [T, ld_qkv] with head h at
 * columns h*128 .. h*128+127 (q and k already L2-normalised by the caller),
 * log_g = log g and beta fp32 [T, H], o elem [T, H*128]; cu_seqlens host
 * [n_seqs+1]; s_init / s_final optional fp32 [n_seqs, H, 128, 128] as in
 * s1k_la_scan.  Synchronises the stream. */
int s1k_gdn_scan(const void* q, const void* k, const void* v, int32_t ld_qkv, const float* log_g, const float* beta,
                 void* o, int32_t T, int32_t H, int32_t n_seqs, const int32_t* cu_seqlens, const float* s_init,
                 float* s_final, void* hip_stream);

/* Causal attention over packed sequences with grouped KV heads:
 *   o_t = sum_{s: pos_s <= pos_t} softmax_s(q_t . k_s / sqrt(hd)) v_s
 * q (elem [Tq, Hq, hd]), k, v (elem [Tkv, Hkv, hd]), o (elem [Tq, Hq, hd]).
 * Sequence i has queries q_row0[i] .. q_row0[i] + q_len[i] - 1; its keys are
 * kv_pre_len[i] prefix rows starting at kv_pre_row0[i] (positions 0 ..) and
 * then its own q_len[i] rows starting at kv_row0[i] (positions
 * kv_pre_len[i] ..); query j has position kv_pre_len[i] + j.  All five
 * arrays are host int32 [n_seqs].  bf16 needs hd = 128; fp32 hd 64 or 128.
 * block_rows: queries per workgroup, 0 to choose by size as the decoder
 * does; bf16 accepts 32, 64 or 128, fp32 16.  piece (bf16 only): 0 runs every
 * query block over its whole key range in one workgroup; a positive multiple
 * of 64 cuts the keys at multiples of it into pieces run by separate
 * workgroups and merged in key order, and lets consecutive sequences that
 * share prefix rows (same kv_pre_row0 and kv_pre_len, contiguous query rows)
 * sweep the prefix keys once for all their queries (RFC #114 section 5:
 * branches share one prefix snapshot); -1 chooses the piece by size as the
 * decoder does.  Query rows of different sequences must not overlap. */
int s1k_attention(int32_t dtype, const void* q, const void* k, const void* v, void* o,
                  int32_t Hq, int32_t Hkv, int32_t hd, int32_t n_seqs, const int32_t* q_row0,
                  const int32_t* q_len, const int32_t* kv_row0, const int32_t* kv_pre_row0,
                  const int32_t* kv_pre_len, int32_t block_rows, int32_t piece, void* hip_stream);

/* The launch plan s1k_attention (and the decoder) would use, on the host
 * only (no device work; usable without a GPU), for checking its coverage.
 * Inputs as s1k_attention (host arrays).  On return blocks[5 * i ..] =
 * (sequence, first query, first key, key end, piece ordinal or -1) for
 * i < *n_blocks, where sequences n_seqs .. *n_seqs_out - 1 are the shared
 * prefix entries whose (q_row0, q_len, kv_row0, kv_pre_row0, kv_pre_len) go
 * to shared[5 * (i - n_seqs) ..]; row_np[r - row_lo] the pieces of query
 * row r, with row_lo the smallest query row.  Capacities: max_blocks
 * blocks, max_shared shared entries, max_rows rows; S1_EINVAL when any is
 * exceeded. */
int s1k_attention_plan(int32_t n_seqs, const int32_t* q_row0, const int32_t* q_len, const int32_t* kv_row0,
                       const int32_t* kv_pre_row0, const int32_t* kv_pre_len, int32_t Hq, int32_t block_rows,
                       int32_t piece, int32_t n_cu, int32_t max_blocks, int32_t* blocks, int32_t* n_blocks,
                       int32_t max_shared, int32_t* shared, int32_t* n_seqs_out, int32_t max_rows,
                       int32_t* row_np, int32_t* piece_out);

/* Decision readout for Q questions: h = RMSNorm(x[rows[j]]; w_final),
 * z_k = h . E[opt_k], p = softmax(z) over the question's options, and the
 * answer fields (layout of s1_decision in s1.h: int32 choice then 5 floats).
 * x fp32 [*, d], E elem [V, d], rows/opt_offsets/opt_ids/q_type device;
 * at most 1024 options per question.
 * (Cua-S1 issue, first plan comment; sys1rust README, "Try it".) */
int s1k_readout(int32_t dtype, const float* x, int32_t d, const float* w_final, float eps,
                const void* E, int32_t Q, const int32_t* rows, const int32_t* opt_offsets,
                const int32_t* opt_ids, const uint8_t* q_type, float* probs, void* decisions,
                void* hip_stream);

/* Full-vocabulary log-sum-exp of R rows of x (fp32 [*, d]) after the final
 * RMSNorm: lse[r] = log sum_v exp(h_r . E[v]), h_r = RMSNorm(x[rows[r]];
 * w_final), over all V rows of E (elem [V, d]); rows device int32 [R], lse
 * device fp32 [R].  bf16: the logits are formed on MFMA from h split into a
 * bf16 pair hi + lo (|h - hi - lo| <= 2^-17 |h|) with fp32 accumulation and
 * need d % 128 == 0; fp32: d % 4 == 0.  Allocates its workspace on the stream
 * (stream-ordered) and returns without synchronising.  (RFC #114, section 4,
 * note under the semantics table: vocabulary work in bounded chunks.) */
int s1k_vocab_lse(int32_t dtype, const float* x, int32_t d, const float* w_final, float eps, const void* E,
                  int32_t V, int32_t R, const int32_t* rows, float* lse, void* hip_stream);

/* Token log-probabilities and candidate normalisation over rows of x (fp32
 * [n_rows, d]), as s1_plan_set_features in s1.h describes, with rows[] indexing
 * x directly.  rows, tokens, cand_offsets and cand_group are host arrays;
 * logp [n_targets], cand_logp and cand_norm [n_cands] device fp32.
 * Synchronises the stream before returning. */
int s1k_token_logprobs(int32_t dtype, const float* x, int32_t n_rows, int32_t d, const float* w_final, float eps,
                       const void* E, int32_t V, int32_t n_targets, const int32_t* rows, const int32_t* tokens,
                       int32_t n_cands, const int32_t* cand_offsets, const int32_t* cand_group, float* logp,
                       float* cand_logp, float* cand_norm, void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* S1_KERNELS_H */
