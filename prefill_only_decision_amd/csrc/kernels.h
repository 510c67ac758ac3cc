// Host-side launch interface of the HIP kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <vector>

namespace s1 {

// ---------------------------------------------------------------- GEMM
// C = A[M,K] x W[N,K]^T with a fused epilogue.
enum Epi {
  EPI_F32 = 0,   // out0 fp32 [M, ld0]
  EPI_RESID,     // out0 fp32 [M, ld0] += C            (residual add)
  EPI_GATE,      // cols < nsplit: out0 elem [M, ld0]; cols >= nsplit:
                 //   out1 fp32 [M, ld1] = log(sigmoid(C))   (decay gate);
                 //   with out2 set, cols >= nsplit2: out2 fp32 [M, ld1] =
                 //   sigmoid(C)                            (write strength)
  EPI_SWIGLU,    // column groups of 64 = [32 gate | 32 up]:
                 //   out0 elem [M, ld0][f] = silu(gate) * up, f < n_valid
  EPI_QKV,       // cols < nsplit: q (rope) -> out0; < nsplit2: k (rope) ->
                 //   out1; else v -> out2.  Head dims permuted (see executor)
  EPI_PARTIAL,   // out0 fp32 slab per K split (split-K partial sums)
  EPI_COUNT
};

struct GemmArgs {
  const void* A;
  const void* W;
  int M, N, K;
  int lda, ldw;          // row strides in elements
  int k_split;           // K elements per split (multiple of the K tile)
  void* out0;
  void* out1;
  void* out2;
  int ld0, ld1, ld2;
  int nsplit, nsplit2;
  int n_valid;
  int head_dim;
  const int* pos;        // EPI_QKV: position of each row
  const float2* rope;    // EPI_QKV: (cos, sin) [max_pos][head_dim / 2]
  long long split_stride;  // EPI_PARTIAL: elements between split slabs
  // EPI_RESID run with a K split: when norm_w is set, the reduction also
  // writes RMSNorm(updated row) * norm_w (epsilon norm_eps) to norm_out
  // (elem, row stride N).
  const float* norm_w;
  void* norm_out;
  float norm_eps;
  int staged;            // set by launch_gemm: bf16 outputs staged through LDS
  // EPI_SWIGLU, EPI_GATE, EPI_QKV (bf16): when row_scale is set, the
  // accumulators of row r are multiplied by row_scale[r] before the epilogue
  // (the 1 / rms of an RMSNorm whose gain has been folded into W).
  const float* row_scale;
  // EPI_RESID (bf16) with rs_out set: the RMSNorm gain is left to the next
  // GEMM (folded into its weights), norm_w unused; rs_out[r] = 1 /
  // sqrt(mean(row^2) + norm_eps).  With a K split the reduction writes the
  // normalised rows (row * rs_out, bf16) to norm_out (row stride N); without
  // one the rows rounded to bf16, and the next GEMM scales its accumulator
  // rows by rs_out.  Without a K split the epilogue writes the rows' sums of squares over
  // aligned groups of 32 * 2^k columns to ss_parts ([N / 32][ss_ld] floats,
  // ss_ld a multiple of 32) and the last workgroup to finish a row block (by
  // `tickets`, one counter per row block, zero between launches) sums them
  // in a fixed tree order that does not depend on the tile configuration.
  float* rs_out;
  float* ss_parts;
  int ss_ld;
  unsigned int* tickets;
};

// Runs the GEMM.  tile_cfg >= 0 picks a tile configuration (0 .. 
// gemm_tile_configs() - 1; configurations the shape cannot use fall back to
// 0) and `split` is the K split; GEMM_AUTO picks both by shape, with `split`
// the largest K split allowed (1 without a workspace).  With split > 1
// (EPI_F32 or EPI_RESID only) partial tiles go to `ws` (split * M * N
// floats) and a reduction kernel applies the epilogue in a fixed order.
// `normed` (optional) reports what an EPI_RESID launch left in norm_out.
enum NormOut {
  NORM_NONE = 0,       // nothing: the norm was not fused
  NORM_ROWS = 1,       // the normalised rows (times norm_w; without a gain when rs_out is set): the
                       // K split's reduction had whole rows
  NORM_DEFERRED = 2,   // the rows rounded to bf16 and rs_out: the consumer scales its rows
};
constexpr int GEMM_AUTO = -1;
hipError_t launch_gemm(bool bf16, Epi epi, const GemmArgs& a, int split, float* ws,
                       hipStream_t s, int tile_cfg = GEMM_AUTO, int* normed = nullptr);
// Weight-direct GEMM (bf16): W is a fragment-order copy made by
// launch_frag_pack (frag_bytes(N, K) bytes); K a positive multiple of 64;
// EPI_F32, EPI_RESID, EPI_SWIGLU over a copy packed with gu16 (gate/up
// interleaved in blocks of 16 rows; ld0 and n_valid multiples of 8), or,
// with tile 2 only, EPI_GATE / EPI_QKV on destinations the staged epilogue
// accepts.  No K split.
size_t frag_bytes(int N, int K);
hipError_t launch_frag_pack(const void* W, int N, int K, int ld, bool gu16, void* out, hipStream_t s);
// tile 1: 128 x 384 workgroup tiles (a wave 128 x 96); tile 2: 256 x 256 (a
// wave 256 x 64); tile 3: 192 x 256 (a wave 192 x 64; EPI_SWIGLU and EPI_F32
// only); tile 4: 224 x 256 (a wave 224 x 64).  gemm_wd_tiles gives the
// workgroup count, gemm_wd_panel the operand rows a workgroup streams per K
// step (BM + BN).
bool gemm_wd_ok(Epi epi, const GemmArgs& a);
int gemm_wd_tiles(int tile, int M, int N);
int gemm_wd_panel(int tile);
hipError_t launch_gemm_wd(Epi epi, const GemmArgs& a, int tile, hipStream_t s);
// Number of tile configurations.
int gemm_tile_configs();
// The K tile (elements) of the register-staged GEMM for the element type.
int gemm_k_tile(bool bf16);

// --------------------------------------------------- achievable peaks
// blocks workgroups of four waves, each wave 8 * iters bf16 32x32x16 matrix
// instructions on registers (out: blocks * 256 floats); a copy of `bytes`
// (multiple of 16) from src to dst, non-temporal.
hipError_t launch_mfma_peak(const void* seed, int blocks, int iters, float* out, hipStream_t s);
hipError_t launch_stream_copy(const void* src, void* dst, long long bytes, hipStream_t s);
// Reads `bytes` (multiple of 16) of src; sink: 4096 bytes, written only when
// a lane's xor of what it read equals a fixed pattern.
hipError_t launch_stream_read(const void* src, long long bytes, void* sink, hipStream_t s);

// ------------------------------------------------------------ elementwise
hipError_t launch_embed(bool bf16, const int32_t* ids, const void* E, float* x, int T, int d,
                        hipStream_t s);
// out = RMSNorm(x) * w.  With w == NULL and rs set (the gain folded into the
// next GEMM's weights): out = x * rs[t] (no gain) and rs[t] = 1 / sqrt(mean(
// x[t]^2) + eps).
hipError_t launch_rmsnorm(bool bf16, const float* x, const float* w, void* out, int T, int d,
                          float eps, hipStream_t s, float* rs = nullptr);
// x = E[ids] (fp32) and xn = RMSNorm(x) * w (elem), T rows of width d
// (d % 4 == 0, d <= 16384; else hipErrorInvalidValue); w == NULL with rs:
// no gain, as launch_rmsnorm.
hipError_t launch_embed_norm(bool bf16, const int32_t* ids, const void* E, float* x, int T, int d,
                             const float* w, void* xn, float eps, hipStream_t s, float* rs = nullptr);
// out[dst_row(o)] = (W[o] + scale * B[o] A) * gain ; row_map may be NULL
// (identity); gain (fp32 [in_dim], an RMSNorm gain folded into the columns)
// may be NULL.  W, A, B may be fp32 or bf16 (same as out); A == NULL means
// no adapter.  fp32 arithmetic, one rounding.
hipError_t launch_merge(bool bf16, const void* W, const void* A, const void* B, void* out,
                        int out_dim, int in_dim, int rank, float scale, const int* row_map,
                        hipStream_t s, const float* gain = nullptr);
hipError_t launch_to_f32(bool bf16, const void* in, float* out, long long n, hipStream_t s);
hipError_t launch_rope_table(float2* table, int max_pos, int head_dim, double base,
                             hipStream_t s);
// out[dst[j]] = x[rows[j]] for j < n_rows (rows of d floats); dst may be NULL.
hipError_t launch_gather_rows(const float* x, int d, const int32_t* rows, const int32_t* dst,
                              int n_rows, float* out, hipStream_t s);

// ------------------------------------------------------------------- scan
struct ScanSeq {
  int row0;   // first row (in the q/k/v/o/log_g arrays)
  int len;
  int s_in;   // initial state slot, or -1 (zero)
  int s_out;  // final state slot, or -1
};
hipError_t launch_scan(bool bf16, const void* q, const void* k, const void* v, int ld_qkv,
                       const float* log_g, int ld_g, void* o, int ld_o, const ScanSeq* seqs,
                       int n_seqs, float* states, int H, int dk, int dv, hipStream_t s, int max_len);
// Chunk-parallel form for few (sequence, head) chains (bf16, dk = dv = 128):
// `chunks` lists every chunk of up to 64 tokens (its s_in / s_out are its own
// index); `cseqs` gives each sequence's chunk range and its initial / final
// state slots in `states`.  cstates [n_chunks][H][128][128] and gamma
// [n_chunks][H] are workspace.  max_nc: the most chunks of one sequence
// (chooses between two and three launches; the results are the same).
// Gated DeltaNet scan: one sequence (rows row0 .. row0 + len - 1, chunks
// c0 .. in the chunk list, state slots as ScanSeq).
struct GdnSeq {
  int row0, len, c0;
  int s_in, s_out;
};
size_t gdn_ws_bytes(int n_chunks, int H);
// q, k, v bf16 [T, ld_qkv] (head h at column h * 128), log_g and beta fp32
// [T, ld_g]; chunks: every 64-token chunk of every sequence (row0, len);
// ws: gdn_ws_bytes(n_chunks, H).
// Short convolution of the Gated DeltaNet inputs for the T rows of a pass
// starting at row r0: y = silu(depthwise causal conv of x, width 4, taps w
// fp32 [C][4]) over C = 3 H 128 channels (q | k | v), q and k L2-normalised
// per head, q scaled by qscale.  row_seq[T] gives each row's sequence in
// seqs; rows before a sequence's start come from hist[s_in] (the last three
// pre-convolution rows of its prefix, bf16 [slots][3][C]) or are zero, and a
// sequence with s_out >= 0 leaves its own last three rows in hist[s_out].
hipError_t launch_gdn_conv(const void* x, void* y, int ld, const float* w, int H, int r0, int T,
                           const int32_t* row_seq, const GdnSeq* seqs, void* hist, float qscale, hipStream_t s);
hipError_t launch_gdn_scan(const void* q, const void* k, const void* v, int ld_qkv, const float* log_g,
                           const float* beta, int ld_g, void* o, int ld_o, const ScanSeq* chunks, int n_chunks,
                           const GdnSeq* seqs, int n_seqs, float* states, int H, float* ws, hipStream_t s);

struct ChunkSeq {
  int c0, nc;    // chunk range
  int s_in;      // initial state slot in `states`, or -1
  int s_out;     // final state slot, or -1
};
hipError_t launch_scan_chunked(const void* q, const void* k, const void* v, int ld_qkv, const float* log_g,
                               int ld_g, void* o, int ld_o, const ScanSeq* chunks, int n_chunks,
                               const ChunkSeq* cseqs, int n_cseqs, float* cstates, float* gamma,
                               float* states, int H, hipStream_t s, int max_nc);

// -------------------------------------------------------------- attention
struct AttnSeq {
  int q_row0;       // first query row (q and o arrays)
  int len;          // queries (= own keys)
  int kv_row0;      // first own key row (k, v arrays)
  int kv_pre_row0;  // first prefix key row
  int kv_pre_len;   // prefix keys (positions 0 ..); queries start at this position
};
struct AttnBlock {
  int seq;          // index into the sequence table
  int q0;           // first query (within the sequence) of this block
  int k_lo, k_hi;   // the keys this workgroup reads, [k_lo, k_hi) in the sequence's key
                    // order (prefix keys first); the causal mask applies within
  int part;         // -1: the block's whole key range, O is written; else the ordinal
                    // of this key piece: (m, l, unnormalised O) go to a partial slot
};
// Queries per attention workgroup for sequences of these lengths: bf16 takes
// the largest of 128, 64, 32 that still gives 512 workgroups over Hq heads
// (else 32); fp32 uses 16.
int attn_block_rows(bool bf16, const int* lens, int n, int Hq);
bool attn_block_rows_valid(bool bf16, int rows);

// Launch plan of one attention pass whose query rows lie in [row_base,
// row_base + n_rows).  piece == 0: one workgroup per query block over its
// whole causal key range (no partial results).  piece > 0 (a multiple of
// 64): keys are cut at multiples of `piece`, each query block's pieces run
// as separate workgroups writing partial (max, sum, O) triples that a
// combine kernel merges in piece order, and consecutive sequences that
// continue the same prefix with contiguous query rows share one sweep of the
// prefix keys (all their queries see every prefix key).  piece < 0: the
// piece is chosen from the key blocks per workgroup chain against the chip
// (n_cu compute units), or no split when the chains are already short and
// no sequence has prefix keys.
struct AttnPlanHost {
  std::vector<AttnSeq> seqs;        // the input sequences, then one entry per shared prefix
  std::vector<AttnBlock> blocks;
  std::vector<int32_t> row_slot;    // [n_rows]: first partial slot of a row (-1: written directly)
  std::vector<int32_t> row_np;      // [n_rows]: the row's pieces
  std::vector<int32_t> comb_rows;   // rows (absolute) the combine kernel writes
  int slots = 0;                    // partial slots, each Hq x (128 + 2) floats
  int piece = 0;
};
void plan_attention(const AttnSeq* seqs, int n, int row_base, int n_rows, int Hq, int bq, int piece, int n_cu,
                    AttnPlanHost* out);
// Partial results of split attention: pO fp32 [slots][Hq][hd], pML (max in
// log2 units, sum) [slots][Hq]; row_slot indexed by row - row_base.
struct AttnPartials {
  const int32_t* row_slot = nullptr;
  const int32_t* row_np = nullptr;
  int row_base = 0;
  float* pO = nullptr;
  float2* pML = nullptr;
};
hipError_t launch_attention(bool bf16, const void* q, int ld_q, const void* k, const void* v,
                            int ld_kv, void* o, int ld_o, const AttnSeq* seqs,
                            const AttnBlock* blocks, int n_blocks, int Hq, int Hkv, int hd, int block_rows,
                            const AttnPartials& part, hipStream_t s);
// Merge the partial results of the listed rows in piece order into o (bf16).
hipError_t launch_attn_combine(const int32_t* rows, int n_rows, const AttnPartials& part, void* o, int ld_o,
                               int Hq, hipStream_t s);

// ---------------------------------------------------------------- readout
hipError_t launch_readout(bool bf16, const float* x, int d, const float* w_final, float eps,
                          const void* E, int Q, const int32_t* rows, const int32_t* opt_offsets,
                          const int32_t* opt_ids, const uint8_t* q_type, float* probs,
                          void* decisions, int max_k, hipStream_t s);

// ------------------------------------------- full-vocabulary log-probs
// Workspace of the feature kernels for R distinct rows (byte offsets into
// one device block): normalised rows hn fp32 [Rp, d], their bf16 hi / lo
// split [Rp, d] each (bf16 models), per-block partial (max, sum) pairs
// [Rp, nb] and lse [Rp]; Rp = R rounded up to 32.
struct FeatWs {
  int Rp = 0, nb = 0;
  size_t hn = 0, hi = 0, lo = 0, part = 0, lse = 0, bytes = 0;
};
FeatWs feat_ws_layout(bool bf16, int R, int V, int d);
// Shapes the feature kernels take: bf16 d % 128 == 0, fp32 d % 4 == 0.
bool feat_shape_ok(bool bf16, int d);

// Device metadata of a feature request: R distinct rows of x (rows[R]);
// target t reads row rows[t_ri[t]] and scores token t_tok[t]; candidate c
// owns targets cand_off[c] .. cand_off[c+1]-1; group g lists its
// candidates grp_cands[grp_off[g] .. grp_off[g+1]-1].
struct FeatArgs {
  int R = 0, n_targets = 0, n_groups = 0;
  const int32_t* rows = nullptr;
  const int32_t* t_ri = nullptr;
  const int32_t* t_tok = nullptr;
  const int32_t* cand_off = nullptr;
  const int32_t* grp_off = nullptr;
  const int32_t* grp_cands = nullptr;
};
// Final RMSNorm of the R rows into the workspace (hn, and hi / lo for bf16).
hipError_t launch_feat_norm(bool bf16, const float* x, int d, const int32_t* rows, int R, const float* w_final,
                            float eps, int V, void* ws, hipStream_t s);
// Per-block partial (max, sum exp) pairs of hn[r] . E[v] over the V rows of
// E, from the workspace's normalised rows; launch_lse_merge then forms
// lse[r] = log sum_v exp(hn[r] . E[v]) in the workspace's lse array.
hipError_t launch_vocab_lse(bool bf16, const void* E, int V, int d, int R, void* ws, hipStream_t s);
hipError_t launch_lse_merge(bool bf16, int V, int d, int R, void* ws, hipStream_t s);
// Per-target logp = hn . E[token] - lse, then the candidate scores and
// their normalisation per group (after launch_vocab_lse).
hipError_t launch_feat_targets(bool bf16, int d, const void* E, int V, const FeatArgs& f, float* logp,
                               float* cand_lp, float* cand_norm, void* ws, hipStream_t s);
// The whole feature computation: logp[n_targets], cand_lp and cand_norm
// [number of candidates].
hipError_t launch_features(bool bf16, const float* x, int d, const float* w_final, float eps, const void* E,
                           int V, const FeatArgs& f, float* logp, float* cand_lp, float* cand_norm, void* ws,
                           hipStream_t s);

}  // namespace s1
