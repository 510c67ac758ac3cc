/*
 * s1.h -- C ABI of the prefill-only decision library for AMD MI355X (gfx950).
 *
 * A decision model answers closed questions from one prefill pass, with no
 * decoding (System1-Omni README, introduction; Cua-S1 4B 0.2 issue #10, first
 * plan comment: a single pass, then a softmax over the option logits).
 * The model is a hybrid decoder -- gated linear-attention layers and full
 * causal-attention layers, 3:1 -- with a LoRA adapter merged into the weights
 * at load (RFC #114 "Native Rust/CUDA support for OmniJev-4B v1.1", sections
 * 1 and 3).  The library takes token ids (Cua-S1 issue, last comment: the
 * native engine only takes token ids), per-question marker positions and
 * option-token id lists, and returns per-option probabilities and the answer
 * fields of the sys1rust README ("Try it": choice, score, noul,
 * answer_confidence, confidence).
 *
 * Conventions
 *  - Every int-returning call returns S1_OK (0) or a negative S1_E* code;
 *    s1_last_error() then gives a message for the calling thread.
 *  - Inputs are validated before any device work; an invalid request
 *    enqueues nothing (RFC #114 section 2: validate counts, lengths and
 *    budgets before dispatch and return explicit errors).
 *  - On a device error the call synchronises its stream before returning,
 *    so no kernel still reads caller memory (RFC #114 section 2: keep
 *    resource ownership until device work finishes, error paths included).
 *  - One call per model at a time; calls on different models may overlap.
 *  - Streams are HIP stream handles passed as void*; NULL selects the
 *    library's own stream.
 */
#ifndef S1_H
#define S1_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  S1_OK = 0,
  S1_EINVAL = -1,   /* malformed argument or request */
  S1_ENOMEM = -2,   /* device or host allocation failed */
  S1_EDEVICE = -3,  /* a HIP call failed */
  S1_EBUDGET = -4   /* request exceeds a budget fixed at load */
};

typedef enum { S1_F32 = 0, S1_BF16 = 1 } s1_dtype;
typedef enum { S1_CHOICE = 0, S1_SCORE = 1, S1_NOUL = 2 } s1_qtype;

/*
 * Linear-attention layer kinds (s1_config.la_kind).
 *  S1_LA_GLA: gated linear attention, S_t = g_t S_{t-1} + k_t v_t^T,
 *    o_t = S_t^T q_t (the stand-in recurrence; RFC #114 sections 4-5 name
 *    Gated DeltaNet without printing it).
 *  S1_LA_GDN: Gated DeltaNet (Yang, Kautz, Hatamizadeh, ICLR 2025): the
 *    q | k | v projections pass a depthwise causal convolution of width 4
 *    (taps `.la.conv` [2 la_heads la_dk + la_heads la_dv, 4], the last tap on
 *    the current token) and SiLU; q and k are L2-normalised per head (eps
 *    1e-6 under the root), q scaled by 1/sqrt(la_dk); beta = sigmoid(u .
 *    w_b) per head from `.la.b` [la_heads, d];
 *    S_t = g_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T.  A branch
 *    continues from its prefix's state and last three pre-convolution rows.
 *    bf16 models only.
 */
enum { S1_LA_GLA = 0, S1_LA_GDN = 1 };

/* LoRA target bits of s1_config.lora_targets. */
enum {
  S1_LORA_Q = 1 << 0, S1_LORA_K = 1 << 1, S1_LORA_V = 1 << 2, S1_LORA_O = 1 << 3,
  S1_LORA_GATE = 1 << 4, S1_LORA_UP = 1 << 5, S1_LORA_DOWN = 1 << 6
};

/*
 * Model shape and budgets, fixed at load.
 *  layer l is full attention iff l % full_every == full_every - 1
 *  linear attention: la_heads heads, key dim la_dk, value dim la_dv, one
 *    scalar decay gate per (token, head)
 *  full attention: fa_q_heads query heads sharing fa_kv_heads key/value heads
 *    in contiguous groups, head dim fa_head_dim, rotate-half RoPE (rope_base)
 *  dtype: S1_BF16 (GEMM operands bf16, fp32 accumulation, fp32 residual
 *    stream, fp32 recurrent state) or S1_F32 (everything fp32).
 *  bf16 models need la_dk == la_dv == fa_head_dim == 128, d_model, ffn and
 *  la_heads*la_dv multiples of 64.  fp32 models need head dims in {64, 128}
 *  and d_model, ffn multiples of 4.
 * Budgets: a request with more tokens, sequences, questions, options per
 * question, prefix sequences or positions than these fails with S1_EBUDGET.
 */
typedef struct {
  int32_t n_layers, full_every;
  int32_t d_model, ffn, vocab;
  int32_t la_heads, la_dk, la_dv;
  int32_t fa_q_heads, fa_kv_heads, fa_head_dim;
  float rope_base, rms_eps;
  int32_t lora_rank;
  float lora_alpha;
  uint32_t lora_targets;
  int32_t dtype;              /* s1_dtype */
  int64_t max_tokens;         /* packed tokens per request */
  int32_t max_seqs;
  int32_t max_questions;
  int32_t max_options;        /* per question */
  int32_t max_prefixes;       /* distinct prefix sequences per request */
  int64_t max_positions;      /* prefix length + branch length */
  int32_t la_kind;            /* linear-attention layers: S1_LA_GLA or S1_LA_GDN */
} s1_config;

/*
 * One weight tensor, caller-owned; the library copies it during
 * s1_load_weights.  data is host memory, or device memory when on_device is
 * non-zero.  dtype must equal the model dtype.  Row-major; projections are
 * [out, in] (y = x W^T).  Names:
 *   embed [vocab, d] (tied: also the readout rows), final_norm [d]
 *   layers.{l}.attn_norm [d], layers.{l}.ffn_norm [d]
 *   layers.{l}.la.{q,k,v,g,o}   (linear-attention layers; g is [la_heads, d];
 *                                Gated DeltaNet layers also .b and .conv)
 *   layers.{l}.fa.{q,k,v,o}     (full-attention layers)
 *   layers.{l}.ffn.{gate,up,down}
 *   <projection>.lora_A [r, in] and <projection>.lora_B [out, r] for every
 *   projection whose target bit is set (the decay gate g is never a target).
 */
typedef struct {
  const char* name;
  int32_t dtype;
  int32_t ndim;
  int64_t shape[2];
  const void* data;
  int32_t on_device;
} s1_tensor;

/*
 * A packed request (no padding; RFC #114 "Plan" comment: rows run unpadded).
 *  cu_seqlens[n_seqs+1]: sequence i is tokens cu_seqlens[i] .. cu_seqlens[i+1]-1
 *  token_ids[cu_seqlens[n_seqs]] in [0, vocab)
 *  prefix_of[n_seqs] (may be NULL = all -1): -1, or the index of another
 *    sequence whose tokens logically precede this one.  Such a branch
 *    continues from the prefix's full-attention keys/values and final
 *    linear-attention state, and its token j has position len(prefix) + j
 *    (RFC #114 section 4 "Branching" and section 5: encode the common prefix
 *    once; every branch starts from the same immutable snapshot).  A prefix
 *    must itself have prefix_of == -1 and carries no questions (S1_EINVAL:
 *    it is encoded once for its branches).  Sequences never see each other
 *    otherwise.
 *  Question q reads token q_marker[q] (0-based, inside sequence q_seq[q]) and
 *    has options opt_ids[opt_offsets[q] .. opt_offsets[q+1]-1], K >= 2 of
 *    them, in caller order; q_type S1_NOUL needs exactly [yes, no].
 * All pointers are host memory, read during the call only.
 */
typedef struct {
  int32_t n_seqs;
  const int32_t* cu_seqlens;
  const int32_t* token_ids;
  const int32_t* prefix_of;
  int32_t n_questions;
  const int32_t* q_seq;
  const int32_t* q_marker;
  const uint8_t* q_type;
  const int32_t* opt_offsets;
  const int32_t* opt_ids;
} s1_batch;

/*
 * Answer fields of one question, from its option probabilities p (sys1rust
 * README, "Try it"): choice = index of the largest p (lowest index on a tie);
 * score = sum_k k p_k with levels 0..K-1, the expected level; noul = p[0],
 * P(yes); answer_confidence = max p; entropy_confidence = 1 - H(p)/ln K
 * (0 for an even split, 1 for a one-hot); confidence = entropy_confidence for
 * choice and score, answer_confidence for noul.  Every field is filled for
 * every question type.
 */
typedef struct {
  int32_t choice;
  float score;
  float noul;
  float answer_confidence;
  float confidence;
  float entropy_confidence;
} s1_decision;

typedef struct {
  int64_t tokens_processed;   /* packed tokens: each prefix once plus every branch */
  double wall_us;             /* host wall time of the call */
  double device_us;           /* HIP-event time of the device work */
} s1_timing;

typedef struct s1_model s1_model;
typedef struct s1_plan s1_plan;

/* Load a model: the executor owns the weights and device buffers from here
 * until s1_free (RFC #114, section 2, "Ownership and serving interface").
 * Copies the caller's tensors, merges each adapter into its projection,
 * W' = W + (alpha/r) B A in fp32 with one rounding to the model dtype (the
 * rank-32 / alpha-64 adapter merged into BF16 weights: RFC #114 section 1;
 * merged at load: Cua-S1 issue #10, plan comment, step 3), lays the weights
 * out for the kernels (gate/up interleaved, RoPE pairs permuted) and
 * allocates the workspace for the budgets in cfg on the current HIP device.
 * tensors: n_tensors caller-owned entries (host, or device with on_device),
 * read during the call only.  hip_stream: the stream the copies and merges
 * run on (NULL: the library's own).  Errors, with nothing left allocated:
 * S1_EINVAL (config, names, shapes, dtypes, missing tensors), S1_ENOMEM,
 * S1_EDEVICE.  *out is set only on success. */
int s1_load_weights(const s1_config* cfg, const s1_tensor* tensors, int32_t n_tensors,
                    void* hip_stream, s1_model** out);

/* Answer every question of the request from one prefill pass (System1-Omni
 * README, introduction: decisions from a single forward pass, no decoding;
 * Cua-S1 issue #10, plan comment: a softmax over the answer-option logits).
 * Input is token ids (Cua-S1 issue #10, last comment), per-question marker
 * positions and option-token id lists (s1_batch); the readout runs only at
 * the marker rows (sys1rust README, "How it works") and fills the answer
 * fields of sys1rust README "Try it" (s1_decision).  probs[sum K] receives
 * the option probabilities in question order, out[n_questions] the fields;
 * both host memory, caller-owned.  timing may be NULL (its wall_us covers the
 * whole call, including the host-to-device copy of the request and the
 * device-to-host copy of the results; device_us the device work alone).
 * Synchronous: returns once the outputs are written.  The request is
 * validated on the host before any device work (RFC #114 section 2:
 * validate counts, lengths and budgets before dispatch, explicit errors):
 * S1_EINVAL (malformed, ids out of range, K < 2, noul K != 2, a marker
 * outside its sequence, bad prefix links, a question on a prefix), S1_EBUDGET
 * (beyond a load-time budget), both with nothing enqueued; S1_EDEVICE after
 * the stream has been synchronised (resource ownership kept until device work
 * finishes, RFC #114 section 2); S1_ENOMEM.  Device memory: a block owned
 * by the model, grown only when a request needs more than every earlier one
 * (no allocation in the steady state).  One call per model at a time. */
int s1_prefill_decide(s1_model* m, const s1_batch* b, float* probs, s1_decision* out,
                      s1_timing* timing, void* hip_stream);

/* Free the model and all its device memory, after the device is idle (RFC
 * #114 section 2: ownership until device work finishes).  NULL is a no-op.
 * The caller must not have a call in flight on the model. */
void s1_free(s1_model* m);

/* Message of the last failed call on this thread ("" if none): the explicit
 * error of RFC #114 section 2.  The pointer stays valid until the next call
 * on this thread. */
const char* s1_last_error(void);

/* Validate a request against a config, on the host only (no device work,
 * usable without a GPU).  Returns S1_OK, S1_EINVAL or S1_EBUDGET. */
int s1_validate(const s1_config* cfg, const s1_batch* b);

/*
 * Resident-input path.  s1_plan_create validates the request, builds its
 * launch plan and copies the token ids and metadata to device memory owned by
 * the plan.  s1_plan_run enqueues the whole forward and readout on hip_stream
 * and returns without synchronising; d_probs[sum K] and d_out[n_questions]
 * are device memory.  A plan belongs to its model and can be run any number
 * of times.  s1_plan_free(NULL) is a no-op.
 */
int s1_plan_create(s1_model* m, const s1_batch* b, s1_plan** out);
int s1_plan_run(s1_model* m, s1_plan* p, float* d_probs, s1_decision* d_out, void* hip_stream);
void s1_plan_free(s1_plan* p);

/*
 * Length buckets (RFC #114 comment "Plan: native OmniJev-4B v1.1" and the
 * Cua-S1 issue's timing comments: graphs captured over length buckets).
 * s1_plan_create_bucket builds a plan for one sequence of max_tokens tokens,
 * max_questions questions and up to max_options options in all (>= 2 per
 * question); s1_plan_update refills it with a request of one sequence (no
 * prefix) that fits, without touching any device pointer, so a HIP graph
 * captured from the plan is replayed as is.  The request's tokens are
 * followed by token 0 up to max_tokens (causal mixers: padding rows never
 * reach a request row) and its questions by two-way placeholder questions;
 * a run writes s1_plan_questions() = max_questions decisions and
 * s1_plan_options() <= max_options + 2 * max_questions probabilities, the
 * request's first (size the outputs for the bound).  s1_plan_update copies synchronously and
 * must not overlap a run of the plan.  Errors: S1_EINVAL (not a bucket plan,
 * more than one sequence, malformed), S1_EBUDGET (the request does not fit).
 */
int s1_plan_create_bucket(s1_model* m, int32_t max_tokens, int32_t max_questions, int32_t max_options,
                          s1_plan** out);
int s1_plan_update(s1_plan* p, const s1_batch* b);
/* Questions and option probabilities a run of the plan writes. */
int32_t s1_plan_questions(const s1_plan* p);
int64_t s1_plan_options(const s1_plan* p);

/* Replay the plan as one HIP graph (enable != 0) instead of issuing every
 * kernel launch from the host.  The graph is captured on the first run and
 * captured again when the output or capture pointers change; the stream must
 * not be the null stream (NULL selects the library's own stream, which is
 * fine).  Default: off.  Profiling always runs launch by launch. */
int s1_plan_set_graph(s1_plan* p, int32_t enable);

/* Row-invariant execution (enable != 0): every row's arithmetic is the same
 * whatever else the request holds -- no K split in any projection GEMM (the
 * tile shapes already accumulate K in one fixed order) and the chunk-parallel
 * scan schedule in every pass -- so a sequence packed with others, run alone,
 * or continued as a branch gives bitwise the same outputs as the plain
 * forward of its tokens (RFC #114 comment "Plan: native OmniJev-4B v1.1":
 * GEMM rows that do not depend on M keep batched rows order-invariant).
 * Slower for short requests (no K split).  Default: off. */
int s1_plan_set_invariant(s1_plan* p, int32_t enable);

/* Tokens the plan processes (each prefix once plus every other sequence). */
int64_t s1_plan_tokens(const s1_plan* p);

/*
 * Capture residual-stream rows for inspection: after the embedding and after
 * every layer, the rows listed (packed token indices of the request) are
 * copied into d_hidden[(n_layers + 1) * n_rows * d_model] (fp32, device
 * memory) by the next s1_plan_run calls.  n_rows = 0 switches capture off.
 */
int s1_plan_set_capture(s1_plan* p, int32_t n_rows, const int32_t* rows, float* d_hidden);

/*
 * Layer-local inputs (a test hook for per-layer parity, RFC #114 section 6:
 * compare the selected hidden rows of every stage).  Before layer l runs,
 * residual-stream row rows[j] (a packed token index of the request, each
 * listed at most once) is replaced by d_src[(l * n_rows + j) * d_model ..]
 * (fp32, device memory, n_layers * n_rows * d_model floats) and the layer's
 * normalised input is recomputed from the replaced stream, so that every
 * layer runs from caller-supplied inputs instead of its predecessor's
 * output.  Rows not listed keep the path's own values; list every row of
 * a sequence (and of its prefix) whose outputs are compared.  With capture
 * on, captured layer l + 1 is then layer l's output from the replaced
 * input.  n_rows = 0 switches it off.  Errors: S1_EINVAL (NULL, range,
 * duplicates), S1_ENOMEM, S1_EDEVICE.
 */
int s1_plan_set_layer_inputs(s1_plan* p, int32_t n_rows, const int32_t* rows, const float* d_src);

/*
 * Full-vocabulary language-model features (RFC #114, section 4, note under
 * the semantics table: token log-probabilities normalised over the whole
 * vocabulary, then across the candidates of the same question; RFC #114
 * comment "Plan: native OmniJev-4B v1.1": the log-softmax runs over every
 * row of the tied embedding, in fp32).  Target n reads the final hidden state
 * of packed token rows[n] (0-based index into the request's token_ids) and
 * scores token tokens[n] in [0, vocab):
 *   h = RMSNorm(x_final[rows[n]]; final_norm), z_v = h . E[v] for every v,
 *   logp[n] = z_tokens[n] - log sum_v exp(z_v).
 * Candidate c owns targets cand_offsets[c] .. cand_offsets[c+1]-1
 * (non-decreasing offsets, last <= n_targets) and scores the sum of their
 * logp (0 when it owns none); candidates with equal cand_group form one
 * question and cand_norm[c] = cand_logp[c] - log sum over its question of
 * exp(cand_logp).  Host arrays, copied during the call.
 */
typedef struct {
  int32_t n_targets;
  const int32_t* rows;
  const int32_t* tokens;
  int32_t n_cands;
  const int32_t* cand_offsets;   /* [n_cands + 1] */
  const int32_t* cand_group;     /* [n_cands] */
} s1_features;

/* Compute the features on every following s1_plan_run, after the readout, on
 * the same stream: d_logp[n_targets], d_cand_logp[n_cands] and
 * d_cand_norm[n_cands] are device memory (the candidate buffers may be NULL
 * when n_cands = 0).  f = NULL or n_targets = 0 switches them off.  The plan
 * allocates the feature workspace here (about 8 * 32 * ceil(vocab / 128)
 * bytes per 32 distinct rows plus 8 * d_model bytes per row).  bf16 models
 * need d_model % 128 == 0.  Errors: S1_EINVAL (ranges, offsets, NULL
 * outputs), S1_ENOMEM, S1_EDEVICE. */
int s1_plan_set_features(s1_plan* p, const s1_features* f, float* d_logp, float* d_cand_logp,
                         float* d_cand_norm);

/*
 * Per-kernel timing.  Runs the plan once like s1_plan_run, with a HIP event
 * recorded on hip_stream after every kernel launch, synchronises, and returns
 * the time between consecutive events summed per kernel family (names such as
 * "gemm_gate_up", "la_scan", "attention", "readout", "vocab_lse"), with the number of
 * launches.  out has room for max_out entries; *n_out receives the count.
 */
typedef struct {
  char name[32];
  int32_t launches;
  double total_us;
} s1_kernel_time;

int s1_plan_profile(s1_model* m, s1_plan* p, float* d_probs, s1_decision* d_out, void* hip_stream,
                    s1_kernel_time* out, int32_t max_out, int32_t* n_out);

#ifdef __cplusplus
}
#endif

#endif /* S1_H */
