// Host-side model and plan structures of the library (internal).
#pragma once

#include <hip/hip_runtime.h>

#include <string>
#include <vector>

#include "../../include/s1.h"
#include "kernels.h"

namespace s1 {

// Thread-local error reporting for the C ABI.
int set_error(int code, const std::string& msg);
std::string hip_msg(hipError_t e, const char* what);

// Device allocation, used by every allocating path of the library.  Test
// hook (forced from the host, no device fault involved): with
// S1_TEST_FAIL_ALLOC=n (or n@tag) in the environment, the n-th allocation
// counted from the last change of that variable's text fails as if the
// device were out of memory, so that every ENOMEM cleanup path can be
// exercised; a new tag restarts the count for the same n.
hipError_t dev_alloc(void** p, size_t bytes);
hipError_t dev_alloc_async(void** p, size_t bytes, hipStream_t s);

struct LayerW {
  bool full = false;
  int la_idx = -1, fa_idx = -1;
  float* attn_norm = nullptr;   // fp32 [d]
  float* ffn_norm = nullptr;    // fp32 [d]
  void* w_in = nullptr;         // LA: [q | k | v | g] rows; FA: [q | k | v], q/k rows RoPE-permuted
  int n_in = 0;
  void* w_o = nullptr;          // [d, heads * head_dim]
  int k_o = 0;
  void* w_gu = nullptr;         // gate/up interleaved in blocks of 32 rows, [2 * ffn_pad, d]
  void* w_gu_frag = nullptr;    // bf16: w_gu in fragment order, gate/up interleaved in blocks of 16
  void* w_down_frag = nullptr;  // bf16: w_down in fragment order (the down GEMM at many rows)
  void* w_o_frag = nullptr;     // bf16: w_o in fragment order (the out-projection at many rows)
  void* w_in_frag = nullptr;    // bf16: w_in in fragment order (the in-projection at many rows)
  int n_gu = 0;
  void* w_down = nullptr;       // [d, ffn]
  float* conv = nullptr;        // Gated DeltaNet: convolution taps fp32 [3 H 128][4]
};

// Kernel families timed by s1_plan_profile.
enum KernelClass {
  KC_EMBED = 0, KC_RMSNORM, KC_GEMM_LA_IN, KC_LA_SCAN, KC_GEMM_FA_QKV, KC_ATTENTION, KC_GEMM_O,
  KC_GEMM_GATE_UP, KC_GEMM_DOWN, KC_CAPTURE, KC_READOUT, KC_VOCAB_LSE, KC_FEATURES, KC_COUNT
};
const char* kernel_class_name(int c);

// Events recorded after each launch while profiling.
struct Profiler {
  std::vector<hipEvent_t> ev;
  std::vector<int> cls;
  int used = 0;
  bool overflow = false;
  ~Profiler();
  int reserve(int n);
  void begin(hipStream_t s);
  void mark(int c, hipStream_t s);
};

struct Model {
  s1_config cfg{};
  bool bf16 = true;
  size_t esz = 2;
  int device = 0;
  hipStream_t own_stream = nullptr;
  int ffn_pad = 0;
  int n_cu = 256;                // compute units of the device (set at load)
  int n_la = 0, n_fa = 0;

  void* embed = nullptr;        // [V, d]
  float* final_norm = nullptr;  // fp32 [d]
  std::vector<LayerW> layers;
  float2* rope = nullptr;       // [max_positions, head_dim / 2]

  // workspace, sized for cfg budgets
  float* x = nullptr;           // residual stream fp32 [T, d]
  void* xn = nullptr;           // normalised activations [T, d]; with the deferred norm: x rounded to bf16
  // Deferred RMSNorm (bf16 models): the pre-norm gains are folded into the
  // columns of the in-projection and gate/up weights, the GEMMs that update
  // x write xn = bf16(x) and rstd = 1 / rms of each row, and the consuming
  // GEMMs scale their accumulator rows by rstd.
  bool fold = false;
  float* rstd = nullptr;        // [T]
  float* ssq = nullptr;         // partial sums of squares [d / 32][ss_ld]
  int ss_ld = 0;
  unsigned int* tickets = nullptr;   // one per row block, zero between launches
  void* qkv = nullptr;          // LA: q | k | v; FA: q          [T, ld_qkv]
  int ld_qkv = 0;
  float* lg = nullptr;          // log decay gate fp32 [T, H]
  float* beta = nullptr;        // Gated DeltaNet write strength fp32 [T, H]
  void* qkv2 = nullptr;         // Gated DeltaNet: convolved, normalised q | k | v [T, ld_qkv]
  void* conv_hist = nullptr;    // [n_la][max_prefixes][3][3 H 128]: prefix pre-convolution rows
  float* gdn_ws = nullptr;      // W | Ut per (chunk, head)
  void* att = nullptr;          // mixer output [T, ld_att]
  int ld_att = 0;
  void* hbuf = nullptr;         // SwiGLU output [T, ffn]
  void* kc = nullptr;           // [n_fa][T][Hkv * hd]
  void* vc = nullptr;
  float* states = nullptr;      // [n_la][max_prefixes][H][dk][dv] fp32
  float* cstates = nullptr;     // chunk states of the chunk-parallel scan [max_chunks][H][dk][dv]
  float* gamma = nullptr;       // chunk log-decays [max_chunks][H]
  int max_chunks = 0;
  float* splitws = nullptr;     // split-K partials
  long long splitws_elems = 0;
  int split_max_rows = 0;

  // s1_prefill_decide's plan and result block, kept from call to call and
  // grown when a request needs more (no allocation in the steady state),
  // and its two timing events
  void* decide_dev = nullptr;
  size_t decide_bytes = 0;
  hipEvent_t decide_ev[2] = {nullptr, nullptr};
  // s1_prefill_decide replays a HIP graph when a batch repeats the previous
  // call's structure (everything but the token and option ids): the plan's
  // device layout in decide_dev is then the same, so only its contents are
  // uploaded again.  decide_sig is that structure (with the block's address
  // and size); the graph is captured on the second call of a structure.
  std::vector<long long> decide_sig;
  hipGraph_t decide_graph = nullptr;
  hipGraphExec_t decide_gexec = nullptr;
  bool decide_eager = false;    // this structure could not be captured
  void drop_decide_graph();
  Profiler* prof = nullptr;     // set only during s1_plan_profile's run
  Profiler* prof_store = nullptr;   // its events, kept between profiled runs
  std::vector<void*> allocs;
  ~Model();
  void* alloc(size_t bytes);    // throws std::bad_alloc on failure
};

struct PassPlan {
  int r0 = 0, T = 0;
  int n_seqs = 0;
  ScanSeq* scan = nullptr;      // device [n_seqs]
  AttnSeq* attn = nullptr;      // device [n_seqs]
  AttnBlock* blocks = nullptr;  // device [n_blocks]: keys split into pieces, prefixes shared
  int n_blocks = 0;
  AttnBlock* blocks_inv = nullptr;  // device: one workgroup per query block (row-invariant mode)
  int n_blocks_inv = 0;
  int32_t* comb_rows = nullptr; // device [n_comb]: rows whose pieces are merged
  int n_comb = 0;
  AttnPartials attn_part;       // partial results of the split attention
  int attn_rows = 0;            // queries per attention workgroup
  bool chunked = false;         // scan runs chunk-parallel (few chains)
  ScanSeq* chunks = nullptr;    // device [n_chunks]
  int n_chunks = 0;
  ChunkSeq* cseqs = nullptr;    // device [n_seqs]
  int max_nc = 0;               // most chunks of one sequence (INT_MAX: an empty one keeps a state)
  int max_len = 0;              // longest sequence of the pass
  GdnSeq* gseqs = nullptr;      // device [n_seqs]: sequences with their first chunk
  int32_t* row_seq = nullptr;   // device [T]: each row's sequence in gseqs
  int32_t* cap_rows = nullptr;  // device [n_cap]: rows captured in this pass
  int32_t* cap_dst = nullptr;   // device [n_cap]: index in the capture list
  int n_cap = 0;
  int32_t* inj_rows = nullptr;  // device [n_inj]: rows whose layer inputs are replaced in this pass
  int32_t* inj_idx = nullptr;   // device [n_inj]: index in the caller's row list
  int n_inj = 0;
};

// Host form of a feature request, validated: distinct rows (internal row
// order), per-target row index and token, candidate spans and the
// candidates of each group (ascending candidate index).
struct FeatHost {
  std::vector<int32_t> rows, t_ri, t_tok, cand_off, grp_off, grp_cands;
  int n_cands = 0;
  size_t meta_bytes() const;
  // copy the metadata to device memory dst (meta_bytes() bytes, 256-aligned)
  // and fill a with device pointers into it
  hipError_t upload(void* dst, FeatArgs* a, hipStream_t s) const;
};
// Validate and build a feature request.  rows[] index 0 .. n_rows-1 and are
// mapped through row_map when it is not NULL.
int build_features(int n_rows, const std::vector<int>* row_map, int V, int n_targets, const int32_t* rows,
                   const int32_t* tokens, int n_cands, const int32_t* cand_offsets, const int32_t* cand_group,
                   const char* who, FeatHost* out);

struct Plan {
  Model* m = nullptr;
  int T = 0, n_seqs = 0, Q = 0, total_opts = 0, max_k = 0;
  int n_passes = 0;
  PassPlan pass[2];
  int32_t* ids = nullptr;       // device [T] (internal row order)
  int32_t* pos = nullptr;       // device [T]
  int32_t* q_row = nullptr;     // device [Q]
  int32_t* opt_off = nullptr;   // device [Q + 1]
  int32_t* opt_ids = nullptr;   // device [sum K]
  uint8_t* q_type = nullptr;    // device [Q]
  std::vector<int> row_of;      // caller packed row -> internal row
  std::vector<int> pass_of_row; // internal row -> pass
  float* cap_out = nullptr;     // device [(n_layers + 1) * n_cap * d]
  int n_cap = 0;
  void* dev = nullptr;          // one device block for the arrays above
  bool dev_owned = true;        // false: the model's reusable block (s1_prefill_decide)
  void* extra = nullptr;        // extra_bytes requested at creation, after the arrays
  void* cap_dev = nullptr;      // device block for capture row lists
  // layer-input replacement (test hook): before layer l, row list entry j
  // takes inj_src[(l * n_inj + j) * d]
  const float* inj_src = nullptr;
  int n_inj = 0;
  void* inj_dev = nullptr;
  // HIP graph of the whole forward, replayed by s1_plan_run when enabled;
  // re-captured when the output or capture pointers change
  bool use_graph = false;
  // row-invariant mode: no K split in any GEMM and the chunk-parallel scan in
  // every pass, so a row's arithmetic does not depend on the rest of the batch
  bool invariant = false;
  // length-bucket plan: created for up to T tokens, Q questions and
  // bucket_opts options, refilled by update_bucket_plan between runs
  bool bucket = false;
  int bucket_opts = 0, real_T = 0, real_Q = 0;
  int opts_cap = 0;             // option ids the device slot holds (bucket plans)
  hipGraph_t graph = nullptr;
  hipGraphExec_t gexec = nullptr;
  float* g_probs = nullptr;
  void* g_dec = nullptr;
  float* g_cap = nullptr;
  const float* g_inj = nullptr;
  // full-vocabulary log-probability features, computed after the readout by
  // every run when set
  void* feat_dev = nullptr;     // metadata + workspace
  FeatArgs feat;
  void* feat_ws = nullptr;
  float* feat_logp = nullptr;
  float* feat_cand_lp = nullptr;
  float* feat_cand_norm = nullptr;
  void drop_graph();
  ~Plan();
};

int validate_config(const s1_config* c);
int validate_batch(const s1_config* c, const s1_batch* b);
int load_model(const s1_config* cfg, const s1_tensor* t, int n, hipStream_t s, Model** out);
// model_block: place the plan's device arrays (and extra_bytes more, at
// p->extra) in the model's reusable block instead of a new allocation.
int create_plan(Model* m, const s1_batch* b, Plan** out, int opts_capacity = 0, bool model_block = false,
                size_t extra_bytes = 0);
int create_bucket_plan(Model* m, int T_b, int Q_b, int O_b, Plan** out);
int update_bucket_plan(Plan* p, const s1_batch* b);
int run_plan(Model* m, Plan* p, float* d_probs, void* d_dec, hipStream_t s);
int set_capture(Plan* p, int n_rows, const int32_t* rows, float* d_hidden);
int set_layer_inputs(Plan* p, int n_rows, const int32_t* rows, const float* d_src);
int set_features(Plan* p, const s1_features* f, float* d_logp, float* d_cand_lp, float* d_cand_norm);
int run_plan_graph(Model* m, Plan* p, float* d_probs, void* d_dec, hipStream_t s);

}  // namespace s1
