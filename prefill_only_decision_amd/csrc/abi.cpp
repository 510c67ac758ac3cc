// C ABI of the library: argument validation, error reporting, entry points.
#include <algorithm>
#include <climits>
#include <chrono>
#include <cstdlib>
#include <mutex>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/s1.h"
#include "../../include/s1_kernels.h"
#include "internal.h"

namespace s1 {

namespace {
thread_local std::string g_err;
}

int set_error(int code, const std::string& msg) {
  g_err = msg;
  return code;
}

std::string hip_msg(hipError_t e, const char* what) {
  return std::string(what) + ": " + hipGetErrorString(e);
}

namespace {
std::mutex g_alloc_mu;
std::string g_alloc_env;   // the hook's value when the count started
long long g_alloc_count = 0;

// True when the S1_TEST_FAIL_ALLOC hook says this allocation fails.
bool injected_failure() {
  std::lock_guard<std::mutex> lock(g_alloc_mu);
  const char* e = std::getenv("S1_TEST_FAIL_ALLOC");
  const std::string v = e ? e : "";
  if (v != g_alloc_env) {
    g_alloc_env = v;
    g_alloc_count = 0;
  }
  if (v.empty()) return false;
  const long long n = std::atoll(v.c_str());
  return ++g_alloc_count == n;
}
}  // namespace

hipError_t dev_alloc(void** p, size_t bytes) {
  *p = nullptr;
  if (injected_failure()) return hipErrorOutOfMemory;
  const hipError_t e = hipMalloc(p, bytes);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    *p = nullptr;
  }
  return e;
}

hipError_t dev_alloc_async(void** p, size_t bytes, hipStream_t s) {
  *p = nullptr;
  if (injected_failure()) return hipErrorOutOfMemory;
  const hipError_t e = hipMallocAsync(p, bytes, s);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    *p = nullptr;
  }
  return e;
}

int validate_config(const s1_config* c) {
  if (!c) return set_error(S1_EINVAL, "config is NULL");
  if (c->dtype != S1_F32 && c->dtype != S1_BF16) return set_error(S1_EINVAL, "dtype must be S1_F32 or S1_BF16");
  if (c->n_layers < 1 || c->full_every < 1 || c->d_model < 1 || c->ffn < 1 || c->vocab < 1 ||
      c->la_heads < 1 || c->la_dk < 1 || c->la_dv < 1 || c->fa_q_heads < 1 || c->fa_kv_heads < 1 ||
      c->fa_head_dim < 1)
    return set_error(S1_EINVAL, "every shape field must be positive");
  if (c->fa_q_heads % c->fa_kv_heads) return set_error(S1_EINVAL, "fa_q_heads must be a multiple of fa_kv_heads");
  if (!(c->rope_base > 0.f) || !(c->rms_eps >= 0.f)) return set_error(S1_EINVAL, "rope_base must be > 0 and rms_eps >= 0");
  if (c->lora_rank < 0 || c->lora_rank > 64 || (c->lora_targets && c->lora_rank < 1))
    return set_error(S1_EINVAL, "lora_rank must be in [1, 64] when targets are set");
  if (c->lora_targets & ~0x7Fu) return set_error(S1_EINVAL, "unknown LoRA target bits");
  if (c->max_tokens < 1 || c->max_seqs < 1 || c->max_questions < 1 || c->max_options < 2 ||
      c->max_prefixes < 1 || c->max_positions < 1)
    return set_error(S1_EINVAL, "budgets must be positive (max_options >= 2)");
  if (c->max_tokens > (1LL << 30) || c->max_positions > (1LL << 24))
    return set_error(S1_EINVAL, "max_tokens or max_positions too large");
  if (c->la_kind != S1_LA_GLA && c->la_kind != S1_LA_GDN) return set_error(S1_EINVAL, "unknown la_kind");
  if (c->la_kind == S1_LA_GDN && c->dtype != S1_BF16)
    return set_error(S1_EINVAL, "Gated DeltaNet layers need a bf16 model");
  if (c->d_model + c->max_options > 16384)
    return set_error(S1_EINVAL, "d_model + max_options must not exceed 16384 (readout LDS)");
  if (c->dtype == S1_BF16) {
    if (c->la_dk != 128 || c->la_dv != 128 || c->fa_head_dim != 128)
      return set_error(S1_EINVAL, "bf16 models need la_dk = la_dv = fa_head_dim = 128");
    if (c->d_model % 64 || c->ffn % 64)
      return set_error(S1_EINVAL, "bf16 models need d_model and ffn to be multiples of 64");
  } else {
    if (c->fa_head_dim != 64 && c->fa_head_dim != 128)
      return set_error(S1_EINVAL, "fp32 models need fa_head_dim 64 or 128");
    if ((c->la_dk != 64 && c->la_dk != 128) || (c->la_dv != 64 && c->la_dv != 128))
      return set_error(S1_EINVAL, "fp32 models need la_dk and la_dv of 64 or 128");
    if (c->d_model % 4 || c->ffn % 4 || (c->la_heads * c->la_dv) % 4)
      return set_error(S1_EINVAL, "fp32 models need d_model, ffn, la_heads*la_dv multiples of 4");
  }
  return S1_OK;
}

int validate_batch(const s1_config* c, const s1_batch* b) {
  if (!c || !b) return set_error(S1_EINVAL, "config or batch is NULL");
  const int n = b->n_seqs;
  if (n < 0) return set_error(S1_EINVAL, "n_seqs < 0");
  if (n > c->max_seqs) return set_error(S1_EBUDGET, "more sequences than max_seqs");
  if (n > 0 && !b->cu_seqlens) return set_error(S1_EINVAL, "cu_seqlens is NULL");
  if (n > 0 && b->cu_seqlens[0] != 0) return set_error(S1_EINVAL, "cu_seqlens[0] must be 0");
  for (int i = 0; i < n; ++i)
    if (b->cu_seqlens[i + 1] < b->cu_seqlens[i]) return set_error(S1_EINVAL, "cu_seqlens must be non-decreasing");
  const long long T = n > 0 ? b->cu_seqlens[n] : 0;
  if (T > c->max_tokens) return set_error(S1_EBUDGET, "more tokens than max_tokens");
  if (T > 0 && !b->token_ids) return set_error(S1_EINVAL, "token_ids is NULL");
  for (long long t = 0; t < T; ++t)
    if (b->token_ids[t] < 0 || b->token_ids[t] >= c->vocab)
      return set_error(S1_EINVAL, "token id out of range at " + std::to_string(t));
  auto len = [&](int i) { return b->cu_seqlens[i + 1] - b->cu_seqlens[i]; };
  std::vector<char> is_prefix(n, 0);
  int n_prefix = 0;
  for (int i = 0; i < n; ++i) {
    const int p = b->prefix_of ? b->prefix_of[i] : -1;
    if (p < -1 || p >= n || p == i) return set_error(S1_EINVAL, "prefix_of[" + std::to_string(i) + "] is invalid");
    if (p >= 0) {
      if (b->prefix_of[p] != -1) return set_error(S1_EINVAL, "a prefix must not itself be a branch");
      if (!is_prefix[p]) ++n_prefix;
      is_prefix[p] = 1;
    }
    const long long positions = (long long)len(i) + (p >= 0 ? len(p) : 0);
    if (positions > c->max_positions) return set_error(S1_EBUDGET, "sequence longer than max_positions");
  }
  if (n_prefix > c->max_prefixes) return set_error(S1_EBUDGET, "more prefix sequences than max_prefixes");
  const int Q = b->n_questions;
  if (Q < 0) return set_error(S1_EINVAL, "n_questions < 0");
  if (Q > c->max_questions) return set_error(S1_EBUDGET, "more questions than max_questions");
  if (Q > 0 && (!b->q_seq || !b->q_marker || !b->q_type || !b->opt_offsets || !b->opt_ids))
    return set_error(S1_EINVAL, "question arrays are NULL");
  if (Q > 0 && b->opt_offsets[0] != 0) return set_error(S1_EINVAL, "opt_offsets[0] must be 0");
  for (int j = 0; j < Q; ++j) {
    const std::string at = " (question " + std::to_string(j) + ")";
    const int s = b->q_seq[j];
    if (s < 0 || s >= n) return set_error(S1_EINVAL, "q_seq out of range" + at);
    // a prefix is encoded once for its branches and answers nothing itself
    // (its questions belong to the branches that continue it)
    if (is_prefix[s]) return set_error(S1_EINVAL, "a question on a prefix sequence" + at);
    if (b->q_marker[j] < 0 || b->q_marker[j] >= len(s)) return set_error(S1_EINVAL, "marker outside its sequence" + at);
    if (b->q_type[j] > S1_NOUL) return set_error(S1_EINVAL, "unknown question type" + at);
    const int K = b->opt_offsets[j + 1] - b->opt_offsets[j];
    if (K < 2) return set_error(S1_EINVAL, "a question needs at least 2 options" + at);
    if (b->q_type[j] == S1_NOUL && K != 2) return set_error(S1_EINVAL, "a noul question needs exactly 2 options" + at);
    if (K > c->max_options) return set_error(S1_EBUDGET, "more options than max_options" + at);
    for (int k = b->opt_offsets[j]; k < b->opt_offsets[j + 1]; ++k)
      if (b->opt_ids[k] < 0 || b->opt_ids[k] >= c->vocab) return set_error(S1_EINVAL, "option id out of range" + at);
  }
  return S1_OK;
}

}  // namespace s1

using namespace s1;

struct s1_model {
  Model* m;
};
struct s1_plan {
  Plan* p;
  s1_model* owner;
};

extern "C" {

const char* s1_last_error(void) { return g_err.c_str(); }

int s1_validate(const s1_config* cfg, const s1_batch* b) {
  int rc = validate_config(cfg);
  if (rc) return rc;
  return validate_batch(cfg, b);
}

int s1_load_weights(const s1_config* cfg, const s1_tensor* tensors, int32_t n_tensors,
                    void* hip_stream, s1_model** out) {
  if (!out) return set_error(S1_EINVAL, "out is NULL");
  Model* m = nullptr;
  const int rc = load_model(cfg, tensors, n_tensors, static_cast<hipStream_t>(hip_stream), &m);
  if (rc) return rc;
  s1_model* h = new (std::nothrow) s1_model{m};
  if (!h) {
    delete m;
    return set_error(S1_ENOMEM, "host allocation failed");
  }
  *out = h;
  g_err.clear();
  return S1_OK;
}

void s1_free(s1_model* m) {
  if (!m) return;
  (void)hipDeviceSynchronize();
  delete m->m;
  delete m;
}

int s1_plan_create(s1_model* m, const s1_batch* b, s1_plan** out) {
  if (!m || !out) return set_error(S1_EINVAL, "model or out is NULL");
  Plan* p = nullptr;
  const int rc = create_plan(m->m, b, &p);
  if (rc) return rc;
  s1_plan* h = new (std::nothrow) s1_plan{p, m};
  if (!h) {
    delete p;
    return set_error(S1_ENOMEM, "host allocation failed");
  }
  *out = h;
  return S1_OK;
}

int s1_plan_create_bucket(s1_model* m, int32_t max_tokens, int32_t max_questions, int32_t max_options,
                          s1_plan** out) {
  if (!m || !out) return set_error(S1_EINVAL, "model or out is NULL");
  Plan* p = nullptr;
  const int rc = create_bucket_plan(m->m, max_tokens, max_questions, max_options, &p);
  if (rc) return rc;
  s1_plan* h = new (std::nothrow) s1_plan{p, m};
  if (!h) {
    delete p;
    return set_error(S1_ENOMEM, "host allocation failed");
  }
  *out = h;
  return S1_OK;
}

int s1_plan_update(s1_plan* p, const s1_batch* b) {
  if (!p || !b) return set_error(S1_EINVAL, "plan or batch is NULL");
  return update_bucket_plan(p->p, b);
}

int32_t s1_plan_questions(const s1_plan* p) { return p ? p->p->Q : 0; }

int64_t s1_plan_options(const s1_plan* p) { return p ? p->p->total_opts : 0; }

void s1_plan_free(s1_plan* p) {
  if (!p) return;
  delete p->p;
  delete p;
}

int64_t s1_plan_tokens(const s1_plan* p) { return p ? p->p->T : 0; }

int s1_plan_set_capture(s1_plan* p, int32_t n_rows, const int32_t* rows, float* d_hidden) {
  if (!p) return set_error(S1_EINVAL, "plan is NULL");
  return set_capture(p->p, n_rows, rows, d_hidden);
}

int s1_plan_set_layer_inputs(s1_plan* p, int32_t n_rows, const int32_t* rows, const float* d_src) {
  if (!p) return set_error(S1_EINVAL, "plan is NULL");
  return set_layer_inputs(p->p, n_rows, rows, d_src);
}

int s1_plan_set_features(s1_plan* p, const s1_features* f, float* d_logp, float* d_cand_logp,
                         float* d_cand_norm) {
  if (!p) return set_error(S1_EINVAL, "plan is NULL");
  return set_features(p->p, f, d_logp, d_cand_logp, d_cand_norm);
}

int s1_plan_run(s1_model* m, s1_plan* p, float* d_probs, s1_decision* d_out, void* hip_stream) {
  if (!m || !p) return set_error(S1_EINVAL, "model or plan is NULL");
  if (p->owner != m) return set_error(S1_EINVAL, "plan belongs to another model");
  if (p->p->Q > 0 && (!d_probs || !d_out)) return set_error(S1_EINVAL, "output buffers are NULL");
  hipStream_t s = hip_stream ? static_cast<hipStream_t>(hip_stream) : m->m->own_stream;
  const int rc = p->p->use_graph ? run_plan_graph(m->m, p->p, d_probs, d_out, s)
                                 : run_plan(m->m, p->p, d_probs, d_out, s);
  if (rc) (void)hipStreamSynchronize(s);
  return rc;
}

int s1_plan_set_invariant(s1_plan* p, int32_t enable) {
  if (!p) return set_error(S1_EINVAL, "plan is NULL");
  p->p->invariant = enable != 0;
  p->p->drop_graph();
  return S1_OK;
}

int s1_plan_set_graph(s1_plan* p, int32_t enable) {
  if (!p) return set_error(S1_EINVAL, "plan is NULL");
  p->p->use_graph = enable != 0;
  if (!enable) p->p->drop_graph();
  return S1_OK;
}

int s1_plan_profile(s1_model* m, s1_plan* p, float* d_probs, s1_decision* d_out, void* hip_stream,
                    s1_kernel_time* out, int32_t max_out, int32_t* n_out) {
  if (!m || !p || !out || !n_out || max_out < 1) return set_error(S1_EINVAL, "NULL argument");
  if (p->owner != m) return set_error(S1_EINVAL, "plan belongs to another model");
  Model* mm = m->m;
  hipStream_t s = hip_stream ? static_cast<hipStream_t>(hip_stream) : mm->own_stream;
  if (!mm->prof_store) mm->prof_store = new (std::nothrow) Profiler();
  if (!mm->prof_store || mm->prof_store->reserve(16 * mm->cfg.n_layers + 64) != S1_OK)
    return set_error(S1_EDEVICE, "profiler events");
  // events are recorded during this run only (other runs, graph captures
  // included, record none)
  Profiler* pr = mm->prof_store;
  mm->prof = pr;
  int rc = run_plan(mm, p->p, d_probs, d_out, s);
  mm->prof = nullptr;
  const hipError_t se = hipStreamSynchronize(s);
  if (rc) return rc;
  if (se != hipSuccess) return set_error(S1_EDEVICE, hip_msg(se, "profiled run"));
  if (pr->overflow) return set_error(S1_EDEVICE, "profiler ran out of events");
  double tot[KC_COUNT] = {0};
  int cnt[KC_COUNT] = {0};
  for (int i = 1; i < pr->used; ++i) {
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, pr->ev[i - 1], pr->ev[i]) != hipSuccess) return set_error(S1_EDEVICE, "event time");
    const int c = pr->cls[i];
    if (c >= 0 && c < KC_COUNT) {
      tot[c] += ms * 1000.0;
      cnt[c] += 1;
    }
  }
  int k = 0;
  for (int c = 0; c < KC_COUNT && k < max_out; ++c) {
    if (!cnt[c]) continue;
    std::memset(out[k].name, 0, sizeof(out[k].name));
    std::strncpy(out[k].name, kernel_class_name(c), sizeof(out[k].name) - 1);
    out[k].launches = cnt[c];
    out[k].total_us = tot[c];
    ++k;
  }
  *n_out = k;
  return S1_OK;
}

// Everything of a batch that decides its plan's device layout and launch
// arguments: sequence lengths, prefixes, questions (sequence, type, marker)
// and option counts.  Token and option ids are contents.
static std::vector<long long> decide_signature(const s1_batch* b) {
  std::vector<long long> v;
  const int n = b->n_seqs, Q = b->n_questions;
  v.push_back(n);
  for (int i = 0; i <= n; ++i) v.push_back(b->cu_seqlens[i]);
  for (int i = 0; i < n; ++i) v.push_back(b->prefix_of ? b->prefix_of[i] : -1);
  v.push_back(Q);
  for (int j = 0; j < Q; ++j) {
    v.push_back(b->q_seq[j]);
    v.push_back(b->q_type[j]);
    v.push_back(b->q_marker[j]);
    v.push_back(b->opt_offsets[j + 1] - b->opt_offsets[j]);
  }
  return v;
}

int s1_prefill_decide(s1_model* m, const s1_batch* b, float* probs, s1_decision* out,
                      s1_timing* timing, void* hip_stream) {
  const auto t0 = std::chrono::steady_clock::now();
  if (!m) return set_error(S1_EINVAL, "model is NULL");
  int rc = validate_batch(&m->m->cfg, b);
  if (rc) return rc;
  if (b->n_questions > 0 && (!probs || !out)) return set_error(S1_EINVAL, "output arrays are NULL");
  Model* mm = m->m;
  hipStream_t s = hip_stream ? static_cast<hipStream_t>(hip_stream) : mm->own_stream;
  for (hipEvent_t& e : mm->decide_ev)
    if (!e && hipEventCreate(&e) != hipSuccess) {
      e = nullptr;
      return set_error(S1_EDEVICE, "event creation failed");
    }
  const int nopt = b->n_questions > 0 ? b->opt_offsets[b->n_questions] : 0;
  const size_t pbytes = ((size_t)nopt * sizeof(float) + 15) / 16 * 16;
  // the plan and the results share the model's reusable device block
  Plan* p = nullptr;
  rc = create_plan(mm, b, &p, 0, true, pbytes + (size_t)b->n_questions * sizeof(s1_decision) + 16);
  if (rc) return rc;
  const int Q = p->Q;
  auto fail = [&](int code, const std::string& msg) {
    (void)hipStreamSynchronize(s);
    delete p;
    return msg.empty() ? code : set_error(code, msg);
  };
  float* dprobs = static_cast<float*>(p->extra);
  s1_decision* ddec = reinterpret_cast<s1_decision*>(static_cast<char*>(p->extra) + pbytes);
  // the batch's structure: a repeat of the previous call's runs as a HIP graph
  std::vector<long long> sig = decide_signature(b);
  sig.push_back(reinterpret_cast<long long>(mm->decide_dev));
  sig.push_back((long long)mm->decide_bytes);
  const bool repeat = sig == mm->decide_sig;
  if (!repeat) {
    mm->drop_decide_graph();
    mm->decide_sig = sig;
    mm->decide_eager = false;
  }
  if (hipEventRecord(mm->decide_ev[0], s) != hipSuccess) return fail(S1_EDEVICE, "event record failed");
  if (repeat && !mm->decide_gexec && !mm->decide_eager) {   // second call of this structure: capture it
    // a stream that cannot be captured (or a failed instantiation) leaves
    // this structure on eager launches
    hipGraph_t g = nullptr;
    hipGraphExec_t x = nullptr;
    hipError_t e = hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal);
    if (e == hipSuccess) {
      rc = run_plan(mm, p, dprobs, ddec, s);
      e = hipStreamEndCapture(s, &g);
      if (rc) {
        if (g) (void)hipGraphDestroy(g);
        mm->decide_sig.clear();
        return fail(rc, "");
      }
      if (e == hipSuccess) e = hipGraphInstantiate(&x, g, nullptr, nullptr, 0);
    }
    if (e == hipSuccess) {
      mm->decide_graph = g;
      mm->decide_gexec = x;
    } else {
      (void)hipGetLastError();
      if (g) (void)hipGraphDestroy(g);
      mm->decide_eager = true;
    }
  }
  if (mm->decide_gexec) {
    const hipError_t e = hipGraphLaunch(mm->decide_gexec, s);
    if (e != hipSuccess) {
      mm->drop_decide_graph();
      mm->decide_sig.clear();
      return fail(S1_EDEVICE, hip_msg(e, "graph launch"));
    }
  } else {
    rc = run_plan(mm, p, dprobs, ddec, s);
    if (rc) return fail(rc, "");
  }
  if (hipEventRecord(mm->decide_ev[1], s) != hipSuccess) return fail(S1_EDEVICE, "event record failed");
  if (Q > 0) {
    if (hipMemcpyAsync(probs, dprobs, (size_t)nopt * 4, hipMemcpyDeviceToHost, s) != hipSuccess ||
        hipMemcpyAsync(out, ddec, (size_t)Q * sizeof(s1_decision), hipMemcpyDeviceToHost, s) != hipSuccess)
      return fail(S1_EDEVICE, "copy results to host failed");
  }
  const hipError_t se = hipStreamSynchronize(s);
  if (se != hipSuccess) return fail(S1_EDEVICE, hip_msg(se, "device work failed"));
  float ms = 0.f;
  const double dev_us = hipEventElapsedTime(&ms, mm->decide_ev[0], mm->decide_ev[1]) == hipSuccess ? ms * 1000.0 : 0.0;
  const long long T = p->T;
  delete p;
  if (timing) {
    timing->tokens_processed = T;
    timing->device_us = dev_us;
    timing->wall_us =
        std::chrono::duration<double, std::micro>(std::chrono::steady_clock::now() - t0).count();
  }
  return S1_OK;
}

// ----------------------------------------------------------- kernel level
static hipStream_t strm(void* s) { return static_cast<hipStream_t>(s); }
static int dev_status(hipError_t e, const char* what) {
  return e == hipSuccess ? S1_OK : set_error(S1_EDEVICE, hip_msg(e, what));
}

namespace {
int gemm_entry(int32_t dtype, const void* A, const void* W, float* C, int32_t M, int32_t N, int32_t K,
               int32_t split_k, int32_t tile_cfg, void* hip_stream) {
  const bool bf16 = dtype == S1_BF16;
  if ((dtype != S1_BF16 && dtype != S1_F32) || M < 0 || N < 0 || K < 1 || split_k < 1 ||
      K % (bf16 ? 8 : 4) || (split_k > 1 && N % 4) || !A || !W || !C || tile_cfg < GEMM_AUTO ||
      tile_cfg >= gemm_tile_configs())
    return set_error(S1_EINVAL, "s1k_gemm: unsupported arguments");
  GemmArgs g{};
  g.A = A;
  g.W = W;
  g.M = M;
  g.N = N;
  g.K = K;
  g.lda = K;
  g.ldw = K;
  g.out0 = C;
  g.ld0 = N;
  float* ws = nullptr;
  if (split_k > 1) {
    if (dev_alloc_async(reinterpret_cast<void**>(&ws), (size_t)split_k * M * N * sizeof(float) + 256, strm(hip_stream)) != hipSuccess)
      return set_error(S1_ENOMEM, "s1k_gemm: workspace allocation failed");
  }
  const hipError_t e = launch_gemm(bf16, EPI_F32, g, split_k, ws, strm(hip_stream), tile_cfg);
  if (ws) (void)hipFreeAsync(ws, strm(hip_stream));
  return dev_status(e, "s1k_gemm");
}
}  // namespace

int s1k_gemm(int32_t dtype, const void* A, const void* W, float* C, int32_t M, int32_t N, int32_t K,
             int32_t split_k, void* hip_stream) {
  return gemm_entry(dtype, A, W, C, M, N, K, split_k, GEMM_AUTO, hip_stream);
}

int s1k_gemm_cfg(int32_t dtype, const void* A, const void* W, float* C, int32_t M, int32_t N, int32_t K,
                 int32_t split_k, int32_t tile_cfg, void* hip_stream) {
  if (tile_cfg < 0) return set_error(S1_EINVAL, "s1k_gemm_cfg: tile_cfg must be >= 0");
  return gemm_entry(dtype, A, W, C, M, N, K, split_k, tile_cfg, hip_stream);
}

int s1k_gemm_resid_norm(const void* A, const void* W, float* x, int32_t M, int32_t N, int32_t K,
                        int32_t split_k, int32_t tile_cfg, float eps, void* hb, float* rs, int32_t* form,
                        void* hip_stream) {
  if (M < 0 || N < 1 || N > 8192 || K < 8 || K % 8 || split_k < 1 || (split_k > 1 && (N % 4 || K % 64)) || !A ||
      !W || !x || !hb || !rs || tile_cfg < GEMM_AUTO || tile_cfg >= gemm_tile_configs())
    return set_error(S1_EINVAL, "s1k_gemm_resid_norm: unsupported arguments");
  if (M == 0) return S1_OK;
  const hipStream_t s = strm(hip_stream);
  const int ld = (M + 31) / 32 * 32, nt = (M / 32 + 2 + 3) / 4 * 4;   // 16-byte aligned split workspace
  const size_t parts = (size_t)((N + 31) / 32) * ld * sizeof(float);
  const size_t split_bytes = split_k > 1 ? (size_t)split_k * M * N * sizeof(float) : 0;
  char* ws = nullptr;
  if (dev_alloc_async(reinterpret_cast<void**>(&ws), parts + nt * sizeof(unsigned) + split_bytes + 256, s) !=
      hipSuccess)
    return set_error(S1_ENOMEM, "s1k_gemm_resid_norm: workspace allocation failed");
  GemmArgs g{};
  g.A = A;
  g.W = W;
  g.M = M;
  g.N = N;
  g.K = K;
  g.lda = K;
  g.ldw = K;
  g.out0 = x;
  g.ld0 = N;
  g.norm_out = hb;
  g.norm_eps = eps;
  g.rs_out = rs;
  g.ss_parts = reinterpret_cast<float*>(ws);
  g.ss_ld = ld;
  g.tickets = reinterpret_cast<unsigned*>(ws + parts);
  float* sws = split_k > 1 ? reinterpret_cast<float*>(ws + parts + nt * sizeof(unsigned)) : nullptr;
  hipError_t e = hipMemsetAsync(g.tickets, 0, nt * sizeof(unsigned), s);
  int normed = NORM_NONE;
  if (e == hipSuccess) e = launch_gemm(true, EPI_RESID, g, split_k, sws, s, tile_cfg, &normed);
  (void)hipFreeAsync(ws, s);
  if (e == hipSuccess && normed == NORM_NONE) return set_error(S1_EINVAL, "s1k_gemm_resid_norm: shape not supported");
  if (e == hipSuccess && form) *form = normed;
  return dev_status(e, "s1k_gemm_resid_norm");
}

int s1k_gemm_tile_configs(void) { return gemm_tile_configs(); }

int s1k_mfma_peak(const void* seed, int32_t blocks, int32_t iters, float* out, void* hip_stream) {
  if (!seed || !out || blocks < 1 || iters < 1) return set_error(S1_EINVAL, "s1k_mfma_peak: unsupported arguments");
  return dev_status(launch_mfma_peak(seed, blocks, iters, out, strm(hip_stream)), "s1k_mfma_peak");
}

int s1k_stream_copy(const void* src, void* dst, int64_t bytes, void* hip_stream) {
  if (!src || !dst || bytes < 0 || bytes % 16) return set_error(S1_EINVAL, "s1k_stream_copy: unsupported arguments");
  return dev_status(launch_stream_copy(src, dst, bytes, strm(hip_stream)), "s1k_stream_copy");
}

int s1k_stream_read(const void* src, int64_t bytes, void* sink, void* hip_stream) {
  if (!src || !sink || bytes < 0 || bytes % 16) return set_error(S1_EINVAL, "s1k_stream_read: unsupported arguments");
  return dev_status(launch_stream_read(src, bytes, sink, strm(hip_stream)), "s1k_stream_read");
}

int64_t s1k_frag_bytes(int32_t N, int32_t K) {
  if (N < 1 || K < 16 || K % 16) return 0;
  return (int64_t)frag_bytes(N, K);
}

int s1k_frag_pack(const void* W, int32_t N, int32_t K, int32_t gate_up16, void* out, void* hip_stream) {
  if (!W || !out || N < 1 || K < 16 || K % 16 || (gate_up16 && N % 64))
    return set_error(S1_EINVAL, "s1k_frag_pack: unsupported arguments");
  return dev_status(launch_frag_pack(W, N, K, K, gate_up16 != 0, out, strm(hip_stream)), "s1k_frag_pack");
}

int s1k_gemm_wfrag(const void* A, const void* Wfrag, void* out, int32_t M, int32_t N, int32_t K,
                   int32_t swiglu, int32_t tile, void* hip_stream) {
  if (!A || !Wfrag || !out || M < 0 || N < 1 || K < 64 || K % 64 || (swiglu && N % 64) || tile < 1 || tile > 4)
    return set_error(S1_EINVAL, "s1k_gemm_wfrag: unsupported arguments");
  GemmArgs g{};
  g.A = A;
  g.W = Wfrag;
  g.M = M;
  g.N = N;
  g.K = K;
  g.lda = K;
  g.ldw = K;
  g.out0 = out;
  g.ld0 = swiglu ? N / 2 : N;
  g.n_valid = N / 2;
  return dev_status(launch_gemm_wd(swiglu ? EPI_SWIGLU : EPI_F32, g, tile, strm(hip_stream)), "s1k_gemm_wfrag");
}

int s1k_rmsnorm(int32_t dtype, const float* x, const float* w, void* out, int32_t T, int32_t d, float eps,
                void* hip_stream) {
  if ((dtype != S1_BF16 && dtype != S1_F32) || T < 0 || d < 4 || d % 4 || !x || !w || !out)
    return set_error(S1_EINVAL, "s1k_rmsnorm: unsupported arguments");
  return dev_status(launch_rmsnorm(dtype == S1_BF16, x, w, out, T, d, eps, strm(hip_stream)), "s1k_rmsnorm");
}

int s1k_embed(int32_t dtype, const int32_t* ids, const void* E, float* x, int32_t T, int32_t d,
              void* hip_stream) {
  if ((dtype != S1_BF16 && dtype != S1_F32) || T < 0 || d < 4 || d % 4 || !ids || !E || !x)
    return set_error(S1_EINVAL, "s1k_embed: unsupported arguments");
  return dev_status(launch_embed(dtype == S1_BF16, ids, E, x, T, d, strm(hip_stream)), "s1k_embed");
}

int s1k_lora_merge(int32_t dtype, const void* W, const void* A, const void* B, void* out, int32_t out_dim,
                   int32_t in_dim, int32_t rank, float scale, void* hip_stream) {
  if ((dtype != S1_BF16 && dtype != S1_F32) || out_dim < 0 || in_dim < 0 || !W || !out ||
      ((A == nullptr) != (B == nullptr)) || (A && (rank < 1 || rank > 64)))
    return set_error(S1_EINVAL, "s1k_lora_merge: unsupported arguments");
  return dev_status(launch_merge(dtype == S1_BF16, W, A, B, out, out_dim, in_dim, rank, scale, nullptr,
                                 strm(hip_stream)),
                    "s1k_lora_merge");
}

int s1k_la_scan(int32_t dtype, const void* q, const void* k, const void* v, int32_t ld_qkv,
                const float* log_g, void* o, int32_t T, int32_t H, int32_t dk, int32_t dv, int32_t n_seqs,
                const int32_t* cu_seqlens, const float* s_init, float* s_final, void* hip_stream) {
  const bool bf16 = dtype == S1_BF16;
  if ((dtype != S1_BF16 && dtype != S1_F32) || n_seqs < 0 || H < 1 || !cu_seqlens || !q || !k || !v ||
      !log_g || !o || (bf16 && (dk != 128 || dv != 128)) ||
      (!bf16 && ((dk != 64 && dk != 128) || (dv != 64 && dv != 128))))
    return set_error(S1_EINVAL, "s1k_la_scan: unsupported arguments");
  if (n_seqs > 0 && (cu_seqlens[0] != 0 || cu_seqlens[n_seqs] > T))
    return set_error(S1_EINVAL, "s1k_la_scan: cu_seqlens out of range");
  if (n_seqs == 0) return S1_OK;
  // one state buffer: initial states copied into slots 0 .. n_seqs - 1, final
  // states written to slots n_seqs .. 2 n_seqs - 1 (the fp32 short-sequence
  // kernel writes a final state while other workgroups read the initial one)
  std::vector<ScanSeq> seqs(n_seqs);
  int max_len = 0;
  for (int i = 0; i < n_seqs; ++i) {
    if (cu_seqlens[i + 1] < cu_seqlens[i]) return set_error(S1_EINVAL, "s1k_la_scan: cu_seqlens decreasing");
    seqs[i] = {cu_seqlens[i], cu_seqlens[i + 1] - cu_seqlens[i], s_init ? i : -1, s_final ? n_seqs + i : -1};
    max_len = std::max(max_len, seqs[i].len);
  }
  const size_t sbytes = (size_t)n_seqs * H * dk * dv * sizeof(float);
  float* st = nullptr;
  ScanSeq* dseq = nullptr;
  hipStream_t s = strm(hip_stream);
  if (dev_alloc(reinterpret_cast<void**>(&st), 2 * sbytes) != hipSuccess ||
      dev_alloc(reinterpret_cast<void**>(&dseq), seqs.size() * sizeof(ScanSeq)) != hipSuccess) {
    (void)hipGetLastError();
    if (st) (void)hipFree(st);
    return set_error(S1_ENOMEM, "s1k_la_scan: allocation failed");
  }
  hipError_t e = hipMemcpy(dseq, seqs.data(), seqs.size() * sizeof(ScanSeq), hipMemcpyHostToDevice);
  if (e == hipSuccess && s_init) e = hipMemcpyAsync(st, s_init, sbytes, hipMemcpyDeviceToDevice, s);
  if (e == hipSuccess)
    e = launch_scan(bf16, q, k, v, ld_qkv, log_g, H, o, H * dv, dseq, n_seqs, st, H, dk, dv, s, max_len);
  if (e == hipSuccess && s_final)
    e = hipMemcpyAsync(s_final, reinterpret_cast<char*>(st) + sbytes, sbytes, hipMemcpyDeviceToDevice, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  (void)hipFree(st);
  (void)hipFree(dseq);
  return dev_status(e, "s1k_la_scan");
}

int s1k_la_scan_chunked(const void* q, const void* k, const void* v, int32_t ld_qkv, const float* log_g, void* o,
                        int32_t T, int32_t H, int32_t n_seqs, const int32_t* cu_seqlens, const float* s_init,
                        float* s_final, void* hip_stream) {
  if (n_seqs < 0 || H < 1 || !cu_seqlens || !q || !k || !v || !log_g || !o)
    return set_error(S1_EINVAL, "s1k_la_scan_chunked: unsupported arguments");
  if (n_seqs == 0) return S1_OK;
  if (cu_seqlens[0] != 0 || cu_seqlens[n_seqs] > T) return set_error(S1_EINVAL, "s1k_la_scan_chunked: cu_seqlens out of range");
  std::vector<ScanSeq> chunks;
  std::vector<ChunkSeq> cseqs;
  int max_nc = 0;
  for (int i = 0; i < n_seqs; ++i) {
    const int len = cu_seqlens[i + 1] - cu_seqlens[i];
    if (len < 0) return set_error(S1_EINVAL, "s1k_la_scan_chunked: cu_seqlens decreasing");
    // final states go to slots of their own (n_seqs + i): in the two-launch
    // schedule one workgroup writes a sequence's final state while others
    // still read its initial one
    ChunkSeq cs{(int)chunks.size(), 0, s_init ? i : -1, s_final ? n_seqs + i : -1};
    for (int t0 = 0; t0 < len; t0 += 64) {
      const int id = (int)chunks.size();
      chunks.push_back({cu_seqlens[i] + t0, std::min(64, len - t0), id, id});
      ++cs.nc;
    }
    max_nc = std::max(max_nc, cs.nc == 0 && cs.s_out >= 0 ? INT_MAX : cs.nc);
    cseqs.push_back(cs);
  }
  const size_t E = 128 * 128;
  const size_t nc = std::max<size_t>(1, chunks.size());
  const size_t bytes = nc * H * E * 4 + nc * H * 4 + (size_t)2 * n_seqs * H * E * 4 +
                       nc * sizeof(ScanSeq) + cseqs.size() * sizeof(ChunkSeq) + 1024;
  char* buf = nullptr;
  hipStream_t s = strm(hip_stream);
  if (dev_alloc(reinterpret_cast<void**>(&buf), bytes) != hipSuccess) {
    (void)hipGetLastError();
    return set_error(S1_ENOMEM, "s1k_la_scan_chunked: allocation failed");
  }
  float* cst = reinterpret_cast<float*>(buf);
  float* gam = cst + nc * H * E;
  float* st = gam + nc * H + 64;
  st = reinterpret_cast<float*>((reinterpret_cast<uintptr_t>(st) + 255) & ~uintptr_t(255));
  ScanSeq* dch = reinterpret_cast<ScanSeq*>(st + (size_t)2 * n_seqs * H * E);
  ChunkSeq* dcs = reinterpret_cast<ChunkSeq*>(dch + nc);
  hipError_t e = hipMemcpy(dch, chunks.data(), chunks.size() * sizeof(ScanSeq), hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemcpy(dcs, cseqs.data(), cseqs.size() * sizeof(ChunkSeq), hipMemcpyHostToDevice);
  const size_t sbytes = (size_t)n_seqs * H * E * 4;
  if (e == hipSuccess && s_init) e = hipMemcpyAsync(st, s_init, sbytes, hipMemcpyDeviceToDevice, s);
  if (e == hipSuccess)
    e = launch_scan_chunked(q, k, v, ld_qkv, log_g, H, o, H * 128, dch, (int)chunks.size(), dcs, n_seqs, cst,
                            gam, st, H, s, max_nc);
  if (e == hipSuccess && s_final)
    e = hipMemcpyAsync(s_final, st + (size_t)n_seqs * H * E, sbytes, hipMemcpyDeviceToDevice, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  (void)hipFree(buf);
  return dev_status(e, "s1k_la_scan_chunked");
}

int s1k_gdn_scan(const void* q, const void* k, const void* v, int32_t ld_qkv, const float* log_g, const float* beta,
                 void* o, int32_t T, int32_t H, int32_t n_seqs, const int32_t* cu_seqlens, const float* s_init,
                 float* s_final, void* hip_stream) {
  if (n_seqs < 0 || H < 1 || T < 0 || !cu_seqlens || !q || !k || !v || !log_g || !beta || !o)
    return set_error(S1_EINVAL, "s1k_gdn_scan: unsupported arguments");
  if (n_seqs > 0 && (cu_seqlens[0] != 0 || cu_seqlens[n_seqs] > T))
    return set_error(S1_EINVAL, "s1k_gdn_scan: cu_seqlens out of range");
  if (n_seqs == 0) return S1_OK;
  std::vector<ScanSeq> chunks;
  std::vector<GdnSeq> seqs(n_seqs);
  for (int i = 0; i < n_seqs; ++i) {
    const int a = cu_seqlens[i], len = cu_seqlens[i + 1] - a;
    if (len < 0) return set_error(S1_EINVAL, "s1k_gdn_scan: cu_seqlens decreasing");
    seqs[i] = {a, len, (int)chunks.size(), s_init ? i : -1, s_final ? i : -1};
    for (int t0 = 0; t0 < len; t0 += 64) chunks.push_back({a + t0, std::min(64, len - t0), -1, -1});
  }
  if (chunks.empty()) return S1_OK;
  const size_t sbytes = (size_t)n_seqs * H * 128 * 128 * sizeof(float);
  const size_t wbytes = gdn_ws_bytes((int)chunks.size(), H);
  const size_t b1 = chunks.size() * sizeof(ScanSeq), b2 = seqs.size() * sizeof(GdnSeq);
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  char* dm = nullptr;
  if (dev_alloc(reinterpret_cast<void**>(&dm), al(sbytes) + al(wbytes) + al(b1) + al(b2)) != hipSuccess) {
    (void)hipGetLastError();
    return set_error(S1_ENOMEM, "s1k_gdn_scan: allocation failed");
  }
  float* st = reinterpret_cast<float*>(dm);
  float* ws = reinterpret_cast<float*>(dm + al(sbytes));
  auto* dch = reinterpret_cast<ScanSeq*>(dm + al(sbytes) + al(wbytes));
  auto* dsq = reinterpret_cast<GdnSeq*>(dm + al(sbytes) + al(wbytes) + al(b1));
  hipStream_t s = strm(hip_stream);
  hipError_t e = hipMemcpy(dch, chunks.data(), b1, hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemcpy(dsq, seqs.data(), b2, hipMemcpyHostToDevice);
  if (e == hipSuccess && s_init) e = hipMemcpyAsync(st, s_init, sbytes, hipMemcpyDeviceToDevice, s);
  if (e == hipSuccess)
    e = launch_gdn_scan(q, k, v, ld_qkv, log_g, beta, H, o, H * 128, dch, (int)chunks.size(), dsq, n_seqs, st, H,
                        ws, s);
  if (e == hipSuccess && s_final) e = hipMemcpyAsync(s_final, st, sbytes, hipMemcpyDeviceToDevice, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  (void)hipFree(dm);
  return dev_status(e, "s1k_gdn_scan");
}

int s1k_attention(int32_t dtype, const void* q, const void* k, const void* v, void* o, int32_t Hq, int32_t Hkv,
                  int32_t hd, int32_t n_seqs, const int32_t* q_row0, const int32_t* q_len,
                  const int32_t* kv_row0, const int32_t* kv_pre_row0, const int32_t* kv_pre_len,
                  int32_t block_rows, int32_t piece, void* hip_stream) {
  const bool bf16 = dtype == S1_BF16;
  if ((dtype != S1_BF16 && dtype != S1_F32) || Hq < 1 || Hkv < 1 || Hq % Hkv || n_seqs < 0 || !q || !k ||
      !v || !o || (bf16 && hd != 128) || (!bf16 && hd != 64 && hd != 128) ||
      (n_seqs > 0 && (!q_row0 || !q_len || !kv_row0 || !kv_pre_row0 || !kv_pre_len)) ||
      (block_rows != 0 && !attn_block_rows_valid(bf16, block_rows)) || (!bf16 && piece != 0) ||
      (piece > 0 && piece % 64))
    return set_error(S1_EINVAL, "s1k_attention: unsupported arguments");
  int row_lo = 0, row_hi = 0;
  for (int i = 0; i < n_seqs; ++i) {
    if (q_len[i] < 0 || kv_pre_len[i] < 0 || q_row0[i] < 0) return set_error(S1_EINVAL, "s1k_attention: negative length");
    if (q_len[i] == 0) continue;
    row_lo = row_hi > row_lo ? std::min(row_lo, q_row0[i]) : q_row0[i];
    row_hi = std::max(row_hi, q_row0[i] + q_len[i]);
  }
  std::vector<AttnSeq> seqs(n_seqs);
  for (int i = 0; i < n_seqs; ++i) seqs[i] = {q_row0[i], q_len[i], kv_row0[i], kv_pre_row0[i], kv_pre_len[i]};
  const int bq = block_rows ? block_rows : attn_block_rows(bf16, q_len, n_seqs, Hq);
  int n_cu = 256;
  int dev = 0;
  if (hipGetDevice(&dev) == hipSuccess) (void)hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
  AttnPlanHost ap;
  plan_attention(seqs.data(), n_seqs, row_lo, row_hi - row_lo, Hq, bq, piece, n_cu, &ap);
  if (ap.blocks.empty()) return S1_OK;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o_ = off;
    off += (bytes + 255) / 256 * 256;
    return o_;
  };
  const size_t o_s = take(ap.seqs.size() * sizeof(AttnSeq)), o_b = take(ap.blocks.size() * sizeof(AttnBlock));
  const size_t o_rs = take(ap.row_slot.size() * 4), o_rn = take(ap.row_np.size() * 4);
  const size_t o_c = take(ap.comb_rows.size() * 4), o_po = take((size_t)ap.slots * Hq * hd * 4);
  const size_t o_pm = take((size_t)ap.slots * Hq * 8);
  void* dm = nullptr;
  if (dev_alloc(&dm, off + 256) != hipSuccess) {
    (void)hipGetLastError();
    return set_error(S1_ENOMEM, "s1k_attention: allocation failed");
  }
  char* d = static_cast<char*>(dm);
  AttnPartials part;
  part.row_slot = reinterpret_cast<const int32_t*>(d + o_rs);
  part.row_np = reinterpret_cast<const int32_t*>(d + o_rn);
  part.row_base = row_lo;
  part.pO = reinterpret_cast<float*>(d + o_po);
  part.pML = reinterpret_cast<float2*>(d + o_pm);
  hipError_t e = hipMemcpy(d + o_s, ap.seqs.data(), ap.seqs.size() * sizeof(AttnSeq), hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemcpy(d + o_b, ap.blocks.data(), ap.blocks.size() * sizeof(AttnBlock), hipMemcpyHostToDevice);
  if (e == hipSuccess && !ap.row_slot.empty()) {
    e = hipMemcpy(d + o_rs, ap.row_slot.data(), ap.row_slot.size() * 4, hipMemcpyHostToDevice);
    if (e == hipSuccess) e = hipMemcpy(d + o_rn, ap.row_np.data(), ap.row_np.size() * 4, hipMemcpyHostToDevice);
  }
  if (e == hipSuccess && !ap.comb_rows.empty())
    e = hipMemcpy(d + o_c, ap.comb_rows.data(), ap.comb_rows.size() * 4, hipMemcpyHostToDevice);
  if (e == hipSuccess)
    e = launch_attention(bf16, q, Hq * hd, k, v, Hkv * hd, o, Hq * hd, reinterpret_cast<AttnSeq*>(d + o_s),
                         reinterpret_cast<AttnBlock*>(d + o_b), (int)ap.blocks.size(), Hq, Hkv, hd, bq, part,
                         strm(hip_stream));
  if (e == hipSuccess)
    e = launch_attn_combine(reinterpret_cast<int32_t*>(d + o_c), (int)ap.comb_rows.size(), part, o, Hq * hd, Hq,
                            strm(hip_stream));
  if (e == hipSuccess) e = hipStreamSynchronize(strm(hip_stream));
  (void)hipFree(dm);
  return dev_status(e, "s1k_attention");
}

int s1k_attention_plan(int32_t n_seqs, const int32_t* q_row0, const int32_t* q_len, const int32_t* kv_row0,
                       const int32_t* kv_pre_row0, const int32_t* kv_pre_len, int32_t Hq, int32_t block_rows,
                       int32_t piece, int32_t n_cu, int32_t max_blocks, int32_t* blocks, int32_t* n_blocks,
                       int32_t max_shared, int32_t* shared, int32_t* n_seqs_out, int32_t max_rows,
                       int32_t* row_np, int32_t* piece_out) {
  if (n_seqs < 0 || Hq < 1 || n_cu < 1 || (piece > 0 && piece % 64) || !attn_block_rows_valid(true, block_rows) ||
      (n_seqs > 0 && (!q_row0 || !q_len || !kv_row0 || !kv_pre_row0 || !kv_pre_len)) || !blocks || !n_blocks ||
      !shared || !n_seqs_out || !row_np || !piece_out)
    return set_error(S1_EINVAL, "s1k_attention_plan: bad arguments");
  int row_lo = 0, row_hi = 0;
  std::vector<AttnSeq> seqs(n_seqs);
  for (int i = 0; i < n_seqs; ++i) {
    if (q_len[i] < 0 || kv_pre_len[i] < 0 || q_row0[i] < 0) return set_error(S1_EINVAL, "s1k_attention_plan: negative length");
    seqs[i] = {q_row0[i], q_len[i], kv_row0[i], kv_pre_row0[i], kv_pre_len[i]};
    if (q_len[i] == 0) continue;
    row_lo = row_hi > row_lo ? std::min(row_lo, q_row0[i]) : q_row0[i];
    row_hi = std::max(row_hi, q_row0[i] + q_len[i]);
  }
  AttnPlanHost ap;
  plan_attention(seqs.data(), n_seqs, row_lo, row_hi - row_lo, Hq, block_rows, piece, n_cu, &ap);
  if ((int)ap.blocks.size() > max_blocks || (int)ap.seqs.size() - n_seqs > max_shared || row_hi - row_lo > max_rows)
    return set_error(S1_EINVAL, "s1k_attention_plan: capacity exceeded");
  for (size_t i = 0; i < ap.blocks.size(); ++i) {
    const AttnBlock& b = ap.blocks[i];
    const int32_t v[5] = {b.seq, b.q0, b.k_lo, b.k_hi, b.part};
    std::memcpy(blocks + 5 * i, v, sizeof(v));
  }
  *n_blocks = (int)ap.blocks.size();
  for (size_t i = n_seqs; i < ap.seqs.size(); ++i) {
    const AttnSeq& a = ap.seqs[i];
    const int32_t v[5] = {a.q_row0, a.len, a.kv_row0, a.kv_pre_row0, a.kv_pre_len};
    std::memcpy(shared + 5 * (i - n_seqs), v, sizeof(v));
  }
  *n_seqs_out = (int)ap.seqs.size();
  for (int r = 0; r < row_hi - row_lo; ++r) row_np[r] = ap.row_np[r];
  *piece_out = ap.piece;
  return S1_OK;
}

int s1k_readout(int32_t dtype, const float* x, int32_t d, const float* w_final, float eps, const void* E,
                int32_t Q, const int32_t* rows, const int32_t* opt_offsets, const int32_t* opt_ids,
                const uint8_t* q_type, float* probs, void* decisions, void* hip_stream) {
  if ((dtype != S1_BF16 && dtype != S1_F32) || d < 4 || d % 4 || Q < 0 || !x || !w_final || !E ||
      (Q > 0 && (!rows || !opt_offsets || !opt_ids || !q_type || !probs || !decisions)))
    return set_error(S1_EINVAL, "s1k_readout: unsupported arguments");
  // the LDS holds d floats plus the logits of one question (K <= 1024)
  if (d + 1024 > 16384) return set_error(S1_EINVAL, "s1k_readout: d too large");
  return dev_status(launch_readout(dtype == S1_BF16, x, d, w_final, eps, E, Q, rows, opt_offsets, opt_ids,
                                   q_type, probs, decisions, 1024, strm(hip_stream)),
                    "s1k_readout");
}

int s1k_vocab_lse(int32_t dtype, const float* x, int32_t d, const float* w_final, float eps, const void* E,
                  int32_t V, int32_t R, const int32_t* rows, float* lse, void* hip_stream) {
  const bool bf16 = dtype == S1_BF16;
  if ((dtype != S1_BF16 && dtype != S1_F32) || !feat_shape_ok(bf16, d) || V < 1 || R < 0 || !x || !w_final ||
      !E || (R > 0 && (!rows || !lse)))
    return set_error(S1_EINVAL, "s1k_vocab_lse: unsupported arguments");
  if (R == 0) return S1_OK;
  hipStream_t s = strm(hip_stream);
  const FeatWs w = feat_ws_layout(bf16, R, V, d);
  void* ws = nullptr;
  if (dev_alloc_async(&ws, w.bytes, s) != hipSuccess) {
    (void)hipGetLastError();
    return set_error(S1_ENOMEM, "s1k_vocab_lse: allocation failed");
  }
  hipError_t e = launch_feat_norm(bf16, x, d, rows, R, w_final, eps, V, ws, s);
  if (e == hipSuccess) e = launch_vocab_lse(bf16, E, V, d, R, ws, s);
  if (e == hipSuccess) e = launch_lse_merge(bf16, V, d, R, ws, s);
  if (e == hipSuccess)
    e = hipMemcpyAsync(lse, static_cast<char*>(ws) + w.lse, 4 * (size_t)R, hipMemcpyDeviceToDevice, s);
  (void)hipFreeAsync(ws, s);
  return dev_status(e, "s1k_vocab_lse");
}

int s1k_token_logprobs(int32_t dtype, const float* x, int32_t n_rows, int32_t d, const float* w_final, float eps,
                       const void* E, int32_t V, int32_t n_targets, const int32_t* rows, const int32_t* tokens,
                       int32_t n_cands, const int32_t* cand_offsets, const int32_t* cand_group, float* logp,
                       float* cand_logp, float* cand_norm, void* hip_stream) {
  const bool bf16 = dtype == S1_BF16;
  if ((dtype != S1_BF16 && dtype != S1_F32) || !feat_shape_ok(bf16, d) || V < 1 || n_rows < 0 || !x ||
      !w_final || !E || (n_targets > 0 && !logp) || (n_cands > 0 && (!cand_logp || !cand_norm)))
    return set_error(S1_EINVAL, "s1k_token_logprobs: unsupported arguments");
  FeatHost h;
  const int rc = build_features(n_rows, nullptr, V, n_targets, rows, tokens, n_cands, cand_offsets, cand_group,
                                "s1k_token_logprobs", &h);
  if (rc) return rc;
  if (n_targets == 0) return S1_OK;
  hipStream_t s = strm(hip_stream);
  const FeatWs w = feat_ws_layout(bf16, (int)h.rows.size(), V, d);
  const size_t meta = h.meta_bytes();
  void* dm = nullptr;
  if (dev_alloc(&dm, meta + w.bytes) != hipSuccess) {
    (void)hipGetLastError();
    return set_error(S1_ENOMEM, "s1k_token_logprobs: allocation failed");
  }
  FeatArgs a;
  hipError_t e = h.upload(dm, &a, s);
  if (e == hipSuccess)
    e = launch_features(bf16, x, d, w_final, eps, E, V, a, logp, cand_logp, cand_norm,
                        static_cast<char*>(dm) + meta, s);
  const hipError_t se = hipStreamSynchronize(s);
  if (e == hipSuccess) e = se;
  (void)hipFree(dm);
  return dev_status(e, "s1k_token_logprobs");
}

}  // extern "C"
